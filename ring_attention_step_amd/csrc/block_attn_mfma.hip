// Blockwise attention partial on bf16 MFMA (gfx950 / CDNA4), fp32 accumulate.
//
// One ring step of "Ring Attention" (Ultralytics glossary), section "How ring
// attention works": the resident query block against the key/value block held
// at this step, with the running maximum production kernels subtract before
// exponentiating.  Emits the block's partial (m, l, unnormalised o).
//
// Orientation.  Both products are computed transposed so that softmax state
// stays lane-local and P never leaves registers:
//     S^T[key, q] = K . Q^T     (A = K tile from LDS, B = Q held in registers)
//     O^T[d, q]  += V^T . P^T   (A = V^T read transposed from LDS, B = P from
//                                the S^T accumulators, converted to bf16)
// with v_mfma_f32_32x32x16_bf16.  For that instruction lane l supplies row
// (l % 32) of A and column (l % 32) of B, each as 8 consecutive k-elements
// starting at 8 * (l / 32); accumulator register v of lane l holds row
// 8*(v/4) + 4*(l/32) + v%4, column l % 32.  So lane l owns query l % 32: its 16
// S^T registers of a 32-key sub-tile are 16 of that query's keys, and its O^T
// registers are head_dim columns of that query's output row.  The other
// half-wave (l ^ 32) holds the remaining keys / columns of the same query,
// reached with v_permlane32_swap for the row max and the final row sum.
//
// P^T as the B operand: accumulator registers 8kk..8kk+7 of sub-tile `sub`
// hold keys 32sub + 16kk + 8(e/4) + 4h + e%4 (h = l / 32, e = 0..7), i.e. two
// runs of four consecutive keys.  ds_read_b64_tr_b16 returns to each lane of a
// 16-lane group four consecutive rows of one column of a row-major tile (lane
// i of the group gets element i%4 of the 8-byte chunk addressed by group lane
// 4k + i/4, for k = 0..3), so two such reads of the row-major V tile give each
// lane exactly its 8 V^T elements in the same key order.  V therefore stays
// in its natural layout and moves HBM -> LDS untouched.
//
// Data movement.  K and V tiles (64 keys x head_dim) are copied HBM -> LDS by
// global_load_lds_dwordx4 (no register staging), double buffered: the copy of
// tile t+1 is issued before tile t is computed, one barrier per tile.  16-byte
// chunk c of tile row r is stored at chunk position c ^ swz(r); swz permutes
// the chunk positions of 8 consecutive rows so that the K operand reads (8
// rows, one chunk) and the V^T transposed reads (4 rows, two adjacent chunks)
// hit distinct LDS banks.
//
// Online softmax.  The running maximum used as the exponent's reference is
// only moved when a row's maximum grows by more than kTau (log2 units), so the
// O rescale (one multiply per accumulator register) is rare; probabilities are
// then bounded by 2^kTau, harmless in fp32 and bf16.  The true row maximum is
// tracked separately and the partial is re-referenced to it once at the end,
// so the emitted (m, l, o) are exactly the block's partial.
//
// Work decomposition: a workgroup of WAVES waves owns 32*WAVES query rows of
// one (b, q-head); each wave owns 32 rows.  Causal masking uses the block's
// mask offset: tiles past the last visible key are never loaded, waves with no
// visible key in a tile skip it, and the element mask is applied only on
// tiles that straddle the diagonal (or the ragged end of the block).  Tiles
// are dispatched heaviest first and grouped so that one head's workgroups land
// on the same XCD (shared L2 for K/V).
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;

constexpr int kNk = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)((char*)(p)))

// Chunk-position permutation of the 8 rows r, r+1, ... (r % 8 == 0).
__device__ inline int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Combine a lane's value with lane ^ 32's (v_permlane32_swap exchanges halves).
__device__ inline float xhalf_max(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id -> logical tile id so that consecutive logical ids (one head's
// query tiles) share an XCD: the dispatcher deals workgroups round-robin over
// the 8 XCDs.  A bijection on [0, n).
__device__ inline int64_t xcd_remap(int64_t w, int64_t n) {
    const int64_t q = n / 8, r = n % 8, x = w % 8, i = w / 8;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

__device__ inline bf16x8 pack_bf16x8(const f32x16& x, int base) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const f32x2 f = {x[base + e], x[base + e + 1]};
        const bf16x2 p = __builtin_convertvector(f, bf16x2);
        r[e] = p[0];
        r[e + 1] = p[1];
    }
    return r;
}

// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at "no wait").
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16 bytes per lane HBM -> LDS (global_load_lds_dwordx4): lane l's bytes land at
// LDS byte address lds_base + 16 l.  Issued from inline assembly so that the
// compiler's wait-count pass does not treat the prefetch of the next tile as a
// hazard for reads of the current one; completion is awaited explicitly
// (wait_vmem_all) before the barrier that publishes a tile.
__device__ inline void lds_dma16(const void* src, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(src), "s"(lds_base)
        : "memory", "m0");
}

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void block_mfma_kernel(const BlockArgs a) {
    constexpr int kMq = 32 * WAVES;
    constexpr int CPR = D / 8;                 // 16-byte chunks per tile row
    constexpr int TILE_BYTES = kNk * D * 2;    // one K (or V) tile
    constexpr int INSTR = TILE_BYTES / 1024;   // 1 KiB copy instructions per tile
    constexpr int PER_WAVE = INSTR / WAVES;
    static_assert(INSTR % WAVES == 0, "tile copy must split evenly over waves");
    __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE_BYTES];  // [stage][K, V]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qi = lane & 31;
    const int half = lane >> 5;

    const int n_qt = (a.q_len + kMq - 1) / kMq;
    const int64_t n_wg = static_cast<int64_t>(n_qt) * a.Hq * a.B;
    int64_t L = xcd_remap(blockIdx.x, n_wg);
    const int qt_rank = static_cast<int>(L % n_qt);
    L /= n_qt;
    const int h = static_cast<int>(L % a.Hq);
    const int b = static_cast<int>(L / a.Hq);
    const int qt = a.causal ? (n_qt - 1 - qt_rank) : qt_rank;  // heaviest first
    const int hk = h / (a.Hq / a.Hkv);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.qs[0] + h * a.qs[1];
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.ks[0] + hk * a.ks[1];
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.vs[0] + hk * a.vs[1];

    const int r0 = qt * kMq;
    const int q0w = r0 + wave * 32;  // first query row of this wave
    const int row = q0w + qi;        // this lane's query row

    // Q as the B operand: 8 consecutive head_dim elements of this lane's row.
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
        if (row < a.q_len)
            qreg[kb] = *reinterpret_cast<const bf16x8*>(qp + row * a.qs[2] + kb * 16 + half * 8);
        else
            qreg[kb] = bf16x8{};
    }

    int key_end = a.kv_len;
    if (a.causal) key_end = min(key_end, min(a.q_len - 1, r0 + kMq - 1) + a.mask_offset + 1);
    const int n_tiles = key_end > 0 ? (key_end + kNk - 1) / kNk : 0;

    // keys this wave may see, and keys every row of this wave sees
    int wave_key_end = 0, wave_full_end = 0;
    if (q0w < a.q_len) {
        wave_key_end = a.kv_len;
        wave_full_end = a.kv_len;
        if (a.causal) {
            wave_key_end = min(a.kv_len, min(a.q_len - 1, q0w + 31) + a.mask_offset + 1);
            wave_full_end = max(0, min(a.kv_len, q0w + a.mask_offset + 1));
        }
    }

    // Copy of tile t into stage s: instruction i of this wave fills LDS chunk
    // positions [64 i', 64 i' + 64) of the K and V tiles (i' = wave-major index);
    // each lane fetches the global chunk that belongs at its position.  Rows past
    // the block re-read its last row (finite values; they are masked).
    const int64_t ks2 = a.ks[2], vs2 = a.vs[2];
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(char, smem)));
    auto issue_tile = [&](int t, int s) {
        const uint32_t kdst = lds0 + s * 2 * TILE_BYTES;
        const uint32_t vdst = kdst + TILE_BYTES;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int inst = wave * PER_WAVE + i;
            const int pos = inst * 64 + lane;
            const int r = pos / CPR;
            const int c = (pos % CPR) ^ swz(r);
            const int key = min(t * kNk + r, a.kv_len - 1);
            lds_dma16(kp + key * ks2 + c * 8, kdst + inst * 1024);
            lds_dma16(vp + key * vs2 + c * 8, vdst + inst * 1024);
        }
    };

    // per-lane LDS byte offsets of the operand reads
    const int sq = swz(qi);  // K rows sub*32 + qi share swz(qi)
    int koff[D / 16];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) koff[kb] = (qi * CPR + ((2 * kb + half) ^ sq)) * 16;
    const int j = lane & 15;                        // lane within its 16-lane group
    const int dsub = (lane >> 4) & 1;               // which 16 columns of a 32-column block
    const int vrow = 4 * half + (j >> 2);           // row within an 8-row run
    const int sv = swz(vrow);
    int voff[D / 32];
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
        voff[dblk] = (vrow * CPR + ((4 * dblk + 2 * dsub + ((j & 3) >> 1)) ^ sv)) * 16 + (j & 1) * 8;

    const float c2 = a.scale * kLog2e;  // exp(s*scale) = exp2(s*c2)
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_ref = -INFINITY;   // exponent reference (log2 units of the scaled score)
    float m_true = -INFINITY;  // running row maximum
    float l_run = 0.f;         // this lane's share of the running sum

    if (n_tiles > 0) issue_tile(0, 0);
    for (int t = 0; t < n_tiles; ++t) {
        const int kbase = t * kNk;
        wait_vmem_all();
        __syncthreads();
        if (t + 1 < n_tiles) issue_tile(t + 1, (t + 1) & 1);
        if (kbase >= wave_key_end) continue;  // nothing visible to this wave here
        const char* kst = smem + (t & 1) * 2 * TILE_BYTES;
        const char* vst = kst + TILE_BYTES;

        // S^T = K Q^T for two 32-key sub-tiles.
        f32x16 sacc[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            sacc[sub] = f32x16{};
#pragma unroll
            for (int kb = 0; kb < D / 16; ++kb) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kst + sub * 32 * CPR * 16 + koff[kb]);
                sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[kb], sacc[sub], 0, 0, 0);
            }
        }

        // scale, mask (diagonal / ragged tiles only), row max
        const bool need_mask = kbase + kNk > wave_full_end;
        float mx = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float s = sacc[sub][v] * c2;
                if (need_mask) {
                    const int key = kbase + sub * 32 + 8 * (v / 4) + 4 * half + (v % 4);
                    const bool vis = key < a.kv_len && (!a.causal || key <= row + a.mask_offset);
                    s = vis ? s : -INFINITY;
                }
                sacc[sub][v] = s;
                mx = fmaxf(mx, s);
            }
        }
        mx = xhalf_max(mx);
        m_true = fmaxf(m_true, mx);
        const bool move = mx > m_ref + kTau;
        if (__builtin_amdgcn_ballot_w64(move)) {  // rare: re-reference the running state
            const float m_new = move ? mx : m_ref;
            const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;  // 0 when m_ref = -inf
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
            m_ref = m_new;
        }
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        float ls = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(sacc[sub][v] - m_use);
                sacc[sub][v] = p;
                ls += p;
            }
        }
        l_run += ls;

        // O^T += V^T P^T over the 64 keys (4 k-blocks of 16).
        bf16x8 preg[4];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            preg[2 * sub] = pack_bf16x8(sacc[sub], 0);
            preg[2 * sub + 1] = pack_bf16x8(sacc[sub], 8);
        }
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) {
            const int run = (kb2 * 16) * CPR * 16;  // first row of this k-block's 8-row runs
#pragma unroll
            for (int dblk = 0; dblk < D / 32; ++dblk) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vst + run + voff[dblk]));
                const s16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vst + run + 8 * CPR * 16 + voff[dblk]));
                const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                const bf16x8 vop = __builtin_bit_cast(bf16x8, both);
                oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, preg[kb2], oacc[dblk], 0, 0, 0);
            }
        }
    }

    // re-reference to the true row maximum
    const float beta = (m_true == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_true);
    const float l_tot = xhalf_sum(l_run) * beta;
    if (row < a.q_len) {
        const int64_t idx = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len + row;
        float* orow = a.o + idx * D;
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 val = {oacc[dblk][4 * g] * beta, oacc[dblk][4 * g + 1] * beta,
                                   oacc[dblk][4 * g + 2] * beta, oacc[dblk][4 * g + 3] * beta};
                *reinterpret_cast<f32x4*>(orow + dblk * 32 + 8 * g + 4 * half) = val;
            }
        }
        if (half == 0) {
            a.m[idx] = (m_true == -INFINITY) ? -INFINITY : m_true * kLn2;
            a.l[idx] = l_tot;
        }
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kWaves = 8;

}  // namespace

bool mfma_eligible(const BlockArgs& a, int dtype) {
    if (dtype != 1 || (a.D != 64 && a.D != 128)) return false;
    if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.o)) return false;
    for (int i = 0; i < 3; ++i)
        if (a.qs[i] % 8 || a.ks[i] % 8 || a.vs[i] % 8) return false;
    return true;
}

hipError_t launch_block_mfma(const BlockArgs& a, hipStream_t s) {
    if (a.q_len == 0) return hipSuccess;
    constexpr int kMq = 32 * kWaves;
    const int n_qt = (a.q_len + kMq - 1) / kMq;
    const int64_t blocks = static_cast<int64_t>(n_qt) * a.Hq * a.B;
    if (a.D == 128)
        hipLaunchKernelGGL((block_mfma_kernel<128, kWaves>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kWaves),
                           0, s, a);
    else
        hipLaunchKernelGGL((block_mfma_kernel<64, kWaves>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kWaves),
                           0, s, a);
    return hipGetLastError();
}

}  // namespace ra
