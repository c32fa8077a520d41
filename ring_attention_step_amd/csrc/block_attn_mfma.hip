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
//     O^T[d, q]  += V^T . P^T   (A = V^T tile from LDS, B = P from the S^T
//                                accumulators, converted to bf16)
// with v_mfma_f32_32x32x16_bf16.  For that instruction lane l supplies row
// (l % 32) of A and column (l % 32) of B, each as 8 consecutive k-elements
// starting at 8 * (l / 32); accumulator register v of lane l holds row
// 8*(v/4) + 4*(l/32) + v%4, column l % 32.  So lane l owns query l % 32: its
// 16 S^T registers of a 32-key sub-tile are 16 of that query's keys, and its
// O^T registers are head_dim columns of that query's output row.  The other
// half-wave (l ^ 32) holds the remaining keys / columns of the same query,
// reached with v_permlane32_swap for the row max and the final row sum.
//
// Feeding P^T as the B operand of the PV product needs each lane's 8 k-values
// (keys) to match the 8 accumulator registers it already has: registers
// 8kk..8kk+7 of sub-tile `sub` hold keys 32sub + 16kk + 8(e/4) + 4h + e%4.
// V^T is therefore staged with its key columns permuted by swapping bits 2
// and 3 of the in-tile key index (slot = swap23(key)), which makes every A
// operand read of V^T one contiguous 16-byte LDS load.
//
// Work decomposition: a workgroup of 4 waves owns 128 query rows of one
// (b, q-head); each wave owns 32 rows.  Keys are visited in tiles of 64.
// Causal masking uses the block's mask offset: tiles past the last visible key
// are never loaded, waves with no visible key in a tile skip it, and the
// element mask is applied only on tiles that straddle the diagonal (or the
// ragged end of the block).  Tiles are dispatched heaviest first and grouped so
// that workgroups of one head land on the same XCD (shared L2 for K/V).
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kMq = 128;       // query rows per workgroup
constexpr int kNk = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Swap bits 2 and 3 of an in-tile key index (an involution).
__device__ inline int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

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

template <int D>
__global__ __launch_bounds__(kThreads) void block_mfma_kernel(const BlockArgs a) {
    constexpr int KSTR = D + 8;    // K tile row stride in LDS (bf16), 16-byte pad
    constexpr int VSTR = kNk + 8;  // V^T tile row stride in LDS (bf16), 16-byte pad
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kNk * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

    const float c2 = a.scale * kLog2e;  // exp(s*scale) = exp2(s*c2)
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;  // running max, log2 units of the scaled score
    float l_run = 0.f;        // this lane's share of the running sum

    for (int t = 0; t < n_tiles; ++t) {
        const int kbase = t * kNk;
        __syncthreads();
        // K tile -> LDS, row-major: coalesced 16-byte loads and stores.
        for (int c = tid; c < kNk * D / 8; c += kThreads) {
            const int kr = c / (D / 8), kc = c % (D / 8);
            const int key = kbase + kr;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (key < a.kv_len)
                val = *reinterpret_cast<const u32x4*>(kp + static_cast<int64_t>(key) * a.ks[2] + kc * 8);
            *reinterpret_cast<u32x4*>(Ks + kr * KSTR + kc * 8) = val;
        }
        // V tile -> LDS transposed, key columns in swap23 order.  Each item is
        // 4 keys x 8 head_dim elements: 4 coalesced 16-byte loads, a register
        // transpose, 8 8-byte stores.
        for (int it = tid; it < (D / 8) * (kNk / 4); it += kThreads) {
            const int dg = it / (kNk / 4), kg = it % (kNk / 4);
            u32x4 r4[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = kbase + 4 * kg + rr;
                r4[rr] = u32x4{0u, 0u, 0u, 0u};
                if (key < a.kv_len)
                    r4[rr] = *reinterpret_cast<const u32x4*>(vp + static_cast<int64_t>(key) * a.vs[2] + dg * 8);
            }
            const int slot = swap23(4 * kg);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const u32x2 lo = {(r4[0][x] & 0xFFFFu) | (r4[1][x] << 16),
                                  (r4[2][x] & 0xFFFFu) | (r4[3][x] << 16)};
                const u32x2 hi = {(r4[0][x] >> 16) | (r4[1][x] & 0xFFFF0000u),
                                  (r4[2][x] >> 16) | (r4[3][x] & 0xFFFF0000u)};
                *reinterpret_cast<u32x2*>(Vt + (8 * dg + 2 * x) * VSTR + slot) = lo;
                *reinterpret_cast<u32x2*>(Vt + (8 * dg + 2 * x + 1) * VSTR + slot) = hi;
            }
        }
        __syncthreads();
        if (kbase >= wave_key_end) continue;  // nothing visible to this wave here

        // S^T = K Q^T for two 32-key sub-tiles.
        f32x16 sacc[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            sacc[sub] = f32x16{};
#pragma unroll
            for (int kb = 0; kb < D / 16; ++kb) {
                const bf16x8 kop =
                    *reinterpret_cast<const bf16x8*>(Ks + (sub * 32 + qi) * KSTR + kb * 16 + half * 8);
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
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
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
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;

        // O^T += V^T P^T over the 64 keys (4 k-blocks of 16).
        bf16x8 preg[4];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            preg[2 * sub] = pack_bf16x8(sacc[sub], 0);
            preg[2 * sub + 1] = pack_bf16x8(sacc[sub], 8);
        }
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) {
                const bf16x8 vop =
                    *reinterpret_cast<const bf16x8*>(Vt + (dblk * 32 + qi) * VSTR + kb2 * 16 + half * 8);
                oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, preg[kb2], oacc[dblk], 0, 0, 0);
            }
        }
    }

    const float l_tot = xhalf_sum(l_run);
    if (row < a.q_len) {
        const int64_t idx = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len + row;
        float* orow = a.o + idx * D;
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 val = {oacc[dblk][4 * g], oacc[dblk][4 * g + 1], oacc[dblk][4 * g + 2],
                                   oacc[dblk][4 * g + 3]};
                *reinterpret_cast<f32x4*>(orow + dblk * 32 + 8 * g + 4 * half) = val;
            }
        }
        if (half == 0) {
            a.m[idx] = (m_run == -INFINITY) ? -INFINITY : m_run * kLn2;
            a.l[idx] = l_tot;
        }
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
    const int n_qt = (a.q_len + kMq - 1) / kMq;
    const int64_t blocks = static_cast<int64_t>(n_qt) * a.Hq * a.B;
    if (a.D == 128)
        hipLaunchKernelGGL(block_mfma_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(block_mfma_kernel<64>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ra
