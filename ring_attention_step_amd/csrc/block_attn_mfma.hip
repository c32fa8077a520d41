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
// Data movement.  K and V tiles (kNk keys x head_dim) are copied HBM -> LDS by
// global_load_lds_dwordx4 (no register staging) into separate double buffers
// for K and for V.  16-byte chunk c of tile row r is stored at chunk position
// c ^ swz(r).  gfx950's LDS serves 64 four-byte banks: swz is a bijection on
// 16 consecutive rows (so the K operand reads -- 16 rows, one chunk -- use 16
// distinct 16-byte bank groups) and gives 4 consecutive rows disjoint 4-chunk
// spans (so the V^T transposed reads -- 4 rows x 4 chunks per 32 lanes -- are
// conflict free).
//
// Online softmax.  The running maximum used as the exponent's reference is
// only moved when a row's maximum grows by more than kTau (log2 units), so the
// O rescale (one multiply per accumulator register) is rare; probabilities are
// then bounded by 2^kTau, harmless in fp32 and bf16.  The true row maximum is
// tracked separately and the partial is re-referenced to it once at the end,
// so the emitted (m, l, o) are exactly the block's partial.
//
// Work decomposition: a workgroup of WAVES (8) waves owns 32*WAVES query rows
// of one (b, q-head); each wave owns 32 rows.  Keys are visited in tiles of
// kNk.  Waves w and w + 4 share a SIMD; they form two groups run half a tile
// apart ("ping-pong"), so while one wave of a SIMD issues MFMAs (QK^T of the
// current tile, then the PV product of the previous one) the other runs its
// softmax on the vector ALU.  Each MFMA half is one software-pipelined
// stream in which every operand's LDS read is issued a few MFMAs ahead of its
// use.  Causal masking uses the block's mask offset: tiles past the
// workgroup's last visible key are never loaded, and the element mask is
// applied only on tiles that straddle the diagonal (or the ragged end of the
// block).  Tiles are taken heaviest first and grouped so that one head's
// tiles run on the same XCD (shared L2 for K/V); with work queues (the ring's
// launches) one looping workgroup per compute unit claims them, and XCDs that
// finish their share early take over the rest of the others'.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "mfma_common.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace mfma;

// Compile-time tuning knobs (defaults are the measured best on gfx950).
#ifndef RA_MFMA_NK
#define RA_MFMA_NK 128
#endif
#ifndef RA_MFMA_WAVES
#define RA_MFMA_WAVES 8
#endif
#ifndef RA_MFMA_SETPRIO
#define RA_MFMA_SETPRIO 1
#endif
#ifndef RA_MFMA_PINGPONG
#define RA_MFMA_PINGPONG 1
#endif
#ifndef RA_MFMA_PREFETCH
#define RA_MFMA_PREFETCH 3
#endif
constexpr int kNk = RA_MFMA_NK;  // keys per tile (64 or 128)
constexpr int kSub = kNk / 32;   // 32-key sub-tiles per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

// Maximum with NaN propagation (IEEE 754-2019 maximum).  Unlike fmaxf it needs
// no quieting of its operands first, and two of them fuse into one
// three-operand v_maximum3_f32.  Scores are finite or -inf, so the NaN rule
// never applies.
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum of N values as a tree of three-operand maxima: ceil((N - 1) / 2)
// instructions, depth ceil(log3 N).
template <int N>
__device__ inline float max_tree(const float* x) {
    if constexpr (N == 1) {
        return x[0];
    } else if constexpr (N == 2) {
        return vmax(x[0], x[1]);
    } else {
        constexpr int M = (N + 2) / 3;
        float y[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const int b = 3 * i;
            if (b + 2 < N) y[i] = vmax(vmax(x[b], x[b + 1]), x[b + 2]);
            else if (b + 1 < N) y[i] = vmax(x[b], x[b + 1]);
            else y[i] = x[b];
        }
        return max_tree<M>(y);
    }
}

// Combine a lane's value with lane ^ 32's (v_permlane32_swap exchanges halves).
__device__ inline float xhalf_max(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id -> logical tile id so that consecutive logical ids share an
// XCD: the dispatcher deals workgroups round-robin over the 8 XCDs.  A
// bijection on [0, n).  XCD x gets the logical ids [start(x), start(x + 1));
// when those are whole heads (hpx = Hq B / 8 of them, no key splits) they are
// ordered query tile first, head second, so that each XCD's share (one KV
// head's group under GQA, sharing its K/V in L2) runs heaviest first as a
// whole; otherwise head by head.
__device__ inline int xcd_remap(int w, int n) {
    const int q = n / 8, r = n % 8, x = w % 8, i = w / 8;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Dynamic tile order.  The dispatcher deals workgroups to the 8 XCDs round
// robin, so with one workgroup per tile every XCD runs the same share of
// tiles whatever its speed, and a launch lasts as long as its slowest XCD
// (measured: XCDs of one GPU differ by up to 13% in speed, so the fast ones
// idle for the last few percent of every launch).  With work queues the
// launch has one workgroup per compute unit, and each loops: it claims a
// tile, processes it, claims the next.  XCD x's share (the logical ids
// xcd_remap gives it, heaviest first) is a queue that its workgroups drain
// in order, so a head's tiles still share one L2; a workgroup whose own queue
// is empty takes the next tile of another XCD's queue (the lightest tiles
// left there), and one that finds all 8 queues empty is done.  A failed
// claim only ever finds a queue that stays empty, so one pass over the 8
// queues decides, and no workgroup waits for another.  Counters live in
// device memory (queue[0..7] the queue heads, queue[8] the number of
// workgroups done claiming); they are updated with device-scope vector
// atomics from one lane, and the last workgroup done claiming zeroes them for
// the next launch (no workgroup of this launch reads them any more).
// Two waves per SIMD (<= 256 registers): one wave's MFMAs overlap the other's
// softmax arithmetic.
// FULL: every key range the launch visits is a whole number of kNk-key tiles
// (no ragged last tile), so the in-stream tile copies need no row clamp.
template <int D, int WAVES, bool FULL>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void block_mfma_kernel(
    const BlockArgs a) {
    constexpr int kMq = 32 * WAVES;
    constexpr int CPR = D / 8;                 // 16-byte chunks per tile row
    constexpr int TILE_BYTES = kNk * D * 2;    // one K (or V) tile
    constexpr int INSTR = TILE_BYTES / 1024;   // 1 KiB copy instructions per tile
    constexpr int PER_WAVE = INSTR / WAVES;
    static_assert(INSTR % WAVES == 0, "tile copy must split evenly over waves");
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_BYTES];  // K0, K1, V0, V1

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int n_qt = (a.q_len + kMq - 1) / kMq;
    const int n_wg = n_qt * a.Hq * a.B * a.n_splits;  // < 2^31 (the launch grid's limit; checked by the host)
    // (64-bit divisions expand to vector code: the results are made scalar
    // again, as the copy addresses need wave-uniform bases)
    __shared__ int claimed;
    for (;;) {  // one pass per tile: a single pass without work queues
        int L;
        if (a.queue) {
            if (tid == 0) claimed = claim_tile(a.queue, n_wg);
            __syncthreads();
            const int c = __builtin_amdgcn_readfirstlane(claimed);
            __syncthreads();  // every wave has read the claim before the next one is written
            if (c < 0) break;
            L = c;
        } else {
            L = xcd_remap(static_cast<int>(blockIdx.x), n_wg);
        }
        // the lane index, read afresh in every pass (volatile, so that nothing
        // derived from it is kept live across passes, where registers are short)
        int lane;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
        const int qi = lane & 31;
        const int half = lane >> 5;
        // divisors as values of this pass (an empty volatile asm), so that the
        // divisions' reciprocals are not kept live across passes
        int d_split = a.n_splits, d_qt = n_qt, d_h = a.Hq, d_g = a.Hq / a.Hkv;
        asm volatile("" : "+s"(d_split), "+s"(d_qt), "+s"(d_h), "+s"(d_g));
        int split, qt_rank, h, b;
        if (a.n_splits == 1 && (a.Hq * a.B) % 8 == 0) {
            // every XCD's share is whole heads (hpx of them): order it query tile
            // first, head second, so that the share runs heaviest first as a whole
            int d_hpx = a.Hq * a.B / 8;
            asm volatile("" : "+s"(d_hpx));
            const int x = L / (d_qt * d_hpx), i = L - x * (d_qt * d_hpx);
            const int hb = x * d_hpx + i % d_hpx;
            split = 0;
            qt_rank = __builtin_amdgcn_readfirstlane(i / d_hpx);
            h = __builtin_amdgcn_readfirstlane(hb % d_h);
            b = __builtin_amdgcn_readfirstlane(hb / d_h);
        } else {
            split = __builtin_amdgcn_readfirstlane(static_cast<int>(L % d_split));
            L /= d_split;
            qt_rank = __builtin_amdgcn_readfirstlane(static_cast<int>(L % d_qt));
            L /= d_qt;
            h = __builtin_amdgcn_readfirstlane(static_cast<int>(L % d_h));
            b = __builtin_amdgcn_readfirstlane(static_cast<int>(L / d_h));
        }
        const int qt = a.causal ? (n_qt - 1 - qt_rank) : qt_rank;  // heaviest first
        const int hk = h / d_g;
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.qs[0] + h * a.qs[1];
        // A key split sees keys [k_lo, k_lo + kv_len) of the block as a block of
        // its own: key c' of the split is key k_lo + c', so its mask offset is
        // mask_offset - k_lo.
        const int k_lo = split * a.split_tiles * kNk;
        const int kv_len = a.n_splits > 1 ? max(0, min(a.kv_len - k_lo, a.split_tiles * kNk)) : a.kv_len;
        const int mask_offset = a.mask_offset - k_lo;
        const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.ks[0] + hk * a.ks[1] + k_lo * a.ks[2];
        const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.vs[0] + hk * a.vs[1] + k_lo * a.vs[2];

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

        int key_end = kv_len;
        if (a.causal) key_end = min(key_end, min(a.q_len - 1, r0 + kMq - 1) + mask_offset + 1);
        const int n_tiles = key_end > 0 ? (key_end + kNk - 1) / kNk : 0;

        // keys this wave may see, and keys every row of this wave sees
        int wave_key_end = 0, wave_full_end = 0;
        if (q0w < a.q_len) {
            wave_key_end = kv_len;
            wave_full_end = kv_len;
            if (a.causal) {
                wave_key_end = min(kv_len, min(a.q_len - 1, q0w + 31) + mask_offset + 1);
                wave_full_end = max(0, min(kv_len, q0w + mask_offset + 1));
            }
        }

        // Tile copies.  K tiles live in LDS buffers 0/1, V tiles in buffers 2/3.
        // Instruction i of this wave fills chunk positions [64 i', 64 i' + 64) of a
        // tile (i' = wave-major instruction index); each lane fetches the global
        // chunk that belongs at its position.  Rows past the block re-read its last
        // row (finite values; they are masked).
        const int64_t ks2 = a.ks[2], vs2 = a.vs[2];
        const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(RA_LDS_PTR(char, smem)));
        // per-lane byte offsets of this wave's copy instructions within a full tile
        uint32_t kcp[PER_WAVE], vcp[PER_WAVE];
        int crow[PER_WAVE], cchunk[PER_WAVE];
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int pos = (wave * PER_WAVE + i) * 64 + lane;
            crow[i] = pos / CPR;
            cchunk[i] = (pos % CPR) ^ swz<D>(crow[i]);
            kcp[i] = static_cast<uint32_t>(crow[i] * ks2 * 2 + cchunk[i] * 16);
            vcp[i] = static_cast<uint32_t>(crow[i] * vs2 * 2 + cchunk[i] * 16);
        }
        auto issue_copy = [&](const uint16_t* src, int64_t stride, const uint32_t* off, int t, int buf)
                              __attribute__((always_inline)) {
            const uint16_t* base = src + static_cast<int64_t>(t) * kNk * stride;
            const uint32_t dst = lds0 + buf * TILE_BYTES;
            const int last = kv_len - 1 - t * kNk;  // last valid row of this tile
            if (last >= kNk - 1) {
#pragma unroll
                for (int i = 0; i < PER_WAVE; ++i) lds_dma16(base, off[i], dst + (wave * PER_WAVE + i) * 1024);
            } else {  // ragged end of the block: rows past it re-read its last row (masked later)
#pragma unroll
                for (int i = 0; i < PER_WAVE; ++i) {
                    const uint32_t o = static_cast<uint32_t>(min(crow[i], last) * stride * 2 + cchunk[i] * 16);
                    lds_dma16(base, o, dst + (wave * PER_WAVE + i) * 1024);
                }
            }
        };
        auto issue_k = [&](int t) __attribute__((always_inline)) { issue_copy(kp, ks2, kcp, t, t & 1); };
        auto issue_v = [&](int t) __attribute__((always_inline)) { issue_copy(vp, vs2, vcp, t, 2 + (t & 1)); };
        // Ping-pong copies: group 0 copies K tiles, group 1 V tiles, each group's
        // four waves one instruction at a time from inside their MFMA stream.
        // Instruction i of wave slot w (w = wave mod WAVES/2) fills chunk
        // positions [64 (w PER_G + i), +64) of the tile: rows crow0 + RPI i.
        constexpr int PER_G = INSTR / (WAVES / 2);  // copy instructions per wave per tile
        constexpr int RPI = 64 / CPR;               // tile rows per copy instruction
        static_assert(INSTR % (WAVES / 2) == 0, "tile copy must split evenly over a wave group");
        const int wslot = wave % (WAVES / 2);
        const int crow0 = wslot * PER_G * RPI + lane / CPR;
        // The chunk a lane fetches for instruction i depends on i only through
        // swz(crow0 + RPI i), which repeats with period 4 in i (RPI is a
        // multiple of 4), so FULL copies use one of four per-lane byte offsets
        // (row crow0's) and advance the rows through the wave-uniform base
        // address: no vector arithmetic between the MFMAs.  Otherwise each
        // instruction clamps its row to the block's last one.
        constexpr int NOFF = FULL ? (PER_G < 4 ? PER_G : 4) : PER_G;
        uint32_t cc16[NOFF];
#pragma unroll
        for (int i = 0; i < NOFF; ++i) {
            cc16[i] = static_cast<uint32_t>(((lane % CPR) ^ swz<D>(crow0 + RPI * i)) * 16);
            // the tensor this wave's group copies: K for waves 0 .. WAVES/2 - 1, V for the rest
            if (FULL) cc16[i] += static_cast<uint32_t>(crow0 * (wave < WAVES / 2 ? ks2 : vs2) * 2);
        }

        // per-lane LDS byte offsets of the operand reads
        const lds_char* lds = RA_LDS_PTR(char, smem);
        const int sq = swz<D>(qi);  // K rows sub*32 + qi share swz(qi)
        uint32_t koff[D / 16];
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) koff[kb] = (qi * CPR + ((2 * kb + half) ^ sq)) * 16;
        const int j = lane & 15;                        // lane within its 16-lane group
        const int dsub = (lane >> 4) & 1;               // which 16 columns of a 32-column block
        const int vrow = 4 * half + (j >> 2);           // row within a 16-row k-block (first run)
        const int sv_lo = swz<D>(vrow), sv_hi = swz<D>(vrow + 8);
        uint32_t voff_lo[D / 32], voff_hi[D / 32];
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
            const int c = 4 * dblk + 2 * dsub + ((j & 3) >> 1);
            voff_lo[dblk] = (vrow * CPR + (c ^ sv_lo)) * 16 + (j & 1) * 8;
            voff_hi[dblk] = ((vrow + 8) * CPR + (c ^ sv_hi)) * 16 + (j & 1) * 8;
        }

        const float c2 = a.scale * kLog2e;  // exp(s*scale) = exp2(s*c2)
        f32x16 oacc[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
        float m_ref = -INFINITY;   // exponent reference (log2 units of the scaled score)
        float m_true = -INFINITY;  // running row maximum
        float l_run = 0.f;         // this lane's share of the running sum
        f32x16 sacc[kSub];         // S^T of the current tile, then its probabilities
        bf16x8 preg[2 * kSub];     // P^T operand of the tile awaiting its PV product

        auto visible = [&](int t) __attribute__((always_inline)) {
            return t >= 0 && t < n_tiles && t * kNk < wave_key_end;
        };

        // mask, row max, reference move, exponentials, row sum, bf16 P^T.
        auto softmax = [&](int t) __attribute__((always_inline)) {
            const int kbase = t * kNk;
            // mask (diagonal / ragged tiles only) and row max, on the raw scores:
            // the scale is positive, so it is applied once, to the maximum.
            if (kbase + kNk > wave_full_end) {
#pragma unroll
                for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = kbase + sub * 32 + 8 * (v / 4) + 4 * half + (v % 4);
                        const bool vis = key < kv_len && (!a.causal || key <= row + mask_offset);
                        sacc[sub][v] = vis ? sacc[sub][v] : -INFINITY;
                    }
                }
            }
            // row max: this lane's 16 kSub scores, then the other half-wave's
            float mt[16 * kSub];
#pragma unroll
            for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
                for (int v = 0; v < 16; ++v) mt[16 * sub + v] = sacc[sub][v];
            const float mx = xhalf_max(max_tree<16 * kSub>(mt)) * c2;
            m_true = vmax(m_true, mx);
            const bool move = mx > m_ref + kTau;
            if (__builtin_amdgcn_ballot_w64(move)) {  // rare: re-reference the running state
                const float m_new = move ? mx : m_ref;
                const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;  // 0 when m_ref = -inf
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
                m_ref = m_new;
            }
            const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
            float ls[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums
#pragma unroll
            for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sub][v], c2, neg_m));
                    sacc[sub][v] = p;
                    ls[v & 3] += p;
                }
            }
            l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
            for (int sub = 0; sub < kSub; ++sub) {
                preg[2 * sub] = pack_bf16x8(sacc[sub], 0);
                preg[2 * sub + 1] = pack_bf16x8(sacc[sub], 8);
            }
        };

        // One MFMA half as a software-pipelined operand stream: the QK^T MFMAs of
        // tile tq (kb-major, sub-tile-minor) then the PV MFMAs of tile tp
        // (O^T += V^T P^T, 4-k-block x dblk order).  Each operand's LDS read is
        // issued kPf steps before its MFMA, and a scheduling fence after every step
        // keeps that distance, so LDS latency hides behind the MFMAs in flight.
        constexpr int kPf = RA_MFMA_PREFETCH;
        constexpr int NPV = 2 * kSub * (D / 32), NQK = kSub * (D / 16), NT = NPV + NQK;
        bf16x8 ops[kPf];  // operands in flight (the first ones may be issued before a barrier)
        auto load_op_at = [&](const lds_char* vst, const lds_char* kst, int i)
                              __attribute__((always_inline)) -> bf16x8 {
            if (i < NPV) {
                const int kb2 = i / (D / 32), dblk = i % (D / 32);
                const int run = (kb2 * 16) * CPR * 16;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(vst + voff_lo[dblk] + run));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(vst + voff_hi[dblk] + run));
                const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                return __builtin_bit_cast(bf16x8, both);
            }
            const int jq = i - NPV, kb = jq / kSub, sub = jq % kSub;
            return *(const __attribute__((address_space(3))) bf16x8*)(kst + koff[kb] + sub * 32 * CPR * 16);
        };
        // the first kPf operands of a full stream for tile tq (QK^T reads of K(tq))
        auto preload = [&](int tq) __attribute__((always_inline)) {
            const lds_char* kst = lds + (tq & 1) * TILE_BYTES;
#pragma unroll
            for (int n = 0; n < kPf; ++n) ops[n] = load_op_at(nullptr, kst, NPV + n);
        };
        auto mfma_stream = [&]<bool PV, bool QK, bool PRE = false>(int tp, int tq, auto&& hook)
                               __attribute__((always_inline)) {
            constexpr int I0 = PV ? 0 : NPV, I1 = QK ? NT : NPV, N = I1 - I0;
            const lds_char* vst = lds + (2 + (tp & 1)) * TILE_BYTES;
            const lds_char* kst = lds + (tq & 1) * TILE_BYTES;
            auto load_op = [&](int i) __attribute__((always_inline)) -> bf16x8 { return load_op_at(vst, kst, i); };
            auto run_mfma = [&](int i, const bf16x8& op) __attribute__((always_inline)) {
                if (i < NPV) {
                    const int kb2 = i / (D / 32), dblk = i % (D / 32);
                    oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, preg[kb2], oacc[dblk], 0, 0, 0);
                } else {
                    const int jq = i - NPV, kb = jq / kSub, sub = jq % kSub;
                    sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qreg[kb], kb == 0 ? f32x16{} : sacc[sub], 0,
                                                                         0, 0);
                }
            };
            // step n -> operand index: QK^T first, then PV, so that the scores the
            // wave's next softmax half reads are complete when the stream ends
            // (only PV results, not needed until the next MFMA half, drain then)
            auto idx = [&](int n) __attribute__((always_inline)) {
                if constexpr (PV && QK) return n < NQK ? NPV + n : n - NQK;
                else return I0 + n;
            };
            if constexpr (!PRE) {
#pragma unroll
                for (int n = 0; n < kPf && n < N; ++n) ops[n] = load_op(idx(n));
            }
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const bf16x8 op = ops[n % kPf];
                if (n + kPf < N) ops[n % kPf] = load_op(idx(n + kPf));
                run_mfma(idx(n), op);
                hook(n);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto no_hook = [](int) __attribute__((always_inline)) {};

#if RA_MFMA_PINGPONG
        // Two groups of WAVES/2 waves (one wave per SIMD each), half a tile apart.
        // Between consecutive barriers one group runs MFMAs (QK^T of tile t, then
        // PV of tile t-1) while the other runs the softmax of its current tile, so
        // each SIMD's matrix core and vector ALU work at the same time.  K(t+1)
        // and V(t) are copied during iteration t and published by its final
        // barrier; a buffer is refilled only after the barrier that ends its last
        // reader's phase.
        static_assert(WAVES % 8 == 0, "ping-pong needs two groups of one wave per SIMD");
        const int group = wave / (WAVES / 2);
        // The MFMA half runs the full stream even for a tile this wave cannot see:
        // P is then zero (valu_half) and the V tile holds finite block values, so
        // the PV product adds exactly zero, and scores of an unseen tile are never
        // read.  A group's phase lasts as long as its slowest wave, so skipping
        // would not shorten it.  Only the first MFMA half (no PV product yet) and
        // the one after the last tile (no QK^T, no copies) are shortened.
        // Copies.  Group 0's MFMA half of tile t (global phase 2t) copies K(t+1);
        // group 1's (phase 2t+1) copies V(t).  Both buffers' last readers
        // finished in phase 2t-1, each group awaits its copies at the end of its
        // own MFMA half (K(t+1) is published at the end of phase 2t, V(t) at the
        // end of phase 2t+1), and neither tile is read before phase 2t+2 -- except
        // the first operands of the next MFMA stream, which each wave reads from
        // K(t+1) at the end of its softmax half of tile t (phases 2t+1 and 2t+2),
        // before the barrier, so that their LDS latency is not exposed at the
        // start of the stream.  Each wave issues its
        // PER_G instructions one every kStep MFMA steps over the first half of its
        // stream, so no wave stalls on a full memory-request queue.  Everything
        // group-dependent is wave-uniform and selected, not branched on, so both
        // groups run one MFMA stream.  A tile index past the block copies the last
        // tile instead (into a buffer no one reads any more; awaited like the
        // others), and rows past the block re-read its last row.
        constexpr int kStep = (NT / 2) / PER_G;
        static_assert(kStep >= 1 && (NT / 2) % PER_G == 0, "copies must split the first half of the stream evenly");
        auto mfma_half = [&]<bool PV, bool QK, bool PRE = false>(int t) __attribute__((always_inline)) {
            const bool gk = group == 0;
            const int tt = gk ? t + 1 : t;
            const int tc = min(tt, n_tiles - 1);
            const int64_t stride = gk ? ks2 : vs2;
            const uint16_t* src = (gk ? kp : vp) + static_cast<int64_t>(tc) * kNk * stride;
            const uint32_t stride2 = static_cast<uint32_t>(stride * 2);
            const int last = kv_len - 1 - tc * kNk;  // last row of the block within tile tc
            const uint32_t dst = lds0 + (gk ? (tt & 1) : 2 + (tt & 1)) * TILE_BYTES + wslot * PER_G * 1024;
            if (RA_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(1);
            mfma_stream.template operator()<PV, QK, PRE>(t - 1, t, [&](int n) __attribute__((always_inline)) {
                if (QK && n % kStep == 0 && n / kStep < PER_G) {
                    const int i = n / kStep;
                    if constexpr (FULL) {
                        lds_dma16(src + static_cast<int64_t>(RPI * i) * stride, cc16[i % NOFF], dst + i * 1024);
                    } else {
                        const uint32_t o = static_cast<uint32_t>(min(crow0 + RPI * i, last)) * stride2 + cc16[i];
                        lds_dma16(src, o, dst + i * 1024);
                    }
                }
            });
            if (RA_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(0);
        };
        auto valu_half = [&](int t) __attribute__((always_inline)) {
            if (visible(t)) {
                softmax(t);
            } else {
#pragma unroll
                for (int i = 0; i < 2 * kSub; ++i) preg[i] = bf16x8{};
            }
        };
        // Both groups run the same loop body -- MFMA half of tile t, barrier,
        // softmax half of tile t, barrier -- but group 1 first passes one extra
        // barrier (and group 0 one after its final PV half), so group 1 runs one
        // phase behind and both groups pass the same number of barriers.
        // Global phase 2t carries group 0's MFMA half of tile t and group 1's
        // softmax half of tile t-1; phase 2t+1 the other way round.
        // barrier with no wait for outstanding LDS reads (the first operands of
        // the next MFMA stream, read from a tile published one phase earlier); the
        // memory clobber keeps the compiler from moving accesses across it
        auto barrier = []() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
        if (n_tiles > 0) {
            issue_k(0);
            wait_vmem_all();
            __syncthreads();
            if (group == 1) barrier();
            // first tile: no PV product yet
            mfma_half.template operator()<false, true>(0);
            wait_vmem_all();
            barrier();
            valu_half(0);
            if (1 < n_tiles) preload(1);
            barrier();
            for (int t = 1; t < n_tiles; ++t) {
                mfma_half.template operator()<true, true, true>(t);
                wait_vmem_all();
                barrier();
                valu_half(t);
                if (t + 1 < n_tiles) preload(t + 1);
                barrier();
            }
            // PV product of the last tile (no copies).  Group 0 then passes the
            // barrier that ends group 1's last softmax half; group 1 runs its
            // final PV half with no barrier after it, while group 0 writes out.
            mfma_half.template operator()<true, false>(n_tiles);
            if (group == 0) barrier();
        }
#else
        if (n_tiles > 0) {
            issue_k(0);
            issue_v(0);
        }
        for (int t = 0; t < n_tiles; ++t) {
            wait_vmem_all();
            __syncthreads();
            if (t + 1 < n_tiles) {
                issue_k(t + 1);
                issue_v(t + 1);
            }
            if (!visible(t)) continue;  // nothing visible to this wave here
            mfma_stream.template operator()<false, true>(t, t, no_hook);
            softmax(t);
            mfma_stream.template operator()<true, false>(t, t, no_hook);
        }
#endif

        // Epilogue.  The partial (oacc, l_run) is referenced to exp2(m_ref); its
        // row maximum is m_true.  Written as is (re-referenced to m_true), or --
        // with a.accumulate -- merged into the running state (o, m, l) of the row
        // with the same online-softmax rule as ra_lse_merge:
        //   m = max(m_a, m_p);  w_x = exp(m_x - m) (0 if m_x = -inf).
        const float l_ref = xhalf_sum(l_run);
        if (row < a.q_len) {
            const int64_t idx = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len + row;
            float* const mrow = a.m + split * a.part_ml_stride;
            float* const lrow = a.l + split * a.part_ml_stride;
            float* orow = a.o + split * a.part_o_stride + idx * D;
            float m_out = m_true;  // log2 units
            float wa = 0.f, l_a = 0.f;
            float wp = (m_true == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_true);
            f32x4* const dst = reinterpret_cast<f32x4*>(orow + 4 * half);  // + (8 dblk + 2 g) vectors
            if (a.accumulate) {
                // every load of the running state is issued before the first store,
                // so the row's read-modify-write costs one memory round trip
                const float m_a = mrow[idx] * kLog2e;  // -inf stays -inf
                l_a = lrow[idx];
                f32x4 prev[D / 32][4];
#pragma unroll
                for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
                    for (int g = 0; g < 4; ++g) prev[dblk][g] = dst[8 * dblk + 2 * g];
                m_out = fmaxf(m_a, m_true);
                wa = (m_a == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_a - m_out);
                wp = (m_true == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_out);
#pragma unroll
                for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 pv = prev[dblk][g];
                        dst[8 * dblk + 2 * g] = f32x4{__builtin_fmaf(wa, pv[0], oacc[dblk][4 * g] * wp),
                                                      __builtin_fmaf(wa, pv[1], oacc[dblk][4 * g + 1] * wp),
                                                      __builtin_fmaf(wa, pv[2], oacc[dblk][4 * g + 2] * wp),
                                                      __builtin_fmaf(wa, pv[3], oacc[dblk][4 * g + 3] * wp)};
                    }
            } else {
#pragma unroll
                for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        dst[8 * dblk + 2 * g] = f32x4{oacc[dblk][4 * g] * wp, oacc[dblk][4 * g + 1] * wp,
                                                      oacc[dblk][4 * g + 2] * wp, oacc[dblk][4 * g + 3] * wp};
            }
            if (half == 0) {
                mrow[idx] = (m_out == -INFINITY) ? -INFINITY : m_out * kLn2;
                lrow[idx] = __builtin_fmaf(wa, l_a, wp * l_ref);
            }
        }
        if (!a.queue) break;
    }  // tile loop
    if (a.queue && tid == 0) finish_claims(a.queue, gridDim.x);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kWaves = RA_MFMA_WAVES;

}  // namespace

// Compute units of the current device (cached per device id).
int compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}


bool mfma_eligible(const BlockArgs& a, int dtype) {
    if (dtype != 1 || (a.D != 64 && a.D != 128)) return false;
    if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.o)) return false;
    for (int i = 0; i < 3; ++i)
        if (a.qs[i] % 8 || a.ks[i] % 8 || a.vs[i] % 8) return false;
    // the tile copies address key/value rows by 32-bit per-lane byte offsets
    // from the tile's base: row (< kNk) x row stride x 2 bytes must fit
    const int64_t lim = int64_t(1) << 24;
    if (a.ks[2] >= lim || a.vs[2] >= lim) return false;
    return true;
}

int mfma_key_tile() { return kNk; }
int mfma_query_tile() { return 32 * kWaves; }

hipError_t launch_block_mfma(const BlockArgs& a, hipStream_t s) {
    if (a.q_len == 0) return hipSuccess;
    constexpr int kMq = 32 * kWaves;
    const int n_qt = (a.q_len + kMq - 1) / kMq;
    if (a.n_splits < 1 || (a.n_splits > 1 && (a.accumulate || a.split_tiles < 1))) return hipErrorInvalidValue;
    int64_t blocks = static_cast<int64_t>(n_qt) * a.Hq * a.B * a.n_splits;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;  // tile ids are 32-bit
    if (a.queue) blocks = std::min<int64_t>(blocks, compute_units());  // one looping workgroup per CU
    // whole tiles only (every key range a multiple of kNk keys): copies without row clamps
    // (key splits cut at tile boundaries, so their ranges are whole tiles too)
    const bool full = a.kv_len % kNk == 0;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWaves);
    if (a.D == 128) {
        if (full) hipLaunchKernelGGL((block_mfma_kernel<128, kWaves, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((block_mfma_kernel<128, kWaves, false>), grid, block, 0, s, a);
    } else {
        if (full) hipLaunchKernelGGL((block_mfma_kernel<64, kWaves, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((block_mfma_kernel<64, kWaves, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace ra
