// Backward of blockwise attention on bf16 MFMA (gfx950 / CDNA4), fp32 accumulate.
//
// The pages run attention's backward pass ("Context Parallelism", Ultralytics
// glossary, section "Practical use and trade-offs").  For one query block
// against one key/value block, with the rows' full-key-set lse and
// delta = dO . O, this block pair's share of the gradients is
//     p = exp(scale s - lse),  ds = p (dO . v - delta),
//     dQ += scale ds K,  dK += scale ds^T Q,  dV += p^T dO
// over visible pairs.  Two kernels, no atomics:
//
// dq_kernel -- a wave owns 32 query rows, keys stream through LDS in tiles:
//     S^T[key, q]  = K . Q^T         (A: K tile, row reads;   B: Q in registers)
//     dP^T[key, q] = V . dO^T        (A: V tile, row reads;   B: dO in registers)
//     dS^T = P^T (dP^T - delta), P^T = exp2(S^T scale log2e - lse log2e)
//     dQ^T[d, q]  += K^T . dS^T      (A: K tile, transposed reads; B: dS^T from
//                                     the S^T accumulators, converted to bf16)
// dkdv_kernel -- a wave owns 32 keys, query rows of every query head of the
// key/value head's group stream through LDS in tiles:
//     S[q, key]   = Q . K^T          (A: Q tile, row reads;   B: K in registers)
//     dP[q, key]  = dO . V^T         (A: dO tile, row reads;  B: V parked in LDS
//                                     in lane order, one 16-byte read)
//     dV[key, d] += P^T . dO         (A: P^T from the S accumulators; B: dO tile,
//                                     transposed reads)
//     dK[key, d] += dS^T . Q         (A: dS^T; B: Q tile, transposed reads)
// With v_mfma_f32_32x32x16_bf16, lane l supplies row l%32 of A and column
// l%32 of B as 8 consecutive k-elements from 8(l/32); accumulator register v
// holds row 8(v/4) + 4(l/32) + v%4, column l%32.  Registers 8kk..8kk+7 of a
// 32-wide accumulator block therefore hold k-indices 16kk + 8(e/4) + 4h + e%4
// of the next product; the transposed LDS reads (ds_read_b64_tr_b16) fetch
// the other operand in exactly that order, so probabilities never leave
// registers.  Tiles are row-major in LDS with 16-byte chunk c of row r at
// chunk position c ^ swz(r) (conflict-free for both read kinds on gfx950's 64
// banks), copied HBM -> LDS by global_load_lds_dwordx4 into double buffers.
// dq_kernel runs eight waves in the forward kernel's ping-pong (two groups
// of one wave per SIMD, half a tile apart); dkdv_kernel runs eight waves
// (256 keys) that share each query tile, two per SIMD, whose MFMAs and
// vector work interleave as they fall; each wave runs a tile as one
// software-pipelined MFMA stream (operands read two MFMAs ahead) and raises
// its priority while it issues its S and dP chains, so that those win the
// SIMD's issue over the other wave's vector work.
#include <algorithm>
#include <climits>
#include <cmath>
#include <type_traits>
#include <utility>

#include "mfma_common.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace mfma;

// Waves per workgroup of each kernel (compile-time knobs; defaults measured best).
#ifndef RA_BWD_DQ_WAVES
#define RA_BWD_DQ_WAVES 8
#endif
#ifndef RA_BWD_KV_WAVES
#define RA_BWD_KV_WAVES 8
#endif
constexpr int kDqWaves = RA_BWD_DQ_WAVES;
constexpr int kKvWaves = RA_BWD_KV_WAVES;
constexpr int kTile = 64;  // keys (dq_kernel) or query rows (dkdv_kernel) per LDS tile

__device__ inline bf16x8 ld_row(const lds_char* p) { return *(const __attribute__((address_space(3))) bf16x8*)p; }

__device__ inline bf16x8 ld_tr(const lds_char* lo, const lds_char* hi) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)lo);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)hi);
    const s16x8 both = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, both);
}

#define MFMA(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16((a), (b), (c), 0, 0, 0)

#ifndef RA_BWD_XCD_REMAP
#define RA_BWD_XCD_REMAP 1
#endif
// Workgroup id -> logical tile id so that consecutive logical ids (one head's
// tiles, which stream the same operand rows) share an XCD and its L2: the
// dispatcher deals workgroups round-robin over the 8 XCDs.  A bijection on
// [0, n).
__device__ inline int64_t xcd_tile(int64_t w, int64_t n) {
    if (!RA_BWD_XCD_REMAP) return w;
    const int64_t q = n / 8, r = n % 8, x = w % 8, i = w / 8;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Per-lane LDS byte offsets of both read kinds for a tile of D-element rows.
// Row reads: lane l reads row 32 sub + (l%32), chunk 2 kb + l/32, stored at
// chunk position (2 kb + h) ^ swz(l%32) = 2 (kb ^ (swz >> 1)) + (h ^ (swz & 1)),
// i.e. a per-lane base plus 32 (kb ^ x): two registers instead of D/16.
template <int D>
struct TileReads {
    static constexpr int CPR = D / 8;  // 16-byte chunks per row
    uint32_t row_base, row_x;
    // Transposed reads: lane l reads chunk c = 4 dblk + c0 (c0 < 4) of rows
    // vrow and vrow + 8, stored at c ^ swz = 4 (dblk ^ (swz >> 2)) + (c0 ^ (swz & 3)).
    uint32_t lo_base, lo_x, hi_base, hi_x;
    __device__ void init(int lane) {
        const int qi = lane & 31, half = lane >> 5;
        const int sq = swz<D>(qi);  // rows 32 sub + qi share swz(qi)
        row_base = (qi * CPR + (half ^ (sq & 1))) * 16;
        row_x = static_cast<uint32_t>(sq >> 1);
        const int j = lane & 15, dsub = (lane >> 4) & 1;
        const int vrow = 4 * half + (j >> 2);
        const int s_lo = swz<D>(vrow), s_hi = swz<D>(vrow + 8);
        const int c0 = 2 * dsub + ((j & 3) >> 1);
        lo_base = (vrow * CPR + (c0 ^ (s_lo & 3))) * 16 + (j & 1) * 8;
        hi_base = ((vrow + 8) * CPR + (c0 ^ (s_hi & 3))) * 16 + (j & 1) * 8;
        lo_x = static_cast<uint32_t>(s_lo >> 2);
        hi_x = static_cast<uint32_t>(s_hi >> 2);
    }
    // A/B operand of 32 rows (32 sub ..) x 16 k at k-block kb
    __device__ bf16x8 rows(const lds_char* tile, int sub, int kb) const {
        return ld_row(tile + row_base + ((static_cast<uint32_t>(kb) ^ row_x) << 5) + sub * 32 * CPR * 16);
    }
    // transposed operand: 32 columns (block dblk) x 16 rows (16 kb2 ..)
    __device__ bf16x8 cols(const lds_char* tile, int kb2, int dblk) const {
        const int run = kb2 * 16 * CPR * 16;
        const uint32_t d = static_cast<uint32_t>(dblk);
        return ld_tr(tile + lo_base + ((d ^ lo_x) << 6) + run, tile + hi_base + ((d ^ hi_x) << 6) + run);
    }
};

// Tile copy plan: a tile of kTile rows x D bf16 is kTile*D*2/1024 copy
// instructions of 1 KiB (RPI = 64 lanes / CPR chunks a row), PER of them for
// each of the WAVES waves.  Instruction i of wave w fills tile rows
// (i WAVES + w) RPI + l / CPR (lane l), so the rows a lane fetches are 16 i'
// apart: they share r & 15, hence the swizzle, hence the lane's byte offset
// within a row.  A full tile then costs one per-lane offset per copy, and
// instruction i only moves the (scalar) base pointer.
template <int D, int WAVES>
struct TileCopy {
    static constexpr int CPR = D / 8;
    static constexpr int RPI = 64 / CPR;
    static constexpr int BYTES = kTile * D * 2;
    static constexpr int PER = BYTES / 1024 / WAVES;
    static_assert((WAVES * RPI) % 16 == 0, "rows a lane fetches must share the swizzle period");
    int crow0, cpos;  // this lane's first row and its chunk position
    __device__ void init(int wave, int lane) {
        crow0 = wave * RPI + lane / CPR;
        cpos = (lane % CPR) ^ swz<D>(crow0);
    }
    // The same plan with the lane index recomputed at the call (volatile, so
    // the compiler cannot hoist it and keep crow0 / cpos live through a loop
    // where registers are short).
    __device__ static TileCopy here(int wave) {
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        TileCopy c;
        c.init(wave, ln);
        return c;
    }
    // rows [r0, r0 + kTile) of src (row stride in elements); rows past n_rows
    // re-read the last row (finite values, masked later)
    __device__ void issue(const uint16_t* src, int64_t stride, int r0, int n_rows, uint32_t lds, int wave) const {
        const uint16_t* base = src + static_cast<int64_t>(r0) * stride;
        const int last = n_rows - 1 - r0;
        const uint32_t s2 = static_cast<uint32_t>(stride * 2);
        if (last >= kTile - 1) {  // whole tile inside the block
            const uint32_t o = crow0 * s2 + cpos * 16;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                lds_dma16(base + static_cast<int64_t>(i) * WAVES * RPI * stride, o, lds + (i * WAVES + wave) * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const uint32_t o = static_cast<uint32_t>(min(crow0 + i * WAVES * RPI, last)) * s2 + cpos * 16;
                lds_dma16(base, o, lds + (i * WAVES + wave) * 1024);
            }
        }
    }
};

// --------------------------------------------------------------------- dQ
// Eight waves in two groups of one wave per SIMD, half a tile apart
// ("ping-pong", as in the forward kernel): between consecutive barriers one
// group runs its MFMA stream -- dQ^T += K^T dS^T of tile t-1, then S^T and
// dP^T of tile t -- while the other computes dS of its current tile on the
// vector ALU.  K tile t is read in phases 2t..2t+3 (S^T, then dQ^T one tile
// later), V tile t in phases 2t..2t+1; K and V have three LDS buffers each.
// Group 0's stream (phase 2t) copies K(t+1) into K buffer (t+1) mod 3, whose
// last reader finished in phase 2t-1; it is awaited by the barrier ending
// phase 2t+1 and first read in phase 2t+2.  Group 1's stream (phase 2t+1)
// copies V(t+2) into V buffer (t+2) mod 3 (last read in phase 2t-1); group 1
// lets a phase's own copies stay in flight and awaits them by the barrier
// ending phase 2t+3, before their first reader in phase 2t+4.  Either way a
// copy has two phases to land.
template <int D>
__global__ __launch_bounds__(64 * kDqWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(const BwdArgs a) {
    constexpr int WAVES = kDqWaves;
    static_assert(WAVES == 8, "ping-pong needs two groups of one wave per SIMD");
    constexpr int kMq = 32 * WAVES;  // query rows per workgroup
    constexpr int SUB = kTile / 32;
    constexpr int CPR = D / 8;
    constexpr int TB = kTile * D * 2;                 // one K or V tile
    constexpr int PER_G = TB / 1024 / (WAVES / 2);    // copy instructions per wave of a group
    constexpr int RPI = 64 / CPR;
    __shared__ __attribute__((aligned(1024))) char smem[6 * TB];  // K0 K1 K2 V0 V1 V2

    const int tid = threadIdx.x, lane = tid & 63, qi = lane & 31, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave / (WAVES / 2), wslot = wave % (WAVES / 2);
    const int n_qt = (a.q_len + kMq - 1) / kMq;
    int64_t L = xcd_tile(blockIdx.x, static_cast<int64_t>(n_qt) * a.Hq * a.B);
    const int qt_rank = __builtin_amdgcn_readfirstlane(static_cast<int>(L % n_qt));
    L /= n_qt;
    const int h = __builtin_amdgcn_readfirstlane(static_cast<int>(L % a.Hq));
    const int b = __builtin_amdgcn_readfirstlane(static_cast<int>(L / a.Hq));
    const int qt = a.causal ? (n_qt - 1 - qt_rank) : qt_rank;  // heaviest first
    const int hk = h / (a.Hq / a.Hkv);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.qs[0] + h * a.qs[1];
    const uint16_t* gp = static_cast<const uint16_t*>(a.dout) + b * a.dos[0] + h * a.dos[1];
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.ks[0] + hk * a.ks[1];
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.vs[0] + hk * a.vs[1];
    const int64_t row0 = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len;

    const int r0 = qt * kMq;
    const int q0w = r0 + wave * 32;
    const int row = q0w + qi;
    const bool row_ok = row < a.q_len;

    bf16x8 qreg[D / 16], greg[D / 16];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
        qreg[kb] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + row * a.qs[2] + kb * 16 + half * 8) : bf16x8{};
        greg[kb] = row_ok ? *reinterpret_cast<const bf16x8*>(gp + row * a.dos[2] + kb * 16 + half * 8) : bf16x8{};
    }
    const float lse2 = row_ok ? a.lse[row0 + row] * kLog2e : -INFINITY;
    const float dlt = row_ok ? a.delta[row0 + row] : 0.f;
    const float c2 = a.scale * kLog2e;

    int key_end = a.kv_len;
    if (a.causal) key_end = max(0, min(key_end, min(a.q_len - 1, r0 + kMq - 1) + a.mask_offset + 1));
    const int n_tiles = (key_end + kTile - 1) / kTile;
    int wave_key_end = 0, wave_full_end = 0;
    if (q0w < a.q_len) {
        wave_key_end = wave_full_end = a.kv_len;
        if (a.causal) {
            wave_key_end = max(0, min(a.kv_len, min(a.q_len - 1, q0w + 31) + a.mask_offset + 1));
            wave_full_end = max(0, min(a.kv_len, q0w + a.mask_offset + 1));
        }
    }

    TileReads<D> rd;
    rd.init(lane);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(RA_LDS_PTR(char, smem)));
    const lds_char* lds = RA_LDS_PTR(char, smem);
    // copy plan of one group: instruction i of wave slot w covers rows crow0 + RPI i
    const int crow0 = wslot * PER_G * RPI + lane / CPR;
    const int cpos = lane % CPR;

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
    f32x16 s[SUB], dp[SUB];
    bf16x8 dsr[2 * SUB];
#pragma unroll
    for (int i = 0; i < 2 * SUB; ++i) dsr[i] = bf16x8{};

    // MFMA stream of one phase: dQ of tile tp (K buffer kbp), then S^T and dP^T
    // of tile tq (K buffer kbq, V buffer vbq), software-pipelined: each LDS
    // operand is read kPf steps ahead of its MFMA.
    constexpr int kPf = 4;
    constexpr int NDQ = (kTile / 16) * (D / 32), NSP = 2 * SUB * (D / 16), NT = NDQ + NSP;
    auto mfma_stream = [&](int kbp, int kbq, int vbq, auto&& hook) __attribute__((always_inline)) {
        const lds_char* kp_t = lds + kbp * TB;
        const lds_char* kq_t = lds + kbq * TB;
        const lds_char* vq_t = lds + (3 + vbq) * TB;  // vbq: V buffer 0..2
        auto load_op = [&](int i) __attribute__((always_inline)) -> bf16x8 {
            if (i < NDQ) return rd.cols(kp_t, i / (D / 32), i % (D / 32));
            const int j = i - NDQ, kb = j / (2 * SUB), r = j % (2 * SUB);
            return rd.rows(r < SUB ? kq_t : vq_t, r % SUB, kb);
        };
        auto run = [&](int i, const bf16x8& op) __attribute__((always_inline)) {
            if (i < NDQ) {
                const int kb2 = i / (D / 32), dblk = i % (D / 32);
                acc[dblk] = MFMA(op, dsr[kb2], acc[dblk]);
            } else {
                const int j = i - NDQ, kb = j / (2 * SUB), r = j % (2 * SUB), sub = r % SUB;
                if (r < SUB) s[sub] = MFMA(op, qreg[kb], kb == 0 ? f32x16{} : s[sub]);
                else dp[sub] = MFMA(op, greg[kb], kb == 0 ? f32x16{} : dp[sub]);
            }
        };
        bf16x8 ops[kPf];
#pragma unroll
        for (int n = 0; n < kPf; ++n) ops[n] = load_op(n);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const bf16x8 op = ops[n % kPf];
            if (n + kPf < NT) ops[n % kPf] = load_op(n + kPf);
            run(n, op);
            hook(n);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // dS of tile t from this wave's S^T, dP^T (zero where nothing is visible).
    // Masked scores become -inf before one branch-free exp2 loop.
    const float nl2 = lse2 == -INFINITY ? -INFINITY : -lse2;
    auto valu_half = [&](int t) __attribute__((always_inline)) {
        const int kbase = t * kTile;
        if (t < n_tiles && kbase < wave_key_end) {
            if (kbase + kTile > wave_full_end) {  // diagonal or ragged tile
                const int k_lim = a.kv_len - kbase - 4 * half;
                const int c_lim = a.causal ? row + a.mask_offset - kbase - 4 * half : k_lim;
#pragma unroll
                for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int j = sub * 32 + 8 * (v / 4) + (v % 4);
                        s[sub][v] = ((j < k_lim) & (j <= c_lim)) ? s[sub][v] : -INFINITY;
                    }
            }
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    s[sub][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][v], c2, nl2)) * (dp[sub][v] - dlt);
                dsr[2 * sub] = pack_bf16x8(s[sub], 0);
                dsr[2 * sub + 1] = pack_bf16x8(s[sub], 8);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2 * SUB; ++i) dsr[i] = bf16x8{};
        }
    };

    constexpr int kStep = (NT / 2) / PER_G;
    static_assert(kStep >= 1 && (NT / 2) % PER_G == 0, "copies must split the first half of the stream evenly");
    if (n_tiles > 0) {
        // finite K buffer for the dQ product of "tile -1" (dS = 0 there)
        for (int i = tid; i < TB / 16; i += 64 * WAVES)
            *(__attribute__((address_space(3))) s16x8*)(lds + 2 * TB + i * 16) = s16x8{};
        // K(0), V(0), V(1), copied by all eight waves (indices clamped to the block)
        {
            const int per = TB / 1024 / WAVES;
            for (int i = 0; i < per; ++i) {
                const int pos = (wave * per + i) * 64 + lane;
                const int cr = pos / CPR, cc = (pos % CPR) ^ swz<D>(cr);
                const uint32_t dst = (wave * per + i) * 1024;
                lds_dma16(kp, static_cast<uint32_t>(min(cr, a.kv_len - 1) * a.ks[2] * 2 + cc * 16), lds0 + dst);
                lds_dma16(vp, static_cast<uint32_t>(min(cr, a.kv_len - 1) * a.vs[2] * 2 + cc * 16),
                          lds0 + 3 * TB + dst);
                const int t1 = min(1, n_tiles - 1);
                lds_dma16(vp + static_cast<int64_t>(t1) * kTile * a.vs[2],
                          static_cast<uint32_t>(min(cr, a.kv_len - 1 - t1 * kTile) * a.vs[2] * 2 + cc * 16),
                          lds0 + 4 * TB + dst);
            }
        }
        wait_vmem_all();
        __syncthreads();
        if (group == 1) __syncthreads();
        int kb_prev = 2, kb_cur = 0;  // K buffers of tiles t-1 and t (t mod 3)
        int vb_cur = 0, vb_next2 = 2;  // V buffers of tiles t and t+2
        for (int t = 0; t <= n_tiles; ++t) {
            const int kb_next = kb_cur == 2 ? 0 : kb_cur + 1;
            // this group's copy: K(t+1) (group 0) or V(t+2) (group 1); index clamped
            const bool gk = group == 0;
            const int tc = min(t + (gk ? 1 : 2), n_tiles - 1);
            const int64_t stride = gk ? a.ks[2] : a.vs[2];
            const uint16_t* src = (gk ? kp : vp) + static_cast<int64_t>(tc) * kTile * stride;
            const uint32_t stride2 = static_cast<uint32_t>(stride * 2);
            const int last = a.kv_len - 1 - tc * kTile;
            const uint32_t dst = lds0 + (gk ? kb_next : 3 + vb_next2) * TB + wslot * PER_G * 1024;
            __builtin_amdgcn_s_setprio(1);
            mfma_stream(kb_prev, kb_cur, vb_cur, [&](int n) __attribute__((always_inline)) {
                if (n % kStep == 0 && n / kStep < PER_G) {
                    const int i = n / kStep;
                    const int crow = crow0 + RPI * i;
                    const uint32_t o = static_cast<uint32_t>(min(crow, last)) * stride2 +
                                       static_cast<uint32_t>((cpos ^ swz<D>(crow)) * 16);
                    lds_dma16(src, o, dst + i * 1024);
                }
            });
            __builtin_amdgcn_s_setprio(0);
            if (group == 1) wait_vmem_leave<PER_G>();  // the previous phase's V copies have landed
            __syncthreads();
            valu_half(t);
            if (group == 0) wait_vmem_all();
            __syncthreads();
            kb_prev = kb_cur;
            kb_cur = kb_next;
            vb_cur = vb_cur == 2 ? 0 : vb_cur + 1;
            vb_next2 = vb_next2 == 2 ? 0 : vb_next2 + 1;
        }
        if (group == 0) __syncthreads();
        wait_vmem_all();  // group 1's last copies land before the workgroup's LDS is released
    }

    if (row_ok) {
        float* out = a.dq + (row0 + row) * D;
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4* dstp = reinterpret_cast<f32x4*>(out + dblk * 32 + 8 * g + 4 * half);
                const f32x4 prev = *dstp;
                *dstp = f32x4{__builtin_fmaf(a.scale, acc[dblk][4 * g], prev[0]),
                              __builtin_fmaf(a.scale, acc[dblk][4 * g + 1], prev[1]),
                              __builtin_fmaf(a.scale, acc[dblk][4 * g + 2], prev[2]),
                              __builtin_fmaf(a.scale, acc[dblk][4 * g + 3], prev[3])};
            }
    }
}

// --------------------------------------------------------------------- dK, dV
template <int D>
__global__ __launch_bounds__(64 * kKvWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_kernel(
    const BwdArgs a) {
    constexpr int kMk = 32 * kKvWaves;  // keys per workgroup
    constexpr int QB = kTile / 32;    // 32-row query blocks per tile
    constexpr int TB = TileCopy<D, kKvWaves>::BYTES;
    constexpr int BUF = 2 * TB + 2 * kTile * 4;                     // Q, dO tiles, lse, delta
    constexpr int VW = 64 * D;                                       // one wave's V operands
    // two tile buffers, then each wave's V operands
    __shared__ __attribute__((aligned(1024))) char smem[2 * BUF + kKvWaves * VW];

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_kt = (a.kv_len + kMk - 1) / kMk;
    int64_t L = xcd_tile(blockIdx.x, static_cast<int64_t>(n_kt) * a.Hkv * a.B);
    const int kt_rank = __builtin_amdgcn_readfirstlane(static_cast<int>(L % n_kt));
    L /= n_kt;
    const int hk = __builtin_amdgcn_readfirstlane(static_cast<int>(L % a.Hkv));
    const int b = __builtin_amdgcn_readfirstlane(static_cast<int>(L / a.Hkv));
    const int kt = kt_rank;  // causal: earlier keys see more rows, so these come first
    const int grp = a.Hq / a.Hkv;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.ks[0] + hk * a.ks[1];
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.vs[0] + hk * a.vs[1];

    const int c0 = kt * kMk;
    const int c0w = c0 + wave * 32;
    const int key = c0w + (lane & 31);  // this lane's key (B operand column, accumulator column)
    const bool key_ok = key < a.kv_len;

    bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
        kreg[kb] = key_ok ? *reinterpret_cast<const bf16x8*>(kp + key * a.ks[2] + kb * 16 + half * 8) : bf16x8{};
        vreg[kb] = key_ok ? *reinterpret_cast<const bf16x8*>(vp + key * a.vs[2] + kb * 16 + half * 8) : bf16x8{};
    }
    // V operands parked in LDS in lane order (one 16-byte read per MFMA, no
    // swizzle: 64 lanes read 1 KiB contiguous), freeing their registers
    const lds_char* vlane = RA_LDS_PTR(char, smem) + 2 * BUF + wave * VW + lane * 16;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) *(__attribute__((address_space(3))) bf16x8*)(vlane + kb * 1024) = vreg[kb];
    const float c2 = a.scale * kLog2e;

    // rows that see some key of this workgroup / this wave, and rows that see all of this wave's keys
    const int row_start = a.causal ? max(0, min(a.q_len, c0 - a.mask_offset)) : 0;
    int wave_row_start = a.q_len, wave_row_full = a.q_len;
    if (c0w < a.kv_len) {
        wave_row_start = a.causal ? max(0, min(a.q_len, c0w - a.mask_offset)) : 0;
        wave_row_full = a.causal ? max(0, min(a.q_len, min(a.kv_len - 1, c0w + 31) - a.mask_offset)) : 0;
    }
    const int n_tiles = (a.q_len - row_start + kTile - 1) / kTile;

    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(RA_LDS_PTR(char, smem)));
    const lds_char* lds = RA_LDS_PTR(char, smem);

    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dk[i] = dv[i] = f32x16{};

    // one step = one query tile of one head of the group
    const int n_steps = grp * n_tiles;
    auto issue = [&](int st) __attribute__((always_inline)) {
        const int hi = st / n_tiles, t = st % n_tiles;
        const int h = hk * grp + hi;
        const int rb = row_start + t * kTile;
        const uint32_t buf = lds0 + (st & 1) * BUF;
        const auto cp = TileCopy<D, kKvWaves>::here(wave);
        cp.issue(static_cast<const uint16_t*>(a.q) + b * a.qs[0] + h * a.qs[1], a.qs[2], rb, a.q_len, buf, wave);
        cp.issue(static_cast<const uint16_t*>(a.dout) + b * a.dos[0] + h * a.dos[1], a.dos[2], rb, a.q_len,
                  buf + TB, wave);
    };
    // lse and delta of the tile's rows, copied like the tiles (rows past the
    // block re-read its last row; they are masked)
    auto stats = [&](int st) __attribute__((always_inline)) {
        const int hi = st / n_tiles, t = st % n_tiles;
        const int h = hk * grp + hi;
        const int rb = row_start + t * kTile;
        const int64_t row0 = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len;
        const uint32_t dst = lds0 + (st & 1) * BUF + 2 * TB;
        if (wave == 0) {
            // lane index recomputed here (volatile, so not hoisted and kept live
            // through the loop, where registers are short)
            int ln;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            const uint32_t o = static_cast<uint32_t>(min(rb + ln, a.q_len - 1)) * 4u;
            lds_dma4(a.lse + row0, o, dst);
            lds_dma4(a.delta + row0, o, dst + kTile * 4);
        }
    };
    if (n_steps > 0) {
        stats(0);
        issue(0);
    }
    for (int st = 0; st < n_steps; ++st) {
        wait_vmem_all();
        static_assert(kTile == 64, "one lane per row of the tile");
        if (wave == 0) {
            // wave 0 copied the tile's lse; turn it in place into the exp2
            // offset -lse log2(e), or -inf for a row whose lse is -inf (so that
            // such a row contributes nothing), before the barrier publishes it
            float* lsw = reinterpret_cast<float*>(smem + (st & 1) * BUF + 2 * TB);
            const float l = lsw[lane];
            lsw[lane] = l == -INFINITY ? -INFINITY : -l * kLog2e;
        }
        __syncthreads();
        if (st + 1 < n_steps) {
            stats(st + 1);
            issue(st + 1);
        }
        const int rb = row_start + (st % n_tiles) * kTile;
        if (rb + kTile <= wave_row_start) continue;  // no row of this tile sees this wave's keys
        // operand-read offsets from a lane index recomputed per tile (volatile:
        // not hoisted, so they are not kept live across the copies and barrier)
        TileReads<D> rd;
        {
            int ln;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            rd.init(ln);
        }
        const lds_char* qt = lds + (st & 1) * BUF;
        const lds_char* gt = qt + TB;
        const float* ls = reinterpret_cast<const float*>(smem + (st & 1) * BUF + 2 * TB);
        // edge tiles: the diagonal, the ragged end of the rows, or keys past the block
        const bool edge = rb < wave_row_full || rb + kTile > a.q_len;
        // One software-pipelined MFMA stream per tile.  For each 32-row block:
        // S = Q K^T (D/16 MFMAs), P on the vector ALU, dV += P^T dO (D/16),
        // dP = dO V^T (D/16), dS on the vector ALU, dK += dS^T Q (D/16).  P^T
        // (bf16) feeds dV at once so that the fp32 scores die before dP is
        // formed.  Every LDS operand is read kPf steps ahead of its MFMA,
        // across chain and block boundaries, with a scheduling fence per step
        // (without the read-ahead each MFMA waited for its operand).
        constexpr int NS = D / 16, NQ = 4 * NS, NT = QB * NQ, kPf = 2;
        constexpr int CS = 0, CV = 1, CP = 2, CK = 3;  // chains in stream order: S, dV, dP, dK
        struct Ops {
            bf16x8 x, y;
        };
        auto load = [&](int n) __attribute__((always_inline)) -> Ops {
            const int qb = n / NQ, c = (n % NQ) / NS, k = n % NS;
            Ops o;
            if (c == CS) {
                o.x = rd.rows(qt, qb, k);
            } else if (c == CP) {
                o.x = rd.rows(gt, qb, k);
                o.y = ld_row(vlane + k * 1024);
            } else {
                o.x = rd.cols(c == CV ? gt : qt, 2 * qb + (k & 1), k >> 1);
            }
            return o;
        };
        f32x16 s = f32x16{}, dp = f32x16{};
        bf16x8 p0 = bf16x8{}, p1 = bf16x8{}, d0 = bf16x8{}, d1 = bf16x8{};
        // the rows' exp2 offsets (nlp) and delta (dlp), read from LDS when the
        // S chain (nlp) or the dP chain (dlp) starts, so that P and dS do not
        // wait for them
        f32x4 nlp[4], dlp[4];
        auto load_stats = [&](int qb, bool delta) __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (delta) dlp[g] = *reinterpret_cast<const f32x4*>(ls + kTile + 32 * qb + 8 * g + 4 * half);
                else nlp[g] = *reinterpret_cast<const f32x4*>(ls + 32 * qb + 8 * g + 4 * half);
            }
        };
        // P; register v holds row rb + 4 half + i of the tile, with the
        // compile-time i = 32 qb + 8 (v/4) + v%4.  Mask (edge tiles only):
        // masked scores become -inf, so that their exp2 is exactly 0; a pair
        // is visible iff i < q_len - rb - 4 half and (causal)
        // i >= key - mask_offset - rb - 4 half.  Keys past the block need no
        // mask: each key's dK / dV column is its own and never stored.
        auto form_p = [&](int qb) __attribute__((always_inline)) {
            if (edge) {
                const int r_lim = a.q_len - rb - 4 * half;
                const int c_lim = a.causal ? key - a.mask_offset - rb - 4 * half : INT_MIN;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int i = 32 * qb + 8 * (v / 4) + v % 4;
                    s[v] = ((i < r_lim) & (i >= c_lim)) ? s[v] : -INFINITY;
                }
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 nl4 = nlp[g];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[4 * g + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + e], c2, nl4[e]));
            }
            p0 = pack_bf16x8(s, 0);
            p1 = pack_bf16x8(s, 8);
        };
        // dS = P (dP - delta), with P taken back from its bf16 copy
        auto form_ds = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 d4 = dlp[g];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * g + e;
                    const float pv = static_cast<float>(v < 8 ? p0[v] : p1[v - 8]);
                    dp[v] = pv * (dp[v] - d4[e]);
                }
            }
            d0 = pack_bf16x8(dp, 0);
            d1 = pack_bf16x8(dp, 8);
        };
        Ops ops[kPf];
#pragma unroll
        for (int n = 0; n < kPf; ++n) ops[n] = load(n);
        // step n of the stream, n a compile-time constant (a fold over 0 .. NT-1
        // below, so that no step is left to a runtime loop)
        auto step = [&]<int n>() __attribute__((always_inline)) {
            constexpr int qb = n / NQ, c = (n % NQ) / NS, k = n % NS;
            const Ops op = ops[n % kPf];
            if constexpr (n + kPf < NT) ops[n % kPf] = load(n + kPf);
            // a wave raises its priority for its S and dP chains, so that they
            // win the SIMD's issue over the other wave's vector work
            if constexpr ((c == CS || c == CP) && k == 0) {
                __builtin_amdgcn_s_setprio(1);
                load_stats(qb, c == CP);
            }
            if constexpr (c == CS) s = MFMA(op.x, kreg[k], k == 0 ? f32x16{} : s);
            else if constexpr (c == CV) dv[k >> 1] = MFMA((k & 1) ? p1 : p0, op.x, dv[k >> 1]);
            else if constexpr (c == CP) dp = MFMA(op.x, op.y, k == 0 ? f32x16{} : dp);
            else dk[k >> 1] = MFMA((k & 1) ? d1 : d0, op.x, dk[k >> 1]);
            if constexpr (k == NS - 1 && c == CS) {
                __builtin_amdgcn_s_setprio(0);
                form_p(qb);
            }
            if constexpr (k == NS - 1 && c == CP) {
                __builtin_amdgcn_s_setprio(0);
                form_ds(qb);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... N>(std::integer_sequence<int, N...>) __attribute__((always_inline)) {
            (step.template operator()<N>(), ...);
        }(std::make_integer_sequence<int, NT>{});
    }
    wait_vmem_all();

    // accumulator register v holds key c0w + 8(v/4) + 4 half + v%4, column d = 32 dblk + lane % 32.
    // The read-modify-write of dK and dV goes in two chunks of eight registers:
    // every load of a chunk is issued before its first store, so each chunk
    // costs one memory round trip.
    const int64_t kv0 = (static_cast<int64_t>(b) * a.Hkv + hk) * a.kv_len;
    constexpr int VC = 8;
#pragma unroll
    for (int v0 = 0; v0 < 16; v0 += VC) {
        float pk[VC][D / 32], pv[VC][D / 32];
#pragma unroll
        for (int e = 0; e < VC; ++e) {
            const int v = v0 + e, c = c0w + 8 * (v / 4) + 4 * half + (v % 4);
            if (c < a.kv_len) {
#pragma unroll
                for (int dblk = 0; dblk < D / 32; ++dblk) {
                    const int64_t o = (kv0 + c) * D + dblk * 32 + (lane & 31);
                    pk[e][dblk] = a.dk[o];
                    pv[e][dblk] = a.dv[o];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < VC; ++e) {
            const int v = v0 + e, c = c0w + 8 * (v / 4) + 4 * half + (v % 4);
            if (c < a.kv_len) {
#pragma unroll
                for (int dblk = 0; dblk < D / 32; ++dblk) {
                    const int64_t o = (kv0 + c) * D + dblk * 32 + (lane & 31);
                    a.dk[o] = __builtin_fmaf(a.scale, dk[dblk][v], pk[e][dblk]);
                    a.dv[o] = pv[e][dblk] + dv[dblk][v];
                }
            }
        }
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool bwd_mfma_eligible(const BwdArgs& a, int dtype) {
    if (dtype != 1 || (a.D != 64 && a.D != 128)) return false;
    if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.dout) || !aligned16(a.dq) ||
        !aligned16(a.dk) || !aligned16(a.dv))
        return false;
    for (int i = 0; i < 3; ++i)
        if (a.qs[i] % 8 || a.ks[i] % 8 || a.vs[i] % 8 || a.dos[i] % 8) return false;
    // per-lane copy offsets within a 64-row tile are 32-bit byte offsets
    const int64_t lim = int64_t(1) << 24;
    if (a.qs[2] >= lim || a.ks[2] >= lim || a.vs[2] >= lim || a.dos[2] >= lim) return false;
    return true;
}

namespace {
int64_t dq_workgroups(const BwdArgs& a) {
    return static_cast<int64_t>((a.q_len + 32 * kDqWaves - 1) / (32 * kDqWaves)) * a.Hq * a.B;
}
int64_t dkdv_workgroups(const BwdArgs& a) {
    return static_cast<int64_t>((a.kv_len + 32 * kKvWaves - 1) / (32 * kKvWaves)) * a.Hkv * a.B;
}
}  // namespace

int64_t bwd_mfma_min_workgroups(const BwdArgs& a) { return std::min(dq_workgroups(a), dkdv_workgroups(a)); }

hipError_t launch_block_bwd_mfma(const BwdArgs& a, hipStream_t s) {
    if (a.q_len == 0 || a.kv_len == 0) return hipSuccess;
    const int64_t qb = dq_workgroups(a);
    const int64_t kb = dkdv_workgroups(a);
    if (qb > INT32_MAX || kb > INT32_MAX) return hipErrorInvalidValue;  // one workgroup per tile: 31-bit grids
    if (a.D == 128) {
        hipLaunchKernelGGL(dq_kernel<128>, dim3(static_cast<unsigned>(qb)), dim3(64 * kDqWaves), 0, s, a);
        hipLaunchKernelGGL(dkdv_kernel<128>, dim3(static_cast<unsigned>(kb)), dim3(64 * kKvWaves), 0, s, a);
    } else {
        hipLaunchKernelGGL(dq_kernel<64>, dim3(static_cast<unsigned>(qb)), dim3(64 * kDqWaves), 0, s, a);
        hipLaunchKernelGGL(dkdv_kernel<64>, dim3(static_cast<unsigned>(kb)), dim3(64 * kKvWaves), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace ra
