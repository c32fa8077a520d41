// Backward of blockwise attention on the vector ALU (fp32 arithmetic).
//
// The pages run attention's backward pass ("Context Parallelism", Ultralytics
// glossary, section "Practical use and trade-offs": q, k, v require gradients
// and a loss is back-propagated through the causal attention).  For one query
// block against one key/value block, with the rows' full-key-set lse and
// delta = dO . O, the chain rule gives this block pair's share of the
// gradients:
//     p_rc  = exp(scale s_rc - lse_r)          (the forward's softmax weights)
//     dp_rc = dO_r . v_c
//     ds_rc = p_rc (dp_rc - delta_r)
//     dQ_r += scale sum_c ds_rc k_c
//     dK_c += scale sum_r ds_rc q_r
//     dV_c += sum_r p_rc dO_r
// over visible pairs (key c visible to row r iff c <= r + mask_offset when
// causal).  Shares of different key blocks add up to the full gradients, so a
// ring accumulates them step by step.
//
// Two kernels, neither needing atomics: dq_kernel owns query rows and loops
// over keys; dkdv_kernel owns key rows and loops over the query heads that
// share its key/value head and over their rows.  Layout of the work follows
// the forward vector-ALU kernel: four waves of four rows (keys) per
// workgroup, the other side staged through LDS in chunks, per-pair dot
// products split over lane groups, per-column accumulation in lanes.
#include <algorithm>
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr int kPerWave = 4;
constexpr int kPerBlock = kWaves * kPerWave;
constexpr int kMaxD = 256;
constexpr int kColsPerLane = kMaxD / 64;

template <typename T>
__device__ inline float ld(const T* p, int64_t i);
template <>
__device__ inline float ld<float>(const float* p, int64_t i) {
    return p[i];
}
template <>
__device__ inline float ld<uint16_t>(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// softmax weight of a visible pair; 0 for an invisible one or a row without keys
__device__ inline float weight(float s, float scale, float lse, bool vis) {
    return (vis && lse != -INFINITY) ? expf(s * scale - lse) : 0.f;
}

// --------------------------------------------------------------------- dQ
template <typename T, int KC>
__global__ __launch_bounds__(256) void dq_kernel(const BwdArgs a) {
    extern __shared__ float smem[];
    const int D = a.D;
    const int ks = D + 1;
    float* Ks = smem;                    // [KC][D+1]
    float* Vs = Ks + KC * ks;            // [KC][D+1]
    float* Qs = Vs + KC * ks;            // [kPerBlock][D]
    float* Gs = Qs + kPerBlock * D;      // [kPerBlock][D]  (dO rows)
    float* Ps = Gs + kPerBlock * D;      // [kWaves][KC]    (ds of the current row)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_qt = (a.q_len + kPerBlock - 1) / kPerBlock;
    int64_t bid = blockIdx.x;
    const int qt = static_cast<int>(bid % n_qt);
    bid /= n_qt;
    const int h = static_cast<int>(bid % a.Hq);
    const int b = static_cast<int>(bid / a.Hq);
    const int hk = h / (a.Hq / a.Hkv);
    const T* q = static_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1];
    const T* g = static_cast<const T*>(a.dout) + b * a.dos[0] + h * a.dos[1];
    const T* k = static_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
    const T* v = static_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
    const int64_t row0 = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len;
    const int r0 = qt * kPerBlock;

    for (int i = tid; i < kPerBlock * D; i += 256) {
        const int rr = i / D, j = i % D, r = r0 + rr;
        const bool ok = r < a.q_len;
        Qs[i] = ok ? ld(q, static_cast<int64_t>(r) * a.qs[2] + j) : 0.f;
        Gs[i] = ok ? ld(g, static_cast<int64_t>(r) * a.dos[2] + j) : 0.f;
    }
    float lse[kPerWave], dlt[kPerWave], acc[kPerWave][kColsPerLane];
#pragma unroll
    for (int rr = 0; rr < kPerWave; ++rr) {
        const int r = r0 + wave * kPerWave + rr;
        lse[rr] = r < a.q_len ? a.lse[row0 + r] : -INFINITY;
        dlt[rr] = r < a.q_len ? a.delta[row0 + r] : 0.f;
#pragma unroll
        for (int t = 0; t < kColsPerLane; ++t) acc[rr][t] = 0.f;
    }

    const int last_row = min(a.q_len - 1, r0 + kPerBlock - 1);
    int key_end = a.kv_len;
    if (a.causal) key_end = max(0, min(key_end, last_row + a.mask_offset + 1));

    constexpr int kParts = 64 / KC;
    const int c_lane = lane % KC, part = lane / KC;
    const int dpart = (D + kParts - 1) / kParts;
    const int j0 = min(D, part * dpart), j1 = min(D, j0 + dpart);

    for (int base = 0; base < key_end; base += KC) {
        __syncthreads();
        for (int i = tid; i < KC * D; i += 256) {
            const int c = i / D, j = i % D, key = base + c;
            const bool ok = key < a.kv_len;
            Ks[c * ks + j] = ok ? ld(k, static_cast<int64_t>(key) * a.ks[2] + j) : 0.f;
            Vs[c * ks + j] = ok ? ld(v, static_cast<int64_t>(key) * a.vs[2] + j) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < kPerWave; ++rr) {
            const int lr = wave * kPerWave + rr, r = r0 + lr;
            if (r >= a.q_len) break;  // wave-uniform
            float s = 0.f, dp = 0.f;
            for (int j = j0; j < j1; ++j) {
                s += Qs[lr * D + j] * Ks[c_lane * ks + j];
                dp += Gs[lr * D + j] * Vs[c_lane * ks + j];
            }
#pragma unroll
            for (int off = KC; off < 64; off <<= 1) {
                s += __shfl_xor(s, off);
                dp += __shfl_xor(dp, off);
            }
            const int key = base + c_lane;
            const bool vis = key < a.kv_len && (!a.causal || key <= r + a.mask_offset);
            const float p = weight(s, a.scale, lse[rr], vis);
            if (part == 0) Ps[wave * KC + c_lane] = p * (dp - dlt[rr]);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < kColsPerLane; ++t) {
                const int j = lane + 64 * t;
                if (j < D) {
                    float x = acc[rr][t];
                    for (int c = 0; c < KC; ++c) x += Ps[wave * KC + c] * Ks[c * ks + j];
                    acc[rr][t] = x;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
#pragma unroll
    for (int rr = 0; rr < kPerWave; ++rr) {
        const int r = r0 + wave * kPerWave + rr;
        if (r >= a.q_len) break;
        float* out = a.dq + (row0 + r) * D;
#pragma unroll
        for (int t = 0; t < kColsPerLane; ++t) {
            const int j = lane + 64 * t;
            if (j < D) out[j] += a.scale * acc[rr][t];
        }
    }
}

// --------------------------------------------------------------------- dK, dV
template <typename T, int QC>
__global__ __launch_bounds__(256) void dkdv_kernel(const BwdArgs a) {
    extern __shared__ float smem[];
    const int D = a.D;
    const int qs = D + 1;
    float* Qs = smem;                   // [QC][D+1]
    float* Gs = Qs + QC * qs;           // [QC][D+1]   (dO rows)
    float* Ks = Gs + QC * qs;           // [kPerBlock][D]
    float* Vs = Ks + kPerBlock * D;     // [kPerBlock][D]
    float* Ls = Vs + kPerBlock * D;     // [QC] lse
    float* Ds = Ls + QC;                // [QC] delta
    float* Ps = Ds + QC;                // [kWaves][QC] p
    float* Ss = Ps + kWaves * QC;       // [kWaves][QC] ds

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_kt = (a.kv_len + kPerBlock - 1) / kPerBlock;
    int64_t bid = blockIdx.x;
    const int kt = static_cast<int>(bid % n_kt);
    bid /= n_kt;
    const int hk = static_cast<int>(bid % a.Hkv);
    const int b = static_cast<int>(bid / a.Hkv);
    const int grp = a.Hq / a.Hkv;
    const T* k = static_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
    const T* v = static_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
    const int c0 = kt * kPerBlock;

    for (int i = tid; i < kPerBlock * D; i += 256) {
        const int cc = i / D, j = i % D, c = c0 + cc;
        const bool ok = c < a.kv_len;
        Ks[i] = ok ? ld(k, static_cast<int64_t>(c) * a.ks[2] + j) : 0.f;
        Vs[i] = ok ? ld(v, static_cast<int64_t>(c) * a.vs[2] + j) : 0.f;
    }
    float ak[kPerWave][kColsPerLane], av[kPerWave][kColsPerLane];
#pragma unroll
    for (int kk = 0; kk < kPerWave; ++kk)
#pragma unroll
        for (int t = 0; t < kColsPerLane; ++t) ak[kk][t] = av[kk][t] = 0.f;

    // rows that see some key of this block: r >= c0 - mask_offset
    const int row_start = a.causal ? max(0, min(a.q_len, c0 - a.mask_offset)) : 0;

    constexpr int kParts = 64 / QC;
    const int r_lane = lane % QC, part = lane / QC;
    const int dpart = (D + kParts - 1) / kParts;
    const int j0 = min(D, part * dpart), j1 = min(D, j0 + dpart);

    for (int hi = 0; hi < grp; ++hi) {
        const int h = hk * grp + hi;
        const T* q = static_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1];
        const T* g = static_cast<const T*>(a.dout) + b * a.dos[0] + h * a.dos[1];
        const int64_t row0 = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len;
        for (int base = row_start; base < a.q_len; base += QC) {
            __syncthreads();
            for (int i = tid; i < QC * D; i += 256) {
                const int rr = i / D, j = i % D, r = base + rr;
                const bool ok = r < a.q_len;
                Qs[rr * qs + j] = ok ? ld(q, static_cast<int64_t>(r) * a.qs[2] + j) : 0.f;
                Gs[rr * qs + j] = ok ? ld(g, static_cast<int64_t>(r) * a.dos[2] + j) : 0.f;
            }
            for (int i = tid; i < QC; i += 256) {
                const int r = base + i;
                Ls[i] = r < a.q_len ? a.lse[row0 + r] : -INFINITY;
                Ds[i] = r < a.q_len ? a.delta[row0 + r] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < kPerWave; ++kk) {
                const int lc = wave * kPerWave + kk, c = c0 + lc;
                if (c >= a.kv_len) break;  // wave-uniform
                float s = 0.f, dp = 0.f;
                for (int j = j0; j < j1; ++j) {
                    s += Qs[r_lane * qs + j] * Ks[lc * D + j];
                    dp += Gs[r_lane * qs + j] * Vs[lc * D + j];
                }
#pragma unroll
                for (int off = QC; off < 64; off <<= 1) {
                    s += __shfl_xor(s, off);
                    dp += __shfl_xor(dp, off);
                }
                const int r = base + r_lane;
                const bool vis = r < a.q_len && (!a.causal || c <= r + a.mask_offset);
                const float p = weight(s, a.scale, Ls[r_lane], vis);
                if (part == 0) {
                    Ps[wave * QC + r_lane] = p;
                    Ss[wave * QC + r_lane] = p * (dp - Ds[r_lane]);
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int t = 0; t < kColsPerLane; ++t) {
                    const int j = lane + 64 * t;
                    if (j < D) {
                        float xv = av[kk][t], xk = ak[kk][t];
                        for (int rr = 0; rr < QC; ++rr) {
                            xv += Ps[wave * QC + rr] * Gs[rr * qs + j];
                            xk += Ss[wave * QC + rr] * Qs[rr * qs + j];
                        }
                        av[kk][t] = xv;
                        ak[kk][t] = xk;
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
#pragma unroll
    for (int kk = 0; kk < kPerWave; ++kk) {
        const int c = c0 + wave * kPerWave + kk;
        if (c >= a.kv_len) break;
        const int64_t off = ((static_cast<int64_t>(b) * a.Hkv + hk) * a.kv_len + c) * D;
#pragma unroll
        for (int t = 0; t < kColsPerLane; ++t) {
            const int j = lane + 64 * t;
            if (j < D) {
                a.dk[off + j] += a.scale * ak[kk][t];
                a.dv[off + j] += av[kk][t];
            }
        }
    }
}

// --------------------------------------------------------------------- delta
template <typename T>
__global__ __launch_bounds__(256) void delta_kernel(int64_t rows, int D, const T* o, const T* g, float* delta) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    float x = 0.f;
    for (int j = lane; j < D; j += 64) x += ld(o, r * D + j) * ld(g, r * D + j);
    x = wave_sum(x);
    if (lane == 0) delta[r] = x;
}

template <typename Kern>
hipError_t launch_dyn(Kern k, int64_t blocks, size_t bytes, hipStream_t s, const BwdArgs& a) {
    if (bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(bytes));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(blocks)), dim3(256), bytes, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const BwdArgs& a, hipStream_t s) {
    const int D = a.D;
    const int64_t q_blocks = static_cast<int64_t>((a.q_len + kPerBlock - 1) / kPerBlock) * a.Hq * a.B;
    const int64_t k_blocks = static_cast<int64_t>((a.kv_len + kPerBlock - 1) / kPerBlock) * a.Hkv * a.B;
    if (q_blocks > INT32_MAX || k_blocks > INT32_MAX) return hipErrorInvalidValue;  // 31-bit grids
    hipError_t e = hipSuccess;
    if (D <= 128) {
        constexpr int C = 32;
        const size_t dq_bytes = sizeof(float) * (2 * C * (D + 1) + 2 * kPerBlock * D + kWaves * C);
        const size_t kv_bytes = sizeof(float) * (2 * C * (D + 1) + 2 * kPerBlock * D + 2 * C + 2 * kWaves * C);
        if (a.kv_len > 0) e = launch_dyn(dq_kernel<T, C>, q_blocks, dq_bytes, s, a);
        if (e == hipSuccess && a.q_len > 0) e = launch_dyn(dkdv_kernel<T, C>, k_blocks, kv_bytes, s, a);
    } else {
        constexpr int C = 16;
        const size_t dq_bytes = sizeof(float) * (2 * C * (D + 1) + 2 * kPerBlock * D + kWaves * C);
        const size_t kv_bytes = sizeof(float) * (2 * C * (D + 1) + 2 * kPerBlock * D + 2 * C + 2 * kWaves * C);
        if (a.kv_len > 0) e = launch_dyn(dq_kernel<T, C>, q_blocks, dq_bytes, s, a);
        if (e == hipSuccess && a.q_len > 0) e = launch_dyn(dkdv_kernel<T, C>, k_blocks, kv_bytes, s, a);
    }
    return e;
}

}  // namespace

hipError_t launch_block_bwd_simt(const BwdArgs& a, int dtype, hipStream_t s) {
    if (a.q_len == 0 || a.kv_len == 0) return hipSuccess;
    return dtype == 0 ? launch_typed<float>(a, s) : launch_typed<uint16_t>(a, s);
}

hipError_t launch_block_bwd(const BwdArgs& a, int dtype, int force_simt, hipStream_t s) {
    if (!force_simt && bwd_mfma_eligible(a, dtype)) return launch_block_bwd_mfma(a, s);
    return launch_block_bwd_simt(a, dtype, s);
}

namespace {
// x[0 .. n) = 0: 16-byte stores when x is 16-byte aligned, else 4-byte stores
template <bool kVec>
__global__ __launch_bounds__(256) void fill_zero_kernel(float* x, int64_t n) {
    constexpr int W = kVec ? 4 : 1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * W;
    for (int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * W; i < n; i += stride) {
        if (kVec && i + 4 <= n) {
            *reinterpret_cast<float4*>(x + i) = float4{0.f, 0.f, 0.f, 0.f};
        } else {
            for (int64_t j = i; j < i + W && j < n; ++j) x[j] = 0.f;
        }
    }
}
}  // namespace

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 1023) / 1024, 8192);
    if (reinterpret_cast<uintptr_t>(x) % 16 == 0)
        hipLaunchKernelGGL(fill_zero_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, n);
    else
        hipLaunchKernelGGL(fill_zero_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, n);
    return hipGetLastError();
}

hipError_t launch_bwd_delta(int64_t rows, int32_t D, int dtype, const void* o, const void* dout, float* delta,
                            hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int64_t blocks = (rows + 3) / 4;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;  // four rows a workgroup: 31-bit grids
    if (dtype == 0)
        hipLaunchKernelGGL(delta_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, rows, D,
                           static_cast<const float*>(o), static_cast<const float*>(dout), delta);
    else
        hipLaunchKernelGGL(delta_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, rows, D,
                           static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), delta);
    return hipGetLastError();
}

}  // namespace ra
