// Blockwise attention partial on the vector ALU (fp32 arithmetic).
//
// One query block against one key/value block, as in one step of the ring of
// "Ring Attention" (Ultralytics glossary), section "How ring attention works":
// scores of the resident queries against the held keys, a running maximum
// subtracted before exponentiating, and running sums of the exponentials and
// of the exponential-weighted values.  Output is the block's partial
// (m, l, unnormalised o); ra_lse_merge combines partials.
//
// Used for binary32 inputs (the exact-parity path) and for bfloat16 inputs
// whose head_dim the MFMA kernel does not cover.  Layout of the work:
//   * a workgroup (4 waves) owns 16 consecutive query rows of one (b, h);
//   * keys are visited in chunks of KC staged through LDS by coalesced loads;
//   * per row, lane c (mod KC) scores key c, the 64/KC lane groups splitting
//     head_dim; max and sum are wavefront reductions; each lane accumulates
//     its own head_dim columns (lane, lane+64, ...) of the numerator.
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
constexpr int kMaxD = 256;
constexpr int kColsPerLane = kMaxD / 64;

template <typename T>
__device__ inline float load_as_float(const T* p, int64_t i);
template <>
__device__ inline float load_as_float<float>(const float* p, int64_t i) {
    return p[i];
}
template <>
__device__ inline float load_as_float<uint16_t>(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <typename T, int KC>
__global__ __launch_bounds__(256) void block_simt_kernel(const BlockArgs a) {
    extern __shared__ float smem[];
    const int D = a.D;
    const int kstride = D + 1;               // odd stride: lanes hit distinct banks
    float* Ks = smem;                        // [KC][D+1]
    float* Vs = Ks + KC * kstride;           // [KC][D+1]
    float* Qs = Vs + KC * kstride;           // [kRowsPerBlock][D]
    float* Ps = Qs + kRowsPerBlock * D;      // [kWaves][KC]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n_qt = (a.q_len + kRowsPerBlock - 1) / kRowsPerBlock;
    int64_t bid = blockIdx.x;
    const int qt = static_cast<int>(bid % n_qt);
    bid /= n_qt;
    const int h = static_cast<int>(bid % a.Hq);
    const int b = static_cast<int>(bid / a.Hq);
    const int hk = h / (a.Hq / a.Hkv);
    const T* q = static_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1];
    const T* k = static_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
    const T* v = static_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
    const int r0 = qt * kRowsPerBlock;

    for (int i = tid; i < kRowsPerBlock * D; i += 256) {
        const int rr = i / D, j = i % D;
        const int r = r0 + rr;
        Qs[i] = (r < a.q_len) ? load_as_float(q, static_cast<int64_t>(r) * a.qs[2] + j) : 0.f;
    }

    // keys that any row of this block may see
    const int last_row = min(a.q_len - 1, r0 + kRowsPerBlock - 1);
    int key_end = a.kv_len;
    if (a.causal) key_end = min(key_end, last_row + a.mask_offset + 1);

    float m_run[kRowsPerWave], l_run[kRowsPerWave], acc[kRowsPerWave][kColsPerLane];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        m_run[rr] = -INFINITY;
        l_run[rr] = 0.f;
#pragma unroll
        for (int t = 0; t < kColsPerLane; ++t) acc[rr][t] = 0.f;
    }

    constexpr int kParts = 64 / KC;          // lane groups sharing one key's dot product
    const int c_lane = lane % KC;
    const int part = lane / KC;
    const int dpart = (D + kParts - 1) / kParts;
    const int j0 = min(D, part * dpart), j1 = min(D, j0 + dpart);

    for (int base = 0; base < key_end; base += KC) {
        __syncthreads();
        for (int i = tid; i < KC * D; i += 256) {
            const int c = i / D, j = i % D;
            const int key = base + c;
            const bool ok = key < a.kv_len;
            Ks[c * kstride + j] = ok ? load_as_float(k, static_cast<int64_t>(key) * a.ks[2] + j) : 0.f;
            Vs[c * kstride + j] = ok ? load_as_float(v, static_cast<int64_t>(key) * a.vs[2] + j) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < kRowsPerWave; ++rr) {
            const int lr = wave * kRowsPerWave + rr;
            const int r = r0 + lr;
            if (r >= a.q_len) break;  // wave-uniform
            const float* qrow = Qs + lr * D;
            float s = 0.f;
            for (int j = j0; j < j1; ++j) s += qrow[j] * Ks[c_lane * kstride + j];
#pragma unroll
            for (int off = KC; off < 64; off <<= 1) s += __shfl_xor(s, off);
            s *= a.scale;
            const int key = base + c_lane;
            const bool vis = key < a.kv_len && (!a.causal || key <= r + a.mask_offset);
            s = vis ? s : -INFINITY;
            const float m_new = fmaxf(m_run[rr], wave_max(s));
            if (m_new == -INFINITY) continue;  // nothing visible yet (wave-uniform)
            const float alpha = expf(m_run[rr] - m_new);  // 0 while m_run is -inf
            const float p = vis ? expf(s - m_new) : 0.f;
            l_run[rr] = l_run[rr] * alpha + wave_sum(part == 0 ? p : 0.f);
            m_run[rr] = m_new;
            if (part == 0) Ps[wave * KC + c_lane] = p;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < kColsPerLane; ++t) {
                const int j = lane + 64 * t;
                if (j < D) {
                    float o = acc[rr][t] * alpha;
                    for (int c = 0; c < KC; ++c) o += Ps[wave * KC + c] * Vs[c * kstride + j];
                    acc[rr][t] = o;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }

    // Epilogue: write the partial, or (a.accumulate) merge it into the row's
    // running state (o, m, l) with the online-softmax rule of ra_lse_merge.
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int r = r0 + wave * kRowsPerWave + rr;
        if (r >= a.q_len) break;
        const int64_t idx = (static_cast<int64_t>(b) * a.Hq + h) * a.q_len + r;
        float m_out = m_run[rr], wa = 0.f, wp = 1.f, l_a = 0.f;
        if (a.accumulate) {
            const float m_a = a.m[idx];
            l_a = a.l[idx];
            m_out = fmaxf(m_a, m_run[rr]);
            wa = (m_a == -INFINITY) ? 0.f : expf(m_a - m_out);
            wp = (m_run[rr] == -INFINITY) ? 0.f : expf(m_run[rr] - m_out);
        }
#pragma unroll
        for (int t = 0; t < kColsPerLane; ++t) {
            const int j = lane + 64 * t;
            if (j < D) {
                float val = acc[rr][t] * wp;
                if (a.accumulate) val = fmaf(wa, a.o[idx * D + j], val);
                a.o[idx * D + j] = val;
            }
        }
        __builtin_amdgcn_wave_barrier();  // every lane has read (m, l) before lane 0 writes them
        if (lane == 0) {
            a.m[idx] = m_out;
            a.l[idx] = fmaf(wa, l_a, wp * l_run[rr]);
        }
    }
}

template <typename T, int KC>
hipError_t launch_t(const BlockArgs& a, hipStream_t s) {
    const int n_qt = (a.q_len + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t blocks = static_cast<int64_t>(n_qt) * a.Hq * a.B;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;  // one workgroup per query tile: 31-bit grids
    const size_t lds = sizeof(float) * (2 * KC * (a.D + 1) + kRowsPerBlock * a.D + kWaves * KC);
    hipLaunchKernelGGL((block_simt_kernel<T, KC>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_simt(const BlockArgs& a, int dtype, hipStream_t s) {
    if (a.q_len == 0) return hipSuccess;
    const bool small = a.D <= 128;
    if (dtype == 0) return small ? launch_t<float, 32>(a, s) : launch_t<float, 16>(a, s);
    return small ? launch_t<uint16_t, 32>(a, s) : launch_t<uint16_t, 16>(a, s);
}

}  // namespace ra
