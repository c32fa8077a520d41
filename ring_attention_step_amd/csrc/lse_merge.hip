// Merge of two blockwise partials with the running softmax, and finalisation.
//
// "Ring Attention" (Ultralytics glossary), section "How ring attention works":
// per-step partial results are combined with the same running softmax flash
// attention uses and the running numerator is divided by the running
// denominator at the end.  For partials (m_a, l_a, o_a) and (m_p, l_p, o_p):
//     m = max(m_a, m_p),  w_x = exp(m_x - m)  (0 when m_x = -inf),
//     l = w_a l_a + w_p l_p,  o = w_a o_a + w_p o_p,
// and finalisation gives o / l (0 when l = 0) and lse = m + ln l.
//
// Several partials (the key splits of one block) can fold in one pass, and
// the running state may be declared empty (a position's first step).
//
// HBM-bound streaming kernel.  All lanes that handle one row sit in the same
// wavefront, and every lane reads the row's (m, l) before any lane of the
// wavefront writes them back, so the in-place update of (m_acc, l_acc) is
// race-free.  Head_dim columns move as 16-byte vectors when alignment allows.
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// MAXP bounds the partials one launch folds; a two-way merge compiles with
// MAXP = 1 so it keeps the register budget of a plain streaming kernel.
template <int VEC, int MAXP>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeArgs a, int tpr) {
    const int lane = threadIdx.x & 63;
    const int rows_per_wave = 64 / tpr;
    const int64_t wave_id = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
    const int64_t row = wave_id * rows_per_wave + lane / tpr;
    const int g = lane % tpr;
    if (row >= a.rows) return;

    // running state (or empty) and the partials' weights w_x = exp(m_x - m)
    const float ma = a.acc_valid ? a.m_acc[row] : -INFINITY;
    const float la = a.acc_valid ? a.l_acc[row] : 0.f;
    const bool fold = a.o_p != nullptr;
    const int np = fold ? a.n_parts : 0;
    float m = ma;
#pragma unroll
    for (int i = 0; i < MAXP; ++i)
        if (i < np) m = fmaxf(m, a.m_p[i * a.part_ml_stride + row]);
    const float wa = (ma == -INFINITY) ? 0.f : expf(ma - m);
    float l = wa * la;
    float wp[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
        wp[i] = 0.f;
        if (i < np) {
            const float mp = a.m_p[i * a.part_ml_stride + row];
            wp[i] = (mp == -INFINITY) ? 0.f : expf(mp - m);
            l += wp[i] * a.l_p[i * a.part_ml_stride + row];
        }
    }
    const bool finalize = a.o_out != nullptr || a.lse_out != nullptr;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t base = row * a.D;
    for (int c = g * VEC; c < a.D; c += tpr * VEC) {
        float o[VEC];
        if (VEC == 4) {
            f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
            if (a.acc_valid) x = *reinterpret_cast<const f32x4*>(a.o_acc + base + c) * (fold ? wa : 1.f);
#pragma unroll
            for (int i = 0; i < MAXP; ++i)
                if (i < np) x += wp[i] * *reinterpret_cast<const f32x4*>(a.o_p + i * a.part_o_stride + base + c);
            o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
        } else {
            float x = a.acc_valid ? a.o_acc[base + c] * (fold ? wa : 1.f) : 0.f;
#pragma unroll
            for (int i = 0; i < MAXP; ++i)
                if (i < np) x += wp[i] * a.o_p[i * a.part_o_stride + base + c];
            o[0] = x;
        }
        if (finalize) {
            if (a.o_out != nullptr) {
                if (a.out_dtype == 1) {
                    __bf16* out = static_cast<__bf16*>(a.o_out) + base + c;
                    if (VEC == 4) {
                        const bf16x2 p0 = __builtin_convertvector((f32x2{o[0] * inv, o[1] * inv}), bf16x2);
                        const bf16x2 p1 = __builtin_convertvector((f32x2{o[2] * inv, o[3] * inv}), bf16x2);
                        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                        *reinterpret_cast<bf16x4*>(out) = bf16x4{p0[0], p0[1], p1[0], p1[1]};
                    } else {
                        const bf16x2 p0 = __builtin_convertvector((f32x2{o[0] * inv, 0.f}), bf16x2);
                        out[0] = p0[0];
                    }
                } else {
                    float* out = static_cast<float*>(a.o_out) + base + c;
                    if (VEC == 4)
                        *reinterpret_cast<f32x4*>(out) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
                    else
                        out[0] = o[0] * inv;
                }
            }
        } else if (fold) {
            if (VEC == 4)
                *reinterpret_cast<f32x4*>(a.o_acc + base + c) = f32x4{o[0], o[1], o[2], o[3]};
            else
                a.o_acc[base + c] = o[0];
        }
    }
    if (g == 0) {
        if (finalize) {
            if (a.lse_out != nullptr) a.lse_out[row] = l > 0.f ? m + logf(l) : -INFINITY;
        } else if (fold) {
            a.m_acc[row] = m;
            a.l_acc[row] = l;
        }
    }
}

// Finalisation knobs (measured best on gfx950, 1M rows x d 128: 6.6 TB/s):
// row groups per wave, and non-temporal loads of the fp32 state.
#ifndef RA_FIN_U
#define RA_FIN_U 2
#endif
#ifndef RA_FIN_NT
#define RA_FIN_NT 1
#endif

// Finalisation alone (no partial to fold), the last pass of the fused ring
// schedule: O / l and lse = m + ln l.  A wave covers U groups of 64 / (D / 4)
// rows, one 16-byte chunk of a row per lane, and issues all its loads before
// its first store, so each lane keeps U loads in flight; the fp32 state is
// read once, so its loads bypass the caches' retention (non-temporal).
template <int D>
__global__ __launch_bounds__(256) void finalize_kernel(const MergeArgs a) {
    constexpr int TPR = D / 4;      // lanes per row
    constexpr int RPW = 64 / TPR;   // rows per wave and group
    constexpr int U = RA_FIN_U;     // row groups per wave
    const int lane = threadIdx.x & 63;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
    const int64_t r0 = wave * (U * RPW) + lane / TPR;
    const int c = (lane % TPR) * 4;
    f32x4 x[U];
    float m[U], l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t row = r0 + u * RPW;
        if (row < a.rows) {
            if (RA_FIN_NT)
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.o_acc + row * D + c));
            else
                x[u] = *reinterpret_cast<const f32x4*>(a.o_acc + row * D + c);
            m[u] = a.m_acc[row];
            l[u] = a.l_acc[row];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t row = r0 + u * RPW;
        if (row >= a.rows) continue;
        const float inv = l[u] > 0.f ? 1.f / l[u] : 0.f;
        if (a.o_out != nullptr) {
            if (a.out_dtype == 1) {
                const bf16x2 p0 = __builtin_convertvector((f32x2{x[u][0] * inv, x[u][1] * inv}), bf16x2);
                const bf16x2 p1 = __builtin_convertvector((f32x2{x[u][2] * inv, x[u][3] * inv}), bf16x2);
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o_out) + row * D + c) =
                    bf16x4{p0[0], p0[1], p1[0], p1[1]};
            } else {
                *reinterpret_cast<f32x4*>(static_cast<float*>(a.o_out) + row * D + c) = x[u] * inv;
            }
        }
        if (c == 0 && a.lse_out != nullptr) a.lse_out[row] = l[u] > 0.f ? m[u] + logf(l[u]) : -INFINITY;
    }
}

bool aligned(const void* p, uintptr_t n) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    const bool vec = (a.D % 4 == 0) && aligned(a.o_acc, 16) && aligned(a.o_p, 16) &&
                     aligned(a.o_out, a.out_dtype == 1 ? 8 : 16) && (a.part_o_stride % 4 == 0);
    const int units = vec ? a.D / 4 : a.D;
    int tpr = 1;
    while (tpr < units && tpr < 64) tpr <<= 1;
    const int64_t rows_per_block = 256 / tpr;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;  // grid-per-rows launches: 31-bit grids
    const bool finalize_only = a.o_p == nullptr && a.acc_valid && (a.o_out != nullptr || a.lse_out != nullptr);
    if (vec && finalize_only && (a.D == 128 || a.D == 64)) {
        const int64_t rows_per_block = 4 * RA_FIN_U * (256 / a.D);  // 4 waves x U groups x 64 / (D / 4) rows
        const dim3 g(static_cast<unsigned>((a.rows + rows_per_block - 1) / rows_per_block));
        if (a.D == 128)
            hipLaunchKernelGGL(finalize_kernel<128>, g, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(finalize_kernel<64>, g, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>(blocks));
    const bool multi = a.o_p != nullptr && a.n_parts > 1;
    if (a.o_p != nullptr && (a.n_parts < 1 || a.n_parts > kMaxMergeParts)) return hipErrorInvalidValue;
    if (vec && multi)
        hipLaunchKernelGGL((lse_merge_kernel<4, kMaxMergeParts>), grid, dim3(256), 0, s, a, tpr);
    else if (vec)
        hipLaunchKernelGGL((lse_merge_kernel<4, 1>), grid, dim3(256), 0, s, a, tpr);
    else if (multi)
        hipLaunchKernelGGL((lse_merge_kernel<1, kMaxMergeParts>), grid, dim3(256), 0, s, a, tpr);
    else
        hipLaunchKernelGGL((lse_merge_kernel<1, 1>), grid, dim3(256), 0, s, a, tpr);
    return hipGetLastError();
}

}  // namespace ra
