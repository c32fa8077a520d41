// Shard layout of the ring: contiguous chunks or striped (round-robin) tokens.
//
// "Ring Attention" (Ultralytics glossary), section "How ring attention works":
// the sequence is cut into N blocks, one per ring position; for causal
// attention the striped layout instead gives each position tokens spread
// evenly along the sequence.  Token t of a length-S sequence (Sb = S / N):
//     contiguous: position t / Sb, local row t % Sb
//     striped:    position t % N,  local row t / N
// Forward: [BH, S, row] -> [N, BH, Sb, row]; inverse the other way.  A row is
// one token's head_dim elements and moves as a unit (pure copy, bit-exact).
//
// HBM-bound: each thread moves 16 bytes (or 4 / 2 when the row size or
// alignment does not allow it); output addresses are consecutive across
// threads, input rows are whole, contiguous runs.
#include "ra_internal.h"

namespace ra {
namespace {

template <typename V, typename I>
__global__ __launch_bounds__(256) void permute_kernel(int striped, int inverse, I BH, I S, I N, I vpr,
                                                       const V* __restrict__ x, V* __restrict__ y) {
    const I Sb = S / N;
    const I total = BH * S * vpr;
    for (I i = static_cast<I>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<I>(gridDim.x) * 256) {
        const I c = i % vpr;
        const I R = i / vpr;  // output row
        I src;
        if (!inverse) {  // y[n][bh][r] <- x[bh][t]
            const I r = R % Sb;
            const I rest = R / Sb;
            const I bh = rest % BH;
            const I n = rest / BH;
            const I t = striped ? r * N + n : n * Sb + r;
            src = bh * S + t;
        } else {  // y[bh][t] <- x[n][bh][r]
            const I t = R % S;
            const I bh = R / S;
            const I n = striped ? t % N : t / Sb;
            const I r = striped ? t / N : t % Sb;
            src = (n * BH + bh) * Sb + r;
        }
        y[i] = x[src * vpr + c];
    }
}

template <typename V>
hipError_t launch_v(int striped, int inverse, int64_t BH, int64_t S, int32_t N, int64_t row_bytes,
                    const void* x, void* y, hipStream_t s) {
    const int64_t vpr = row_bytes / static_cast<int64_t>(sizeof(V));
    const int64_t total = BH * S * vpr;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 64);
    if (total < (int64_t(1) << 31)) {
        hipLaunchKernelGGL((permute_kernel<V, uint32_t>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           striped, inverse, static_cast<uint32_t>(BH), static_cast<uint32_t>(S),
                           static_cast<uint32_t>(N), static_cast<uint32_t>(vpr), static_cast<const V*>(x),
                           static_cast<V*>(y));
    } else {
        hipLaunchKernelGGL((permute_kernel<V, uint64_t>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           striped, inverse, static_cast<uint64_t>(BH), static_cast<uint64_t>(S),
                           static_cast<uint64_t>(N), static_cast<uint64_t>(vpr), static_cast<const V*>(x),
                           static_cast<V*>(y));
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stripe_permute(int layout, int inverse, int64_t BH, int64_t S, int32_t N,
                                 int64_t row_bytes, const void* x, void* y, hipStream_t s) {
    if (BH == 0 || S == 0) return hipSuccess;
    const uintptr_t ax = reinterpret_cast<uintptr_t>(x), ay = reinterpret_cast<uintptr_t>(y);
    const int striped = layout == 1;
    if (row_bytes % 16 == 0 && ax % 16 == 0 && ay % 16 == 0)
        return launch_v<uint4>(striped, inverse, BH, S, N, row_bytes, x, y, s);
    if (row_bytes % 4 == 0 && ax % 4 == 0 && ay % 4 == 0)
        return launch_v<uint32_t>(striped, inverse, BH, S, N, row_bytes, x, y, s);
    return launch_v<uint16_t>(striped, inverse, BH, S, N, row_bytes, x, y, s);
}

}  // namespace ra
