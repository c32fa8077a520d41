// Internal launch interface between the host runtime (ra_host.cpp) and the
// HIP kernels.  Not part of the public ABI (include/ra.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

#include "ra.h"
#include <cstdint>

namespace ra {

// One query block against one key/value block.  All lengths fit in int32
// (checked by the host); mask_offset is clamped to [-q_len, kv_len] so that it
// fits as well without changing which keys are visible.
struct BlockArgs {
    const void* q;
    const void* k;
    const void* v;
    float* o;  // [B, Hq, q_len, D] unnormalised numerator
    float* m;  // [B, Hq, q_len] running max (natural log units)
    float* l;  // [B, Hq, q_len] sum of exponentials
    int32_t B, Hq, Hkv, D;
    int32_t q_len, kv_len;
    int64_t qs[3], ks[3], vs[3];  // element strides for (b, h, row)
    float scale;                  // softmax scale (already resolved)
    int32_t causal;
    int32_t mask_offset;  // key c visible to row r iff c <= r + mask_offset
    int32_t accumulate;   // 0: write the block's partial to (o, m, l);
                          // 1: (o, m, l) hold a running state; merge the partial into it
    // Key split (MFMA kernel only): n_splits > 1 cuts the block's keys into
    // ranges of split_tiles key tiles; split i writes its own partial to
    // o + i part_o_stride, m / l + i part_ml_stride (accumulate must be 0).
    int32_t n_splits = 1;
    int32_t split_tiles = 0;
    int64_t part_o_stride = 0, part_ml_stride = 0;
    // Work queues (MFMA kernel only): NULL keeps the fixed workgroup -> tile
    // order.  Otherwise kQueueWords zeroed counters in device memory: each
    // workgroup claims its tile from its XCD's queue (heaviest first) and,
    // once that queue is empty, from the others; the launch leaves them zeroed.
    // Launches that may run at the same time need counters of their own.
    uint32_t* queue = nullptr;
};
constexpr int kQueueWords = 16;  // 8 per-XCD queue heads, the claim count, padding
// Compute units of the current device (one persistent workgroup each).
int compute_units();

// Vector-ALU kernel: binary32 or bfloat16 inputs, any D in [1, 256], fp32 math.
hipError_t launch_block_simt(const BlockArgs& a, int dtype, hipStream_t s);

// bf16 MFMA kernel (gfx950): D in {64, 128}; 16-byte aligned rows.
bool mfma_eligible(const BlockArgs& a, int dtype);
int mfma_key_tile();    // keys per LDS tile of the MFMA kernel
int mfma_query_tile();  // query rows per workgroup of the MFMA kernel
hipError_t launch_block_mfma(const BlockArgs& a, hipStream_t s);

// Backward of one query block against one key/value block: this pair's share
// of the gradients, added into dq [B, Hq, q_len, D] and dk, dv
// [B, Hkv, kv_len, D] (fp32, contiguous).  lse and delta ([B, Hq, q_len],
// fp32) belong to the rows' full key set: p = exp(scale s - lse), and
// delta = dO . O.  dk/dv of a key/value head sum its query heads.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    const float* delta;
    float* dq;
    float* dk;
    float* dv;
    int32_t B, Hq, Hkv, D;
    int32_t q_len, kv_len;
    int64_t qs[3], ks[3], vs[3], dos[3];  // element strides for (b, h, row)
    float scale;
    int32_t causal;
    int32_t mask_offset;  // key c visible to row r iff c <= r + mask_offset
};

// Vector-ALU backward: binary32 or bfloat16 inputs, any D in [1, 256].
hipError_t launch_block_bwd_simt(const BwdArgs& a, int dtype, hipStream_t s);
// bf16 MFMA backward (gfx950): D in {64, 128}; 16-byte aligned rows and outputs.
bool bwd_mfma_eligible(const BwdArgs& a, int dtype);
hipError_t launch_block_bwd_mfma(const BwdArgs& a, hipStream_t s);
// workgroups of the smaller of the two MFMA backward launches (dQ, dK/dV)
int64_t bwd_mfma_min_workgroups(const BwdArgs& a);
// Kernel selection for the backward (MFMA where eligible unless force_simt).
hipError_t launch_block_bwd(const BwdArgs& a, int dtype, int force_simt, hipStream_t s);
// x[0 .. n) = 0 (fp32), a fill kernel rather than a memset node.
hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t s);

// delta[r] = sum_j dout[r, j] * o[r, j] for rows x D (contiguous, dtype), fp32 out.
hipError_t launch_bwd_delta(int64_t rows, int32_t D, int dtype, const void* o, const void* dout, float* delta,
                            hipStream_t s);

struct MergeArgs {
    int64_t rows;
    int32_t D;
    float* o_acc;
    float* m_acc;
    float* l_acc;
    const float* o_p;  // NULL: no partial to fold in
    const float* m_p;
    const float* l_p;
    void* o_out;  // finalise when o_out or lse_out is non-NULL
    int32_t out_dtype;
    float* lse_out;
    // Several partials (o_p + i part_o_stride, ... for i < n_parts, at most
    // kMaxMergeParts) fold in one pass; acc_valid = 0 treats the running state
    // as empty (it is not read) -- the first step of a split-key position.
    int32_t n_parts = 1;
    int32_t acc_valid = 1;
    int64_t part_o_stride = 0, part_ml_stride = 0;
};
constexpr int kMaxMergeParts = 8;
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s);

// Row moves between [BH, S, row] and [N, BH, S/N, row] under a token map.
hipError_t launch_stripe_permute(int layout, int inverse, int64_t BH, int64_t S, int32_t N,
                                 int64_t row_bytes, const void* x, void* y, hipStream_t s);

// Records a message for ra_last_error() and returns s.
ra_status set_error(ra_status s, const char* msg);

// The ring forward with every launch on `stream` itself: no library stream or
// event is created or recorded (stats and emulate_copy are refused).  Same
// arguments and workspace layout as ra_ring_forward with n_streams = 1.
ra_status ring_forward_on_stream(const ra_ring_desc* d, const void* q, const void* k, const void* v, void* o,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace ra
