/*
 * ra.h -- ring attention's per-step blockwise forward on AMD Instinct MI355X
 * (gfx950 / CDNA4).  C ABI: plain pointers and sizes, no framework types.
 *
 * The problem, as the pages state it ("Ring Attention", Ultralytics glossary,
 * section "How ring attention works"): a sequence is cut into N blocks, one
 * per ring position.  Position i keeps its query block for the whole
 * computation; at each of N steps it attends to the key/value block it holds,
 * which then moves one hop along the ring, so at step s it holds block
 * (i - s) mod N.  Per-step partial results are combined with the same running
 * softmax flash attention uses (running sums of exponentiated scores and of
 * weighted values, a running maximum subtracted before exponentiating,
 * division at the end), and the result is exactly full softmax attention
 * softmax(q k^T / sqrt(d)) v up to rounding.  Under a causal mask early
 * positions idle; the striped layout spreads every position's tokens evenly
 * along the sequence to balance the work.  The causal mask is the
 * `is_causal=True` rule of "Context Parallelism" (Ultralytics glossary),
 * section "Practical use and trade-offs": a key is visible to a query iff its
 * global position is not after the query's.
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE memory owned by the caller; the library never
 *    allocates, frees or retains them.  Scratch memory for ra_ring_forward
 *    comes from the caller's `workspace`.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call is asynchronous on it; ra_ring_forward forks onto library-owned
 *    streams and joins back to `stream` before returning, so it stays
 *    stream-ordered for the caller.
 *  - Element types: RA_F32 (binary32) or RA_BF16 (bfloat16).  Partials and
 *    log-sum-exp values are always binary32.
 *  - Argument errors are found before anything is launched and return
 *    RA_ERR_INVALID / RA_ERR_UNSUPPORTED / RA_ERR_WORKSPACE with no side
 *    effect; launch failures return RA_ERR_HIP.  Faults inside kernels surface
 *    at the caller's next synchronisation, as usual in HIP.  ra_last_error()
 *    returns a thread-local message for the last non-OK status.
 *  - Log-sum-exp and running maxima are natural-log quantities of the scaled
 *    scores s = scale * q.k.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_ABI_VERSION 5

typedef enum ra_status {
    RA_OK = 0,
    RA_ERR_INVALID = 1,     /* malformed argument (null pointer, bad size, ...)  */
    RA_ERR_UNSUPPORTED = 2, /* well formed but not implemented (dtype, head_dim) */
    RA_ERR_HIP = 3,         /* the HIP runtime reported an error                 */
    RA_ERR_WORKSPACE = 4    /* caller's workspace is too small                   */
} ra_status;

typedef enum ra_dtype { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* How global token t maps to ring position and local row (S = N * Sb):
 * CONTIGUOUS: position t / Sb, row t % Sb (equal chunks of the sequence).
 * STRIPED:    position t % N,  row t / N  (round-robin; the pages' striped
 *             layout, read as tokens dealt out evenly in turn).            */
typedef enum ra_layout { RA_CONTIGUOUS = 0, RA_STRIPED = 1 } ra_layout;

/* ra_block_desc.flags */
#define RA_BLOCK_FORCE_SIMT 1u /* use the vector-ALU kernel even where the MFMA kernel applies */
#define RA_BLOCK_ACCUMULATE 2u /* (o, m, l) hold a running state on entry; see ra_block_attn_fwd */

/*
 * One query block against one key/value block.
 *
 * q: [batch, q_heads, q_len, head_dim] at element strides q_strides = {b, h, row}
 * k, v: [batch, kv_heads, kv_len, head_dim] at strides k_strides / v_strides;
 * head_dim is always contiguous.  Query head h reads key/value head
 * h / (q_heads / kv_heads) (grouped-query attention, consecutive grouping).
 *
 * Global position of local query row r is q_pos0 + r * pos_stride, of local
 * key row c is k_pos0 + c * pos_stride (contiguous shards: stride 1,
 * pos0 = i * Sb; striped shards: stride N, pos0 = i).  With causal != 0 key c
 * is visible to row r iff k_pos0 + c*stride <= q_pos0 + r*stride, i.e.
 * c <= r + floor((q_pos0 - k_pos0) / stride).
 */
typedef struct ra_block_desc {
    int32_t batch, q_heads, kv_heads, head_dim;
    int64_t q_len, kv_len;
    int32_t dtype;  /* ra_dtype of q, k, v                                     */
    int32_t causal; /* 0 or 1                                                  */
    float scale;    /* softmax scale; <= 0 selects 1/sqrt(head_dim)            */
    uint32_t flags; /* RA_BLOCK_* bits; unknown bits are RA_ERR_UNSUPPORTED    */
    int64_t q_pos0, k_pos0, pos_stride; /* pos_stride >= 1                     */
    int64_t q_strides[3], k_strides[3], v_strides[3];
} ra_block_desc;

/*
 * ra_block_attn_fwd -- one ring step's blockwise attention ("Ring Attention",
 * section "How ring attention works": attention between the resident query
 * block and the key/value block held at this step, with the running maximum
 * of production kernels).
 *
 * Writes, for every query row r of every (b, h), the partial of this block:
 *   m[r]    = max over visible keys c of s_rc          (-inf if none visible)
 *   l[r]    = sum_c exp(s_rc - m[r])                   (0 if none)
 *   o[r, :] = sum_c exp(s_rc - m[r]) * v_c             (0 if none; NOT divided by l)
 * with s_rc = scale * q_r . k_c.
 * o: [batch, q_heads, q_len, head_dim] binary32, dense;
 * m, l: [batch, q_heads, q_len] binary32, dense.
 *
 * Kernels: bfloat16 with head_dim 64 or 128 runs on bf16 MFMA with fp32
 * accumulation (exponentials of the bf16-rounded probabilities feed the P.V
 * product; l sums the unrounded ones); every other supported case (binary32,
 * or bfloat16 with another head_dim) runs a vector-ALU kernel in fp32.
 * head_dim must be in [1, 256].  Empty blocks (q_len == 0) are a no-op;
 * kv_len == 0 yields the empty partial (m = -inf, l = 0, o = 0).
 */
ra_status ra_block_attn_fwd(const ra_block_desc* desc, const void* q, const void* k,
                            const void* v, float* o, float* m, float* l, void* stream);
/*
 * ra_block_attn_fwd_kernel -- which kernel ra_block_attn_fwd would run for the
 * same arguments, decided on the host with no GPU work: 1 = the bf16 MFMA
 * kernel, 0 = the vector-ALU kernel (also for a valid empty call), -1 = the
 * call would be rejected (ra_last_error says why).  The MFMA kernel needs
 * bfloat16, head_dim 64 or 128, 16-byte aligned q, k, v, o, strides that are
 * multiples of 8 elements, and key/value row strides below 2^24 elements.
 */
int32_t ra_block_attn_fwd_kernel(const ra_block_desc* desc, const void* q, const void* k, const void* v,
                                 const float* o, const float* m, const float* l);

/* With RA_BLOCK_ACCUMULATE, (o, m, l) hold a running state (a partial of some
 * other key set, in the same layout) on entry, and on return hold the merge of
 * that state with this block's partial -- the result ra_lse_merge would give
 * for (running state, this partial), computed in the kernel's epilogue without
 * writing the partial out.  The running state must be initialised (e.g. by a
 * call without the flag, or to m = -inf, l = 0, o = 0). */

/*
 * ra_lse_merge -- combine two partials with the running softmax ("Ring
 * Attention", section "How ring attention works": partial results are merged
 * with flash attention's running softmax and divided at the end).
 *
 * rows = number of (b, h, row) triples, all arrays dense and row-major:
 * o_* [rows, head_dim], m_* / l_* [rows], binary32.
 *
 * If o_part, m_part, l_part are all non-NULL the partial is folded into the
 * running state (a):  m = max(m_a, m_p);  w_x = exp(m_x - m) (0 if m_x = -inf);
 *   l = w_a l_a + w_p l_p;  o = w_a o_a + w_p o_p.
 * If all three are NULL the running state is taken as is.  A mix is invalid.
 *
 * If o_out == NULL and lse_out == NULL the result is written back to
 * (o_acc, m_acc, l_acc).  Otherwise the call FINALISES instead: o_out
 * [rows, head_dim] in out_dtype receives o / l (0 for rows with l == 0;
 * bfloat16 is rounded to nearest even) and lse_out [rows] receives m + ln l
 * (-inf for rows with l == 0); either may be NULL; the running state is then
 * left unchanged.  The merge may be done in place (o_part may not alias
 * o_acc).  rows == 0 is a no-op.
 */
ra_status ra_lse_merge(int64_t rows, int32_t head_dim, float* o_acc, float* m_acc, float* l_acc,
                       const float* o_part, const float* m_part, const float* l_part,
                       void* o_out, int32_t out_dtype, float* lse_out, void* stream);

/* Timing and work counters of one ra_ring_forward call (see ra_ring_desc.stats). */
typedef struct ra_ring_stats {
    double block_ms, merge_ms, copy_ms; /* summed kernel / copy durations, HIP events   */
    int64_t block_launches, merge_launches, copy_launches;
    int64_t blocks_skipped;             /* (position, step) pairs fully masked, skipped */
    double unmasked_pairs;              /* (query row, key) pairs attended, all heads   */
    double flops;                       /* ra_ring_forward: 4 * head_dim * unmasked_pairs;
                                           ra_ring_backward: 10 * head_dim * unmasked_pairs */
    int64_t kv_splits;                  /* ra_ring_forward: key ranges per block launch (1: none) */
} ra_ring_stats;

/*
 * N virtual ring positions run on one GPU.
 *
 * Positions first_pos .. first_pos + n_run - 1 are computed (n_run = 1 runs one
 * position's share; n_run = n_pos the whole ring).  Position i at step s
 * attends to key/value block j = (i - visit_order[s]) mod n_pos
 * (visit_order = NULL means visit_order[s] = s, the ring's own order: the
 * block that arrived from the previous position).  Any permutation gives the
 * same result up to rounding.
 */
typedef struct ra_ring_desc {
    int32_t batch, q_heads, kv_heads, head_dim;
    int32_t n_pos;      /* N >= 1                                                 */
    int32_t first_pos;  /* 0 <= first_pos, first_pos + n_run <= N                 */
    int32_t n_run;      /* >= 1                                                   */
    int32_t layout;     /* ra_layout of the shards (decides the causal mask)      */
    int64_t block_len;  /* Sb = S / N tokens per position                         */
    int32_t dtype;      /* ra_dtype of q, k, v and of the output o                */
    int32_t causal;
    float scale;        /* <= 0 selects 1/sqrt(head_dim)                          */
    int32_t emulate_copy; /* 0: step s reads block j where it lies;
                             1: blocks travel through two per-position slots
                                (double buffer) by device-to-device copies on
                                a copy stream, ordered by HIP events, as a ring
                                transfer would be                              */
    int32_t n_streams;  /* compute streams; 0 = min(n_run, 8).  A single position
                           (n_run = 1) whose block launches hold at least twice
                           as many query tiles as the GPU has compute units
                           (bf16, head_dim 64 or 128, fused schedule, no
                           emulate_copy) runs its computed steps alternately on
                           two running states on two streams when n_streams is
                           0 or >= 2, and the final merge pass folds the second
                           into the first; n_streams = 1 keeps one state      */
    int32_t separate_merge; /* 0: each step after a position's first merges its
                               partial into the running state inside the block
                               kernel (RA_BLOCK_ACCUMULATE) and one finalising
                               ra_lse_merge pass ends the position;
                               1: each step writes a partial and ra_lse_merge
                               folds it in (the last fold also finalises)     */
    int32_t kv_splits;  /* fused schedule, bf16, head_dim 64 or 128 only: each
                           block launch cuts the block's keys into this many
                           ranges (one workgroup per query tile, head and
                           range), and one ra_lse_merge pass per step folds
                           the ranges' partials into the running state.
                           0: automatic (used when a step's launches would
                           fill fewer workgroups than the GPU has compute
                           units); 1: off; 2..8: that many ranges (capped at
                           the block's 128-key tiles).  Ignored otherwise.   */
    const int32_t* visit_order; /* host array [n_pos] (a permutation) or NULL     */
    ra_ring_stats* stats;       /* host pointer or NULL.  When set, every launch is
                                   timed with HIP events and the call waits for
                                   its own work to finish before returning.      */
} ra_ring_desc;

/* Bytes of device workspace ra_ring_forward needs for `desc` (256-byte aligned
 * base required). */
ra_status ra_ring_workspace_size(const ra_ring_desc* desc, size_t* bytes);

/*
 * ra_ring_forward -- the ring schedule of "Ring Attention", section "How ring
 * attention works", for N virtual positions on one GPU: no inter-GPU transfer,
 * no collective, no sharding.  Per position, the first computed step writes
 * its partial straight into the running state; every later step merges its
 * block into that state (in the block kernel, or -- with separate_merge -- by
 * a partial plus an ra_lse_merge fold); a final ra_lse_merge pass normalises
 * (fused schedule) or the last fold does (separate schedule).  With key splits
 * (kv_splits) every step writes one partial per key range and one merge pass
 * folds them all into the running state, the last one also normalising.  Fully masked
 * (position, block) pairs are skipped (contiguous causal: blocks after the
 * query block).  Positions are spread over n_streams library-owned streams.
 *
 * q: [n_run, batch, q_heads, Sb, head_dim]   (query shards of the run positions)
 * k, v: [n_pos, batch, kv_heads, Sb, head_dim] (all key/value shards)
 * o: [n_run, batch, q_heads, Sb, head_dim] in dtype (normalised output)
 * lse: [n_run, batch, q_heads, Sb] binary32 (may be NULL)
 * All dense, position-major (the layout ra_stripe_permute produces).
 * workspace: device memory of at least ra_ring_workspace_size bytes: the
 * running states (fp32 O, m, l) of the run positions, partials, emulated
 * transfer slots, and per library stream a block of tile-queue counters (the
 * bf16 block kernel's workgroups claim query tiles from per-XCD queues and
 * take over other XCDs' tiles once their own are done; the call zeroes the
 * counters first and every launch leaves them zeroed).  Its contents need no
 * initialisation; calls that may run at the same time need separate
 * workspaces.
 * Concurrent calls are serialised on an internal mutex.
 * With stats == NULL the call only enqueues work -- kernel launches, event
 * records and waits (and, with emulate_copy, device-to-device copies) -- on
 * `stream` and on library streams forked from it and joined back, so it may
 * be captured into a HIP graph once an eager call with the same n_streams has
 * created those streams and events on the device.
 */
ra_status ra_ring_forward(const ra_ring_desc* desc, const void* q, const void* k, const void* v,
                          void* o, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * ra_ring_forward_noalloc -- ra_ring_forward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, layouts and results as
 * ra_ring_forward with n_streams = 1, without the workspace: the scratch
 * (running states, key-range partials, tile-queue counters) is a device array
 * the library holds, ra_ring_noalloc_max_bytes() bytes (256 MiB: enough for
 * one position's share of the 256K-token, 8-head, head_dim 128 ring) per GPU,
 * from the first call on that GPU until the process ends: that first call
 * looks the array's address up, and the HIP runtime backs it with device
 * memory then (make it before capture or a no-allocation section begins).
 * Every later call creates no stream, event or device memory; every launch
 * goes to `stream`, in order.
 * Refused before anything is launched: desc->stats or desc->emulate_copy
 * (RA_ERR_UNSUPPORTED, they need library events and streams), and shapes
 * whose scratch (ra_ring_workspace_size with n_streams = 1) exceeds the array
 * (RA_ERR_WORKSPACE).  Every call on one GPU shares that GPU's array and
 * leaves its last contents there; calls whose GPU work may overlap on one GPU
 * (other streams, other threads) race on it and give wrong results.
 */
ra_status ra_ring_forward_noalloc(const ra_ring_desc* desc, const void* q, const void* k, const void* v,
                                  void* o, float* lse, void* stream);
/* Bytes of scratch ra_ring_forward_noalloc holds per GPU. */
size_t ra_ring_noalloc_max_bytes(void);

/*
 * ra_stripe_permute -- build (or undo) the per-position shard layout: the
 * contiguous split of the pages' ring (N equal blocks) or the striped layout
 * ("Ring Attention", section "How ring attention works": each position gets
 * tokens spread evenly along the sequence).
 *
 * inverse == 0: x [batch, heads, seq_len, head_dim] -> y [n_pos, batch, heads, seq_len/n_pos, head_dim]
 * inverse != 0: x [n_pos, batch, heads, seq_len/n_pos, head_dim] -> y [batch, heads, seq_len, head_dim]
 * with the token maps of ra_layout.  Pure data movement: bit-exact.
 * seq_len % n_pos must be 0; x and y must not overlap.  head_dim = 1 with
 * RA_F32 moves log-sum-exp arrays.
 */
ra_status ra_stripe_permute(int32_t layout, int32_t inverse, int32_t dtype, int32_t batch,
                            int32_t heads, int64_t seq_len, int32_t head_dim, int32_t n_pos,
                            const void* x, void* y, void* stream);

/*
 * Backward pass.  The pages run it: "Context Parallelism" (Ultralytics
 * glossary), section "Practical use and trade-offs", marks q, k, v as
 * requiring gradients and back-propagates a loss through the causal
 * attention.  For an upstream gradient dO = dL/dO, with p_rc the forward's
 * softmax weights exp(s_rc - lse_r) and delta_r = dO_r . O_r, the chain rule
 * gives  dp_rc = dO_r . v_c,  ds_rc = p_rc (dp_rc - delta_r),
 *   dQ_r = scale sum_c ds_rc k_c,  dK_c = scale sum_r ds_rc q_r,
 *   dV_c = sum_r p_rc dO_r   (sums over visible pairs).
 * Summed over key blocks these give the full gradients, so a ring adds each
 * step's share: dQ stays with its position, dK and dV travel with their block.
 */

/* ra_attn_bwd_delta -- delta[r] = sum_j dout[r, j] * o[r, j] (binary32) for
 * rows x head_dim arrays o, dout in dtype (dense, row-major).  o is the
 * forward's normalised output. */
ra_status ra_attn_bwd_delta(int64_t rows, int32_t head_dim, int32_t dtype, const void* o,
                            const void* dout, float* delta, void* stream);

/*
 * ra_block_attn_bwd -- one query block against one key/value block: ADDS this
 * block pair's share of the gradients into dq, dk, dv.
 *
 * desc, q, k, v: as for ra_block_attn_fwd (flags: only RA_BLOCK_FORCE_SIMT).
 * dout: [batch, q_heads, q_len, head_dim] in dtype at q's strides.
 * lse, delta: [batch, q_heads, q_len] binary32, dense: the rows' log-sum-exp
 *   over their FULL key set (ra_ring_forward's lse) and ra_attn_bwd_delta.
 *   Rows with lse = -inf contribute nothing.
 * dq: [batch, q_heads, q_len, head_dim]; dk, dv: [batch, kv_heads, kv_len,
 *   head_dim]; binary32, dense, accumulated into (+=).  A key/value head's
 *   dk, dv sum over the query heads that read it; no atomics are used, so
 *   concurrent calls must not share an output array.
 * q_len == 0 or kv_len == 0 is a no-op.
 */
ra_status ra_block_attn_bwd(const ra_block_desc* desc, const void* q, const void* k,
                            const void* v, const void* dout, const float* lse,
                            const float* delta, float* dq, float* dk, float* dv, void* stream);

/* ra_block_attn_bwd_kernel -- which kernels ra_block_attn_bwd would run for
 * the same arguments (host only): 1 = bf16 MFMA, 0 = vector ALU (also for a
 * valid empty call), -1 = rejected.  MFMA needs bfloat16, head_dim 64 or 128,
 * 16-byte aligned tensors, strides that are multiples of 8 elements and row
 * strides below 2^24 elements. */
int32_t ra_block_attn_bwd_kernel(const ra_block_desc* desc, const void* q, const void* k, const void* v,
                                 const void* dout, const float* lse, const float* delta, const float* dq,
                                 const float* dk, const float* dv);

/* Bytes of device workspace ra_ring_backward needs (256-byte aligned base). */
ra_status ra_ring_bwd_workspace_size(const ra_ring_desc* desc, size_t* bytes);

/*
 * ra_ring_backward -- the ring backward for N virtual positions on one GPU.
 * Steps run in lockstep as on a real ring: at step s position i holds block
 * j = (i - visit_order[s]) mod n_pos (distinct across positions) and adds its
 * share into its own dq and into the block's dk, dv.  Fully masked pairs are
 * skipped.  The positions of one step write disjoint outputs and run on
 * n_streams library streams (position p on stream p mod n_streams), forked
 * from `stream` before each step and joined back to it after.  n_streams = 0
 * picks one stream (the caller's) when each launch's dQ and dK/dV kernels
 * both hold at least one workgroup per compute unit (bf16, head_dim 64 or
 * 128), else min(n_run, 8).  emulate_copy and separate_merge are ignored.  With desc->stats,
 * backward launches are timed (block_ms, block_launches; spans of launches on
 * different streams may overlap) and flops counts the five products.
 *
 * q, o, dout: [n_run, batch, q_heads, Sb, head_dim] in dtype (o and lse from
 *   ra_ring_forward on the same desc);  lse: [n_run, batch, q_heads, Sb];
 * k, v: [n_pos, batch, kv_heads, Sb, head_dim] in dtype;
 * dq: [n_run, batch, q_heads, Sb, head_dim] binary32 (overwritten);
 * dk, dv: [n_pos, batch, kv_heads, Sb, head_dim] binary32 (overwritten with
 *   the run positions' share: the full gradients when n_run == n_pos).
 */
ra_status ra_ring_backward(const ra_ring_desc* desc, const void* q, const void* k,
                           const void* v, const void* o, const void* dout, const float* lse,
                           float* dq, float* dk, float* dv, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Host-side helpers (no GPU work; usable on a machine without a GPU). */

/* floor((q_pos0 - k_pos0) / pos_stride): key c is visible to row r iff c <= r + offset. */
int64_t ra_mask_offset(int64_t q_pos0, int64_t k_pos0, int64_t pos_stride);

/* Number of (row, key) pairs of a q_len x kv_len block that the mask leaves
 * visible (causal: key c visible to row r iff c <= r + offset). */
int64_t ra_unmasked_pairs(int64_t q_len, int64_t kv_len, int32_t causal, int64_t offset);

/* Mask offset between position i's queries and block j's keys in a ring of
 * n_pos positions of block_len tokens with the given layout. */
int64_t ra_ring_pair_offset(int32_t layout, int32_t n_pos, int64_t block_len, int32_t i, int32_t j);

const char* ra_last_error(void);
int32_t ra_abi_version(void);
/* Frees library-owned streams and events (they are recreated on demand). */
void ra_release(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
