// Host runtime behind include/ra.h: argument validation, mask-offset and
// work accounting, kernel selection, and the virtual ring scheduler.
//
// The ring schedule follows "Ring Attention" (Ultralytics glossary), section
// "How ring attention works": position i keeps its query block and at step s
// works on key/value block (i - s) mod N, folding each step's partial into a
// running state with the online softmax; the division happens at the end.
// Here the N positions are virtual: they share one GPU, each position's work
// runs on one of a small pool of library-owned HIP streams, and the "transfer"
// of a block to the next position is either nothing (the position simply reads
// block j where it lies) or, in emulate-copy mode, a device-to-device copy
// into a per-position double buffer ordered by HIP events exactly as a real
// ring's receive would be.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "ra.h"
#include "ra_internal.h"

namespace {

thread_local std::string g_err;

ra_status fail(ra_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

ra_status hip_fail(hipError_t e, const char* what) {
    return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define RA_HIP(expr)                                 \
    do {                                             \
        hipError_t e_ = (expr);                      \
        if (e_ != hipSuccess) return hip_fail(e_, #expr); \
    } while (0)

int64_t floor_div(int64_t a, int64_t b) {
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
    return q;
}

size_t elem_size(int32_t dtype) { return dtype == RA_BF16 ? 2 : 4; }
bool valid_dtype(int32_t d) { return d == RA_F32 || d == RA_BF16; }
bool aligned_to(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
constexpr int64_t kMaxLen = (int64_t(1) << 31) - 1;

// Shared shape checks of the block and ring descriptors.
ra_status check_heads(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t dtype) {
    if (batch < 1 || hq < 1 || hkv < 1) return fail(RA_ERR_INVALID, "batch and head counts must be >= 1");
    if (hq % hkv != 0) return fail(RA_ERR_INVALID, "q_heads (%d) must be a multiple of kv_heads (%d)", hq, hkv);
    if (d < 1) return fail(RA_ERR_INVALID, "head_dim must be >= 1");
    if (d > 256) return fail(RA_ERR_UNSUPPORTED, "head_dim %d > 256 is not supported", d);
    if (!valid_dtype(dtype)) return fail(RA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    return RA_OK;
}

float resolve_scale(float scale, int32_t d) {
    return scale > 0.f ? scale : static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
}

int32_t clamp_offset(int64_t off, int64_t q_len, int64_t kv_len) {
    return static_cast<int32_t>(std::min<int64_t>(std::max<int64_t>(off, -q_len), kv_len));
}

ra_status launch_block(const ra::BlockArgs& a, int32_t dtype, uint32_t flags, hipStream_t s) {
    hipError_t e;
    if (!(flags & RA_BLOCK_FORCE_SIMT) && ra::mfma_eligible(a, dtype))
        e = ra::launch_block_mfma(a, s);
    else if (a.n_splits > 1)
        return fail(RA_ERR_UNSUPPORTED, "key splits need the MFMA kernel");
    else
        e = ra::launch_block_simt(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "block attention launch");
    return RA_OK;
}


// Validates a forward block call and fills its kernel arguments.  q_len == 0
// is valid (a no-op) and returns RA_OK with the arguments unset.
ra_status block_fwd_args(const ra_block_desc* d, const void* q, const void* k, const void* v, float* o, float* m,
                         float* l, ra::BlockArgs* out) {
    if (!d) return fail(RA_ERR_INVALID, "null descriptor");
    ra_status st = check_heads(d->batch, d->q_heads, d->kv_heads, d->head_dim, d->dtype);
    if (st != RA_OK) return st;
    if (d->q_len < 0 || d->kv_len < 0 || d->q_len > kMaxLen || d->kv_len > kMaxLen)
        return fail(RA_ERR_INVALID, "q_len / kv_len out of range");
    if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_INVALID, "causal must be 0 or 1");
    if (d->flags & ~(RA_BLOCK_FORCE_SIMT | RA_BLOCK_ACCUMULATE))
        return fail(RA_ERR_UNSUPPORTED, "unknown flags 0x%x", d->flags);
    if (d->pos_stride < 1) return fail(RA_ERR_INVALID, "pos_stride must be >= 1");
    if (!std::isfinite(d->scale)) return fail(RA_ERR_INVALID, "scale must be finite");
    for (int i = 0; i < 3; ++i)
        if (d->q_strides[i] < 0 || d->k_strides[i] < 0 || d->v_strides[i] < 0)
            return fail(RA_ERR_INVALID, "strides must be non-negative");
    if (d->q_len == 0) return RA_OK;
    if (!q || !o || !m || !l) return fail(RA_ERR_INVALID, "null q / o / m / l pointer");
    if (d->kv_len > 0 && (!k || !v)) return fail(RA_ERR_INVALID, "null k / v pointer");
    const size_t es = elem_size(d->dtype);
    if (!aligned_to(q, es) || (k && !aligned_to(k, es)) || (v && !aligned_to(v, es)) || !aligned_to(o, 4) ||
        !aligned_to(m, 4) || !aligned_to(l, 4))
        return fail(RA_ERR_INVALID, "misaligned pointer");
    ra::BlockArgs& a = *out;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.m = m;
    a.l = l;
    a.B = d->batch;
    a.Hq = d->q_heads;
    a.Hkv = d->kv_heads;
    a.D = d->head_dim;
    a.q_len = static_cast<int32_t>(d->q_len);
    a.kv_len = static_cast<int32_t>(d->kv_len);
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = d->q_strides[i];
        a.ks[i] = d->k_strides[i];
        a.vs[i] = d->v_strides[i];
    }
    a.scale = resolve_scale(d->scale, d->head_dim);
    a.causal = d->causal;
    a.mask_offset = clamp_offset(ra_mask_offset(d->q_pos0, d->k_pos0, d->pos_stride), d->q_len, d->kv_len);
    a.accumulate = (d->flags & RA_BLOCK_ACCUMULATE) ? 1 : 0;
    return RA_OK;
}

}  // namespace

extern "C" {

int64_t ra_mask_offset(int64_t q_pos0, int64_t k_pos0, int64_t pos_stride) {
    if (pos_stride < 1) return 0;
    return floor_div(q_pos0 - k_pos0, pos_stride);
}

int64_t ra_unmasked_pairs(int64_t q_len, int64_t kv_len, int32_t causal, int64_t offset) {
    if (q_len <= 0 || kv_len <= 0) return 0;
    if (!causal) return q_len * kv_len;
    // row r sees min(kv_len, max(0, r + offset + 1)) keys
    const int64_t lo = std::min(std::max<int64_t>(-offset, 0), q_len);              // rows < lo see none
    const int64_t hi = std::min(std::max<int64_t>(kv_len - offset - 1, lo), q_len);  // rows >= hi see all
    const int64_t n = hi - lo;
    const int64_t partial = n * (offset + 1) + (lo + hi - 1) * n / 2;
    return partial + (q_len - hi) * kv_len;
}

int64_t ra_ring_pair_offset(int32_t layout, int32_t n_pos, int64_t block_len, int32_t i, int32_t j) {
    if (layout == RA_STRIPED) return ra_mask_offset(i, j, n_pos);  // 0 if j <= i else -1
    return ra_mask_offset(static_cast<int64_t>(i) * block_len, static_cast<int64_t>(j) * block_len, 1);
}

const char* ra_last_error(void) { return g_err.c_str(); }
int32_t ra_abi_version(void) { return RA_ABI_VERSION; }

ra_status ra_block_attn_fwd(const ra_block_desc* d, const void* q, const void* k, const void* v, float* o,
                            float* m, float* l, void* stream) {
    ra::BlockArgs a{};
    const ra_status st = block_fwd_args(d, q, k, v, o, m, l, &a);
    if (st != RA_OK || d->q_len == 0) return st;
    return launch_block(a, d->dtype, d->flags, static_cast<hipStream_t>(stream));
}

int32_t ra_block_attn_fwd_kernel(const ra_block_desc* d, const void* q, const void* k, const void* v,
                                 const float* o, const float* m, const float* l) {
    ra::BlockArgs a{};
    if (block_fwd_args(d, q, k, v, const_cast<float*>(o), const_cast<float*>(m), const_cast<float*>(l), &a) != RA_OK)
        return -1;
    return (!(d->flags & RA_BLOCK_FORCE_SIMT) && ra::mfma_eligible(a, d->dtype)) ? 1 : 0;
}

ra_status ra_lse_merge(int64_t rows, int32_t head_dim, float* o_acc, float* m_acc, float* l_acc,
                       const float* o_part, const float* m_part, const float* l_part, void* o_out,
                       int32_t out_dtype, float* lse_out, void* stream) {
    if (rows < 0) return fail(RA_ERR_INVALID, "rows must be >= 0");
    if (head_dim < 1) return fail(RA_ERR_INVALID, "head_dim must be >= 1");
    if (!valid_dtype(out_dtype)) return fail(RA_ERR_UNSUPPORTED, "unknown out_dtype %d", out_dtype);
    const int given = (o_part != nullptr) + (m_part != nullptr) + (l_part != nullptr);
    if (given != 0 && given != 3) return fail(RA_ERR_INVALID, "o_part, m_part, l_part must be all set or all NULL");
    if (rows == 0) return RA_OK;
    if (!o_acc || !m_acc || !l_acc) return fail(RA_ERR_INVALID, "null running state");
    if (o_part != nullptr && o_part == o_acc) return fail(RA_ERR_INVALID, "o_part aliases o_acc");
    if (!aligned_to(o_acc, 4) || !aligned_to(m_acc, 4) || !aligned_to(l_acc, 4) ||
        (o_out && !aligned_to(o_out, elem_size(out_dtype))) || (lse_out && !aligned_to(lse_out, 4)) ||
        (o_part && (!aligned_to(o_part, 4) || !aligned_to(m_part, 4) || !aligned_to(l_part, 4))))
        return fail(RA_ERR_INVALID, "misaligned pointer");
    ra::MergeArgs a{rows, head_dim, o_acc, m_acc, l_acc, o_part, m_part, l_part, o_out, out_dtype, lse_out};
    hipError_t e = ra::launch_lse_merge(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lse merge launch");
    return RA_OK;
}

ra_status ra_stripe_permute(int32_t layout, int32_t inverse, int32_t dtype, int32_t batch, int32_t heads,
                            int64_t seq_len, int32_t head_dim, int32_t n_pos, const void* x, void* y,
                            void* stream) {
    if (layout != RA_CONTIGUOUS && layout != RA_STRIPED) return fail(RA_ERR_INVALID, "unknown layout %d", layout);
    if (!valid_dtype(dtype)) return fail(RA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (batch < 1 || heads < 1 || head_dim < 1 || n_pos < 1 || seq_len < 0)
        return fail(RA_ERR_INVALID, "batch, heads, head_dim, n_pos must be >= 1 and seq_len >= 0");
    if (seq_len % n_pos != 0)
        return fail(RA_ERR_INVALID, "seq_len (%lld) must be a multiple of n_pos (%d)", (long long)seq_len, n_pos);
    if (seq_len == 0) return RA_OK;
    if (!x || !y) return fail(RA_ERR_INVALID, "null pointer");
    const int64_t row_bytes = static_cast<int64_t>(head_dim) * static_cast<int64_t>(elem_size(dtype));
    const int64_t total = static_cast<int64_t>(batch) * heads * seq_len * row_bytes;
    const char* xb = static_cast<const char*>(x);
    const char* yb = static_cast<const char*>(y);
    if (xb < yb + total && yb < xb + total) return fail(RA_ERR_INVALID, "x and y overlap");
    if (!aligned_to(x, elem_size(dtype)) || !aligned_to(y, elem_size(dtype)))
        return fail(RA_ERR_INVALID, "misaligned pointer");
    hipError_t e = ra::launch_stripe_permute(layout, inverse, static_cast<int64_t>(batch) * heads, seq_len, n_pos,
                                             row_bytes, x, y, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "stripe permute launch");
    return RA_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ ring
namespace {

struct RingPlanStep {
    int32_t step, block;
    int64_t offset;  // mask offset between the position's queries and the block's keys
    bool skip;       // causal and fully masked
};

struct RingGeometry {
    int64_t rows;       // B * Hq * Sb
    int64_t q_elems;    // B * Hq * Sb * D   (one position's query shard / output)
    int64_t kv_elems;   // B * Hkv * Sb * D  (one key or value shard)
    int32_t n_streams;
    int32_t n_chains;               // accumulation chains of a single position (1 or 2)
    int32_t n_splits, split_tiles;  // key splits of every block launch (1: none)
    int32_t n_part;                 // partials per stream (0, 1 or n_splits)
    size_t acc_o, acc_ml, part_o, part_ml, slot;  // bytes, each 256-aligned
    size_t queue;                                 // per stream: the block kernel's tile-queue counters
    size_t total;
};

ra_status check_ring(const ra_ring_desc* d) {
    if (!d) return fail(RA_ERR_INVALID, "null descriptor");
    ra_status st = check_heads(d->batch, d->q_heads, d->kv_heads, d->head_dim, d->dtype);
    if (st != RA_OK) return st;
    if (d->n_pos < 1) return fail(RA_ERR_INVALID, "n_pos must be >= 1");
    if (d->n_run < 1 || d->first_pos < 0 || static_cast<int64_t>(d->first_pos) + d->n_run > d->n_pos)
        return fail(RA_ERR_INVALID, "positions [first_pos, first_pos + n_run) must lie in [0, n_pos)");
    if (d->layout != RA_CONTIGUOUS && d->layout != RA_STRIPED) return fail(RA_ERR_INVALID, "unknown layout");
    if (d->block_len < 1 || d->block_len > kMaxLen) return fail(RA_ERR_INVALID, "block_len out of range");
    if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_INVALID, "causal must be 0 or 1");
    if (d->emulate_copy != 0 && d->emulate_copy != 1) return fail(RA_ERR_INVALID, "emulate_copy must be 0 or 1");
    if (d->n_streams < 0 || d->n_streams > 64) return fail(RA_ERR_INVALID, "n_streams must be in [0, 64]");
    if (d->separate_merge != 0 && d->separate_merge != 1) return fail(RA_ERR_INVALID, "separate_merge must be 0 or 1");
    if (d->kv_splits < 0 || d->kv_splits > ra::kMaxMergeParts)
        return fail(RA_ERR_INVALID, "kv_splits must be in [0, %d]", ra::kMaxMergeParts);
    if (!std::isfinite(d->scale)) return fail(RA_ERR_INVALID, "scale must be finite");
    if (d->visit_order) {
        std::vector<char> seen(d->n_pos, 0);
        for (int s = 0; s < d->n_pos; ++s) {
            const int32_t x = d->visit_order[s];
            if (x < 0 || x >= d->n_pos || seen[x]) return fail(RA_ERR_INVALID, "visit_order is not a permutation");
            seen[x] = 1;
        }
    }
    return RA_OK;
}

RingGeometry geometry(const ra_ring_desc* d) {
    RingGeometry g{};
    const int64_t Sb = d->block_len;
    g.rows = static_cast<int64_t>(d->batch) * d->q_heads * Sb;
    g.q_elems = g.rows * d->head_dim;
    g.kv_elems = static_cast<int64_t>(d->batch) * d->kv_heads * Sb * d->head_dim;
    g.n_streams = d->n_streams > 0 ? std::min(d->n_streams, d->n_run) : std::min(d->n_run, 8);
    g.acc_o = round_up(static_cast<size_t>(g.q_elems) * 4, 256);
    g.acc_ml = round_up(static_cast<size_t>(g.rows) * 4, 256);
    // Key splits (fused schedule, MFMA shapes): when one step's block launches
    // fill few workgroups, each launch cuts the keys into n_splits ranges of
    // split_tiles tiles, one workgroup per (query tile, head, range), and a
    // multi-partial ra_lse_merge pass folds the ranges into the running state.
    g.n_splits = 1;
    g.split_tiles = 0;
    if (!d->separate_merge && d->kv_splits != 1 && d->dtype == RA_BF16 &&
        (d->head_dim == 64 || d->head_dim == 128)) {
        const int64_t tiles = (Sb + ra::mfma_key_tile() - 1) / ra::mfma_key_tile();
        int64_t want = d->kv_splits;
        if (want == 0) {  // automatic: about one workgroup per compute unit, >= 2 key tiles per range
            const int64_t cus = ra::compute_units();
            const int64_t wg = (Sb + ra::mfma_query_tile() - 1) / ra::mfma_query_tile() * d->q_heads * d->batch *
                               std::min(g.n_streams, d->n_run);
            want = wg >= cus ? 1 : std::min<int64_t>((cus + wg - 1) / wg, tiles / 2);
        }
        want = std::max<int64_t>(1, std::min<int64_t>({want, tiles, ra::kMaxMergeParts}));
        if (want > 1) {
            g.split_tiles = static_cast<int32_t>((tiles + want - 1) / want);
            g.n_splits = static_cast<int32_t>((tiles + g.split_tiles - 1) / g.split_tiles);  // no empty range
        }
    }
    // Accumulation chains.  One position's fused steps run one after another
    // on one stream, each launch folding into the running state, so every
    // launch's start (claims, Q loads, first tile copies) and end (compute
    // units running out of tiles) are paid in full.  When a single position
    // runs large launches (the work queues' threshold), its computed steps
    // alternate between two running states on two streams instead: the
    // launches of one chain overlap the start and end of the other's, and the
    // final merge pass folds the second state into the first and normalises.
    g.n_chains = 1;
    if (d->n_run == 1 && !d->separate_merge && g.n_splits == 1 && !d->emulate_copy && d->n_pos >= 2 &&
        (d->n_streams == 0 || d->n_streams >= 2) && d->dtype == RA_BF16 && (d->head_dim == 64 || d->head_dim == 128)) {
        const int64_t launch_tiles =
            (Sb + ra::mfma_query_tile() - 1) / ra::mfma_query_tile() * d->q_heads * d->batch;
        if (launch_tiles >= 2 * static_cast<int64_t>(ra::compute_units())) g.n_chains = 2;
    }
    if (g.n_chains > 1) g.n_streams = g.n_chains;
    g.n_part = d->separate_merge ? 1 : (g.n_splits > 1 ? g.n_splits : 0);
    g.part_o = g.n_part ? g.acc_o : 0;
    g.part_ml = g.n_part ? g.acc_ml : 0;
    g.slot = d->emulate_copy ? round_up(static_cast<size_t>(g.kv_elems) * elem_size(d->dtype), 256) : 0;
    g.queue = round_up(ra::kQueueWords * sizeof(uint32_t), 256);
    // per run position: n_chains running states o, m, l (+ 2 slots x {K, V});
    // per stream: n_part partials o, m, l and the tile-queue counters of its
    // block launches
    g.total = static_cast<size_t>(d->n_run) * (g.n_chains * (g.acc_o + 2 * g.acc_ml) + 4 * g.slot) +
              static_cast<size_t>(g.n_streams) * (g.n_part * (g.part_o + 2 * g.part_ml) + g.queue);
    return g;
}

std::vector<RingPlanStep> plan_position(const ra_ring_desc* d, int32_t i) {
    std::vector<RingPlanStep> out(d->n_pos);
    for (int32_t s = 0; s < d->n_pos; ++s) {
        const int32_t off = d->visit_order ? d->visit_order[s] : s;
        const int32_t j = ((i - off) % d->n_pos + d->n_pos) % d->n_pos;
        const int64_t delta = ra_ring_pair_offset(d->layout, d->n_pos, d->block_len, i, j);
        const bool skip = d->causal && ra_unmasked_pairs(d->block_len, d->block_len, 1, delta) == 0;
        out[s] = {s, j, delta, skip};
    }
    return out;
}

struct DeviceState {
    std::vector<hipStream_t> compute, copy;
    std::vector<hipEvent_t> sync_events;    // timing disabled
    std::vector<hipEvent_t> timing_events;  // timing enabled
    std::vector<hipEvent_t> bwd_events;     // timing disabled: the ring backward's per-step fork and join
};

std::mutex g_mutex;
std::map<int, DeviceState> g_devices;

ra_status ensure_streams(DeviceState& ds, int n) {
    while (static_cast<int>(ds.compute.size()) < n) {
        hipStream_t s;
        RA_HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
        ds.compute.push_back(s);
        RA_HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
        ds.copy.push_back(s);
    }
    return RA_OK;
}

ra_status ensure_events(std::vector<hipEvent_t>& pool, size_t n, unsigned flags) {
    while (pool.size() < n) {
        hipEvent_t e;
        RA_HIP(hipEventCreateWithFlags(&e, flags));
        pool.push_back(e);
    }
    return RA_OK;
}

// Times one launch with a pair of events when stats are requested.
struct Timer {
    std::vector<hipEvent_t>* pool = nullptr;
    size_t next = 0;
    std::vector<std::pair<size_t, int>> spans;  // (event index, kind)
    ra_status begin(hipStream_t s, size_t& idx) {
        if (!pool) return RA_OK;
        ra_status st = ensure_events(*pool, next + 2, hipEventDefault);
        if (st != RA_OK) return st;
        idx = next;
        next += 2;
        RA_HIP(hipEventRecord((*pool)[idx], s));
        return RA_OK;
    }
    ra_status end(hipStream_t s, size_t idx, int kind) {
        if (!pool) return RA_OK;
        RA_HIP(hipEventRecord((*pool)[idx + 1], s));
        spans.emplace_back(idx, kind);
        return RA_OK;
    }
};

}  // namespace

extern "C" {

ra_status ra_ring_workspace_size(const ra_ring_desc* d, size_t* bytes) {
    ra_status st = check_ring(d);
    if (st != RA_OK) return st;
    if (!bytes) return fail(RA_ERR_INVALID, "null bytes pointer");
    *bytes = geometry(d).total;
    return RA_OK;
}

}  // extern "C"

namespace {

// The ring forward.  own_streams: positions run on library-owned streams
// forked from and joined back to `stream` with events (created on first use);
// otherwise every launch goes to `stream` itself, in order, and no stream or
// event is created or recorded (stats and emulate_copy must then be off).
ra_status ring_forward_run(const ra_ring_desc* d, const void* q, const void* k, const void* v, void* o,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream, bool own_streams) {
    ra_status st = check_ring(d);
    if (st != RA_OK) return st;
    if (!q || !k || !v || !o) return fail(RA_ERR_INVALID, "null q / k / v / o pointer");
    const size_t es = elem_size(d->dtype);
    if (!aligned_to(q, es) || !aligned_to(k, es) || !aligned_to(v, es) || !aligned_to(o, es) ||
        (lse && !aligned_to(lse, 4)))
        return fail(RA_ERR_INVALID, "misaligned pointer");
    const RingGeometry g = geometry(d);
    if (!workspace || workspace_bytes < g.total)
        return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", g.total,
                    workspace ? workspace_bytes : size_t(0));
    if (!aligned_to(workspace, 256)) return fail(RA_ERR_INVALID, "workspace must be 256-byte aligned");

    const int32_t N = d->n_pos, D = d->head_dim;
    const int64_t Sb = d->block_len;
    const hipStream_t caller = static_cast<hipStream_t>(stream);

    // carve the workspace
    char* ws = static_cast<char*>(workspace);
    struct PosBufs {
        float *o[2], *m[2], *l[2];  // running state of each accumulation chain
        char* slot[2][2];           // [parity][K=0 / V=1]
    };
    std::vector<PosBufs> pos(d->n_run);
    for (int p = 0; p < d->n_run; ++p) {
        for (int c = 0; c < g.n_chains; ++c) {
            pos[p].o[c] = reinterpret_cast<float*>(ws);
            ws += g.acc_o;
            pos[p].m[c] = reinterpret_cast<float*>(ws);
            ws += g.acc_ml;
            pos[p].l[c] = reinterpret_cast<float*>(ws);
            ws += g.acc_ml;
        }
        for (int par = 0; par < 2; ++par)
            for (int kv = 0; kv < 2; ++kv) {
                pos[p].slot[par][kv] = d->emulate_copy ? ws : nullptr;
                ws += g.slot;
            }
    }
    struct StreamBufs {
        float *o, *m, *l;
        uint32_t* queue;
    };
    std::vector<StreamBufs> part(g.n_streams);  // partial i at o + i part_o, m / l + i part_ml
    for (int s = 0; s < g.n_streams; ++s) {
        part[s].o = reinterpret_cast<float*>(ws);
        ws += g.n_part * g.part_o;
        part[s].m = reinterpret_cast<float*>(ws);
        ws += g.n_part * g.part_ml;
        part[s].l = reinterpret_cast<float*>(ws);
        ws += g.n_part * g.part_ml;
        part[s].queue = reinterpret_cast<uint32_t*>(ws);
        ws += g.queue;
    }

    std::vector<std::vector<RingPlanStep>> plan(d->n_run);
    std::vector<int> n_computed(d->n_run, 0);
    ra_ring_stats stats{};
    for (int p = 0; p < d->n_run; ++p) {
        plan[p] = plan_position(d, d->first_pos + p);
        for (const auto& ps : plan[p]) {
            if (ps.skip) {
                ++stats.blocks_skipped;
            } else {
                ++n_computed[p];
                stats.unmasked_pairs += static_cast<double>(ra_unmasked_pairs(Sb, Sb, d->causal, ps.offset)) *
                                        d->batch * d->q_heads;
            }
        }
    }
    stats.flops = 4.0 * D * stats.unmasked_pairs;
    stats.kv_splits = 1;

    if (!own_streams && (d->stats || d->emulate_copy))
        return fail(RA_ERR_UNSUPPORTED, "stats and emulate_copy need library streams and events");
    std::lock_guard<std::mutex> lock(g_mutex);
    int dev = 0;
    RA_HIP(hipGetDevice(&dev));
    DeviceState no_state;
    DeviceState& ds = own_streams ? g_devices[dev] : no_state;
    if (own_streams) {
        st = ensure_streams(ds, g.n_streams);
        if (st != RA_OK) return st;
        // sync events: fork, per-stream join, per (position, parity) copied /
        // used, and the join of a second accumulation chain
        const size_t n_sync = 2 + g.n_streams + 4 * static_cast<size_t>(d->n_run);
        st = ensure_events(ds.sync_events, n_sync, hipEventDisableTiming);
        if (st != RA_OK) return st;
    }
    auto ev_fork = [&]() { return ds.sync_events[0]; };
    auto ev_join = [&](int s) { return ds.sync_events[1 + s]; };
    auto ev_copied = [&](int p, int par) { return ds.sync_events[1 + g.n_streams + 4 * p + par]; };
    auto ev_used = [&](int p, int par) { return ds.sync_events[1 + g.n_streams + 4 * p + 2 + par]; };
    auto ev_chain = [&]() { return ds.sync_events[1 + g.n_streams + 4 * static_cast<size_t>(d->n_run)]; };
    // the stream position p's work (and the queue counters of stream slot s) run on
    auto compute_stream = [&](int s) { return own_streams ? ds.compute[s] : caller; };

    Timer timer;
    if (d->stats) timer.pool = &ds.timing_events;

    // Work queues pay off when a block launch has many more query tiles than
    // the GPU has compute units (each workgroup then loops over several and
    // the XCDs can even out); a launch with fewer tiles keeps one workgroup
    // per tile in the fixed order, as the claims would only add latency.
    const int64_t launch_tiles = (Sb + ra::mfma_query_tile() - 1) / ra::mfma_query_tile() * d->q_heads *
                                 d->batch * g.n_splits;
    const bool use_queue = launch_tiles >= 2 * static_cast<int64_t>(ra::compute_units());

    if (own_streams) RA_HIP(hipEventRecord(ev_fork(), caller));
    for (int s = 0; s < g.n_streams; ++s) {
        if (own_streams) {
            RA_HIP(hipStreamWaitEvent(ds.compute[s], ev_fork(), 0));
            if (d->emulate_copy) RA_HIP(hipStreamWaitEvent(ds.copy[s], ev_fork(), 0));
        }
        // the stream's tile-queue counters start at zero (each block launch
        // leaves them so); a fill kernel, not a memset, so that the call can be
        // captured in a graph
        if (use_queue) {
            const hipError_t e = ra::launch_fill_zero(reinterpret_cast<float*>(part[s].queue),
                                                      static_cast<int64_t>(g.queue / 4), compute_stream(s));
            if (e != hipSuccess) return hip_fail(e, "queue reset launch");
        }
    }

    const char* kb = static_cast<const char*>(k);
    const char* vb = static_cast<const char*>(v);
    const size_t kv_bytes = static_cast<size_t>(g.kv_elems) * es;
    std::vector<char> used_parity(2 * d->n_run, 0);

    // emulated transfer of block j into position p's slot `par`
    auto issue_copy = [&](int p, int par, int32_t j) -> ra_status {
        const hipStream_t xs = ds.copy[p % g.n_streams];
        if (used_parity[2 * p + par]) RA_HIP(hipStreamWaitEvent(xs, ev_used(p, par), 0));
        size_t t0 = 0;
        ra_status s2 = timer.begin(xs, t0);
        if (s2 != RA_OK) return s2;
        RA_HIP(hipMemcpyAsync(pos[p].slot[par][0], kb + static_cast<size_t>(j) * kv_bytes, kv_bytes,
                              hipMemcpyDeviceToDevice, xs));
        RA_HIP(hipMemcpyAsync(pos[p].slot[par][1], vb + static_cast<size_t>(j) * kv_bytes, kv_bytes,
                              hipMemcpyDeviceToDevice, xs));
        s2 = timer.end(xs, t0, 2);
        if (s2 != RA_OK) return s2;
        RA_HIP(hipEventRecord(ev_copied(p, par), xs));
        return RA_OK;
    };

    if (d->emulate_copy)
        for (int p = 0; p < d->n_run; ++p) {
            st = issue_copy(p, 0, plan[p][0].block);
            if (st != RA_OK) return st;
        }

    std::vector<int> done(d->n_run, 0);
    const char* qbase = static_cast<const char*>(q);
    char* obase = static_cast<char*>(o);
    for (int32_t s = 0; s < N; ++s) {
        for (int p = 0; p < d->n_run; ++p) {
            const RingPlanStep& ps = plan[p][s];
            // the chain (and stream) of this position's next computed step
            const int chain = done[p] % g.n_chains;
            const int sid = g.n_chains > 1 ? chain : p % g.n_streams;
            const hipStream_t cs = compute_stream(sid);
            const int par = s & 1;
            const void* kp = kb + static_cast<size_t>(ps.block) * kv_bytes;
            const void* vp = vb + static_cast<size_t>(ps.block) * kv_bytes;
            if (d->emulate_copy) {
                kp = pos[p].slot[par][0];
                vp = pos[p].slot[par][1];
            }
            if (!ps.skip) {
                if (d->emulate_copy) RA_HIP(hipStreamWaitEvent(cs, ev_copied(p, par), 0));
                const bool first = done[p] < g.n_chains;  // the chain's first step: it writes its state
                const bool last = done[p] + 1 == n_computed[p];
                const bool fused = !d->separate_merge;
                ra::BlockArgs a{};
                a.q = qbase + static_cast<size_t>(p) * g.q_elems * es;
                a.k = kp;
                a.v = vp;
                const bool into_acc = first || fused;
                a.o = into_acc ? pos[p].o[chain] : part[sid].o;
                a.m = into_acc ? pos[p].m[chain] : part[sid].m;
                a.l = into_acc ? pos[p].l[chain] : part[sid].l;
                a.accumulate = (fused && !first) ? 1 : 0;
                a.B = d->batch;
                a.Hq = d->q_heads;
                a.Hkv = d->kv_heads;
                a.D = D;
                a.q_len = static_cast<int32_t>(Sb);
                a.kv_len = static_cast<int32_t>(Sb);
                a.qs[0] = static_cast<int64_t>(d->q_heads) * Sb * D;
                a.qs[1] = Sb * D;
                a.qs[2] = D;
                a.ks[0] = a.vs[0] = static_cast<int64_t>(d->kv_heads) * Sb * D;
                a.ks[1] = a.vs[1] = Sb * D;
                a.ks[2] = a.vs[2] = D;
                a.scale = resolve_scale(d->scale, D);
                a.causal = d->causal;
                a.mask_offset = clamp_offset(ps.offset, Sb, Sb);
                a.queue = use_queue ? part[sid].queue : nullptr;  // launches on one stream run in turn
                const bool split = g.n_splits > 1 && ra::mfma_eligible(a, d->dtype);
                if (split) {  // the block's key ranges as partials, folded by the merge below
                    stats.kv_splits = g.n_splits;
                    a.o = part[sid].o;
                    a.m = part[sid].m;
                    a.l = part[sid].l;
                    a.accumulate = 0;
                    a.n_splits = g.n_splits;
                    a.split_tiles = g.split_tiles;
                    a.part_o_stride = static_cast<int64_t>(g.part_o / 4);
                    a.part_ml_stride = static_cast<int64_t>(g.part_ml / 4);
                }
                size_t t0 = 0;
                st = timer.begin(cs, t0);
                if (st != RA_OK) return st;
                st = launch_block(a, d->dtype, 0u, cs);
                if (st != RA_OK) return st;
                st = timer.end(cs, t0, 0);
                if (st != RA_OK) return st;
                if (d->emulate_copy) {
                    RA_HIP(hipEventRecord(ev_used(p, par), cs));
                    used_parity[2 * p + par] = 1;
                }
                if ((!first && !fused) || last || split) {
                    ra::MergeArgs ma{};
                    ma.rows = g.rows;
                    ma.D = D;
                    ma.o_acc = pos[p].o[chain];
                    ma.m_acc = pos[p].m[chain];
                    ma.l_acc = pos[p].l[chain];
                    if ((!first && !fused) || split) {
                        ma.o_p = part[sid].o;
                        ma.m_p = part[sid].m;
                        ma.l_p = part[sid].l;
                    }
                    if (last && g.n_chains > 1 && n_computed[p] > 1) {
                        // the other chain's state is the partial folded in by
                        // the finalising pass, once that chain's stream is done
                        const int other = 1 - chain;
                        RA_HIP(hipEventRecord(ev_chain(), compute_stream(other)));
                        RA_HIP(hipStreamWaitEvent(cs, ev_chain(), 0));
                        ma.o_p = pos[p].o[other];
                        ma.m_p = pos[p].m[other];
                        ma.l_p = pos[p].l[other];
                    }
                    if (split) {
                        ma.n_parts = g.n_splits;
                        ma.part_o_stride = static_cast<int64_t>(g.part_o / 4);
                        ma.part_ml_stride = static_cast<int64_t>(g.part_ml / 4);
                        ma.acc_valid = first ? 0 : 1;
                    }
                    if (last) {
                        ma.o_out = obase + static_cast<size_t>(p) * g.q_elems * es;
                        ma.out_dtype = d->dtype;
                        ma.lse_out = lse ? lse + static_cast<size_t>(p) * g.rows : nullptr;
                    }
                    st = timer.begin(cs, t0);
                    if (st != RA_OK) return st;
                    hipError_t e = ra::launch_lse_merge(ma, cs);
                    if (e != hipSuccess) return hip_fail(e, "lse merge launch");
                    st = timer.end(cs, t0, 1);
                    if (st != RA_OK) return st;
                }
                ++done[p];
            }
            if (d->emulate_copy && s + 1 < N) {
                st = issue_copy(p, (s + 1) & 1, plan[p][s + 1].block);
                if (st != RA_OK) return st;
            }
        }
    }

    for (int s = 0; s < g.n_streams && own_streams; ++s) {
        if (d->emulate_copy) {
            // the copy stream's tail must also be joined before the caller reuses the slots
            RA_HIP(hipEventRecord(ev_join(s), ds.copy[s]));
            RA_HIP(hipStreamWaitEvent(ds.compute[s], ev_join(s), 0));
        }
        RA_HIP(hipEventRecord(ev_join(s), ds.compute[s]));
        RA_HIP(hipStreamWaitEvent(caller, ev_join(s), 0));
    }

    if (d->stats) {
        RA_HIP(hipStreamSynchronize(caller));
        for (const auto& sp : timer.spans) {
            float ms = 0.f;
            RA_HIP(hipEventElapsedTime(&ms, ds.timing_events[sp.first], ds.timing_events[sp.first + 1]));
            if (sp.second == 0) {
                stats.block_ms += ms;
                ++stats.block_launches;
            } else if (sp.second == 1) {
                stats.merge_ms += ms;
                ++stats.merge_launches;
            } else {
                stats.copy_ms += ms;
                ++stats.copy_launches;
            }
        }
        *d->stats = stats;
    }
    return RA_OK;
}

}  // namespace

namespace ra {
ra_status set_error(ra_status s, const char* msg) { return fail(s, "%s", msg); }

ra_status ring_forward_on_stream(const ra_ring_desc* d, const void* q, const void* k, const void* v, void* o,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    return ring_forward_run(d, q, k, v, o, lse, workspace, workspace_bytes, stream, false);
}
}  // namespace ra

extern "C" {

ra_status ra_ring_forward(const ra_ring_desc* d, const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return ring_forward_run(d, q, k, v, o, lse, workspace, workspace_bytes, stream, true);
}

// ------------------------------------------------------------------ backward
ra_status ra_attn_bwd_delta(int64_t rows, int32_t head_dim, int32_t dtype, const void* o, const void* dout,
                            float* delta, void* stream) {
    if (rows < 0) return fail(RA_ERR_INVALID, "rows must be >= 0");
    if (head_dim < 1) return fail(RA_ERR_INVALID, "head_dim must be >= 1");
    if (!valid_dtype(dtype)) return fail(RA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (rows == 0) return RA_OK;
    if (!o || !dout || !delta) return fail(RA_ERR_INVALID, "null pointer");
    if (!aligned_to(o, elem_size(dtype)) || !aligned_to(dout, elem_size(dtype)) || !aligned_to(delta, 4))
        return fail(RA_ERR_INVALID, "misaligned pointer");
    hipError_t e = ra::launch_bwd_delta(rows, head_dim, dtype, o, dout, delta, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "delta launch");
    return RA_OK;
}

namespace {
// Validates a backward block call and fills its kernel arguments; *empty is
// set when the call is a valid no-op (q_len or kv_len zero).
ra_status block_bwd_args(const ra_block_desc* d, const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, const float* delta, float* dq, float* dk, float* dv, ra::BwdArgs* out,
                         bool* empty) {
    *empty = false;
    if (!d) return fail(RA_ERR_INVALID, "null descriptor");
    ra_status st = check_heads(d->batch, d->q_heads, d->kv_heads, d->head_dim, d->dtype);
    if (st != RA_OK) return st;
    if (d->q_len < 0 || d->kv_len < 0 || d->q_len > kMaxLen || d->kv_len > kMaxLen)
        return fail(RA_ERR_INVALID, "q_len / kv_len out of range");
    if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_INVALID, "causal must be 0 or 1");
    if (d->flags & ~RA_BLOCK_FORCE_SIMT) return fail(RA_ERR_UNSUPPORTED, "unknown flags 0x%x", d->flags);
    if (d->pos_stride < 1) return fail(RA_ERR_INVALID, "pos_stride must be >= 1");
    if (!std::isfinite(d->scale)) return fail(RA_ERR_INVALID, "scale must be finite");
    for (int i = 0; i < 3; ++i)
        if (d->q_strides[i] < 0 || d->k_strides[i] < 0 || d->v_strides[i] < 0)
            return fail(RA_ERR_INVALID, "strides must be non-negative");
    if (d->q_len == 0 || d->kv_len == 0) {
        *empty = true;
        return RA_OK;
    }
    if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv)
        return fail(RA_ERR_INVALID, "null pointer");
    const size_t es = elem_size(d->dtype);
    if (!aligned_to(q, es) || !aligned_to(k, es) || !aligned_to(v, es) || !aligned_to(dout, es) ||
        !aligned_to(lse, 4) || !aligned_to(delta, 4) || !aligned_to(dq, 4) || !aligned_to(dk, 4) || !aligned_to(dv, 4))
        return fail(RA_ERR_INVALID, "misaligned pointer");
    ra::BwdArgs& a = *out;
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = d->batch;
    a.Hq = d->q_heads;
    a.Hkv = d->kv_heads;
    a.D = d->head_dim;
    a.q_len = static_cast<int32_t>(d->q_len);
    a.kv_len = static_cast<int32_t>(d->kv_len);
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = d->q_strides[i];
        a.dos[i] = d->q_strides[i];
        a.ks[i] = d->k_strides[i];
        a.vs[i] = d->v_strides[i];
    }
    a.scale = resolve_scale(d->scale, d->head_dim);
    a.causal = d->causal;
    a.mask_offset = clamp_offset(ra_mask_offset(d->q_pos0, d->k_pos0, d->pos_stride), d->q_len, d->kv_len);
    return RA_OK;
}
}  // namespace

ra_status ra_block_attn_bwd(const ra_block_desc* d, const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, const float* delta, float* dq, float* dk, float* dv, void* stream) {
    ra::BwdArgs a{};
    bool empty = false;
    const ra_status st = block_bwd_args(d, q, k, v, dout, lse, delta, dq, dk, dv, &a, &empty);
    if (st != RA_OK || empty) return st;
    const hipError_t e = ra::launch_block_bwd(a, d->dtype, d->flags & RA_BLOCK_FORCE_SIMT, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "block backward launch");
    return RA_OK;
}

int32_t ra_block_attn_bwd_kernel(const ra_block_desc* d, const void* q, const void* k, const void* v,
                                 const void* dout, const float* lse, const float* delta, const float* dq,
                                 const float* dk, const float* dv) {
    ra::BwdArgs a{};
    bool empty = false;
    if (block_bwd_args(d, q, k, v, dout, lse, delta, const_cast<float*>(dq), const_cast<float*>(dk),
                       const_cast<float*>(dv), &a, &empty) != RA_OK)
        return -1;
    if (empty) return 0;
    return (!(d->flags & RA_BLOCK_FORCE_SIMT) && ra::bwd_mfma_eligible(a, d->dtype)) ? 1 : 0;
}

ra_status ra_ring_bwd_workspace_size(const ra_ring_desc* d, size_t* bytes) {
    ra_status st = check_ring(d);
    if (st != RA_OK) return st;
    if (!bytes) return fail(RA_ERR_INVALID, "null bytes pointer");
    const int64_t rows = static_cast<int64_t>(d->batch) * d->q_heads * d->block_len;
    *bytes = round_up(static_cast<size_t>(d->n_run) * static_cast<size_t>(rows) * 4, 256);
    return RA_OK;
}

ra_status ra_ring_backward(const ra_ring_desc* d, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, float* dq, float* dk, float* dv, void* workspace,
                           size_t workspace_bytes, void* stream) {
    ra_status st = check_ring(d);
    if (st != RA_OK) return st;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return fail(RA_ERR_INVALID, "null pointer");
    const size_t es = elem_size(d->dtype);
    if (!aligned_to(q, es) || !aligned_to(k, es) || !aligned_to(v, es) || !aligned_to(o, es) ||
        !aligned_to(dout, es) || !aligned_to(lse, 4) || !aligned_to(dq, 4) || !aligned_to(dk, 4) || !aligned_to(dv, 4))
        return fail(RA_ERR_INVALID, "misaligned pointer");
    size_t need = 0;
    ra_ring_bwd_workspace_size(d, &need);
    if (!workspace || workspace_bytes < need)
        return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : size_t(0));
    if (!aligned_to(workspace, 256)) return fail(RA_ERR_INVALID, "workspace must be 256-byte aligned");

    const int32_t N = d->n_pos, D = d->head_dim;
    const int64_t Sb = d->block_len;
    const int64_t rows = static_cast<int64_t>(d->batch) * d->q_heads * Sb;
    const int64_t q_elems = rows * D;
    const int64_t kv_elems = static_cast<int64_t>(d->batch) * d->kv_heads * Sb * D;
    const hipStream_t caller = static_cast<hipStream_t>(stream);
    float* delta = static_cast<float*>(workspace);

    std::vector<std::vector<RingPlanStep>> plan(d->n_run);
    ra_ring_stats stats{};
    for (int p = 0; p < d->n_run; ++p) {
        plan[p] = plan_position(d, d->first_pos + p);
        for (const auto& ps : plan[p]) {
            if (ps.skip) ++stats.blocks_skipped;
            else
                stats.unmasked_pairs += static_cast<double>(ra_unmasked_pairs(Sb, Sb, d->causal, ps.offset)) *
                                        d->batch * d->q_heads;
        }
    }
    stats.flops = 10.0 * D * stats.unmasked_pairs;  // five products of 2 d FLOPs per pair

    std::lock_guard<std::mutex> lock(g_mutex);
    int dev = 0;
    RA_HIP(hipGetDevice(&dev));
    DeviceState& ds = g_devices[dev];
    Timer timer;
    if (d->stats) timer.pool = &ds.timing_events;
    // the positions of one step write disjoint dq and dk / dv, so they may run
    // on n_streams library streams, forked from the caller's stream before
    // every step and joined back after it (the next step hands every block to
    // another position).  Automatic: one stream when each of a launch's two
    // kernels already holds a workgroup per compute unit (concurrent launches
    // then only contend for the same units: measured slower), else
    // min(n_run, 8).
    int n_streams = d->n_streams > 0 ? std::min(d->n_streams, d->n_run) : std::min(d->n_run, 8);
    if (d->n_streams == 0 && d->dtype == RA_BF16 && (D == 64 || D == 128)) {
        ra::BwdArgs g{};
        g.B = d->batch;
        g.Hq = d->q_heads;
        g.Hkv = d->kv_heads;
        g.q_len = g.kv_len = static_cast<int32_t>(Sb);
        if (ra::bwd_mfma_min_workgroups(g) >= ra::compute_units()) n_streams = 1;
    }
    if (n_streams > 1) {
        st = ensure_streams(ds, n_streams);
        if (st != RA_OK) return st;
        st = ensure_events(ds.bwd_events, 1 + static_cast<size_t>(n_streams), hipEventDisableTiming);
        if (st != RA_OK) return st;
    }

    // gradients start at zero (fill kernels: no memset nodes under graph capture)
    hipError_t e = ra::launch_fill_zero(dq, static_cast<int64_t>(d->n_run) * q_elems, caller);
    if (e == hipSuccess) e = ra::launch_fill_zero(dk, static_cast<int64_t>(N) * kv_elems, caller);
    if (e == hipSuccess) e = ra::launch_fill_zero(dv, static_cast<int64_t>(N) * kv_elems, caller);
    if (e == hipSuccess) e = ra::launch_bwd_delta(static_cast<int64_t>(d->n_run) * rows, D, d->dtype, o, dout, delta, caller);
    if (e != hipSuccess) return hip_fail(e, "backward set-up launch");

    // Lockstep over steps, as on a real ring: at step s position i holds block
    // j = (i - visit[s]) mod N, distinct across positions, and adds its share
    // into that block's dK, dV (which travel with the block) and into its own
    // dQ.  Position p's launches go to stream p mod n_streams.
    for (int32_t s = 0; s < N; ++s) {
        if (n_streams > 1) {
            RA_HIP(hipEventRecord(ds.bwd_events[0], caller));
            for (int i = 0; i < n_streams; ++i) RA_HIP(hipStreamWaitEvent(ds.compute[i], ds.bwd_events[0], 0));
        }
        for (int p = 0; p < d->n_run; ++p) {
            const RingPlanStep& ps = plan[p][s];
            if (ps.skip) continue;
            const hipStream_t ps_stream = n_streams > 1 ? ds.compute[p % n_streams] : caller;
            ra::BwdArgs a{};
            const char* qb = static_cast<const char*>(q) + static_cast<size_t>(p) * q_elems * es;
            a.q = qb;
            a.dout = static_cast<const char*>(dout) + static_cast<size_t>(p) * q_elems * es;
            a.k = static_cast<const char*>(k) + static_cast<size_t>(ps.block) * kv_elems * es;
            a.v = static_cast<const char*>(v) + static_cast<size_t>(ps.block) * kv_elems * es;
            a.lse = lse + p * rows;
            a.delta = delta + p * rows;
            a.dq = dq + p * q_elems;
            a.dk = dk + ps.block * kv_elems;
            a.dv = dv + ps.block * kv_elems;
            a.B = d->batch;
            a.Hq = d->q_heads;
            a.Hkv = d->kv_heads;
            a.D = D;
            a.q_len = static_cast<int32_t>(Sb);
            a.kv_len = static_cast<int32_t>(Sb);
            a.qs[0] = static_cast<int64_t>(d->q_heads) * Sb * D;
            a.qs[1] = Sb * D;
            a.qs[2] = D;
            for (int i = 0; i < 3; ++i) a.dos[i] = a.qs[i];
            a.ks[0] = a.vs[0] = static_cast<int64_t>(d->kv_heads) * Sb * D;
            a.ks[1] = a.vs[1] = Sb * D;
            a.ks[2] = a.vs[2] = D;
            a.scale = resolve_scale(d->scale, D);
            a.causal = d->causal;
            a.mask_offset = clamp_offset(ps.offset, Sb, Sb);
            size_t ti = 0;
            st = timer.begin(ps_stream, ti);
            if (st != RA_OK) return st;
            e = ra::launch_block_bwd(a, d->dtype, 0, ps_stream);
            if (e != hipSuccess) return hip_fail(e, "block backward launch");
            st = timer.end(ps_stream, ti, 0);
            if (st != RA_OK) return st;
        }
        if (n_streams > 1) {
            for (int i = 0; i < n_streams; ++i) {
                RA_HIP(hipEventRecord(ds.bwd_events[1 + i], ds.compute[i]));
                RA_HIP(hipStreamWaitEvent(caller, ds.bwd_events[1 + i], 0));
            }
        }
    }
    if (d->stats) {
        RA_HIP(hipStreamSynchronize(caller));
        for (const auto& sp : timer.spans) {
            float ms = 0.f;
            RA_HIP(hipEventElapsedTime(&ms, ds.timing_events[sp.first], ds.timing_events[sp.first + 1]));
            stats.block_ms += ms;
            ++stats.block_launches;
        }
        *d->stats = stats;
    }
    return RA_OK;
}

void ra_release(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_devices) {
        (void)hipSetDevice(kv.first);
        for (auto s : kv.second.compute) (void)hipStreamDestroy(s);
        for (auto s : kv.second.copy) (void)hipStreamDestroy(s);
        for (auto e : kv.second.sync_events) (void)hipEventDestroy(e);
        for (auto e : kv.second.timing_events) (void)hipEventDestroy(e);
        for (auto e : kv.second.bwd_events) (void)hipEventDestroy(e);
    }
    g_devices.clear();
    (void)hipSetDevice(cur);
}

}  // extern "C"
