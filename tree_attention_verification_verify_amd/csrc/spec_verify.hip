// Host side of libspecverify: C ABI, validation, workspace and launch order.
//
// A run enqueues, on the caller's stream and without synchronising:
//   tree attention (MFMA or VALU kernel) -> split merge (when split)
//   row statistics of every target / draft logits row (one read)
//   selection (ratios, decisions, longest accepted path, final draw at v*)
// The attention and the vocabulary work read disjoint inputs: when the
// attention grid leaves at least half of the CUs idle (one sequence, few KV
// heads) and the rows need no top-p cut, the attention launch also carries the
// row statistics in workgroups of their own, so both run at once.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "spec_verify.h"

namespace sv {
int valu_rows_for(int R);
}

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return SPEC_VERIFY_ERR_HIP;
}

constexpr int kTimingRing = 1024;
constexpr int kEventsPerRun = SPEC_VERIFY_NUM_STAGES + 1;
constexpr int kTargetWaves = 2048;   // two waves per SIMD on 256 CUs
// Each prefix split takes at least this many keys: at the llama7b-medusa-greedy
// shape (2112 slots, 32 KV heads, one sequence) 6 splits (192 attention
// workgroups, with the 64 row-statistics workgroups beside them on 256 CUs)
// take 19.7 us per step against 20.2 us for 4 or 5; 7 would leave no room
// for the statistics.
constexpr int kMinSplitKeys = 352;
// The vector-ALU kernels' workgroups are small and latency-bound: one 64-key
// tile per split already pays (the tiny fp32 chain, 133 slots on 4 heads).
constexpr int kMinSplitKeysValu = 64;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnPlan {
    bool mfma = false;
    bool tiled = false;     // VALU path: 4-wave tiled kernel (few rows per KV head)
    int waves = 1;          // waves per block
    int rows_per_block = 0;
    int rowblocks = 1;
    int Rpad = 0;
    int nsplit = 1;
    int chunk = 0;
    size_t part_rows = 0;   // pairs * nsplit * Rpad
    bool stream = false;    // K/V tiles loaded with the non-temporal policy
};

// K/V tiles stream with the non-temporal cache policy when no other workgroup
// reads them (one row block) and the call's caches are too large to stay in
// the last-level cache anyway (more than a quarter of its 256 MiB, taking the
// capacity as the bound).  Smaller caches keep the default policy, so calls
// that follow each other over the same cache find it there (measured at the
// llama7b Medusa shape, 35 MB of K/V: 29.9 us per step non-temporal, 27.9
// with the default policy; at the long-context shape, 2.1 GB: 471 us with the
// default policy, 426 us non-temporal).
constexpr size_t kStreamMinBytes = size_t(64) << 20;

// max_part_rows: the split partials must fit this many rows (fewer splits
// otherwise; one split needs none).
AttnPlan plan_attention(const spec_verify_config& c, int B, int T, size_t max_part_rows = SIZE_MAX) {
    AttnPlan p;
    const int g = c.num_q_heads / c.num_kv_heads;
    const int R = g * T;
    p.mfma = (c.dtype == SPEC_VERIFY_BF16) && R >= 16;
    if (p.mfma) {
        p.waves = std::min(4, (R + 31) / 32);
        p.rows_per_block = 32 * p.waves;
    } else {
        p.tiled = sv::valu_tiled_supported(c.dtype == SPEC_VERIFY_BF16, c.head_dim, R);
        p.waves = p.tiled ? 4 : 1;
        p.rows_per_block = sv::valu_rows_for(R);
    }
    p.rowblocks = (R + p.rows_per_block - 1) / p.rows_per_block;
    p.Rpad = p.rowblocks * p.rows_per_block;
    const size_t elem = c.dtype == SPEC_VERIFY_BF16 ? 2 : 4;
    const size_t kv_bytes = 2 * (size_t)B * c.num_kv_heads * (size_t)c.kv_capacity * c.head_dim * elem;
    p.stream = p.rowblocks == 1 && kv_bytes > kStreamMinBytes;
    const long pairs = (long)B * c.num_kv_heads;
    const long base_waves = pairs * p.rowblocks * p.waves * (p.mfma ? sv::kMfmaHalves : 1);
    long want = (kTargetWaves + base_waves - 1) / base_waves;
    const long keys = c.kv_capacity;
    const long max_split = std::max(1L, keys / (p.mfma ? kMinSplitKeys : kMinSplitKeysValu));
    long ns = std::max(1L, std::min(want, max_split));
    for (;;) {
        long chunk = (keys + ns - 1) / ns;
        chunk = ((chunk + 63) / 64) * 64;
        const long n = (keys + chunk - 1) / chunk;
        p.nsplit = (int)n;
        p.chunk = (int)chunk;
        p.part_rows = n > 1 ? (size_t)pairs * n * p.Rpad : 0;
        if (p.part_rows <= max_part_rows || ns == 1) break;
        --ns;
    }
    return p;
}

// Checks of a paged cache description against the config; fills pt and the
// slots a sequence can address.  SPEC_VERIFY_OK or INVALID_ARG.
int check_paged(const spec_verify_config& c, const spec_verify_paged_kv* pg, sv::PageTable* pt, int* slots) {
    if (!pg) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "paged is NULL");
    if (!pg->k_pool || !pg->v_pool || !pg->block_table)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "k_pool, v_pool and block_table must be non-NULL");
    if ((((uintptr_t)pg->k_pool) & 15u) || (((uintptr_t)pg->v_pool) & 15u))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "k_pool and v_pool must be 16-byte aligned");
    if (((uintptr_t)pg->block_table) & 3u) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
    if (pg->num_blocks < 1) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "num_blocks must be >= 1");
    const int bs = pg->block_size;
    if (bs < 16 || bs > 65536 || (bs & (bs - 1)) != 0)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "block_size must be a power of two in [16, 65536]");
    if (pg->table_width < 1) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "table_width must be >= 1");
    if ((long long)pg->table_width * bs > c.kv_capacity)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "table_width * block_size exceeds kv_capacity");
    int lg = 0;
    while ((1 << lg) < bs) ++lg;
    pt->table = pg->block_table;
    pt->width = pg->table_width;
    pt->bs_log2 = lg;
    pt->num_blocks = pg->num_blocks;
    *slots = pg->table_width * bs;
    return SPEC_VERIFY_OK;
}

// Every host-checkable fault of a configuration (before any HIP call).
int validate_config(const spec_verify_config& c) {
    if (c.max_batch < 1) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "max_batch must be >= 1");
    if (c.max_nodes < 1 || c.max_nodes > 64) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "max_nodes must be in [1, 64]");
    if (c.num_q_heads < 1 || c.num_kv_heads < 1) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "head counts must be >= 1");
    if (c.num_q_heads % c.num_kv_heads != 0)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
    if ((long)(c.num_q_heads / c.num_kv_heads) * c.max_nodes > 65536)
        return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "too many query rows per KV head");
    if (c.head_dim != 64 && c.head_dim != 128) return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (c.kv_capacity < c.max_nodes) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "kv_capacity must be >= max_nodes");
    if (c.vocab < 1 || c.vocab > sv::kVocabChunk * 128)
        return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "vocab must be in [1, 4194304]");
    if (c.dtype != SPEC_VERIFY_F32 && c.dtype != SPEC_VERIFY_BF16)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "dtype must be SPEC_VERIFY_F32 or SPEC_VERIFY_BF16");
    if (c.mode != SPEC_VERIFY_GREEDY && c.mode != SPEC_VERIFY_SAMPLING)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "mode must be SPEC_VERIFY_GREEDY or SPEC_VERIFY_SAMPLING");
    if (c.mode == SPEC_VERIFY_SAMPLING) {
        if (!(c.temperature > 0.f) || !std::isfinite(c.temperature))
            return fail(SPEC_VERIFY_ERR_INVALID_ARG, "temperature must be a finite value > 0");
        if (!(c.top_p > 0.f && c.top_p <= 1.f)) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "top_p must be in (0, 1]");
    }
    if (!(c.softmax_scale >= 0.f) || !std::isfinite(c.softmax_scale))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    constexpr uint32_t kKnownFlags = SPEC_VERIFY_FLAG_TIMING | SPEC_VERIFY_FLAG_LOSSLESS_TREE |
                                     SPEC_VERIFY_FLAG_SKIP_ATTENTION | SPEC_VERIFY_FLAG_SKIP_VOCAB |
                                     SPEC_VERIFY_FLAG_WRITE_PROBS | SPEC_VERIFY_FLAG_WALK_NO_WAIT;
    if ((c.flags & ~kKnownFlags) != 0u) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "unknown flag bits");
    if ((c.flags & SPEC_VERIFY_FLAG_LOSSLESS_TREE) && c.mode != SPEC_VERIFY_SAMPLING)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "SPEC_VERIFY_FLAG_LOSSLESS_TREE needs sampling mode");
    if ((c.flags & SPEC_VERIFY_FLAG_SKIP_ATTENTION) && (c.flags & SPEC_VERIFY_FLAG_SKIP_VOCAB))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "SKIP_ATTENTION and SKIP_VOCAB together leave nothing to run");
    if ((c.flags & SPEC_VERIFY_FLAG_WRITE_PROBS) && c.mode != SPEC_VERIFY_SAMPLING)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "SPEC_VERIFY_FLAG_WRITE_PROBS needs sampling mode");
    if ((c.flags & SPEC_VERIFY_FLAG_WRITE_PROBS) && (c.flags & SPEC_VERIFY_FLAG_SKIP_VOCAB))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "SPEC_VERIFY_FLAG_WRITE_PROBS needs the vocabulary pass");
    if ((c.flags & SPEC_VERIFY_FLAG_WALK_NO_WAIT) && !(c.flags & SPEC_VERIFY_FLAG_LOSSLESS_TREE))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "SPEC_VERIFY_FLAG_WALK_NO_WAIT needs SPEC_VERIFY_FLAG_LOSSLESS_TREE");
    // the attention kernels address one (sequence, KV head) slice of a cache
    // through a buffer resource with a 32-bit byte range
    const long long slab_bytes = (long long)c.kv_capacity * c.head_dim * (c.dtype == SPEC_VERIFY_BF16 ? 2 : 4);
    if (slab_bytes >= (1LL << 31))
        return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "kv_capacity * head_dim * element size must be below 2^31 bytes");

    return SPEC_VERIFY_OK;
}

}  // namespace

// Device workspace of a run: the handle's (allocated by create) or carved out
// of the static scratch array (spec_verify_run_noalloc).
struct Workspace {
    size_t part_rows_cap = 0;
    float* part_o = nullptr;
    float2* part_ml = nullptr;
    sv::RowStat* stats = nullptr;     // batch * 2 * nodes row statistics
    double2* slice_tot = nullptr;     // batch * slices final-draw slice totals
    double2* slice_pre = nullptr;     // batch * slices * 256 per-thread slice prefixes (few slices only; may be NULL)
    int32_t* arrive = nullptr;        // batch final-draw arrival counters (zero between runs)
    float* resid_ws = nullptr;        // max_batch * 2 * vocab residual rows (lossless tree walk)
    int32_t* walk_sync = nullptr;     // max_batch * 4 walk counters (lossless tree walk)
    double* walk_part = nullptr;      // max_batch * 2 * walk_k walk slice totals
    float* walk_rx = nullptr;         // max_batch * 4 walk test values
    int walk_k = 0;
    int walk_cap = 0;                 // largest B * walk_k launched across workgroups (all resident at once)
    int walk_spin = 0;                // polls of a walk wait before it gives up
    int cus = 0;                      // compute units of the device (0: never fuse the row statistics)
};

// Workgroups of the attention launch of a plan.
long attention_blocks(const AttnPlan& p, int B, int Hkv) {
    const long groups = (long)B * Hkv * p.nsplit;
    if (p.mfma) return p.rowblocks == 1 ? groups : ((groups + 7) / 8) * 8 * p.rowblocks;
    return p.tiled ? groups : groups * p.rowblocks;
}

// Whether the attention launch carries the row statistics (dense caches, no
// top-p cut, no per-stage timing):
//  * 256-thread attention workgroups (the statistics' size) with room on the
//    CUs for both grids at once: the statistics run beside the attention (at
//    the llama7b Medusa shape 128 attention and 64 statistics workgroups on
//    256 CUs);
//  * 512-thread MFMA workgroups that fill every CU, with rows of at most
//    rows::CHUNK logits and one workgroup of two rows per CU at most:
//    these follow the attention in the same launch and start on each CU as
//    its attention workgroup ends, with no launch boundary between the two
//    (the 70B GQA tree shape in greedy mode: 0.1542 -> 0.1526 ms per step).
//    A second round would hold one such workgroup per CU (the attention's
//    LDS), half the statistics kernel's loads in flight: in sampling mode
//    (1016 rows) that cost what the boundary saved.
bool fuse_row_stats(const Workspace& ws, const AttnPlan& p, int B, int Hkv, const sv::StatsParams& tp, bool paged,
                    bool timing) {
    const int threads = p.mfma ? p.waves * 64 * sv::kMfmaHalves : (p.tiled ? sv::kStatsThreads : 64);
    const long stats_blocks = (long)B * (tp.sampling ? 2 * tp.T : tp.T);
    if (paged || timing || ws.cus <= 0 || !sv::row_stats_streams(tp)) return false;
    if (threads == sv::kStatsThreads) return attention_blocks(p, B, Hkv) + stats_blocks <= ws.cus;
    return p.mfma && threads == 2 * sv::kStatsThreads && tp.V <= sv::kVocabChunk &&
           attention_blocks(p, B, Hkv) >= ws.cus && (stats_blocks + 1) / 2 <= ws.cus;
}

struct spec_verify_handle {
    spec_verify_config cfg;
    int device = 0;
    Workspace ws;
    int32_t* commit_arrive = nullptr; // max_batch KV-commit finish counters (zero between calls)
    unsigned long long* tree_cand = nullptr;   // tree building: per-slice best keys of every row
    int32_t* tree_arrive = nullptr;            // tree building: finished slices per row (zero between calls)
    bool timing = false;
    std::vector<hipEvent_t> events;   // kTimingRing * kEventsPerRun
    long runs_recorded = 0;           // since the last read
    long ring_head = 0;               // total runs recorded
};

extern "C" {

const char* spec_verify_last_error(void) { return g_err.c_str(); }

int spec_verify_create(const spec_verify_config* cfg, spec_verify_handle** out) {
    g_err.clear();
    if (!cfg || !out) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "cfg and out must be non-NULL");
    *out = nullptr;
    const spec_verify_config& c = *cfg;
    if (int rc = validate_config(c)) return rc;

    // workspace: the largest split-prefix partial buffer over every (B, T) a run may use
    size_t cap = 0;
    for (int B = 1; B <= c.max_batch; ++B)
        for (int T = 1; T <= c.max_nodes; ++T) cap = std::max(cap, plan_attention(c, B, T).part_rows);

    spec_verify_handle* h = new (std::nothrow) spec_verify_handle();
    if (!h) return fail(SPEC_VERIFY_ERR_OOM, "host allocation failed");
    h->cfg = c;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, "hipGetDevice");
    }
    h->ws.part_rows_cap = cap;
    e = hipDeviceGetAttribute(&h->ws.cus, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, "hipDeviceGetAttribute");
    }
    if (cap > 0) {
        e = hipMalloc((void**)&h->ws.part_o, cap * c.head_dim * sizeof(float));
        if (e == hipSuccess) e = hipMalloc((void**)&h->ws.part_ml, cap * sizeof(float2));
        if (e != hipSuccess) {
            (void)hipFree(h->ws.part_o);
            delete h;
            (void)hipGetLastError();
            return fail(SPEC_VERIFY_ERR_OOM, "workspace allocation failed");
        }
    }
    e = hipMalloc((void**)&h->ws.stats, (size_t)c.max_batch * 2 * c.max_nodes * sizeof(sv::RowStat));
    const int slices = (c.vocab + sv::kSelectSlice - 1) / sv::kSelectSlice;
    if (e == hipSuccess) e = hipMalloc((void**)&h->ws.slice_tot, (size_t)c.max_batch * slices * sizeof(double2));
    if (e == hipSuccess && c.mode == SPEC_VERIFY_SAMPLING && slices <= sv::kSelectKeepSlices)
        e = hipMalloc((void**)&h->ws.slice_pre, (size_t)c.max_batch * slices * sv::kSelectThreads * sizeof(double2));
    if (e == hipSuccess) e = hipMalloc((void**)&h->ws.arrive, (size_t)c.max_batch * sizeof(int32_t));
    if (e == hipSuccess) e = hipMemset(h->ws.arrive, 0, (size_t)c.max_batch * sizeof(int32_t));
    if (e == hipSuccess) e = hipMalloc((void**)&h->commit_arrive, (size_t)c.max_batch * sizeof(int32_t));
    if (e == hipSuccess) e = hipMemset(h->commit_arrive, 0, (size_t)c.max_batch * sizeof(int32_t));
    {
        const size_t rows = (size_t)c.max_batch * std::max(1, c.max_nodes - 1);   // (sequence, depth) rows
        if (e == hipSuccess) e = hipMalloc((void**)&h->tree_cand, rows * sv::kTreeMaxSlices * 32 * sizeof(unsigned long long));
        if (e == hipSuccess) e = hipMalloc((void**)&h->tree_arrive, rows * sizeof(int32_t));
        if (e == hipSuccess) e = hipMemset(h->tree_arrive, 0, rows * sizeof(int32_t));
    }
    if (e == hipSuccess && (c.flags & SPEC_VERIFY_FLAG_LOSSLESS_TREE)) {
        // the walk across workgroups waits for all of a sequence's workgroups,
        // so it is launched only while the grid fits twice per CU; larger
        // grids use one workgroup per sequence (with residual rows in HBM
        // beyond one on-chip chunk)
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device);
        h->ws.walk_k = (c.vocab + sv::kWalkSlice - 1) / sv::kWalkSlice;
        // as many workgroups as the CUs hold at once by the kernel's own resource use
        int per_cu = 0;
        if (e == hipSuccess) e = sv::walk_coop_blocks_per_cu(&per_cu);
        h->ws.walk_cap = per_cu * cus;
        h->ws.walk_spin = (c.flags & SPEC_VERIFY_FLAG_WALK_NO_WAIT) ? 0 : sv::kWalkSpinLimit;
        if (e == hipSuccess) e = hipMalloc((void**)&h->ws.walk_sync, (size_t)c.max_batch * 4 * sizeof(int32_t));
        if (e == hipSuccess) e = hipMemset(h->ws.walk_sync, 0, (size_t)c.max_batch * 4 * sizeof(int32_t));
        if (e == hipSuccess) e = hipMalloc((void**)&h->ws.walk_part, (size_t)c.max_batch * 2 * h->ws.walk_k * sizeof(double));
        if (e == hipSuccess) e = hipMemset(h->ws.walk_part, 0, (size_t)c.max_batch * 2 * h->ws.walk_k * sizeof(double));
        if (e == hipSuccess) e = hipMalloc((void**)&h->ws.walk_rx, (size_t)c.max_batch * 4 * sizeof(float));
        if (e == hipSuccess && (long)c.max_batch * h->ws.walk_k > h->ws.walk_cap && c.vocab > sv::kVocabChunk)
            e = hipMalloc((void**)&h->ws.resid_ws, (size_t)c.max_batch * 2 * c.vocab * sizeof(float));
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(h->ws.stats);
        (void)hipFree(h->ws.slice_tot);
        (void)hipFree(h->ws.slice_pre);
        (void)hipFree(h->ws.arrive);
        (void)hipFree(h->commit_arrive);
        (void)hipFree(h->tree_cand);
        (void)hipFree(h->tree_arrive);
        (void)hipFree(h->ws.resid_ws);
        (void)hipFree(h->ws.walk_sync);
        (void)hipFree(h->ws.walk_part);
        (void)hipFree(h->ws.walk_rx);
        (void)hipFree(h->ws.part_o);
        (void)hipFree(h->ws.part_ml);
        delete h;
        (void)hipGetLastError();
        return fail(SPEC_VERIFY_ERR_OOM, "workspace allocation failed");
    }
    h->timing = (c.flags & SPEC_VERIFY_FLAG_TIMING) != 0u;
    if (h->timing) {
        h->events.resize((size_t)kTimingRing * kEventsPerRun, nullptr);
        for (auto& ev : h->events) {
            e = hipEventCreate(&ev);
            if (e != hipSuccess) {
                spec_verify_destroy(h);
                return hip_fail(e, "hipEventCreate");
            }
        }
    }
    *out = h;
    return SPEC_VERIFY_OK;
}

int spec_verify_destroy(spec_verify_handle* h) {
    g_err.clear();
    if (!h) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "handle is NULL");
    int dev = -1;
    (void)hipGetDevice(&dev);
    if (dev != h->device) (void)hipSetDevice(h->device);
    for (auto& ev : h->events)
        if (ev) (void)hipEventDestroy(ev);
    if (h->ws.part_o) (void)hipFree(h->ws.part_o);
    if (h->ws.part_ml) (void)hipFree(h->ws.part_ml);
    if (h->ws.stats) (void)hipFree(h->ws.stats);
    if (h->ws.slice_tot) (void)hipFree(h->ws.slice_tot);
    if (h->ws.slice_pre) (void)hipFree(h->ws.slice_pre);
    if (h->ws.arrive) (void)hipFree(h->ws.arrive);
    if (h->commit_arrive) (void)hipFree(h->commit_arrive);
    if (h->tree_cand) (void)hipFree(h->tree_cand);
    if (h->tree_arrive) (void)hipFree(h->tree_arrive);
    if (h->ws.resid_ws) (void)hipFree(h->ws.resid_ws);
    if (h->ws.walk_sync) (void)hipFree(h->ws.walk_sync);
    if (h->ws.walk_part) (void)hipFree(h->ws.walk_part);
    if (h->ws.walk_rx) (void)hipFree(h->ws.walk_rx);
    if (dev >= 0 && dev != h->device) (void)hipSetDevice(dev);
    delete h;
    return SPEC_VERIFY_OK;
}

}  // extern "C"

namespace {

// Event ring of a handle created with SPEC_VERIFY_FLAG_TIMING.
struct TimingRing {
    std::vector<hipEvent_t>* events;
    long* ring_head;
    long* runs_recorded;
};

// One verify step with workspace ws; paged == nullptr reads the dense caches of `in`.
int run_impl(const spec_verify_config& c, const Workspace& ws, const TimingRing* timing,
             const spec_verify_inputs* in, const spec_verify_paged_kv* paged,
             const spec_verify_outputs* out, void* stream) {
    if (!in || !out) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "inputs and outputs must be non-NULL");
    const int B = in->batch, T = in->nodes;
    if (B < 1 || B > c.max_batch) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "batch out of range");
    if (T < 1 || T > c.max_nodes) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "nodes out of range");
    const bool sampling = c.mode == SPEC_VERIFY_SAMPLING;
    sv::PageTable pt{};
    int slots = c.kv_capacity;
    const void* kc = in->k_cache;
    const void* vc = in->v_cache;
    if (paged) {
        if (int rc = check_paged(c, paged, &pt, &slots)) return rc;
        kc = paged->k_pool;
        vc = paged->v_pool;
    }
    const bool do_attn = !(c.flags & SPEC_VERIFY_FLAG_SKIP_ATTENTION);
    const bool do_vocab = !(c.flags & SPEC_VERIFY_FLAG_SKIP_VOCAB);
    const bool do_probs = (c.flags & SPEC_VERIFY_FLAG_WRITE_PROBS) != 0u;
    if (!in->kv_len || !in->parent) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "an input pointer is NULL");
    if (do_attn && (!in->q || !kc || !vc || !out->attn_out))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "an attention pointer is NULL");
    if (do_vocab) {
        if (!in->tokens || !in->target_logits || !in->u_accept || !in->u_final)
            return fail(SPEC_VERIFY_ERR_INVALID_ARG, "an input pointer is NULL");
        if (sampling && !in->draft_logits)
            return fail(SPEC_VERIFY_ERR_INVALID_ARG, "draft_logits is NULL in sampling mode");
        if (!out->accept_len || !out->final_node || !out->path || !out->out_tokens || !out->status ||
            !out->node_p || !out->node_q || !out->node_accept || !out->final_from_residual || !out->row_token)
            return fail(SPEC_VERIFY_ERR_INVALID_ARG, "an output pointer is NULL");
        if (do_probs && !out->probs)
            return fail(SPEC_VERIFY_ERR_INVALID_ARG, "probs is NULL with SPEC_VERIFY_FLAG_WRITE_PROBS");
    }
    auto misaligned = [](const void* ptr, uintptr_t a) { return (((uintptr_t)ptr) & (a - 1)) != 0; };
    if (do_attn && (misaligned(in->q, 16) || misaligned(kc, 16) || misaligned(vc, 16) || misaligned(out->attn_out, 16)))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "q, k_cache, v_cache and attn_out must be 16-byte aligned");
    if (misaligned(in->kv_len, 4) || misaligned(in->parent, 4))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "arrays must be aligned to their element size");
    if (do_vocab &&
        (misaligned(in->tokens, 4) || misaligned(in->target_logits, 4) || (sampling && misaligned(in->draft_logits, 4)) ||
         misaligned(in->u_accept, 4) || misaligned(in->u_final, 4) || misaligned(out->accept_len, 4) ||
         misaligned(out->final_node, 4) || misaligned(out->path, 4) || misaligned(out->out_tokens, 4) ||
         misaligned(out->status, 4) || misaligned(out->node_p, 4) || misaligned(out->node_q, 4) ||
         misaligned(out->row_token, 4) || (do_probs && misaligned(out->probs, 4))))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "arrays must be aligned to their element size");
    hipStream_t s = (hipStream_t)stream;

    const int D = c.head_dim;
    const bool bf16 = c.dtype == SPEC_VERIFY_BF16;
    AttnPlan plan = plan_attention(c, B, T, ws.part_rows_cap);
    if (plan.part_rows > ws.part_rows_cap) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "workspace too small (internal)");

    hipEvent_t* ev = nullptr;
    if (timing) {
        ev = &(*timing->events)[(size_t)(*timing->ring_head % kTimingRing) * kEventsPerRun];
        hipError_t e = hipEventRecord(ev[0], s);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    auto mark = [&](int stage) -> int {
        if (!ev) return SPEC_VERIFY_OK;
        hipError_t e = hipEventRecord(ev[stage + 1], s);
        return e == hipSuccess ? SPEC_VERIFY_OK : hip_fail(e, "hipEventRecord");
    };

    sv::AttnParams ap{};
    ap.q = in->q;
    ap.k = kc;
    ap.v = vc;
    ap.kv_len = in->kv_len;
    ap.parent = in->parent;
    ap.out = out->attn_out;
    ap.part_o = ws.part_o;
    ap.part_ml = ws.part_ml;
    ap.B = B;
    ap.T = T;
    ap.Hq = c.num_q_heads;
    ap.Hkv = c.num_kv_heads;
    ap.g = c.num_q_heads / c.num_kv_heads;
    ap.D = D;
    ap.Lcap = slots;
    ap.pt = pt;
    ap.R = ap.g * T;
    ap.Rpad = plan.Rpad;
    ap.rowblocks = plan.rowblocks;
    ap.stream = plan.stream ? 1 : 0;
    ap.nsplit = plan.nsplit;
    ap.chunk = plan.chunk;
    const float scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.0f / std::sqrt((float)D);
    ap.c = scale * kLog2e;

    sv::StatsParams tp{};
    tp.target = in->target_logits;
    tp.draft = in->draft_logits;
    tp.stats = ws.stats;
    tp.B = B;
    tp.T = T;
    tp.V = c.vocab;
    tp.sampling = sampling ? 1 : 0;
    tp.ilog = sampling ? kLog2e / c.temperature : kLog2e;
    tp.top_p = sampling ? c.top_p : 1.f;
    const bool fused = do_attn && do_vocab && fuse_row_stats(ws, plan, B, c.num_kv_heads, tp, paged != nullptr, timing != nullptr);

    hipError_t e = hipSuccess;
    if (do_attn) {
        const sv::StatsParams* fp = fused ? &tp : nullptr;
        e = plan.mfma    ? sv::launch_attention_mfma(ap, plan.waves, s, fp)
            : plan.tiled ? sv::launch_attention_valu_tiled(ap, bf16, s, fp)
                         : sv::launch_attention_valu(ap, bf16, s);
        if (e != hipSuccess) return hip_fail(e, "attention launch");
    }
    if (int rc = mark(SPEC_VERIFY_STAGE_ATTENTION)) return rc;

    if (do_vocab) {
        if (!fused) e = sv::launch_row_stats(tp, s);
        if (e != hipSuccess) return hip_fail(e, "row statistics launch");
        if (do_probs) {
            e = sv::launch_write_probs(tp, out->probs, s);
            if (e != hipSuccess) return hip_fail(e, "probs launch");
        }
    }
    if (int rc = mark(SPEC_VERIFY_STAGE_VOCAB)) return rc;

    sv::SelectParams sp{};
    sp.target = in->target_logits;
    sp.draft = in->draft_logits;
    sp.stats = ws.stats;
    sp.parent = in->parent;
    sp.tokens = in->tokens;
    sp.kv_len = in->kv_len;
    sp.u_accept = in->u_accept;
    sp.u_final = in->u_final;
    sp.node_p = out->node_p;
    sp.node_q = out->node_q;
    sp.row_token = out->row_token;
    sp.accept_len = out->accept_len;
    sp.final_node = out->final_node;
    sp.path = out->path;
    sp.out_tokens = out->out_tokens;
    sp.status = out->status;
    sp.node_accept = out->node_accept;
    sp.final_from_residual = out->final_from_residual;
    sp.B = B;
    sp.T = T;
    sp.V = c.vocab;
    sp.Lcap = slots;
    sp.pt = pt;
    sp.sampling = sampling ? 1 : 0;
    sp.ilog = tp.ilog;
    sp.slice_tot = ws.slice_tot;
    sp.slice_pre = ws.slice_pre;
    sp.arrive = ws.arrive;
    sp.S = (c.vocab + sv::kSelectSlice - 1) / sv::kSelectSlice;
    sp.resid_ws = ws.resid_ws;
    sp.walk_sync = ws.walk_sync;
    sp.walk_part = ws.walk_part;
    sp.walk_rx = ws.walk_rx;
    sp.walk_k = ws.walk_k;
    sp.walk_coop = ((long)B * ws.walk_k <= ws.walk_cap) ? 1 : 0;
    sp.walk_spin = ws.walk_spin;
    const bool walk = do_vocab && sampling && (c.flags & SPEC_VERIFY_FLAG_LOSSLESS_TREE);
    e = sv::launch_finish(sp, ap, do_vocab && !walk, do_attn && plan.nsplit > 1, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "finishing launch");
    if (walk) {
        e = sv::launch_lossless_walk(sp, s);
        if (e != hipSuccess) return hip_fail(e, "lossless walk launch");
    }
    if (int rc = mark(SPEC_VERIFY_STAGE_FINISH)) return rc;

    if (timing) {
        ++*timing->ring_head;
        *timing->runs_recorded = std::min<long>(*timing->runs_recorded + 1, kTimingRing);
    }
    return SPEC_VERIFY_OK;
}

// KV commit; paged == nullptr writes the dense caches of `a`.
int commit_impl(spec_verify_handle* h, const spec_verify_commit_args* a, const spec_verify_paged_kv* paged,
                void* stream) {
    if (!h || !a) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "handle and args must be non-NULL");
    const spec_verify_config& c = h->cfg;
    if (a->batch < 1 || a->batch > c.max_batch) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "batch out of range");
    if (a->nodes < 1 || a->nodes > c.max_nodes) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "nodes out of range");
    sv::PageTable pt{};
    int slots = c.kv_capacity;
    void* kc = a->k_cache;
    void* vc = a->v_cache;
    if (paged) {
        if (int rc = check_paged(c, paged, &pt, &slots)) return rc;
        kc = paged->k_pool;
        vc = paged->v_pool;
    }
    if (!kc || !vc || !a->kv_len || !a->path || !a->accept_len || !a->final_node)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "a commit pointer is NULL");
    auto misaligned = [](const void* ptr, uintptr_t al) { return (((uintptr_t)ptr) & (al - 1)) != 0; };
    if (misaligned(kc, 16) || misaligned(vc, 16))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
    if (misaligned(a->kv_len, 4) || misaligned(a->path, 4) || misaligned(a->accept_len, 4) ||
        misaligned(a->final_node, 4))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "arrays must be aligned to their element size");
    sv::CommitParams cp{};
    cp.k = kc;
    cp.v = vc;
    cp.kv_len = a->kv_len;
    cp.kv_len_out = a->kv_len;
    cp.path = a->path;
    cp.accept_len = a->accept_len;
    cp.final_node = a->final_node;
    cp.B = a->batch;
    cp.T = a->nodes;
    cp.Hkv = c.num_kv_heads;
    cp.Lcap = slots;
    cp.row_bytes = c.head_dim * (c.dtype == SPEC_VERIFY_BF16 ? 2 : 4);
    cp.pt = pt;
    cp.arrive = h->commit_arrive;
    const hipError_t e = sv::launch_kv_commit(cp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "commit launch");
    return SPEC_VERIFY_OK;
}

}  // namespace

namespace {

// ------------------------------------------------------------------ workspace without allocation
//
// spec_verify_run_noalloc takes its workspace from this array instead of a
// handle's hipMalloc'd buffers.  Each GPU the library runs on holds its own
// copy (placed by the runtime when the code object is loaded there) until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per GPU
constexpr int kNoallocMaxBatch = 1024;               // sequences per call (one arrival counter each)
constexpr size_t kCounterBytes = kNoallocMaxBatch * sizeof(int32_t);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words_kernel(int32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Device address of this GPU's scratch array.  The first call on a device
// looks it up and clears the arrival counters on `stream` (every complete run
// leaves them at 0 again: the last workgroup's increment wraps them).
int scratch_for_device(int dev, hipStream_t stream, unsigned char** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(SPEC_VERIFY_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        hipLaunchKernelGGL(zero_words_kernel, dim3(4), dim3(256), 0, stream, (int32_t*)ptr, kNoallocMaxBatch);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
        g_scratch_ptr[dev] = (unsigned char*)ptr;
    }
    *out = g_scratch_ptr[dev];
    return SPEC_VERIFY_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Carve a run's workspace for (B, T) out of the scratch at `base`: arrival
// counters, row statistics and final-draw totals first, the per-thread slice
// prefixes when they fit in half of what is left, and split partials in the
// rest (the attention plan then takes as many prefix splits as fit).
int carve_scratch(const spec_verify_config& c, int B, int T, unsigned char* base, Workspace* ws) {
    const int slices = (c.vocab + sv::kSelectSlice - 1) / sv::kSelectSlice;
    const uintptr_t b0 = (uintptr_t)base;   // 0 for a size check only
    size_t off = kCounterBytes;
    const size_t stats_bytes = round_up((size_t)B * 2 * T * sizeof(sv::RowStat), 256);
    const size_t tot_bytes = round_up((size_t)B * slices * sizeof(double2), 256);
    if (off + stats_bytes + tot_bytes > kScratchBytes)
        return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "the batch needs more than the 16 MiB scratch of spec_verify_run_noalloc");
    ws->arrive = (int32_t*)b0;
    ws->stats = (sv::RowStat*)(b0 + off);
    off += stats_bytes;
    ws->slice_tot = (double2*)(b0 + off);
    off += tot_bytes;
    const size_t pre_bytes = round_up((size_t)B * slices * sv::kSelectThreads * sizeof(double2), 256);
    ws->slice_pre = nullptr;
    if (c.mode == SPEC_VERIFY_SAMPLING && slices <= sv::kSelectKeepSlices && 2 * pre_bytes <= kScratchBytes - off) {
        ws->slice_pre = (double2*)(b0 + off);
        off += pre_bytes;
    }
    // partial rows: D floats of O and one (m, l) pair each; 256 bytes kept for aligning the pairs
    const size_t row_bytes = (size_t)c.head_dim * sizeof(float) + sizeof(float2);
    const size_t left = kScratchBytes - off;
    ws->part_rows_cap = left > 256 ? (left - 256) / row_bytes : 0;
    ws->part_o = (float*)(b0 + off);
    ws->part_ml = (float2*)(b0 + off + round_up(ws->part_rows_cap * c.head_dim * sizeof(float), 256));
    return SPEC_VERIFY_OK;
}

}  // namespace

extern "C" {

int spec_verify_run(spec_verify_handle* h, const spec_verify_inputs* in, const spec_verify_outputs* out,
                    void* stream) {
    g_err.clear();
    if (!h) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "handle is NULL");
    TimingRing tr{&h->events, &h->ring_head, &h->runs_recorded};
    return run_impl(h->cfg, h->ws, h->timing ? &tr : nullptr, in, nullptr, out, stream);
}

int spec_verify_run_paged(spec_verify_handle* h, const spec_verify_inputs* in, const spec_verify_paged_kv* paged,
                          const spec_verify_outputs* out, void* stream) {
    g_err.clear();
    if (!h) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "handle is NULL");
    if (!paged) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "paged is NULL");
    TimingRing tr{&h->events, &h->ring_head, &h->runs_recorded};
    return run_impl(h->cfg, h->ws, h->timing ? &tr : nullptr, in, paged, out, stream);
}

int spec_verify_run_noalloc(const spec_verify_config* cfg, const spec_verify_inputs* in,
                            const spec_verify_outputs* out, void* stream) {
    g_err.clear();
    if (!cfg || !in || !out) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "cfg, inputs and outputs must be non-NULL");
    const spec_verify_config& c = *cfg;
    if (int rc = validate_config(c)) return rc;
    if (c.flags & (SPEC_VERIFY_FLAG_TIMING | SPEC_VERIFY_FLAG_LOSSLESS_TREE | SPEC_VERIFY_FLAG_WALK_NO_WAIT))
        return fail(SPEC_VERIFY_ERR_UNSUPPORTED,
                    "spec_verify_run_noalloc takes neither SPEC_VERIFY_FLAG_TIMING nor SPEC_VERIFY_FLAG_LOSSLESS_TREE");
    if (in->batch < 1 || in->batch > c.max_batch) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "batch out of range");
    if (in->nodes < 1 || in->nodes > c.max_nodes) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "nodes out of range");
    if (in->batch > kNoallocMaxBatch)
        return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "spec_verify_run_noalloc takes at most 1024 sequences");
    Workspace ws;
    if (int rc = carve_scratch(c, in->batch, in->nodes, nullptr, &ws)) return rc;   // size check only
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    unsigned char* base = nullptr;
    if (int rc = scratch_for_device(dev, (hipStream_t)stream, &base)) return rc;
    carve_scratch(c, in->batch, in->nodes, base, &ws);
    e = hipDeviceGetAttribute(&ws.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    return run_impl(c, ws, nullptr, in, nullptr, out, stream);
}

int spec_verify_commit(spec_verify_handle* h, const spec_verify_commit_args* a, void* stream) {
    g_err.clear();
    return commit_impl(h, a, nullptr, stream);
}

int spec_verify_commit_paged(spec_verify_handle* h, const spec_verify_commit_args* a,
                             const spec_verify_paged_kv* paged, void* stream) {
    g_err.clear();
    if (!paged) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "paged is NULL");
    return commit_impl(h, a, paged, stream);
}

int spec_verify_build_tree(spec_verify_handle* h, const spec_verify_tree_args* a, void* stream) {
    g_err.clear();
    if (!h || !a) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "handle and args must be non-NULL");
    const spec_verify_config& c = h->cfg;
    const int B = a->batch, T = a->nodes;
    if (B < 1 || B > c.max_batch) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "batch out of range");
    if (T < 1 || T > c.max_nodes) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "nodes out of range");
    if (!a->cand_logits || !a->root_token || !a->tree_parent || !a->tree_rank || !a->parent || !a->tokens)
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "a tree-build pointer is NULL");
    auto misaligned = [](const void* ptr) { return (((uintptr_t)ptr) & 3u) != 0; };
    if (misaligned(a->cand_logits) || misaligned(a->root_token) || misaligned(a->parent) || misaligned(a->tokens))
        return fail(SPEC_VERIFY_ERR_INVALID_ARG, "arrays must be aligned to their element size");
    sv::TreeParams tp{};
    int depth[64];
    int levels = 0;
    for (int i = 0; i < T; ++i) {
        const int p = a->tree_parent[i];
        if (i == 0 ? p != -1 : (p < 0 || p >= i))
            return fail(SPEC_VERIFY_ERR_INVALID_ARG, "tree_parent is not a topologically ordered tree");
        depth[i] = i == 0 ? 0 : depth[p] + 1;
        levels = std::max(levels, depth[i]);
        const int r = i == 0 ? 0 : a->tree_rank[i];
        if (r < 0) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "tree_rank must be >= 0");
        if (r >= 32) return fail(SPEC_VERIFY_ERR_UNSUPPORTED, "a depth needs more than 32 top-k entries");
        tp.tpar[i] = (int8_t)p;
        tp.trank[i] = (int8_t)r;
        tp.tdep[i] = (int8_t)depth[i];
    }
    if (levels > a->depth) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "the template is deeper than depth");
    int kmax = 0;
    for (int i = 1; i < T; ++i) {
        tp.kd[depth[i]] = (int8_t)std::max<int>(tp.kd[depth[i]], tp.trank[i] + 1);
        kmax = std::max<int>(kmax, tp.kd[depth[i]]);
    }
    if (kmax > c.vocab) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "more top-k entries needed than the vocabulary has");
    tp.logits = a->cand_logits;
    tp.root_token = a->root_token;
    tp.parent = a->parent;
    tp.tokens = a->tokens;
    tp.B = B;
    tp.T = T;
    tp.V = c.vocab;
    tp.rows = a->depth;
    tp.levels = levels;
    // long rows are split over up to kTreeMaxSlices workgroups of >= 4096 ids
    tp.slices = levels ? std::max(1, std::min(sv::kTreeMaxSlices, c.vocab / 4096)) : 1;
    tp.cand = h->tree_cand;
    tp.arrive = h->tree_arrive;
    const hipError_t e = sv::launch_tree_build(tp, kmax, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "tree-build launch");
    return SPEC_VERIFY_OK;
}

int spec_verify_tree_template(const int32_t* caps, int32_t ncaps, int32_t nodes, int32_t* parent, int32_t* rank) {
    g_err.clear();
    if (!caps || !parent || !rank) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "NULL argument");
    if (ncaps < 1 || ncaps > 63) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "ncaps must be in [1, 63]");
    if (nodes < 1 || nodes > 64) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "nodes must be in [1, 64]");
    long long tuples = 0, level = 1;
    for (int k = 0; k < ncaps; ++k) {
        if (caps[k] < 1) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "caps must be >= 1");
        level = std::min<long long>(level * caps[k], 1LL << 40);
        tuples = std::min<long long>(tuples + level, 1LL << 40);
    }
    if (nodes - 1 > tuples) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "nodes exceed 1 + the number of rank tuples");
    // Best-first over the rank tuples: every tuple but (0) is reached from a
    // smaller key, as the first child t+(0) of t (same product, one deeper)
    // or as the next sibling of (.., r) (larger product), so popping the
    // smallest key and pushing those two successors yields the tuples in key order.
    struct Cand {
        unsigned long long prod;
        std::vector<int> t;
    };
    auto less = [](const Cand& x, const Cand& y) {
        if (x.prod != y.prod) return x.prod < y.prod;
        if (x.t.size() != y.t.size()) return x.t.size() < y.t.size();
        return x.t < y.t;
    };
    std::vector<Cand> open{Cand{1ull, {0}}};
    std::vector<std::vector<int>> kept;
    while ((int)kept.size() < nodes - 1) {
        size_t best = 0;
        for (size_t q = 1; q < open.size(); ++q)
            if (less(open[q], open[best])) best = q;
        Cand cur = open[best];
        open.erase(open.begin() + best);
        if ((int)cur.t.size() < ncaps) {
            Cand child{cur.prod, cur.t};
            child.t.push_back(0);
            open.push_back(child);
        }
        const int r = cur.t.back();
        if (r + 1 < caps[cur.t.size() - 1]) {
            Cand sib{cur.prod / (unsigned long long)(r + 1) * (unsigned long long)(r + 2), cur.t};
            sib.t.back() = r + 1;
            open.push_back(sib);
        }
        kept.push_back(cur.t);
    }
    std::sort(kept.begin(), kept.end(), [](const std::vector<int>& x, const std::vector<int>& y) {
        if (x.size() != y.size()) return x.size() < y.size();
        return x < y;
    });
    parent[0] = -1;
    rank[0] = 0;
    for (int i = 1; i < nodes; ++i) {
        const std::vector<int>& t = kept[i - 1];
        int p = 0;
        if (t.size() > 1) {
            const std::vector<int> up(t.begin(), t.end() - 1);
            for (int j = 1; j < i; ++j)
                if (kept[j - 1] == up) p = j;
        }
        parent[i] = p;
        rank[i] = t.back();
    }
    return SPEC_VERIFY_OK;
}

int spec_verify_describe(spec_verify_handle* h, int32_t batch, int32_t nodes, char* buf, int32_t buf_len) {
    g_err.clear();
    if (!h || !buf || buf_len < 1) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "NULL argument or empty buffer");
    const spec_verify_config& c = h->cfg;
    if (batch < 1 || batch > c.max_batch) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "batch out of range");
    if (nodes < 1 || nodes > c.max_nodes) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "nodes out of range");
    const bool sampling = c.mode == SPEC_VERIFY_SAMPLING;
    const bool do_attn = !(c.flags & SPEC_VERIFY_FLAG_SKIP_ATTENTION);
    const bool do_vocab = !(c.flags & SPEC_VERIFY_FLAG_SKIP_VOCAB);
    const bool walk = do_vocab && sampling && (c.flags & SPEC_VERIFY_FLAG_LOSSLESS_TREE);
    const AttnPlan plan = plan_attention(c, batch, nodes, h->ws.part_rows_cap);
    sv::StatsParams tp{};
    tp.B = batch;
    tp.T = nodes;
    tp.V = c.vocab;
    tp.sampling = sampling ? 1 : 0;
    tp.top_p = sampling ? c.top_p : 1.f;
    sv::SelectParams sp{};
    sp.V = c.vocab;
    sp.walk_coop = ((long)batch * h->ws.walk_k <= h->ws.walk_cap) ? 1 : 0;
    const char* attn = !do_attn ? "" : plan.mfma ? "attn_mfma_kernel" : plan.tiled ? "attn_valu_tiled_kernel"
                                                                                   : "attn_valu_kernel";
    const bool merge = do_attn && plan.nsplit > 1;
    const bool select = do_vocab && !walk;
    const int n = std::snprintf(
        buf, (size_t)buf_len,
        "{\"attention\": \"%s\", \"waves\": %d, \"rowblocks\": %d, \"nsplit\": %d, \"chunk\": %d, \"stream\": %d, "
        "\"vocab\": \"%s\", \"probs\": \"%s\", \"finish\": \"%s\", \"select\": %d, \"merge\": %d, "
        "\"walk\": \"%s\", \"vocab_in_attention_launch\": %d}",
        attn, do_attn ? plan.waves : 0, do_attn ? plan.rowblocks : 0, do_attn ? plan.nsplit : 0,
        do_attn ? plan.chunk : 0, do_attn && plan.stream ? 1 : 0, do_vocab ? sv::row_stats_kernel_name(tp) : "",
        (c.flags & SPEC_VERIFY_FLAG_WRITE_PROBS) ? "write_probs_kernel" : "", (select || merge) ? "finish_kernel" : "",
        select ? 1 : 0, merge ? 1 : 0, walk ? sv::lossless_walk_kernel_name(sp) : "",
        (do_attn && do_vocab && fuse_row_stats(h->ws, plan, batch, c.num_kv_heads, tp, false, h->timing)) ? 1 : 0);
    if (n < 0 || n >= buf_len) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "buffer too small");
    return SPEC_VERIFY_OK;
}

int spec_verify_timing_read(spec_verify_handle* h, float* stage_ms, int32_t* runs) {
    g_err.clear();
    if (!h || !stage_ms || !runs) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "NULL argument");
    if (!h->timing) return fail(SPEC_VERIFY_ERR_INVALID_ARG, "handle was created without SPEC_VERIFY_FLAG_TIMING");
    for (int k = 0; k < SPEC_VERIFY_NUM_STAGES; ++k) stage_ms[k] = 0.f;
    const long n = h->runs_recorded;
    for (long r = 0; r < n; ++r) {
        const long slot = (h->ring_head - n + r) % kTimingRing;
        hipEvent_t* ev = &h->events[(size_t)slot * kEventsPerRun];
        hipError_t e = hipEventSynchronize(ev[kEventsPerRun - 1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        for (int k = 0; k < SPEC_VERIFY_NUM_STAGES; ++k) {
            float ms = 0.f;
            e = hipEventElapsedTime(&ms, ev[k], ev[k + 1]);
            if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
            stage_ms[k] += ms;
        }
    }
    *runs = (int32_t)n;
    h->runs_recorded = 0;
    return SPEC_VERIFY_OK;
}

}  // extern "C"
