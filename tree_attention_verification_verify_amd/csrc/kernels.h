// Internal kernel launch interface of libspecverify (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// Block table of a paged KV cache (table == nullptr: dense caches).  Slot s of
// sequence b is row s & (bs - 1) of page table[b * width + (s >> bs_log2)];
// a page holds bs slots of every KV head: [pages][Hkv][bs][D].
struct PageTable {
    const int32_t* table;
    int width;          // entries per sequence
    int bs_log2;        // log2 of the slots per page
    int num_blocks;     // pages in the pool
};

// Tree attention over the prefix split into `nsplit` key ranges of `chunk`
// keys.  Rows of one (sequence, KV head) pair are r = node * g + (h % g).
struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* kv_len;
    const int32_t* parent;
    void* out;          // [B,T,Hq,D] dtype (written directly when nsplit == 1)
    float* part_o;      // [pairs][nsplit][Rpad][D] un-normalised partial outputs
    float2* part_ml;    // [pairs][nsplit][Rpad] (running max in log2 units, row sum)
    int B, T, Hq, Hkv, g, D, Lcap;
    int R;              // g * T rows per pair
    int Rpad;           // rowblocks * rows_per_block
    int rowblocks;
    int nsplit;
    int chunk;          // keys per split (multiple of 64)
    int groups_per_xcd; // XCD-aware block mapping (mfma path with rowblocks > 1)
    int stream;         // K/V tiles loaded with the non-temporal policy (see plan_attention)
    float c;            // softmax_scale * log2(e)
    PageTable pt;       // paged caches: k, v are the pools; Lcap = pt.width << pt.bs_log2
};

// Statistics of one logits row under temperature (and top-p).
struct RowStat {
    float zmax;      // largest logit
    int argmax;      // smallest token id holding it
    uint32_t thr;    // top-p cut: bit pattern of the smallest kept unnormalised probability
    int cutoff;      // tokens whose value equals the cut are kept when id < cutoff
    double Z;        // sum over the kept tokens of exp((z - zmax) / temperature)
};

// stats[b * 2T + r]: r < T -> target row r; r = T + i -> draft row of node i (i >= 1).
struct StatsParams {
    const float* target;
    const float* draft;
    RowStat* stats;
    int B, T, V;
    int sampling;
    float ilog;         // log2(e) / temperature
    float top_p;
};

struct SelectParams {
    const float* target;
    const float* draft;
    const RowStat* stats;
    const int32_t* parent;
    const int32_t* tokens;
    const int32_t* kv_len;
    const float* u_accept;
    const float* u_final;
    float* node_p;
    float* node_q;
    int32_t* row_token;
    int32_t* accept_len;
    int32_t* final_node;
    int32_t* path;
    int32_t* out_tokens;
    int32_t* status;
    uint8_t* node_accept;
    uint8_t* final_from_residual;
    double2* slice_tot;   // [B][S] (residual, p-only) weight totals per slice of the final draw
    double2* slice_pre;   // [B][S][kSelectThreads] per-thread exclusive prefixes (S <= kSelectKeepSlices)
    float* resid_ws;      // [B][2][V] residual rows of the lossless sibling walk
    int32_t* walk_sync;   // [B][4] sibling walk across workgroups: (unused), finished workgroups, timeout flag
    double* walk_part;    // [B][2][walk_k] per-workgroup residual totals tagged with their pass (two passes
                          // in turn; zero between launches)
    float* walk_rx;       // [B][2][2] the next test's r (new, kept) from the workgroup holding its token
    int walk_k;           // workgroups per sequence of the walk: ceil(V / kWalkSlice)
    int walk_coop;        // 1: the walk over walk_k workgroups per sequence; 0: one workgroup per sequence
    int walk_spin;        // polls of a walk wait before it gives up (status bit 16)
    int32_t* arrive;      // [B] slices done (wraps to 0 at the last one)
    int B, T, V, Lcap;
    int S;                // slices per sequence: ceil(V / kSelectSlice)
    int sampling;
    float ilog;
    PageTable pt;         // paged caches: table entries of the used slots count for status bit 8
};

struct CommitParams {
    void* k;                 // [B,Hkv,Lcap,D] updated in place
    void* v;
    const int32_t* kv_len;   // [B] L before the commit
    int32_t* kv_len_out;     // [B] L + accept_len + 1 (may be kv_len itself)
    const int32_t* path;     // [B,T]
    const int32_t* accept_len;
    const int32_t* final_node;
    int B, T, Hkv, Lcap;
    int row_bytes;           // D * element size (a multiple of 16)
    PageTable pt;            // paged caches: k, v are the pools; Lcap = pt.width << pt.bs_log2
    int32_t* arrive;         // [B] finished workgroups per sequence (zero between calls)
};

// Candidate-tree construction: template by value (T <= 64, depth <= 63,
// ranks < 32), one workgroup per (sequence, depth).
struct TreeParams {
    const float* logits;        // [B][rows][V]: row d-1 = distribution of depth-d candidates
    const int32_t* root_token;  // [B]
    int32_t* parent;            // [B][T] out
    int32_t* tokens;            // [B][T] out
    int B, T, V, rows;
    int levels;                 // deepest template depth (0: root only)
    int8_t tpar[64];            // template parent[] (-1 for the root)
    int8_t trank[64];           // top-k entry each node takes
    int8_t tdep[64];            // depth of each node
    int8_t kd[64];              // entries needed at depth d (max rank + 1)
    int slices;                 // workgroups per row (1: the whole row in one)
    unsigned long long* cand;   // [B][levels][slices][32] per-slice best keys (slices > 1)
    int32_t* arrive;            // [B][levels] finished slices per row (zero between calls)
};

// Returns hipSuccess or the launch error.  fused != nullptr (only where the
// planner allows it): the same launch also runs the streaming row statistics
// of *fused in workgroups of its own after the attention workgroups: one row
// per 256-thread workgroup (beside a grid that leaves CUs idle), or two rows
// per 512-thread workgroup (after a grid that fills the GPU).
hipError_t launch_attention_mfma(const AttnParams& p, int waves, hipStream_t s, const StatsParams* fused = nullptr);
hipError_t launch_attention_valu(const AttnParams& p, bool bf16, hipStream_t s);
// VALU attention with 4 waves sharing double-buffered tiles: R <= 8 rows per KV
// head, K/V rows of 128 or 256 bytes (valu_tiled_supported); Rpad = rows per block.
bool valu_tiled_supported(bool bf16, int D, int R);
hipError_t launch_attention_valu_tiled(const AttnParams& p, bool bf16, hipStream_t s, const StatsParams* fused = nullptr);
hipError_t launch_row_stats(const StatsParams& p, hipStream_t s);
const char* row_stats_kernel_name(const StatsParams& p);   // the kernel launch_row_stats takes
// Whether launch_row_stats takes the streaming kernel (no top-p cut), the one
// an attention launch can carry.
bool row_stats_streams(const StatsParams& p);
// probs[B,T,V] = effective target distribution of every row (after launch_row_stats).
hipError_t launch_write_probs(const StatsParams& p, float* probs, hipStream_t s);
// The step's last launch: selection (decisions, path, final draw) and, when
// `merge`, the merge of the attention splits.
hipError_t launch_finish(const SelectParams& sp, const AttnParams& ap, bool select, bool merge, bool bf16,
                         hipStream_t s);
// Lossless sibling walk (sampling mode, SPEC_VERIFY_FLAG_LOSSLESS_TREE): one workgroup per sequence.
hipError_t launch_lossless_walk(const SelectParams& p, hipStream_t s);
const char* lossless_walk_kernel_name(const SelectParams& p);   // the kernel launch_lossless_walk takes
// Workgroups of the walk across workgroups one CU holds at once (its register,
// LDS and wave use, from the runtime's occupancy calculation).
hipError_t walk_coop_blocks_per_cu(int* blocks);
constexpr int kWalkSpinLimit = 1 << 21;   // polls (s_sleep 1 each, about 0.1 s) before a walk wait gives up
// KV commit of the accepted path: one workgroup per sequence.
hipError_t launch_kv_commit(const CommitParams& p, hipStream_t s);
// Candidate tree: kmax = largest kd over the depths (<= 32).
hipError_t launch_tree_build(const TreeParams& p, int kmax, hipStream_t s);

constexpr int kValuRows = 16;      // rows per block of the VALU attention kernel
constexpr int kMfmaHalves = 2;     // key halves per workgroup of the MFMA attention kernel
constexpr int kTreeMaxSlices = 8;                  // tree building: workgroups per logits row at most
constexpr int kVocabThreads = 1024;               // register-resident row kernels
constexpr int kVocabChunk = kVocabThreads * 32;   // logits held on chip per pass
constexpr int kStatsThreads = 256;                // streaming row-statistics kernel
constexpr int kStatsUnroll = 16;                  // float4 loads in flight per thread
constexpr int kSelectThreads = 256;               // selection / final draw workgroups
constexpr int kSelectSlice = 2048;                // token ids per final-draw slice
constexpr int kSelectMaxSlices = 2048;            // vocab <= 4194304
constexpr int kSelectKeepSlices = 64;             // up to this many slices the draw keeps slice prefixes
constexpr int kWalkThreads = 256;                 // sibling-walk workgroups
constexpr int kWalkSlice = kWalkThreads * 16;     // token ids each walk workgroup holds in registers

}  // namespace sv
