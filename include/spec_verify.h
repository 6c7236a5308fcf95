/*
 * spec_verify.h - C ABI of the MI355X verify-step library (libspecverify.so).
 *
 * The library runs the target-model verify step of speculative decoding and
 * Medusa tree decoding for a batch of sequences, on one HIP stream, in four
 * parts:
 *
 *   1. Tree-masked attention of the T candidate nodes over the shared KV
 *      prefix plus each node's own root path.  Flattening the tree into one
 *      sequence with a mask: "大模型推理加速：推测解码与MTP核心原理与工程实践"
 *      section 3.2; the mask itself: "推测解码技术详解：加速LLM推理的关键" section
 *      "Tree Attention验证"; siblings never see each other: "投机解码的五条路线"
 *      section 4.  Prefix KV reuse: the first page, section 3.1 item 2.
 *   2. Per-node temperature (+ top-p) softmax over the vocabulary: target p,
 *      and draft q where a draft exists ("投机解码的五条路线", section on exact
 *      verification: the effective sampling distributions must be used).
 *   3. Token-level acceptance u < p(x)/q(x), resampling from norm([p-q]_+) on
 *      rejection and a bonus token when a whole path passed (featured article
 *      on the founding speculative-decoding paper, sections 2.1-2.2); greedy
 *      mode accepts a candidate iff it is the target's best token.
 *   4. Selection of the longest root path accepted consecutively from the
 *      root (first page, section 2.3; "投机解码的五条路线", figure 3).
 *
 * All pointers in the input/output structs are DEVICE pointers unless noted;
 * the caller owns them and keeps them alive until the stream work is done.
 * q, k_cache, v_cache and attn_out must be 16-byte aligned, every other array
 * aligned to its element size (SPEC_VERIFY_ERR_INVALID_ARG otherwise).
 * Shapes use B = inputs.batch, T = inputs.nodes, Hq/Hkv/D/Lcap/V from the
 * config; arrays are dense, row-major, in the order of their dimensions.
 *
 * Errors: every entry point returns SPEC_VERIFY_OK (0) or a negative code and
 * sets a thread-local message (spec_verify_last_error).  Host-checkable faults
 * are caught before any HIP call.  Data-dependent faults (bad parent[], token
 * ids, kv_len) are reported per sequence in outputs.status, asynchronously.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_VERIFY_OK 0
#define SPEC_VERIFY_ERR_INVALID_ARG (-1)
#define SPEC_VERIFY_ERR_UNSUPPORTED (-2)
#define SPEC_VERIFY_ERR_HIP (-3)
#define SPEC_VERIFY_ERR_OOM (-4)

#define SPEC_VERIFY_F32 0
#define SPEC_VERIFY_BF16 1

#define SPEC_VERIFY_GREEDY 0
#define SPEC_VERIFY_SAMPLING 1

/* config.flags: record HIP events around each kernel of every run (see
 * spec_verify_timing_read).  Costs a few event records per run, and keeps
 * the three stages in launches of their own (no row statistics inside the
 * attention launch), so each stage's time can be read. */
#define SPEC_VERIFY_FLAG_TIMING 1u
/* config.flags, sampling mode only: lossless multi-candidate tree sampling.
 * Instead of testing every node independently against its parent's p and
 * keeping the longest accepted root path, walk from the root: try the
 * children of the current node in increasing id, accept child c when
 * u_accept[c] < r(x_c)/q_c(x_c), otherwise set r <- norm([r - q_c]_+) (kept if
 * that is all zero) and try the next child; r starts as p of the node reached
 * and the final token is drawn from r.  The output then follows the target's
 * law for any tree, not only for chains ("投机解码的五条路线", section 4:
 * lossless verification; the featured article on the founding
 * speculative-decoding paper, section 2.1, for one rejection step).  For
 * chains both rules give the same outputs.  node_accept/node_p/node_q then
 * describe the tests made (r(x) and q(x) at test time); children never tried
 * get 0.  Costs one pass over the vocabulary per rejected child. */
#define SPEC_VERIFY_FLAG_LOSSLESS_TREE 2u
/* config.flags: run without step 1 (tree attention).  q, k_cache, v_cache
 * (or the paged pools) and attn_out are not read or written and may be NULL;
 * parent and kv_len are still read (status bits 1 and 8). */
#define SPEC_VERIFY_FLAG_SKIP_ATTENTION 4u
/* config.flags: run step 1 only.  target_logits, draft_logits, tokens,
 * u_accept, u_final and every output except attn_out are not read or written
 * and may be NULL.  Not together with SKIP_ATTENTION. */
#define SPEC_VERIFY_FLAG_SKIP_VOCAB 8u
/* config.flags, sampling mode only: also write outputs.probs[B,T,V], the
 * effective target distribution of every row, TopP(softmax(z / temperature))
 * (the full probability rows the page's sampler takes as its input:
 * "推测解码技术详解：加速LLM推理的关键", section "数学保证：无损输出质量").  A
 * debug output: it writes 4 bytes per logit.  probs[b, parent[b,i], x_i]
 * equals node_p[b, i] bit for bit. */
#define SPEC_VERIFY_FLAG_WRITE_PROBS 16u
/* config.flags, for tests of the lossless walk's time-out path only: every
 * wait of the walk for the sequence's other workgroups gives up after one
 * poll (status bit 16 and invalid outputs for a sequence whose workgroups
 * were not all there yet).  Every kernel still runs to its end. */
#define SPEC_VERIFY_FLAG_WALK_NO_WAIT 32u

/* Status bits written to outputs.status[b]. */
#define SPEC_VERIFY_STATUS_BAD_PARENT 1   /* parent[0] != -1 or not 0 <= parent[i] < i   */
#define SPEC_VERIFY_STATUS_BAD_TOKEN 2    /* tokens[b,i] outside [0,V) for some i >= 1    */
#define SPEC_VERIFY_STATUS_ZERO_DRAFT 4   /* q_i(x_i) = 0 for a supplied draft (rejected) */
#define SPEC_VERIFY_STATUS_BAD_KVLEN 8    /* kv_len[b] < 0 or kv_len[b] + T > Lcap        */
#define SPEC_VERIFY_STATUS_WALK_TIMEOUT 16 /* lossless walk: a wait for the sequence's other
                                              workgroups ran out (another launch held the
                                              GPU); that sequence's outputs are not valid */

/* Kernel stages (launches, in order) reported by spec_verify_timing_read. */
#define SPEC_VERIFY_STAGE_ATTENTION 0     /* tree attention main kernel                   */
#define SPEC_VERIFY_STAGE_VOCAB 1         /* per-row softmax statistics (one read)        */
#define SPEC_VERIFY_STAGE_FINISH 2        /* ratios, decisions, path, final draw, and the
                                             merge of split-prefix attention partials     */
#define SPEC_VERIFY_NUM_STAGES 3

typedef struct spec_verify_config {
    int32_t max_batch;      /* >= 1: largest B a run may pass                        */
    int32_t max_nodes;      /* 1..64: largest T (tree nodes incl. the root)          */
    int32_t num_q_heads;    /* Hq >= 1                                               */
    int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0; query head h uses KV head
                               h / (Hq/Hkv) (contiguous groups)                      */
    int32_t head_dim;       /* D: 64 or 128                                          */
    int32_t kv_capacity;    /* Lcap >= max_nodes: slots per (sequence, KV head)      */
    int32_t vocab;          /* V >= 1                                                */
    int32_t dtype;          /* SPEC_VERIFY_F32 or SPEC_VERIFY_BF16: Q, K, V, attn_out */
    int32_t mode;           /* SPEC_VERIFY_GREEDY or SPEC_VERIFY_SAMPLING            */
    float temperature;      /* > 0 (sampling mode); applied to target and draft      */
    float top_p;            /* (0,1]; 1 = off                                        */
    float softmax_scale;    /* attention scale; 0 => 1/sqrt(D)                       */
    uint32_t flags;         /* SPEC_VERIFY_FLAG_*                                    */
} spec_verify_config;

typedef struct spec_verify_inputs {
    const void* q;              /* [B,T,Hq,D] dtype: node i's queries (RoPE applied)     */
    const void* k_cache;        /* [B,Hkv,Lcap,D] dtype: slots 0..L_b-1 = prefix,
                                   slot L_b+i = tree node i's own key                     */
    const void* v_cache;        /* [B,Hkv,Lcap,D] dtype: same slots for values            */
    const int32_t* kv_len;      /* [B]: L_b, prefix length of sequence b                  */
    const int32_t* parent;      /* [B,T]: parent[b,0] = -1, 0 <= parent[b,i] < i           */
    const int32_t* tokens;      /* [B,T]: token of node i (node 0 = current token, unused) */
    const float* target_logits; /* [B,T,V] fp32: row i = target logits after node i       */
    const float* draft_logits;  /* [B,T,V] fp32: row i = logits node i was drafted from
                                   (row 0 unused); sampling mode only, NULL in greedy     */
    const float* u_accept;      /* [B,T] fp32 in [0,1): uniform of node i's accept test   */
    const float* u_final;       /* [B] fp32 in [0,1): uniform of the final token draw     */
    int32_t batch;              /* B: 1..max_batch                                        */
    int32_t nodes;              /* T: 1..max_nodes                                        */
} spec_verify_inputs;

typedef struct spec_verify_outputs {
    void* attn_out;                /* [B,T,Hq,D] dtype: attention output of every node      */
    int32_t* accept_len;           /* [B]: depth of the selected node v* (accepted drafts)  */
    int32_t* final_node;           /* [B]: v* (-1 if the sequence is void)                  */
    int32_t* path;                 /* [B,T]: root..v* node ids, then -1                      */
    int32_t* out_tokens;           /* [B,T]: accepted tokens, then the final token, then -1  */
    int32_t* status;               /* [B]: SPEC_VERIFY_STATUS_* bits                         */
    float* node_p;                 /* [B,T]: p_parent(i)(x_i) (sampling; 0 otherwise)        */
    float* node_q;                 /* [B,T]: q_i(x_i) (sampling; 0 otherwise)                */
    uint8_t* node_accept;          /* [B,T]: per-node test result (node 0 = 1)               */
    uint8_t* final_from_residual;  /* [B]: 1 if the final token came from norm([p-q]_+)      */
    int32_t* row_token;            /* [B,T]: best token of target row v (smallest id on ties) */
    float* probs;                  /* [B,T,V] fp32 with SPEC_VERIFY_FLAG_WRITE_PROBS (else unused,
                                      may be NULL): row v = effective target distribution p_v   */
} spec_verify_outputs;

/* Arguments of spec_verify_commit (device pointers; B = batch, T = nodes). */
typedef struct spec_verify_commit_args {
    void* k_cache;              /* [B,Hkv,Lcap,D] dtype, 16-byte aligned: updated in place            */
    void* v_cache;              /* [B,Hkv,Lcap,D] dtype, 16-byte aligned: updated in place            */
    int32_t* kv_len;            /* [B] in: L_b; out: L_b + accept_len[b] + 1 (unchanged if skipped)    */
    const int32_t* path;        /* [B,T] root..v* node ids then -1 (spec_verify_run's output)          */
    const int32_t* accept_len;  /* [B] (spec_verify_run's output)                                     */
    const int32_t* final_node;  /* [B] (spec_verify_run's output; < 0 = void sequence, skipped)        */
    int32_t batch;              /* B: 1..max_batch                                                    */
    int32_t nodes;              /* T: 1..max_nodes, the T of the run                                  */
} spec_verify_commit_args;

/* A paged KV cache: the slots of every sequence live in pages of a shared
 * pool, found through a per-sequence block table ("大模型推理加速：推测解码与
 * MTP核心原理与工程实践", section 4.2 on the candidates' KV memory and section
 * 6.3: speculative KV is held in pages and released page by page).  Slot s of
 * sequence b (prefix 0..L_b-1, tree node i at L_b+i, as in the dense cache) is
 * row s % block_size of page block_table[b, s / block_size] of each pool.  The
 * slots a sequence can address are table_width * block_size; pages may be
 * shared between sequences (a common prefix): runs only read them, a commit
 * writes slots L_b..L_b+accept_len, which the caller keeps in pages of that
 * sequence alone.  Table entries past a sequence's slots in use are never read.
 * A sequence whose entries for slots 0..L_b+T-1 are not all in
 * [0, num_blocks), or whose L_b + T exceeds its slots, gets status bit
 * SPEC_VERIFY_STATUS_BAD_KVLEN and zero attention output (its decisions are
 * taken as usual). */
typedef struct spec_verify_paged_kv {
    void* k_pool;               /* [num_blocks,Hkv,block_size,D] dtype, 16-byte aligned    */
    void* v_pool;               /* [num_blocks,Hkv,block_size,D] dtype, 16-byte aligned    */
    const int32_t* block_table; /* [B,table_width]: page of slots j*block_size..+block_size-1 */
    int32_t num_blocks;         /* pages in each pool, >= 1                                 */
    int32_t block_size;         /* slots per page: a power of two in [16, 65536]            */
    int32_t table_width;        /* entries per sequence, >= 1;
                                   table_width * block_size <= config.kv_capacity          */
} spec_verify_paged_kv;

/* Arguments of spec_verify_build_tree (B = batch, T = nodes, V from the config). */
typedef struct spec_verify_tree_args {
    const float* cand_logits;   /* [B,depth,V] fp32, device: row d-1 holds the logits the depth-d
                                   candidates are taken from (d = 1: the target's next-token
                                   row; d >= 2: Medusa head d-1)                                */
    const int32_t* root_token;  /* [B], device: token of node 0 (the current token)              */
    const int32_t* tree_parent; /* [T], HOST: template parent[] (parent[0] = -1,
                                   0 <= parent[i] < i)                                           */
    const int32_t* tree_rank;   /* [T], HOST: node i >= 1 takes entry tree_rank[i] (0 = best) of
                                   its depth's top-k list; tree_rank[0] is ignored              */
    int32_t* parent;            /* [B,T], device, out: the template, for every sequence          */
    int32_t* tokens;            /* [B,T], device, out: root_token, then the candidates           */
    int32_t batch;              /* B: 1..max_batch                                              */
    int32_t nodes;              /* T: 1..max_nodes                                              */
    int32_t depth;              /* rows per sequence in cand_logits, >= the template's depth    */
} spec_verify_tree_args;

typedef struct spec_verify_handle spec_verify_handle;

/* Validate cfg, size and allocate the workspace on the current HIP device.
 * *out receives the handle.  No kernel is launched.  The fields follow the
 * verifier's inputs on the pages: the target's sampling settings (temperature,
 * top-p) of the generation config in "Medusa推测解码：为LLM推理加速2-3倍的工程实践",
 * section 4.2, which must also be the settings the drafts were sampled with
 * ("投机解码的五条路线", section on exact verification); the tree size of the
 * candidate tree of "推测解码技术详解：加速LLM推理的关键", section "Tree Attention验证".
 * The handle owns only its workspace (allocated here, freed by destroy); the
 * caller owns every array it passes to the other calls.
 * Errors: INVALID_ARG (bad field, unknown or conflicting flags),
 * UNSUPPORTED (a shape outside what the kernels handle: head_dim not 64 or
 * 128, V > 4194304, one (sequence, KV head) slice of the cache of 2 GiB or
 * more, i.e. kv_capacity * head_dim * element size >= 2^31, ...), OOM, HIP. */
int spec_verify_create(const spec_verify_config* cfg, spec_verify_handle** out);

/* Enqueue one verify step on `stream` (a hipStream_t; NULL = default stream):
 * the four parts listed at the top of this file, for every sequence of the
 * batch.  The call shape follows the page's sampler, which takes the draft
 * and target probability rows and the draft tokens and returns the emitted
 * tokens and their count ("推测解码技术详解：加速LLM推理的关键", section
 * "数学保证：无损输出质量"); here the rows come as logits, the tree as parent[],
 * and the random draws as the uniforms u_accept and u_final.
 * Asynchronous: allocates nothing, never synchronises.  All output arrays are
 * written (entries past T or past a sequence's path are -1), except those a
 * SKIP flag leaves out.  One run per handle may be in flight at a time unless
 * runs share the same stream (the workspace is the handle's).
 * Errors: INVALID_ARG (NULL pointer, B or T out of range, draft_logits NULL in
 * sampling mode, probs NULL with SPEC_VERIFY_FLAG_WRITE_PROBS), HIP (launch
 * failure). */
int spec_verify_run(spec_verify_handle* h, const spec_verify_inputs* in,
                    const spec_verify_outputs* out, void* stream);

/* spec_verify_run for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no handle, no hipMalloc/hipFree, no allocating library call.  The
 * workspace (row statistics, final-draw totals, arrival counters, split
 * partials) lives in a 16 MiB array of static device memory that every GPU
 * the library runs on holds from the library's first use there until the
 * process ends; the first call on a GPU looks its address up and clears its
 * counters on `stream`.  Outputs equal spec_verify_run's for the same cfg
 * (decisions and tokens bit for bit; attention within the stated tolerance:
 * when the split partials would not fit, the prefix is split fewer times).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and give wrong results; calls on
 * one stream are ordered.  cfg is validated as in spec_verify_create.
 * Errors: INVALID_ARG (as spec_verify_create and spec_verify_run),
 * UNSUPPORTED (SPEC_VERIFY_FLAG_TIMING or SPEC_VERIFY_FLAG_LOSSLESS_TREE,
 * more than 1024 sequences, or row statistics and draw totals for the batch
 * above 16 MiB), HIP. */
int spec_verify_run_noalloc(const spec_verify_config* cfg, const spec_verify_inputs* in,
                            const spec_verify_outputs* out, void* stream);

/* Enqueue the KV commit of the accepted paths on `stream`: for every sequence,
 * slot L_b+k of both caches (all KV heads) receives tree node path[b,k]
 * (k = 1..accept_len[b]; the root already sits at slot L_b) and kv_len[b]
 * becomes L_b + accept_len[b] + 1.  The caches are preallocated per sequence,
 * so rolling back the rejected nodes is the new length alone (featured
 * article on the founding speculative-decoding paper, section 4.3;
 * "大模型推理加速：推测解码与MTP核心原理与工程实践", section 3.1 item 4 and
 * section 6.3).  A sequence is skipped (caches and kv_len unchanged) when it
 * is void (final_node < 0), L_b + T > Lcap, or path is not a root path
 * (path[0] = 0, k <= path[k] < T).  Asynchronous; allocates nothing.  The
 * caches and kv_len must not be in use by another call in flight; one commit
 * per handle may be in flight at a time unless commits share the same
 * stream (a per-handle counter joins the KV heads of a sequence).
 * Errors: INVALID_ARG (NULL or misaligned pointer, B or T out of range),
 * HIP (launch failure). */
int spec_verify_commit(spec_verify_handle* h, const spec_verify_commit_args* args, void* stream);

/* spec_verify_run with the caches read through a block table: in->k_cache and
 * in->v_cache are ignored, the keys and values of every slot come from
 * paged->k_pool / v_pool (only read).  Every output is the one spec_verify_run
 * gives for the dense caches holding the same slots.  Errors: as
 * spec_verify_run, and INVALID_ARG for a NULL or misaligned pool or table, a
 * block_size that is not a power of two in [16, 65536], or table_width *
 * block_size > config.kv_capacity. */
int spec_verify_run_paged(spec_verify_handle* h, const spec_verify_inputs* in, const spec_verify_paged_kv* paged,
                          const spec_verify_outputs* out, void* stream);

/* spec_verify_commit through a block table: args->k_cache and args->v_cache
 * are ignored; slot L_b+k (k = 1..accept_len[b]) of the pools receives tree
 * node path[b,k]'s row, every KV head, and kv_len[b] becomes
 * L_b + accept_len[b] + 1.  Skipped sequences as spec_verify_commit, and also
 * those whose entries for slots 0..L_b+T-1 leave the pool.  The written slots
 * must not lie in pages another sequence of the batch reads or writes.
 * Errors: as spec_verify_commit, and the paged checks of spec_verify_run_paged. */
int spec_verify_commit_paged(spec_verify_handle* h, const spec_verify_commit_args* args,
                             const spec_verify_paged_kv* paged, void* stream);

/* Build the candidate trees of a Medusa verify step: tokens[b,i] is entry
 * tree_rank[i] of the top-k list of row depth(i)-1 of sequence b (larger
 * logit first, equal logits by smaller token id, NaN below every number),
 * tokens[b,0] = root_token[b], parent[b,:] = tree_parent.  The per-head top-k
 * lists form the tree's levels and the template fixes which combinations are
 * kept ("推测解码技术详解：加速LLM推理的关键", section "Tree Attention验证": the
 * two-head top-2 product tree; "Medusa推测解码：为LLM推理加速2-3倍的工程实践",
 * sections 2.2 and 4.2: top-k candidates per head).  The outputs are the
 * parent/tokens inputs of spec_verify_run.  Asynchronous; allocates nothing.
 * One tree build per handle may be in flight at a time unless builds share
 * the same stream (per-handle slots join the slices of a long row).
 * Errors: INVALID_ARG (NULL or misaligned pointer, B or T out of range, a
 * template that is not topological, a negative rank, a template deeper than
 * `depth`, or more entries needed at some depth than V), UNSUPPORTED (more
 * than 32 entries of one depth's list), HIP (launch failure). */
int spec_verify_build_tree(spec_verify_handle* h, const spec_verify_tree_args* args, void* stream);

/* Host only, no GPU: the template of a pruned Medusa tree.  Candidates are
 * rank tuples (r_1..r_d), 1 <= d <= ncaps, r_k < caps[k-1]; the nodes-1
 * tuples with the smallest key (prod_k (r_k + 1), d, ranks lexicographically)
 * are kept (a child's key exceeds its parent's, so ancestors are kept) and
 * ordered by (d, ranks) after the root.  When nodes-1 is the size of the full
 * Cartesian product nothing is pruned (the product tree of the page section
 * cited above; the pages give no pruning rule, this ordering is this
 * library's).  Writes parent[nodes] and rank[nodes] (host arrays; rank[0] =
 * 0, rank[i] = r_d of node i).  Errors: INVALID_ARG (NULL pointer, ncaps not
 * in [1, 63], a cap < 1, nodes not in [1, 64] or above 1 + the number of
 * tuples). */
int spec_verify_tree_template(const int32_t* caps, int32_t ncaps, int32_t nodes, int32_t* parent, int32_t* rank);

/* Free the workspace and the handle (the counterpart of spec_verify_create;
 * the pages' verifier keeps no state between calls beyond the KV cache, which
 * the caller owns).  The caller's streams must be idle. */
int spec_verify_destroy(spec_verify_handle* h);

/* Message of the last error on this thread ("" if none).  Valid until the
 * next call into the library on this thread.  No exception or abort crosses
 * the boundary: every failure is a return code plus this message. */
const char* spec_verify_last_error(void);

/* Host only (no kernel is launched): the plan a run on this handle with
 * `batch` sequences of `nodes` nodes would follow, as a JSON object written
 * into buf (host memory, NUL-terminated): the names of the kernels it
 * launches ("" for a part that is skipped), the attention's waves per
 * workgroup, row blocks, prefix splits and keys per split, whether the
 * finishing launch selects and/or merges splits, and whether the row
 * statistics run inside the attention launch ("vocab_in_attention_launch":
 * beside a small attention grid that leaves room on the CUs, or after one
 * that fills them when one round of two-row workgroups follows; dense
 * caches, no top-p cut, handles without SPEC_VERIFY_FLAG_TIMING).  For tools that report
 * per-kernel figures (the pages ask for the latency of each round:
 * "投机解码的五条路线", section "怎么选,以及怎么算收益").  Errors: INVALID_ARG
 * (NULL argument, batch or nodes out of range, buffer too small). */
int spec_verify_describe(spec_verify_handle* h, int32_t batch, int32_t nodes, char* buf, int32_t buf_len);

/* Per-round latency of the verify step, by stage (the pages ask for the
 * latency of each round next to the accept lengths: "投机解码的五条路线",
 * section "怎么选,以及怎么算收益").
 * With SPEC_VERIFY_FLAG_TIMING: wait for the runs recorded since the last
 * read, then write into stage_ms[SPEC_VERIFY_NUM_STAGES] the summed kernel
 * time of each stage over those runs (HIP events on the run's stream) and the
 * run count into *runs (host pointers).  At most 1024 runs are kept between
 * reads (older ones are dropped).  Errors: INVALID_ARG (no timing flag). */
int spec_verify_timing_read(spec_verify_handle* h, float* stage_ms, int32_t* runs);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
