// Tree-masked attention of the T candidate nodes over the shared KV prefix.
//
// What is computed (flattened tree with a root-path mask: "大模型推理加速：推测
// 解码与MTP核心原理与工程实践" section 3.2; mask: "推测解码技术详解：加速LLM推理的关键"
// section "Tree Attention验证"; no sibling visibility: "投机解码的五条路线"
// section 4): for sequence b, query head h, node i, KV head kv = h / g,
//   keys S = {0..L_b-1} U {L_b + j : j on node i's root path, i included}
//   O[b,i,h] = softmax_S(scale * Q[b,i,h] . K[b,kv,S]) V[b,kv,S]
//
// Work decomposition (ours, for gfx950): one workgroup per (sequence, KV
// head, prefix split, row block).  All g*T query rows that share a KV head
// sit in the same workgroup family, so a K/V tile read from HBM is used by
// every tree node and every query head of the group.  The tree mask is a
// per-node 64-bit ancestor set built in registers from parent[]; only tiles
// that reach slot L_b pay for masking.  Online softmax runs in the log2
// domain; the splits are merged by the finishing launch (combine.h).
//
// MFMA path (bf16, >= 16 rows per KV head): S^T = K Q^T and O^T = V^T P^T
// with v_mfma_f32_32x32x16_bf16, so the query index is the MFMA column and a
// lane owns one query: the softmax rescale of O never leaves the lane.  Keys
// are permuted inside each 32-key sub-tile (bits 2 and 3 of the row index
// swapped) so that the S^T accumulator registers of a lane are exactly the
// P^T operand the PV product needs, and V^T is staged transposed in LDS.
//
// VALU path (fp32, or fewer than 16 rows per KV head): one wave per block;
// QK^T with one lane per key (bf16 dot2 or fp32 FMA), PV with one lane per
// head-dim column; these shapes are HBM-bound, not contraction-bound.

#include "device_common.h"
#include "kernels.h"
#include "stats_stream.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swap_bits_2_3(int x) {
    return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Chunk swizzle of V rows: the 4 consecutive keys one transposed read touches
// land in 4 disjoint quarters of the row's chunk range.
template <int CH>
__device__ __forceinline__ int v_swizzle(int key) { return (key & 3) * (CH / 4); }

// Maximum of three scores (v_maximum3_f32: NaN-propagating, so the inputs need
// no quieting first; scores are finite or -inf).
__device__ __forceinline__ float fmax3(float a, float b, float c) {
    return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// ---------------------------------------------------------------- MFMA path

// H halves of WAVES waves each: with H = 2 the halves take the two halves of
// the split's tiles and merge their (O, m, l) through LDS at the end, so a
// workgroup of 8 waves covers what two 4-wave workgroups and a merge pass
// would.  Both halves run the same number of steps (barriers are shared); a
// half with one tile fewer runs its last step on a tile past its range,
// whose loads read zeros and whose keys are all masked.
// STREAM: K/V tiles loaded with the non-temporal policy (chosen by the host:
// one row block, large caches).  Tiles are read by every row block of a
// (sequence, KV head, split); with several row blocks the default policy keeps
// them in L2 for the others (at the 70B GQA tree shape, four row blocks,
// non-temporal tile loads fetched 320 MB instead of 288 MB and took 1.7% longer).
// FUSE: workgroups from attn_blocks on compute the streaming row statistics
// of S instead (one logits row per 256 threads: one row per 256-thread
// workgroup, two per 512-thread workgroup).
template <int D, int WAVES, bool PAGED, int H, bool STREAM, bool FUSE = false>
__global__ __launch_bounds__(WAVES * 64 * H, 2) void attn_mfma_kernel(AttnParams P, StatsParams S, int attn_blocks) {   // 2 waves per SIMD
    if constexpr (FUSE) {
        if ((int)blockIdx.x >= attn_blocks) {
            if constexpr (WAVES * 64 * H == kStatsThreads) {   // one row per workgroup
                if (S.sampling) row_stats_stream_block<true>(S, (int)blockIdx.x - attn_blocks);
                else row_stats_stream_block<false>(S, (int)blockIdx.x - attn_blocks);
            } else {                                           // two rows, one per half
                static_assert(WAVES * 64 * H == 2 * kStatsThreads, "row statistics groups of 256 threads");
                if (S.sampling) row_stats_stream_pair<true>(S, (int)blockIdx.x - attn_blocks);
                else row_stats_stream_pair<false>(S, (int)blockIdx.x - attn_blocks);
            }
            return;
        }
    }
    constexpr int NSUB = 2;                 // 32-key sub-tiles per tile
    constexpr int KT = 32 * NSUB;           // keys per tile
    constexpr int CH = D / 8;               // 16-byte chunks per K/V row
    constexpr int KSTEPS = D / 16;          // k-steps of the QK^T product
    constexpr int DT = D / 32;              // 32-row tiles of O^T
    static_assert((KT * D * 2 / 1024) % WAVES == 0, "whole 1 KB blocks per wave");

    // Two buffers each for K and V, as four separate LDS objects: the compiler
    // then knows that the loads filling one buffer never alias the reads of
    // another and does not wait for the prefetch before reading the current tile.
    __shared__ __align__(16) uint8_t k_lds0_all[H * KT * D * 2];
    __shared__ __align__(16) uint8_t k_lds1_all[H * KT * D * 2];
    __shared__ __align__(16) uint8_t v_lds0_all[H * KT * D * 2];
    __shared__ __align__(16) uint8_t v_lds1_all[H * KT * D * 2];
    __shared__ unsigned long long anc_lds[64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int hv = __builtin_amdgcn_readfirstlane((tid >> 6) / WAVES);   // which half of the split's tiles
    const int wave = (tid >> 6) % WAVES;      // wave within the half
    uint8_t* const k_lds0 = k_lds0_all + hv * (KT * D * 2);
    uint8_t* const k_lds1 = k_lds1_all + hv * (KT * D * 2);
    uint8_t* const v_lds0 = v_lds0_all + hv * (KT * D * 2);
    uint8_t* const v_lds1 = v_lds1_all + hv * (KT * D * 2);
    int group, rb;
    if (P.rowblocks == 1) {
        group = blockIdx.x;
        rb = 0;
    } else {  // row blocks of one (pair, split) go to the same XCD, back to back
        const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
        rb = local % P.rowblocks;
        group = (local / P.rowblocks) * 8 + xcd;
    }
    if (group >= P.B * P.Hkv * P.nsplit) return;
    // workgroups in order of decreasing prefix length (longest first); group
    // becomes the (sequence, KV head, split) slot of the partial results
    const int pair0 = group / P.nsplit, split = group - pair0 * P.nsplit;
    const int rank = pair0 / P.Hkv, kvh = pair0 - rank * P.Hkv;
    const int2 bl = seq_by_length(P.kv_len, P.B, rank);
    const int b = bl.x, L = bl.y;
    const int pair = b * P.Hkv + kvh;
    group = pair * P.nsplit + split;
    const int T = P.T, g = P.g;
    bool kv_ok = (L >= 0) && (L <= P.Lcap - T);
    const int N = L + T;
    if constexpr (PAGED) {   // every table entry of the used slots must name a page of the pool
        const bool bad = kv_ok && page_entries_bad(P.pt, b, N, tid, WAVES * 64 * H);
        kv_ok = kv_ok && !__syncthreads_or(bad);
    }
    const int s0 = split * P.chunk;            // the workgroup's keys [s0, s1)
    const int s1 = min(N, s0 + P.chunk);
    const int nsteps = (s1 - s0 + KT - 1) / KT / H + ((s1 - s0 + KT - 1) / KT % H ? 1 : 0);
    const int k0 = s0 + hv * nsteps * KT;      // this half's keys [k0, k1)
    const int k1 = (hv == H - 1) ? s1 : min(s1, k0 + nsteps * KT);
    const int qcol = lane & 31, half = lane >> 5;
    const int r = rb * (WAVES * 32) + wave * 32 + qcol;
    const bool row_ok = r < P.R;
    const int node = row_ok ? r / g : 0;
    const int head = kvh * g + (row_ok ? r - node * g : 0);
    const size_t part_row = (size_t)group * P.Rpad + r;

    if (!kv_ok || s0 >= s1) {
        if (hv != 0) return;
        if (P.nsplit == 1) {
            if (row_ok) {
                uint16_t* o = (uint16_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * D;
                for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) o[d] = 0;
            }
        } else if (row_ok && half == 0) {
            P.part_ml[part_row] = make_float2(-INFINITY, 0.f);
        }
        return;
    }

    if (tid < kWave) {
        bool bad;
        unsigned long long a = ancestor_mask(P.parent + (size_t)b * T, T, &bad);
        anc_lds[lane] = a;
    }

    // Q^T operand: lane holds Q[row r][16*ks + 8*half .. +7] for every k-step.
    bf16x8_t qb[KSTEPS];
    {
        const uint16_t* qrow = (const uint16_t*)P.q + ((size_t)(b * T + node) * P.Hq + head) * D;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4*)(qrow + 16 * ks + 8 * half);
            qb[ks] = as_bf16x8(v);
        }
    }
    __syncthreads();
    const unsigned long long anc_row = anc_lds[node];

    floatx16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    float neg_m = 0.f;   // -m_run, or 0 while no key has been seen
    const floatx16_t zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int krow = swap_bits_2_3(qcol);   // key (within a 32-key sub-tile) fed to MFMA row qcol

    // Tile staging straight from HBM into LDS: buffer loads with the LDS as
    // destination (each lane's 16 bytes land at the LDS base + 16 * lane).
    // The chunk swizzles of the LDS layout (K: chunk ^ key%CH for the MFMA
    // operand reads, V: chunk ^ v_swizzle(key) for the transposed reads) are
    // applied on the global side: lane i of a 1 KB block loads the logical
    // chunk that belongs at its slot.  The buffer resources end at key k1, so
    // loads past the split read zeros (and those keys are masked or unused).
    //
    // Paged caches: a 1 KB block (4 or 8 rows) never straddles a page (pages
    // hold a power of two >= 16 slots), so each block load gets a resource of
    // its own, based at the block's page and ending at key k1 or the page's
    // end.  The page entries of a step's loads are fetched one step ahead:
    // lane l of the fetched register holds the entry of block load l (-1 past
    // the split); the step reads them into scalar registers.
    constexpr uint32_t kRsrcFlags = 0x00020000;
    constexpr int kTilePolicy = STREAM ? kStreamPolicy : 0;
    const size_t head_off = PAGED ? (size_t)kvh * ((size_t)D << P.pt.bs_log2)
                                  : (size_t)(b * P.Hkv + kvh) * P.Lcap * D;
    const uint16_t* kbase = (const uint16_t*)P.k + head_off;
    const uint16_t* vbase = (const uint16_t*)P.v + head_off;
    // paged: one resource per pool, based at this KV head's slice of page 0;
    // a block wholly inside a page and the split is read through it with the
    // page's offset as the scalar offset (when the pool spans < 4 GiB)
    const int page_bytes = PAGED ? P.Hkv * (D << P.pt.bs_log2) * 2 : 0;
    const bool pool_small = PAGED && (uint64_t)P.pt.num_blocks * (uint64_t)page_bytes < (1ull << 32);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, PAGED ? -1 : k1 * D * 2, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, PAGED ? -1 : k1 * D * 2, kRsrcFlags);
    constexpr int BLOCKS = KT * D * 2 / 1024;          // 1 KB blocks per tile and operand
    constexpr int ROWS_PER_BLOCK = 1024 / (D * 2);
    constexpr int LOADS = 2 * BLOCKS / WAVES;           // K and V blocks one wave loads per tile
    static_assert(LOADS <= 64, "one page entry per lane");
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int32_t* trow = PAGED ? P.pt.table + (size_t)b * P.pt.width : nullptr;
    // page entries of the block loads of a step that loads K at key tk and V at key tv
    auto load_pages = [&](int tk, int tv) -> int {
        int e = -1;
        if (PAGED && lane < LOADS) {
            const bool isk = lane < LOADS / 2;
            const int blk = (isk ? lane : lane - LOADS / 2) * WAVES + wave_u;
            const int key0 = (isk ? tk : tv) + blk * ROWS_PER_BLOCK;
            if (key0 < k1) e = trow[key0 >> P.pt.bs_log2];
        }
        return e;
    };
    // block load l of a tile: l < LOADS/2 -> K of the tile at key tk, else V at key tv
    auto issue_load = [&](int l, int tk, uint8_t* kdst, int tv, uint8_t* vdst, int page) {
        const bool isk = l < LOADS / 2;
        const int blk = (isk ? l : l - LOADS / 2) * WAVES + wave_u;
        const int row = blk * ROWS_PER_BLOCK + lane / CH;
        const int c = (lane % CH) ^ (isk ? (row & (CH - 1)) : v_swizzle<CH>(row));
        auto* dst = (__attribute__((address_space(3))) void*)((isk ? kdst : vdst) + blk * 1024);
        if constexpr (PAGED) {
            const int key0 = (isk ? tk : tv) + blk * ROWS_PER_BLOCK;
            const int in_page = key0 & ((1 << P.pt.bs_log2) - 1);
            if (pool_small && page >= 0 && key0 + ROWS_PER_BLOCK <= k1) {   // wave-uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? krs : vrs, dst, 16, (in_page + lane / CH) * (D * 2) + c * 16,
                                                         (uint32_t)page * (uint32_t)page_bytes, 0, kTilePolicy);
                return;
            }
            const int room = min(max(k1 - (key0 - in_page), 0), 1 << P.pt.bs_log2);
            const size_t page_off = ((size_t)max(page, 0) * P.Hkv) * ((size_t)D << P.pt.bs_log2);
            // every operand of the resource is wave-uniform: keep it in scalar registers
            const uint64_t addr = (uint64_t)((isk ? kbase : vbase) + page_off);
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
            const int bytes = __builtin_amdgcn_readfirstlane(page >= 0 ? room * D * 2 : 0);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(((uint64_t)hi << 32) | lo), 0, bytes, kRsrcFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (in_page + lane / CH) * (D * 2) + c * 16, 0, 0, kTilePolicy);
        } else {
            // a resource based at the tile and ending at key k1 (wave-uniform,
            // built in scalar registers), so the lane offset is the same at
            // every step and loads past the split still read zeros
            const int key = isk ? tk : tv;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)((isk ? kbase : vbase) + (size_t)key * D), 0, max(k1 - key, 0) * (D * 2), kRsrcFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, row * (D * 2) + c * 16, 0, 0, kTilePolicy);
        }
    };

    // MFMA operands.  QK^T product i (i < NQK) is sub-tile i % NSUB, k-step
    // i / NSUB; PV product i (i < NPV) is O^T tile i % DT, 16-key step i / DT.
    constexpr int NQK = NSUB * KSTEPS;
    constexpr int NPV = DT * NSUB * 2;
    auto read_k = [&](const uint8_t* kl, int i) -> bf16x8_t {
        const int kk = (i % NSUB) * 32 + krow;
        const int c = 2 * (i / NSUB) + half;
        return as_bf16x8(*(const u32x4*)(kl + kk * (D * 2) + ((c ^ (kk & (CH - 1))) << 4)));
    };
    // PV operand by transposed LDS reads (ds_read_b64_tr_b16): within each
    // 16-lane group, source lane s addresses 4 columns (4*(s&3)..+3) of key row
    // s>>2 of a 4-key block, and output lane j receives column j of all 4 keys.
    // Lane l = (G = l>>4, s = l&15) therefore reads key 8*(G>>1) + 4*h + (s>>2)
    // of the 16-key step and columns 32*dt + 16*(G&1) + 4*(s&3); it gets the
    // column 32*dt + (l&31) for keys 8*(l>>5) + 4*h + 0..3: with h = 0, 1 these
    // are the 8 k-slots the P^T operand of the lane holds.
    const int tr_key = 8 * (lane >> 5) + (((lane & 15) >> 2));
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto read_v = [&](const uint8_t* vl, int i) -> bf16x8_t {
        const int dt = i % DT, step16 = i / DT;
        const int col = 32 * dt + tr_col;
        const int key0 = 16 * step16 + tr_key;
        const int key1 = key0 + 4;
        const int c = col >> 3;
        const uint8_t* p0 = vl + key0 * (D * 2) + ((c ^ v_swizzle<CH>(key0)) << 4) + (col & 7) * 2;
        const uint8_t* p1 = vl + key1 * (D * 2) + ((c ^ v_swizzle<CH>(key1)) << 4) + (col & 7) * 2;
        const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
        const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p1);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // Scores: accumulator element e of lane (qcol, half) in sub-tile sub holds
    // key sub*32 + 16*(e>>3) + 8*half + (e&7).  Masking is needed only for
    // tiles that reach the tree slots or the end of the split.  Each score is
    // replaced in its own register (a select written as an instruction whose
    // output is tied to its input): written as a plain select, the masked
    // branch produced the scores in new registers and the unmasked path of
    // every step copied all 32 of them to match.
    auto mask_tile = [&](int t, floatx16_t (&s)[NSUB]) {
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = t + sub * 32 + 16 * (e >> 3) + 8 * half + (e & 7);
                const unsigned rel = (unsigned)(key - L);
                const bool tree_vis = (anc_row >> (rel & 63u)) & 1ull;
                const bool vis = (key < k1) & ((key < L) | tree_vis);   // no short circuit: no branch per key
                const unsigned long long hide = __ballot(!vis);   // lanes whose key is hidden
                float x = s[sub][e];
                asm volatile("v_cndmask_b32_e64 %0, %0, %1, %2" : "+v"(x) : "v"(-INFINITY), "s"(hide));
                s[sub][e] = x;
            }
    };
    auto tile_max = [&](const floatx16_t (&s)[NSUB]) {
        float mx = -INFINITY;
#pragma unroll
        for (int f = 0; f < 16 * NSUB; f += 2) mx = fmax3(mx, s[f / 16][f % 16], s[f / 16][f % 16 + 1]);
        return fmaxf(mx, __shfl_xor(mx, 32, kWave));
    };
    // Online softmax in the log2 domain.  The exponent reference m_run is set
    // from the first tile's maximum and raised only when a tile's weights
    // would grow too large (see the step), so no per-tile maximum is taken:
    // weights exp2(s*c - m_run) of a lane stay below 2^64 in sum (exact enough
    // as bf16 products with fp32 sums), and a weight that underflows to 0 lies
    // below 2^-126 of the largest one seen.
    auto raise_reference = [&](float mx) {
        const float mt = mx * P.c;
        if (__any(mt > m_run)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
            m_run = m_new;
            neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
        }
    };
    const bf16x2_t ones2 = {(__bf16)1.0f, (__bf16)1.0f};

    // Software pipeline over tiles, K two tiles ahead of V in LDS.  K(t) sits
    // in k_lds[(t/KT)&1] and V(t) in v_lds[(t/KT)&1]; a buffer is refilled
    // only after the barrier that follows its last read, and the loop is
    // unrolled by two so that every LDS access names its buffer statically.
    // The weights of a tile are taken in two halves (sub-tile 0: keys 0..31,
    // sub-tile 1: keys 32..63), so that every MFMA of both phases has its
    // share of exp2 beside it (one at D = 128, two at D = 64).  Step t:
    //   phase A: the QK^T products of tile t+1, each with the K read two
    //            products ahead, a share of the block loads of K(t+2) and
    //            V(t+1), and its share of tile t's sub-tile 1 weights (exp2;
    //            for each pair the bf16 pack and the row sum by dot2);
    //   check:   a lane whose weights of tile t sum to 2^64 or more (scores far
    //            above the reference), or that has no reference yet, makes the
    //            wave take tile t's maximum, raise the reference and weigh the
    //            tile again (rare: once per row block in practice);
    //   phase B: masking of tile t+1 if it reaches the tree slots or the split
    //            end, then the PV products of tile t (sub-tile 0's weights
    //            first), each with its two transposed V reads two products
    //            ahead and its share of tile t+1's sub-tile 0 weights.
    // Scheduling fences keep this order, so the matrix cores and the vector
    // ALU work side by side within the wave.  Products of a tile past the
    // split read stale or zero data and are never used.
    constexpr int PF = 2;                        // operand reads in flight
    constexpr int WA = 16 / NQK, WB = 16 / NPV;  // weights beside each product of phase A / phase B
    static_assert(WA * NQK == 16 && WB * NPV == 16, "16 weights per sub-tile spread over each phase");
    // weight f (0..31) of a tile: exp2, and for odd f the bf16 pair and its row sum
    // Weight pair q of a tile sits in 32-bit word q % 4 of wp[q / 4], so the
    // four pairs of a 16-key step are the PV operand as they stand (built
    // from separate pairs, the compiler shifted and permuted them into place).
    auto weigh_one = [&](const floatx16_t (&s)[NSUB], float (&w)[2], u32x4 (&wp)[2 * NSUB], float (&ps)[2], int f) {
        w[f & 1] = __builtin_amdgcn_exp2f(fmaf(s[f / 16][f % 16], P.c, neg_m));
        if (f & 1) {
            const bf16x2_t pair = __builtin_convertvector((floatx2_t){w[0], w[1]}, bf16x2_t);
            wp[f / 8][(f / 2) % 4] = __builtin_bit_cast(uint32_t, pair);
            ps[(f / 2) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones2, ps[(f / 2) & 1], false);
        }
    };
    auto weigh_all = [&](const floatx16_t (&s)[NSUB], u32x4 (&wp)[2 * NSUB], float (&ps)[2]) {
        float w[2];
        ps[0] = ps[1] = 0.f;
#pragma unroll
        for (int f = 0; f < 16 * NSUB; ++f) weigh_one(s, w, wp, ps, f);
    };
    auto step = [&](int t, const uint8_t* k_next, const uint8_t* v_cur, uint8_t* k_fill, uint8_t* v_fill,
                    floatx16_t (&s_cur)[NSUB], floatx16_t (&s_next)[NSUB], u32x4 (&wp_cur)[2 * NSUB],
                    u32x4 (&wp_next)[2 * NSUB], float (&ps_cur)[2], float (&ps_next)[2], int pg_cur, int& pg_next) {
        int pages[LOADS];   // wave-uniform page entries of this step's block loads
#pragma unroll
        for (int l = 0; l < LOADS; ++l) pages[l] = PAGED ? __builtin_amdgcn_readlane(pg_cur, l) : -1;
        if constexpr (PAGED) pg_next = load_pages(t + 3 * KT, t + 2 * KT);
        bf16x8_t ka[NQK];
        float w[2];
#pragma unroll
        for (int i = 0; i < PF; ++i) ka[i] = read_k(k_next, i);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            if (i + PF < NQK) ka[i + PF] = read_k(k_next, i + PF);
#pragma unroll
            for (int l = 0; l < LOADS; ++l)
                if (l * NQK / LOADS == i) issue_load(l, t + 2 * KT, k_fill, t + KT, v_fill, pages[l]);
            s_next[i % NSUB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qb[i / NSUB],
                                                                       i < NSUB ? zero16 : s_next[i % NSUB], 0, 0, 0);
#pragma unroll
            for (int f = 16 + WA * i; f < 16 + WA * (i + 1); ++f) weigh_one(s_cur, w, wp_cur, ps_cur, f);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (__any(!(ps_cur[0] + ps_cur[1] < 0x1p64f) || m_run == -INFINITY)) {
            raise_reference(tile_max(s_cur));
            weigh_all(s_cur, wp_cur, ps_cur);
        }
        l_run += ps_cur[0] + ps_cur[1];
        if (t + 2 * KT > L || t + 2 * KT > k1) mask_tile(t + KT, s_next);
        ps_next[0] = ps_next[1] = 0.f;
        bf16x8_t va[NPV];
#pragma unroll
        for (int i = 0; i < PF; ++i) va[i] = read_v(v_cur, i);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + PF < NPV) va[i + PF] = read_v(v_cur, i + PF);
            const bf16x8_t pbj = __builtin_bit_cast(bf16x8_t, wp_cur[i / DT]);   // 16-key step i / DT
            o[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pbj, o[i % DT], 0, 0, 0);
#pragma unroll
            for (int f = WB * i; f < WB * (i + 1); ++f) weigh_one(s_next, w, wp_next, ps_next, f);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The next tile's sub-tile 0 weights are used here, on every path: without
        // this use the compiler sinks them past the loop's exit test between the
        // two unrolled steps, and the first step's PV products then run with no
        // weights beside them while the second step's QK products get twice as many.
        asm volatile("" ::"v"(wp_next[0]), "v"(wp_next[1]), "v"(ps_next[0]), "v"(ps_next[1]));
        __builtin_amdgcn_s_waitcnt(0);    // K(t+2) and V(t+1) have landed
        __syncthreads();
    };

    floatx16_t sa[NSUB], sb[NSUB];
    u32x4 wa[2 * NSUB], wb[2 * NSUB];
    float psa[2] = {0.f, 0.f}, psb[2] = {0.f, 0.f};
    int pga = -1, pgb = -1;
    if constexpr (PAGED) {
        const int p0 = load_pages(k0, k0), p1 = load_pages(k0 + KT, k0 + KT);
        pga = load_pages(k0 + 2 * KT, k0 + KT);   // the first step's loads
        __builtin_amdgcn_s_waitcnt(0);
        pgb = p1;
#pragma unroll
        for (int l = 0; l < LOADS; ++l) issue_load(l, k0, k_lds0, k0, v_lds0, __builtin_amdgcn_readlane(p0, l));
    } else {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) issue_load(l, k0, k_lds0, k0, v_lds0, -1);
    }
#pragma unroll
    for (int l = 0; l < LOADS / 2; ++l)
        issue_load(l, k0 + KT, k_lds1, 0, nullptr, PAGED ? __builtin_amdgcn_readlane(pgb, l) : -1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NQK; ++i)
        sa[i % NSUB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_k(k_lds0, i), qb[i / NSUB],
                                                               i < NSUB ? zero16 : sa[i % NSUB], 0, 0, 0);
    // the reference starts at the first tile's maximum (after its masking);
    // sub-tile 0 of the first tile is weighed here, the rest in the first step
    if (k0 + KT > L || k0 + KT > k1) mask_tile(k0, sa);
    raise_reference(tile_max(sa));
    {
        float w[2];
#pragma unroll
        for (int f = 0; f < 16; ++f) weigh_one(sa, w, wa, psa, f);
    }
    __builtin_amdgcn_s_waitcnt(0);       // every wave is done with K(k0) before it is refilled
    __syncthreads();
    for (int st = 0; st < nsteps; st += 2) {
        const int t = k0 + st * KT;
        step(t, k_lds1, v_lds0, k_lds0, v_lds1, sa, sb, wa, wb, psa, psb, pga, pgb);
        if (st + 1 >= nsteps) break;
        step(t + KT, k_lds0, v_lds1, k_lds1, v_lds0, sb, sa, wb, wa, psb, psa, pgb, pga);
    }

    float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    if constexpr (H == 2) {
        // half 1 hands (O, m, l) to half 0 through the (now idle) tile buffers:
        // O tiles 0..DT/2-1 in the K buffers 0, the rest in K buffers 1, (m, l) in V buffers 0
        auto xo = [&](int dt, int e) -> float* {
            uint8_t* arr = dt < DT / 2 ? k_lds0_all : k_lds1_all;
            return (float*)arr + ((wave * (DT / 2) + dt % (DT / 2)) * 16 + e) * kWave + lane;
        };
        float2* xml = (float2*)v_lds0_all + wave * kWave + lane;
        if (hv == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) *xo(dt, e) = o[dt][e];
            *xml = make_float2(m_run, l_tot);
        }
        __syncthreads();
        if (hv == 1) return;
        const float2 mlb = *xml;
        const float ma = l_tot > 0.f ? m_run : -INFINITY, mb = mlb.y > 0.f ? mlb.x : -INFINITY;
        const float mm = fmaxf(ma, mb);
        const float wa = l_tot > 0.f ? __builtin_amdgcn_exp2f(ma - mm) : 0.f;
        const float wb = mlb.y > 0.f ? __builtin_amdgcn_exp2f(mb - mm) : 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] = wa * o[dt][e] + wb * *xo(dt, e);
        l_tot = wa * l_tot + wb * mlb.y;
        m_run = mm;
    }
    if (!row_ok) return;
    // O^T element e of tile dt: column d = 32*dt + 8*(e>>2) + 4*half + (e&3)
    if (P.nsplit == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = (uint16_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int d = 32 * dt + 8 * e4 + 4 * half;
                u32x2 w = {pack_bf16x2(o[dt][4 * e4] * inv, o[dt][4 * e4 + 1] * inv),
                           pack_bf16x2(o[dt][4 * e4 + 2] * inv, o[dt][4 * e4 + 3] * inv)};
                *(u32x2*)(orow + d) = w;
            }
        }
    } else {
        float* prow = P.part_o + part_row * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int d = 32 * dt + 8 * e4 + 4 * half;
                *(floatx4_t*)(prow + d) = floatx4_t{o[dt][4 * e4], o[dt][4 * e4 + 1], o[dt][4 * e4 + 2],
                                                    o[dt][4 * e4 + 3]};
            }
        }
        if (half == 0) P.part_ml[part_row] = make_float2(m_run, l_tot);
    }
}

// ---------------------------------------------------------------- VALU path

template <bool BF16, int D, int MAXR, bool PAGED>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnParams P) {
    constexpr int KT = 64;
    constexpr int EB = BF16 ? 2 : 4;
    constexpr int ROWB = D * EB;
    constexpr int CH = ROWB / 16;
    constexpr int DPL = D / 64;             // head-dim columns per lane in PV

    __shared__ __align__(16) uint8_t q_lds[MAXR * ROWB];
    __shared__ __align__(16) uint8_t k_lds[KT * ROWB];
    __shared__ __align__(16) float p_lds[KT * MAXR];
    __shared__ unsigned long long anc_lds[64];
    __shared__ size_t row_lds[PAGED ? KT : 1];   // paged: byte offset of each key row of the tile

    const int lane = threadIdx.x;
    const int rb = blockIdx.x % P.rowblocks;
    const int group = blockIdx.x / P.rowblocks;
    const int pair = group / P.nsplit, split = group - pair * P.nsplit;
    const int b = pair / P.Hkv, kvh = pair - b * P.Hkv;
    const int T = P.T, g = P.g;
    const int L = P.kv_len[b];
    bool kv_ok = (L >= 0) && (L <= P.Lcap - T);
    const int N = L + T;
    if constexpr (PAGED) kv_ok = kv_ok && !__any(page_entries_bad(P.pt, b, N, lane, 64));
    const int k0 = split * P.chunk;
    const int k1 = min(N, k0 + P.chunk);
    const int rbase = rb * MAXR;

    if (!kv_ok || k0 >= k1) {
        for (int j = 0; j < MAXR; ++j) {
            const int r = rbase + j;
            if (r >= P.R) break;
            const int node = r / g, head = kvh * g + (r - node * g);
            if (P.nsplit == 1) {
                uint8_t* o = (uint8_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * ROWB;
                for (int x = lane; x < ROWB / 4; x += 64) ((uint32_t*)o)[x] = 0u;
            } else if (lane == 0) {
                P.part_ml[(size_t)group * P.Rpad + r] = make_float2(-INFINITY, 0.f);
            }
        }
        return;
    }

    {
        bool bad;
        anc_lds[lane] = ancestor_mask(P.parent + (size_t)b * T, T, &bad);
    }
    for (int idx = lane; idx < MAXR * CH; idx += 64) {
        const int j = idx / CH, c = idx - j * CH;
        const int r = rbase + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < P.R) {
            const int node = r / g, head = kvh * g + (r - node * g);
            v = *(const u32x4*)((const uint8_t*)P.q + ((size_t)(b * T + node) * P.Hq + head) * ROWB + c * 16);
        }
        *(u32x4*)(q_lds + j * ROWB + c * 16) = v;
    }
    __syncthreads();
    unsigned long long anc_r[MAXR];
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        const int r = rbase + j;
        anc_r[j] = anc_lds[r < P.R ? r / g : 0];
    }

    // Dense: row of key j at kbase + j * ROWB.  Paged: at kbase + row_lds[j - t]
    // for the keys of tile t (page base of this KV head + row in the page).
    const size_t head_off = PAGED ? (size_t)kvh * ((size_t)ROWB << P.pt.bs_log2)
                                  : (size_t)(b * P.Hkv + kvh) * P.Lcap * ROWB;
    const uint8_t* kbase = (const uint8_t*)P.k + head_off;
    const uint8_t* vbase = (const uint8_t*)P.v + head_off;
    const int32_t* trow = PAGED ? P.pt.table + (size_t)b * P.pt.width : nullptr;
    auto row_off = [&](int t, int key) -> size_t {
        if constexpr (PAGED) return row_lds[key];
        else return (size_t)(t + key) * ROWB;
    };

    float m_run[MAXR], l_run[MAXR], o[MAXR][DPL];
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int x = 0; x < DPL; ++x) o[j][x] = 0.f;
    }

    for (int t = k0; t < k1; t += KT) {
        if constexpr (PAGED) {
            const int slot = t + lane;
            size_t off = 0;
            if (slot < k1) {
                const int page = trow[slot >> P.pt.bs_log2];
                off = (size_t)page * P.Hkv * ((size_t)ROWB << P.pt.bs_log2) +
                      (size_t)(slot & ((1 << P.pt.bs_log2) - 1)) * ROWB;
            }
            row_lds[lane] = off;
            __syncthreads();
        }
        for (int idx = lane; idx < KT * CH; idx += 64) {
            const int key = idx / CH, c = idx - key * CH;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t + key < k1) v = *(const u32x4*)(kbase + row_off(t, key) + c * 16);
            *(u32x4*)(k_lds + key * ROWB + ((c ^ (key & (CH - 1))) << 4)) = v;
        }
        __syncthreads();

        // scores: lane = key
        float s[MAXR];
#pragma unroll
        for (int j = 0; j < MAXR; ++j) s[j] = 0.f;
        for (int c = 0; c < CH; ++c) {
            const u32x4 kc = *(const u32x4*)(k_lds + lane * ROWB + ((c ^ (lane & (CH - 1))) << 4));
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {
                const u32x4 qc = *(const u32x4*)(q_lds + j * ROWB + c * 16);
                if constexpr (BF16) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        // copy the lanes out of the vectors first: a bit_cast of a vector
                        // element is lowered as a cast of element 0 by this compiler
                        const uint32_t qw = qc[w], kw = kc[w];
                        s[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw),
                                                               __builtin_bit_cast(bf16x2_t, kw), s[j], false);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) s[j] = fmaf(__uint_as_float(qc[w]), __uint_as_float(kc[w]), s[j]);
                }
            }
        }

        const int key = t + lane;
        const bool tail = key >= L;
#pragma unroll
        for (int j = 0; j < MAXR; ++j) {
            float val = s[j] * P.c;
            const bool vis = key < k1 && (!tail || ((anc_r[j] >> (key - L)) & 1ull));
            if (!vis) val = -INFINITY;
            const float mx = wave_max(val);
            const float m_new = fmaxf(m_run[j], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run[j] - m_use);
            const float p = exp2f(val - m_use);
            m_run[j] = m_new;
            l_run[j] = l_run[j] * alpha + p;
#pragma unroll
            for (int x = 0; x < DPL; ++x) o[j][x] *= alpha;
            p_lds[lane * MAXR + j] = p;
        }
        __syncthreads();

        // PV: lane owns head-dim columns lane*DPL .. +DPL-1
        const int nk = min(KT, k1 - t);
        for (int kk = 0; kk < nk; ++kk) {
            float v[DPL];
            const uint8_t* vrow = vbase + row_off(t, kk);
            if constexpr (BF16) {
                if constexpr (DPL == 2) {
                    const uint32_t w = *(const uint32_t*)(vrow + lane * 4);
                    v[0] = bf16_lo(w);
                    v[1] = bf16_hi(w);
                } else {
                    v[0] = __uint_as_float(((uint32_t) * (const uint16_t*)(vrow + lane * 2)) << 16);
                }
            } else {
#pragma unroll
                for (int x = 0; x < DPL; ++x) v[x] = *(const float*)(vrow + (lane * DPL + x) * 4);
            }
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {
                const float p = p_lds[kk * MAXR + j];
#pragma unroll
                for (int x = 0; x < DPL; ++x) o[j][x] = fmaf(p, v[x], o[j][x]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        const float l_tot = wave_sum(l_run[j]);
        const int r = rbase + j;
        if (r >= P.R) continue;
        const int node = r / g, head = kvh * g + (r - node * g);
        if (P.nsplit == 1) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            uint8_t* orow = (uint8_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * ROWB;
#pragma unroll
            for (int x = 0; x < DPL; ++x) {
                const int d = lane * DPL + x;
                if constexpr (BF16)
                    ((uint16_t*)orow)[d] = (uint16_t)f32_to_bf16_bits(o[j][x] * inv);
                else
                    ((float*)orow)[d] = o[j][x] * inv;
            }
        } else {
            const size_t prow = (size_t)group * P.Rpad + r;
#pragma unroll
            for (int x = 0; x < DPL; ++x) P.part_o[prow * D + lane * DPL + x] = o[j][x];
            if (lane == 0) P.part_ml[prow] = make_float2(m_run[j], l_tot);
        }
    }
}

// ---------------------------------------------------------------- split merge

template <bool BF16, int D, bool PAGED>
void launch_valu_rows_p(const AttnParams& p, int maxr, dim3 grid, hipStream_t s) {
    switch (maxr) {
        case 2: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 2, PAGED>), grid, dim3(64), 0, s, p); break;
        case 4: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 4, PAGED>), grid, dim3(64), 0, s, p); break;
        case 6: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 6, PAGED>), grid, dim3(64), 0, s, p); break;
        case 8: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 8, PAGED>), grid, dim3(64), 0, s, p); break;
        case 12: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 12, PAGED>), grid, dim3(64), 0, s, p); break;
        default: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 16, PAGED>), grid, dim3(64), 0, s, p); break;
    }
}

template <bool BF16, int D>
hipError_t launch_valu_rows(const AttnParams& p, int maxr, dim3 grid, hipStream_t s) {
    if (p.pt.table) launch_valu_rows_p<BF16, D, true>(p, maxr, grid, s);
    else launch_valu_rows_p<BF16, D, false>(p, maxr, grid, s);
    return hipGetLastError();
}

template <int D, bool PAGED, bool STREAM>
void launch_mfma_waves_s(const AttnParams& p, int waves, dim3 grid, hipStream_t s, const StatsParams* fused, int blocks) {
    constexpr int H = kMfmaHalves;
    const StatsParams S = fused ? *fused : StatsParams{};
    const int nrows = S.sampling ? 2 * S.T : S.T;
    if (fused && waves * 64 * H == kStatsThreads) {
        hipLaunchKernelGGL((attn_mfma_kernel<D, kStatsThreads / (64 * H), PAGED, H, STREAM, true>),
                           dim3(blocks + S.B * nrows), dim3(kStatsThreads), 0, s, p, S, blocks);
    } else if (fused && waves * 64 * H == 2 * kStatsThreads) {
        hipLaunchKernelGGL((attn_mfma_kernel<D, 2 * kStatsThreads / (64 * H), PAGED, H, STREAM, true>),
                           dim3(blocks + (S.B * nrows + 1) / 2), dim3(2 * kStatsThreads), 0, s, p, S, blocks);
    } else if (waves == 4) {
        hipLaunchKernelGGL((attn_mfma_kernel<D, 4, PAGED, H, STREAM>), grid, dim3(256 * H), 0, s, p, S, blocks);
    } else if (waves == 2) {
        hipLaunchKernelGGL((attn_mfma_kernel<D, 2, PAGED, H, STREAM>), grid, dim3(128 * H), 0, s, p, S, blocks);
    } else {
        hipLaunchKernelGGL((attn_mfma_kernel<D, 1, PAGED, H, STREAM>), grid, dim3(64 * H), 0, s, p, S, blocks);
    }
}

template <int D, bool PAGED>
void launch_mfma_waves(const AttnParams& p, int waves, dim3 grid, hipStream_t s, const StatsParams* fused) {
    if (p.stream) launch_mfma_waves_s<D, PAGED, true>(p, waves, grid, s, fused, (int)grid.x);
    else launch_mfma_waves_s<D, PAGED, false>(p, waves, grid, s, fused, (int)grid.x);
}

}  // namespace

int valu_rows_for(int R) {
    if (R <= 2) return 2;
    if (R <= 4) return 4;
    if (R <= 6) return 6;
    if (R <= 8) return 8;
    if (R <= 12) return 12;
    return kValuRows;
}

hipError_t launch_attention_mfma(const AttnParams& p, int waves, hipStream_t s, const StatsParams* fused) {
    const int groups = p.B * p.Hkv * p.nsplit;
    int blocks;
    if (p.rowblocks == 1) blocks = groups;
    else blocks = ((groups + 7) / 8) * 8 * p.rowblocks;
    dim3 grid(blocks);
    if (p.pt.table) {   // paged caches: no fused row statistics
        if (p.D == 128) launch_mfma_waves<128, true>(p, waves, grid, s, nullptr);
        else launch_mfma_waves<64, true>(p, waves, grid, s, nullptr);
    } else {
        if (p.D == 128) launch_mfma_waves<128, false>(p, waves, grid, s, fused);
        else launch_mfma_waves<64, false>(p, waves, grid, s, fused);
    }
    return hipGetLastError();
}

hipError_t launch_attention_valu(const AttnParams& p, bool bf16, hipStream_t s) {
    dim3 grid(p.B * p.Hkv * p.nsplit * p.rowblocks);
    const int maxr = p.Rpad / p.rowblocks;
    if (bf16) return p.D == 128 ? launch_valu_rows<true, 128>(p, maxr, grid, s)
                                : launch_valu_rows<true, 64>(p, maxr, grid, s);
    return p.D == 128 ? launch_valu_rows<false, 128>(p, maxr, grid, s)
                      : launch_valu_rows<false, 64>(p, maxr, grid, s);
}


}  // namespace sv
