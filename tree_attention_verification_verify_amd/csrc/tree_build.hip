// Candidate-tree construction for Medusa verification.
//
// The candidates of depth d are the top-k tokens of one logits row per
// sequence (d = 1: the target's own next-token row; d >= 2: Medusa head
// d-1), and the tree is the Cartesian product of those lists, pruned to T
// nodes ("推测解码技术详解：加速LLM推理的关键", section "Tree Attention验证": two
// heads with top-2 each give the 7-node product tree; "Medusa推测解码：为LLM推理
// 加速2-3倍的工程实践", sections 2.2 and 4.2: top-k per head, k = 10).  A
// template (parent[], rank[]) fixes the tree's shape; node i >= 1 takes entry
// rank[i] of its depth's top-k list, so the kernel only has to find each
// row's best few tokens and scatter them.
//
// Rows of at least 8192 ids are split over up to 8 workgroups (slices of
// >= 4096 ids) that each find their slice's k best the way described below;
// the last slice of a row to finish (a per-row counter) ranks the slices' k
// best together.  One 1024-thread workgroup per (sequence, depth, slice),
// two passes over its ids.
// Pass 1: the c = ceil(k/16) best entries of each wave's share; the k-th
// largest of those 16c distinct entries is a lower bound on the row's k-th
// largest.  Pass 2 (from L2): each thread keeps the K best entries at or
// above that bound, sorted, in registers, and appends them to a short list
// in LDS; the rank of each listed key is the number of larger listed keys
// (keys are unique), which places the k best.  If the list overflows (a row
// whose best entries crowd into one wave's share), the exact fallback pulls
// each wave's k best by k rounds of a wave-wide maximum and merges the wave
// lists the same way.  A key is the order-preserving integer image of the
// logit (NaN lowest, -0 == +0) in the high word and the complement of the
// token id in the low word, so keys are unique and the larger key is the
// larger logit, then the smaller id.

#include "device_common.h"
#include "kernels.h"

namespace sv {
namespace {

constexpr int TB = 1024;    // threads per workgroup
constexpr int NW = TB / 64;  // waves
constexpr int CAP = 512;     // keys the LDS list holds before the exact fallback

__device__ __forceinline__ unsigned long long order_key(float v, int id) {
    uint32_t u = __float_as_uint(v);
    if (v == 0.f) u = 0u;                              // -0 ranks with +0
    const uint32_t o = (v != v) ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
    return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long w = __shfl_xor(v, o, kWave);
        v = w > v ? w : v;
    }
    return v;
}

// The block's k best keys (k <= K) from every thread's sorted list `lst`
// (consumed): written to out[0..k-1], best first, visible after the call.
template <int K>
__device__ __forceinline__ void block_topk(unsigned long long (&lst)[K], int k, unsigned long long (*wave_top)[K],
                           unsigned long long* out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = 0; r < k; ++r) {
        const unsigned long long m = wave_max_u64(lst[0]);
        if (m != 0ull && lst[0] == m) {
#pragma unroll
            for (int q = 0; q + 1 < K; ++q) lst[q] = lst[q + 1];
            lst[K - 1] = 0ull;
        }
        if (lane == 0) wave_top[wave][r] = m;
    }
    __syncthreads();
    if (wave == 0) {
        constexpr int PER = (NW * K + kWave - 1) / kWave;
        unsigned long long c[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int idx = q * kWave + lane;
            const int w = idx / K, r = idx - w * K;
            c[q] = (w < NW && r < k) ? wave_top[w][r] : 0ull;
        }
        for (int r = 0; r < k; ++r) {
            unsigned long long best = 0ull;
#pragma unroll
            for (int q = 0; q < PER; ++q) best = c[q] > best ? c[q] : best;
            const unsigned long long m = wave_max_u64(best);
#pragma unroll
            for (int q = 0; q < PER; ++q)
                if (m != 0ull && c[q] == m) c[q] = 0ull;
            if (lane == 0) out[r] = m;
        }
    }
    __syncthreads();
}

// Applies f(key) to every entry of the row in this thread's share: float4
// loads when the row is 16-byte aligned, else scalar loads.
template <typename F>
__device__ __forceinline__ void for_row(const float* row, int V, int id0, F&& f) {
    const int tid = threadIdx.x;
    if ((((uintptr_t)row) & 15u) == 0) {
        const int V4 = V >> 2;
        const floatx4_t* row4 = (const floatx4_t*)row;
        constexpr int U = 4;
        int j = tid;
        for (; j + (U - 1) * TB < V4; j += U * TB) {
            floatx4_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = row4[j + u * TB];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) f(order_key(v[u][e], id0 + 4 * (j + u * TB) + e));
        }
        for (; j < V4; j += TB) {
            const floatx4_t v = row4[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) f(order_key(v[e], id0 + 4 * j + e));
        }
        for (int x = 4 * V4 + tid; x < V; x += TB) f(order_key(row[x], id0 + x));
    } else {
        for (int x = tid; x < V; x += TB) f(order_key(row[x], id0 + x));
    }
}

// Places the keys list[0..n-1] (unique) by rank: out[r] = the key with r larger ones, r < k.
__device__ __forceinline__ void rank_place(const unsigned long long* list, int n, int k, unsigned long long* out) {
    for (int i = threadIdx.x; i < n; i += TB) {
        const unsigned long long c = list[i];
        int r = 0;
        for (int j = 0; j < n; ++j) r += list[j] > c ? 1 : 0;
        if (r < k) out[r] = c;
    }
}

template <int K>
__global__ __launch_bounds__(TB) void tree_build_kernel(TreeParams P) {
    __shared__ unsigned long long wave_top[NW][K];
    __shared__ unsigned long long best[K];
    __shared__ unsigned long long list[CAP];
    __shared__ int nlist, is_last;
    const int tid = threadIdx.x;
    const int levels = P.levels;
    const int G = P.slices;
    const int rowid = blockIdx.x / G, sl = blockIdx.x - rowid * G;   // (sequence, depth) row and its slice
    const int b = levels ? rowid / levels : rowid;
    const int d = levels ? rowid - b * levels + 1 : 0;
    const size_t base = (size_t)b * P.T;

    if (d <= 1 && sl == 0 && tid < P.T) {   // the template and the root token, once per sequence
        P.parent[base + tid] = P.tpar[tid];
        if (tid == 0) P.tokens[base] = P.root_token[b];
    }
    if (d == 0) return;
    const int k = P.kd[d];
    // this workgroup's slice of the row: ids [lo, lo + len), lo a multiple of 4
    const int span = ((P.V + G - 1) / G + 3) & ~3;
    const int lo = min(sl * span, P.V), len = min(P.V - lo, span);
    const float* row = P.logits + ((size_t)b * P.rows + (d - 1)) * P.V + lo;

    const int lane = tid & 63, wave = tid >> 6;
    unsigned long long lst[K];
    // pass 1: the c best entries of each wave's share (c <= 2 per-thread
    // maxima, pulled by c wave-wide maxima); the k-th largest of them bounds the k-th best
    const int c = (k + NW - 1) / NW;
    unsigned long long m0 = 0ull, m1 = 0ull;   // the thread's two best
    for_row(row, len, lo, [&](unsigned long long key) {
        const unsigned long long mn = key > m0 ? m0 : key;
        m0 = key > m0 ? key : m0;
        m1 = mn > m1 ? mn : m1;
    });
    if (tid == 0) {
        nlist = 0;
        best[0] = 0ull;   // bound 0 (every entry) when fewer than k entries were listed
    }
    for (int r = 0; r < c; ++r) {
        const unsigned long long m = wave_max_u64(m0);
        if (m != 0ull && m0 == m) {
            m0 = m1;
            m1 = 0ull;
        }
        if (lane == 0) list[wave * 2 + r] = m;
    }
    __syncthreads();
    if (tid < NW * c) {   // the k-th largest of the NW * c listed keys
        const unsigned long long x = list[(tid / c) * 2 + tid % c];
        int r = 0;
        for (int j = 0; j < NW * c; ++j) r += list[(j / c) * 2 + j % c] > x ? 1 : 0;
        if (r == k - 1) best[0] = x;
    }
    __syncthreads();
    const unsigned long long bound = best[0];
    __syncthreads();

    // pass 2: the K best entries >= bound of this thread's share
#pragma unroll
    for (int q = 0; q < K; ++q) lst[q] = 0ull;
    for_row(row, len, lo, [&](unsigned long long key) {
        if (key >= bound && key > lst[K - 1]) {
#pragma unroll
            for (int q = 0; q < K; ++q) {
                const unsigned long long hi = key > lst[q] ? key : lst[q];
                key = key > lst[q] ? lst[q] : key;
                lst[q] = hi;
            }
        }
    });
    int mine = 0;
#pragma unroll
    for (int q = 0; q < K; ++q) mine += lst[q] != 0ull ? 1 : 0;
    const int at = mine ? atomicAdd(&nlist, mine) : 0;
#pragma unroll
    for (int q = 0; q < K; ++q)
        if (q < mine && at + q < CAP) list[at + q] = lst[q];
    __syncthreads();
    const int n = nlist;
    if (n <= CAP) {
        rank_place(list, n, k, best);
        __syncthreads();
    } else {
        block_topk<K>(lst, k, wave_top, best);
    }
    if (G > 1) {
        // each slice publishes its k best (agent-scope stores, landed before the
        // count); the last slice of the row to finish ranks the G * k keys
        // (unique: distinct ids; every slice has more than k entries)
        unsigned long long* cand = P.cand + (size_t)rowid * G * 32;
        if (tid < k) __hip_atomic_store(cand + sl * 32 + tid, best[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            is_last = arrive_last(P.arrive + rowid, G);
        }
        __syncthreads();
        if (!is_last) return;
        for (int i = tid; i < G * k; i += TB)
            list[i] = __hip_atomic_load(cand + (i / k) * 32 + i % k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        rank_place(list, G * k, k, best);
        __syncthreads();
    }
    if (tid >= 1 && tid < P.T && P.tdep[tid] == d)
        P.tokens[base + tid] = (int)(0xFFFFFFFFu - (uint32_t)(best[P.trank[tid]] & 0xFFFFFFFFull));
}

}  // namespace

hipError_t launch_tree_build(const TreeParams& p, int kmax, hipStream_t s) {
    dim3 grid(p.B * (p.levels ? p.levels : 1) * p.slices);
    if (kmax <= 8) hipLaunchKernelGGL(tree_build_kernel<8>, grid, dim3(TB), 0, s, p);
    else if (kmax <= 16) hipLaunchKernelGGL(tree_build_kernel<16>, grid, dim3(TB), 0, s, p);
    else hipLaunchKernelGGL(tree_build_kernel<32>, grid, dim3(TB), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
