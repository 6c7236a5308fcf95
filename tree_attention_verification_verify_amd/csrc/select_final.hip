// Acceptance decisions, longest accepted root path and the final token.
//
// Node i (>= 1) passes its test when u_i < p_parent(i)(x_i) / q_i(x_i)
// (sampling: featured article on the founding speculative-decoding paper,
// section 2.1; "推测解码技术详解：加速LLM推理的关键" section "数学保证：无损输出质量"
// compares a uniform with the ratio) or when x_i is the target's best token
// after its parent (greedy: "大模型推理加速：推测解码与MTP核心原理与工程实践"
// section 3.1 item 3).  Only a prefix accepted consecutively from the root
// counts and the deepest such node v* is kept (first page, section 2.3;
// "投机解码的五条路线" figure 3); ties between equally deep nodes go to the
// smallest node id.  The emitted tokens are the path's drafts followed by one
// more token drawn at v*: from norm([p_v* - q_c]_+) when v* has children
// (c = its first child, whose draft was rejected) and from p_v* when v* is a
// leaf (bonus token) (featured article, sections 2.1-2.2; greedy: the
// target's best token of row v*).
//
// Work decomposition (ours): a grid of (slice, sequence) workgroups of 256
// threads.  Every workgroup of a sequence first takes the decisions (wave 0,
// lane = node; with the ancestor sets anc*(i) as 64-bit masks, "whole root
// path accepted" is (anc*(i) & ~accepted) == 0 and depth(i) =
// popcount(anc*(i)) - 1); slice 0 writes the per-node outputs.  In sampling
// mode each workgroup then weighs its slice of 2048 token ids (residual
// max(0, p - q) and p alone, both restricted to their nuclei) and publishes
// the two slice totals; the last workgroup of the sequence to arrive finds
// the slice holding u * W by a prefix over the totals in slice order, weighs
// that slice again and locates the token by an inverse CDF in token-id
// order.  Every sum is taken in a fixed order, so the draw does not depend on
// the order in which workgroups arrive.

#include "combine.h"
#include "row_block.h"

namespace sv {
namespace {

constexpr int ST = kSelectThreads;     // threads per workgroup
constexpr int SW = ST / kWave;         // waves per workgroup
constexpr int EPT = kSelectSlice / ST; // consecutive token ids per thread

struct SelectShared {
    int live, vstar, c0, dstar;
    int is_last, winner, found;
    double wtot[SW][2];
    double wpre[SW + 1][2];
    double use_tot;
};

__device__ __forceinline__ float prob_at(const float* row, const RowStat& st, int x, float ilog) {
    const float e = rows::unnorm(row[x], st.zmax, ilog);
    const rows::Nucleus nu{st.thr, st.cutoff};
    return rows::in_nucleus(e, x, nu) ? (float)((double)e / st.Z) : 0.f;
}

// Decisions and path of sequence b (wave 0).  Fills sh; writes the per-node
// outputs only when `write`.
__device__ __forceinline__ void decide(const SelectParams& P, int b, bool write, SelectShared& sh) {
    const int lane = threadIdx.x;
    const int T = P.T, V = P.V;
    const size_t base = (size_t)b * T;
    const int nrows = P.sampling ? 2 * T : T;
    const RowStat* st = P.stats + (size_t)b * nrows;
    const bool live = lane < T;
    bool bad_parent;
    const unsigned long long anc = ancestor_mask(P.parent + base, T, &bad_parent);
    const int tok = live ? P.tokens[base + lane] : 0;
    const bool bad_token = __any(live && lane >= 1 && (tok < 0 || tok >= V));
    const int L = P.kv_len[b];
    bool bad_kv = (L < 0) || (L > P.Lcap - T);
    // paged caches: table entries of the used slots (L + T <= Lcap here); only the status needs it
    bad_kv = bad_kv || (write && __any(page_entries_bad(P.pt, b, L + T, lane, kWave)));
    int status = (bad_parent ? 1 : 0) | (bad_token ? 2 : 0) | (bad_kv ? 8 : 0);
    if (write && live) P.row_token[base + lane] = st[lane].argmax;

    if (bad_parent || bad_token) {
        if (write && live) {
            P.path[base + lane] = -1;
            P.out_tokens[base + lane] = -1;
            P.node_accept[base + lane] = 0;
            P.node_p[base + lane] = 0.f;
            P.node_q[base + lane] = 0.f;
        }
        if (lane == 0) {
            if (write) {
                P.accept_len[b] = 0;
                P.final_node[b] = -1;
                P.final_from_residual[b] = 0;
                P.status[b] = status;
            }
            sh.live = 0;
        }
        return;
    }
    const int par = live ? P.parent[base + lane] : -1;
    bool a = (lane == 0);
    bool zero_q = false;
    float pv = 0.f, qv = 0.f;
    if (live && lane >= 1) {
        if (P.sampling) {
            pv = prob_at(P.target + (base + par) * V, st[par], tok, P.ilog);
            qv = prob_at(P.draft + (base + lane) * V, st[T + lane], tok, P.ilog);
            if (qv > 0.f) a = P.u_accept[base + lane] < pv / qv;
            else zero_q = true;
        } else {
            a = (tok == st[par].argmax);
        }
    }
    if (__any(zero_q)) status |= 4;
    const unsigned long long accepted = __ballot(live && a);
    const bool path_ok = live && ((anc & ~accepted) == 0ull);
    const int depth = live ? (__popcll(anc) - 1) : -1;
    int key = path_ok ? (depth * 64 + (63 - lane)) : -1;   // deepest, then smallest id
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, kWave));
    const int vstar = 63 - (key & 63);
    const int dstar = key >> 6;
    const unsigned long long on_path = __shfl(anc, vstar, kWave);
    const unsigned long long kids = __ballot(live && lane >= 1 && par == vstar);
    if (write && live) {
        P.node_accept[base + lane] = a ? 1 : 0;
        P.node_p[base + lane] = pv;
        P.node_q[base + lane] = qv;
        const bool mine = (on_path >> lane) & 1ull;
        if (lane > dstar) P.path[base + lane] = -1;
        if (mine) P.path[base + depth] = lane;
        if (mine && lane != 0) P.out_tokens[base + depth - 1] = tok;
        if (lane > dstar) P.out_tokens[base + lane] = -1;
    }
    if (lane == 0) {
        if (write) {
            P.accept_len[b] = dstar;
            P.final_node[b] = vstar;
            P.final_from_residual[b] = (P.sampling && kids) ? 1 : 0;
            P.status[b] = status;
        }
        sh.live = 1;
        sh.vstar = vstar;
        sh.dstar = dstar;
        sh.c0 = kids ? __builtin_ctzll(kids) : -1;
    }
}

// Inclusive scans of two values over thread order: incl/excl receive each
// thread's inclusive/exclusive prefixes and total the block totals.
// Wave offsets are accumulated sequentially, so adjacent threads' bounds are
// bitwise equal and a repeated scan of the same values gives the same bits.
__device__ __forceinline__ void block_scan2(const double (&v)[2], double (&incl)[2], double (&excl)[2], double (&total)[2],
                            SelectShared& sh) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        double x = v[k];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double y = __shfl_up(x, o, kWave);
            if (lane >= o) x += y;
        }
        if (lane == kWave - 1) sh.wtot[wave][k] = x;
        double prev = __shfl_up(x, 1, kWave);
        if (lane == 0) prev = 0.0;
        incl[k] = x;
        excl[k] = prev;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
        const int k = threadIdx.x;
        double acc = 0.0;
        for (int w = 0; w < SW; ++w) {
            sh.wpre[w][k] = acc;
            acc += sh.wtot[w][k];
        }
        sh.wpre[SW][k] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        incl[k] += sh.wpre[wave][k];
        excl[k] += sh.wpre[wave][k];
        total[k] = sh.wpre[SW][k];
    }
    __syncthreads();
}

// Draw weights of this thread's EPT token ids of slice s: w[0] residual
// max(0, p - q) (normalised; zero unless resid), w[1] p alone (unnormalised).
__device__ __forceinline__ void slice_weights(const SelectParams& P, int b, int s, const SelectShared& sh, float (&wr)[EPT],
                              float (&wp)[EPT]) {
    const int T = P.T, V = P.V;
    const int x0 = s * kSelectSlice + EPT * threadIdx.x;
    const bool resid = sh.c0 >= 0;
    const RowStat sp = P.stats[(size_t)b * 2 * T + sh.vstar];
    const RowStat sq = resid ? P.stats[(size_t)b * 2 * T + T + sh.c0] : sp;
    const float* zp = P.target + ((size_t)b * T + sh.vstar) * V;
    const float* zq = P.draft + ((size_t)b * T + (resid ? sh.c0 : 0)) * V;
    float lp[EPT], lq[EPT];
    const bool vec = (x0 + EPT <= V) && ((((uintptr_t)(zp + x0)) & 15) == 0) && ((((uintptr_t)(zq + x0)) & 15) == 0);
    if (vec) {
#pragma unroll
        for (int k = 0; k < EPT; k += 4) {
            const float4 a = *(const float4*)(zp + x0 + k);
            lp[k] = a.x; lp[k + 1] = a.y; lp[k + 2] = a.z; lp[k + 3] = a.w;
            if (resid) {
                const float4 c = *(const float4*)(zq + x0 + k);
                lq[k] = c.x; lq[k + 1] = c.y; lq[k + 2] = c.z; lq[k + 3] = c.w;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            lp[k] = (x0 + k < V) ? zp[x0 + k] : -INFINITY;
            if (resid) lq[k] = (x0 + k < V) ? zq[x0 + k] : -INFINITY;
        }
    }
    const rows::Nucleus np{sp.thr, sp.cutoff}, nq{sq.thr, sq.cutoff};
    const float ip = (float)(1.0 / sp.Z);
    const float iq = resid ? (float)(1.0 / sq.Z) : 0.f;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int x = x0 + k;
        float pe = rows::unnorm(lp[k], sp.zmax, P.ilog);
        if (x >= V || !rows::in_nucleus(pe, x, np)) pe = 0.f;
        wp[k] = pe;
        float r = 0.f;
        if (resid) {
            float qe = rows::unnorm(lq[k], sq.zmax, P.ilog);
            if (x >= V || !rows::in_nucleus(qe, x, nq)) qe = 0.f;
            r = rows::resid_weight(pe, ip, qe, iq);
        }
        wr[k] = r;
    }
}

template <bool SAMPLING>
__device__ __forceinline__ void select_block(const SelectParams& P, int s, int b) {
    __shared__ SelectShared sh;
    const int tid = threadIdx.x;
    if (tid < kWave) decide(P, b, s == 0, sh);
    __syncthreads();
    if (!sh.live) return;
    const size_t base = (size_t)b * P.T;
    if (!SAMPLING) {
        const int nrows = P.T;
        if (tid == 0) P.out_tokens[base + sh.dstar] = P.stats[(size_t)b * nrows + sh.vstar].argmax;
        return;
    }

    // this slice's totals
    float wr[EPT], wp[EPT];
    slice_weights(P, b, s, sh, wr, wp);
    double mine[2] = {0.0, 0.0};
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        mine[0] += (double)wr[k];
        mine[1] += (double)wp[k];
    }
    double incl[2], excl[2], tot[2];
    block_scan2(mine, incl, excl, tot, sh);
    // Publication without a device-wide fence (which would write back the whole
    // L2 of this XCD): the totals are stored and later read as agent-scope
    // atomics (write-through, and reads that bypass a stale L2 copy), and the
    // counter is bumped only after both stores have completed (vmcnt 0).
    if (tid == 0) {
        double* slot = (double*)(P.slice_tot + (size_t)b * P.S + s);
        __hip_atomic_store(slot, tot[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 1, tot[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        const int prev = __hip_atomic_fetch_add(P.arrive + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.is_last = (prev == P.S - 1);
    }
    __syncthreads();
    if (!sh.is_last) return;

    // last arriver: prefix over the slice totals in slice order
    if (tid == 0) __hip_atomic_store(P.arrive + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // next launch
    constexpr int SPT = (kSelectMaxSlices + ST - 1) / ST;
    double st_mine[2] = {0.0, 0.0};
    double st_vals[SPT][2];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int j = tid * SPT + k;
        double2 v = make_double2(0.0, 0.0);
        if (j < P.S) {
            const double* src = (const double*)(P.slice_tot + (size_t)b * P.S + j);
            v.x = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v.y = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        st_vals[k][0] = v.x;
        st_vals[k][1] = v.y;
        st_mine[0] += v.x;
        st_mine[1] += v.y;
    }
    double sincl[2], sexcl[2], stot[2];
    block_scan2(st_mine, sincl, sexcl, stot, sh);
    const bool use_resid = (sh.c0 >= 0) && (stot[0] > 0.0);
    const int col = use_resid ? 0 : 1;
    const double W = stot[col];
    const double target = (double)P.u_final[b] * W;
    // s*: the first slice whose running prefix (in slice order) exceeds the
    // target; cum: the prefix before it
    if (tid == 0) { sh.winner = INT_MAX; sh.found = -1; }
    __syncthreads();
    {
        double run = sexcl[col];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int j = tid * SPT + k;
            run += st_vals[k][col];
            if (j < P.S && run > target) atomicMin(&sh.winner, j);
            if (j < P.S && st_vals[k][col] > 0.0) atomicMax(&sh.found, j);
        }
    }
    __syncthreads();
    int sstar = sh.winner;
    if (sstar == INT_MAX) sstar = sh.found;     // rounding at the very end: last slice with weight
    if (sstar < 0) {                            // no weight at all: cannot happen, p always has mass
        if (tid == 0) P.out_tokens[base + sh.dstar] = -1;
        return;
    }
    if (tid == sstar / SPT) {
        double run = sexcl[col];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            if (tid * SPT + k == sstar) sh.use_tot = run;
            run += st_vals[k][col];
        }
    }
    __syncthreads();
    const double cum = sh.use_tot;

    // weigh slice s* again and locate the token
    slice_weights(P, b, sstar, sh, wr, wp);
    double m2[2] = {0.0, 0.0};
    float w[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        w[k] = use_resid ? wr[k] : wp[k];
        m2[0] += (double)wr[k];
        m2[1] += (double)wp[k];
    }
    block_scan2(m2, incl, excl, tot, sh);
    if (tid == 0) { sh.winner = INT_MAX; sh.found = -1; }
    __syncthreads();
    const double lo = cum + excl[col], hi = cum + incl[col];
    if (lo <= target && target < hi) atomicMin(&sh.winner, tid);
    int last_pos = -1;
    const int x0 = sstar * kSelectSlice + EPT * tid;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
        if (w[k] > 0.f) last_pos = x0 + k;
    atomicMax(&sh.found, last_pos);
    __syncthreads();
    if (tid == sh.winner) {
        double run = lo;
        int y = -1;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            run += (double)w[k];
            if (y < 0 && run > target) y = x0 + k;
        }
        P.out_tokens[base + sh.dstar] = (y >= 0) ? y : last_pos;
    } else if (sh.winner == INT_MAX && tid == 0) {
        P.out_tokens[base + sh.dstar] = sh.found;   // rounding left no winner: last positive weight
    }
}

// The launch that ends a step: the selection workgroups first (their
// dependent loads start at once), then the merge of the attention splits,
// which only streams memory and fills the GPU meanwhile.  Greedy mode uses one
// selection workgroup per sequence, sampling mode one per (sequence, slice).
template <bool SAMPLING, bool BF16, int D>
__global__ __launch_bounds__(ST) void finish_kernel(SelectParams P, AttnParams A, int nsel) {
    const int blk = blockIdx.x;
    if (blk < nsel) {
        if (SAMPLING) select_block<true>(P, blk % P.S, blk / P.S);
        else select_block<false>(P, 0, blk);
    } else {
        combine_block<BF16, D>(A, blk - nsel, threadIdx.x);
    }
}

}  // namespace

hipError_t launch_finish(const SelectParams& sp, const AttnParams& ap, bool select, bool merge, bool bf16,
                         hipStream_t s) {
    const int nsel = !select ? 0 : (sp.sampling ? sp.S * sp.B : sp.B);
    int nmerge = 0;
    if (merge) {
        const long rows = (long)ap.B * ap.Hkv * ap.R;
        const long rpb = ap.D == 128 ? combine_rows_per_block<128>() : combine_rows_per_block<64>();
        nmerge = (int)((rows + rpb - 1) / rpb);
    }
    if (nsel + nmerge == 0) return hipSuccess;
    const dim3 grid(nsel + nmerge), block(ST);
#define SV_FINISH(S_, B_, D_) hipLaunchKernelGGL((finish_kernel<S_, B_, D_>), grid, block, 0, s, sp, ap, nsel)
    if (sp.sampling) {
        if (bf16) { if (ap.D == 128) SV_FINISH(true, true, 128); else SV_FINISH(true, true, 64); }
        else { if (ap.D == 128) SV_FINISH(true, false, 128); else SV_FINISH(true, false, 64); }
    } else {
        if (bf16) { if (ap.D == 128) SV_FINISH(false, true, 128); else SV_FINISH(false, true, 64); }
        else { if (ap.D == 128) SV_FINISH(false, false, 128); else SV_FINISH(false, false, 64); }
    }
#undef SV_FINISH
    return hipGetLastError();
}

}  // namespace sv
