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
// popcount(anc*(i)) - 1) in two rounds of dependent loads: every per-node
// input and row statistic first (a parent's statistics then come by lane
// shuffles), then the two logits each test needs; slice 0 writes the
// per-node outputs.  In sampling mode each workgroup then weighs its slice of
// 2048 token ids (residual max(0, p - q) and p alone, both restricted to
// their nuclei), publishes the two slice totals and, for up to 64 slices per
// sequence, its threads' exclusive prefixes; the last workgroup of the
// sequence to arrive finds the slice holding u * W by a prefix over the
// totals in slice order (one wave), and each of its threads takes its own
// bounds within that slice from the kept prefixes and re-weighs its 8 token
// ids: the thread whose bounds hold the target locates the token.  Beyond 64
// slices the last workgroup scans the slice again instead; with a single
// slice (V <= 2048) its one workgroup draws at once.  Every sum is
// taken in a fixed order, so the draw does not depend on the order in which
// workgroups arrive.

#include "combine.h"
#include "row_block.h"

namespace sv {
namespace {

constexpr int ST = kSelectThreads;     // threads per workgroup
constexpr int SW = ST / kWave;         // waves per workgroup
constexpr int EPT = kSelectSlice / ST; // consecutive token ids per thread

struct SelectShared {
    int live, vstar, c0, dstar;
    int is_last, winner, found, sstar, col;
    RowStat sp, sq;                 // statistics of target row v* and of the draft row of its first child
    double wtot[2][SW][2];          // two buffers of per-wave scan totals
    double cum, send, target;       // prefix of the slices before s*, through s*; u * W
};

__device__ __forceinline__ float prob_from(float z, float zmax, uint32_t thr, int cutoff, double Z, int x, float ilog) {
    const float e = rows::unnorm(z, zmax, ilog);
    const rows::Nucleus nu{thr, cutoff};
    return rows::in_nucleus(e, x, nu) ? (float)((double)e / Z) : 0.f;
}

__device__ __forceinline__ RowStat shfl_stat(const RowStat& s, int src) {
    RowStat o;
    o.zmax = __shfl(s.zmax, src, kWave);
    o.argmax = __shfl(s.argmax, src, kWave);
    o.thr = (uint32_t)__shfl((int)s.thr, src, kWave);
    o.cutoff = __shfl(s.cutoff, src, kWave);
    o.Z = __shfl(s.Z, src, kWave);
    return o;
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
    // first round: every load whose address is known up front
    const int par_in = live ? P.parent[base + lane] : -1;
    const int tok = live ? P.tokens[base + lane] : 0;
    RowStat sl{0.f, 0, 0u, 0, 0.0};     // target row of this node
    RowStat sq{0.f, 0, 0u, 0, 1.0};     // draft row this node was drafted from
    float u = 0.f;
    if (live) sl = st[lane];
    if (P.sampling && live && lane >= 1) {
        sq = st[T + lane];
        u = P.u_accept[base + lane];
    }
    const int L = P.kv_len[b];
    bool bad_parent;
    const unsigned long long anc = ancestor_mask_of(par_in, T, &bad_parent);
    const bool bad_token = __any(live && lane >= 1 && (tok < 0 || tok >= V));
    bool bad_kv = (L < 0) || (L > P.Lcap - T);
    // paged caches: table entries of the used slots (L + T <= Lcap here); only the status needs it
    bad_kv = bad_kv || (write && __any(page_entries_bad(P.pt, b, L + T, lane, kWave)));
    int status = (bad_parent ? 1 : 0) | (bad_token ? 2 : 0) | (bad_kv ? 8 : 0);
    if (write && live) P.row_token[base + lane] = sl.argmax;

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
    const int par = par_in;   // valid: parent < node for every node >= 1
    const RowStat spar = shfl_stat(sl, par >= 0 ? par : 0);
    bool a = (lane == 0);
    bool zero_q = false;
    float pv = 0.f, qv = 0.f;
    if (live && lane >= 1) {
        if (P.sampling) {
            // second round: the two logits of the test
            const float zt = P.target[(base + par) * V + tok];
            const float zd = P.draft[(base + lane) * V + tok];
            pv = prob_from(zt, spar.zmax, spar.thr, spar.cutoff, spar.Z, tok, P.ilog);
            qv = prob_from(zd, sq.zmax, sq.thr, sq.cutoff, sq.Z, tok, P.ilog);
            if (qv > 0.f) a = u < pv / qv;
            else zero_q = true;
        } else {
            a = (tok == spar.argmax);
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
    const int c0 = kids ? __builtin_ctzll(kids) : -1;
    const RowStat sp_v = shfl_stat(sl, vstar);
    const RowStat sq_c = shfl_stat(sq, c0 >= 0 ? c0 : 0);
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
        sh.c0 = c0;
        sh.sp = sp_v;
        sh.sq = sq_c;
    }
}

// Inclusive scans of two values over thread order (one barrier): incl/excl
// receive each thread's inclusive/exclusive prefixes and total the block
// totals.  Every thread adds the wave totals before its own wave in wave
// order, so adjacent threads' bounds are bitwise equal (incl_t == excl_t+1)
// and a repeated scan of the same values gives the same bits.  Consecutive
// scans must use different buffers `bufi`.
__device__ __forceinline__ void block_scan2(const double (&v)[2], double (&incl)[2], double (&excl)[2], double (&total)[2],
                                            SelectShared& sh, int bufi) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const double x = wave_scan_d(v[k]);
        if (lane == kWave - 1) sh.wtot[bufi][wave][k] = x;
        double prev = __shfl_up(x, 1, kWave);
        if (lane == 0) prev = 0.0;
        incl[k] = x;
        excl[k] = prev;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        double acc = 0.0, mybase = 0.0;
#pragma unroll
        for (int w = 0; w < SW; ++w) {
            if (w == wave) mybase = acc;
            acc += sh.wtot[bufi][w][k];
        }
        incl[k] += mybase;
        excl[k] += mybase;
        total[k] = acc;
    }
}

// Draw weights of this thread's EPT token ids of slice s: w[0] residual
// max(0, p - q) (normalised; zero unless resid), w[1] p alone (unnormalised).
__device__ __forceinline__ void slice_weights(const SelectParams& P, int b, int s, const SelectShared& sh, float (&wr)[EPT],
                                              float (&wp)[EPT]) {
    const int T = P.T, V = P.V;
    const int x0 = s * kSelectSlice + EPT * threadIdx.x;
    const bool resid = sh.c0 >= 0;
    const RowStat sp = sh.sp;
    const RowStat sq = sh.sq;
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
    const bool pall = rows::keeps_all(np), qall = rows::keeps_all(nq);
    const float ip = (float)(1.0 / sp.Z);
    const float iq = resid ? (float)(1.0 / sq.Z) : 0.f;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int x = x0 + k;
        float pe = rows::unnorm(lp[k], sp.zmax, P.ilog);
        if (x >= V || !(pall || rows::in_nucleus(pe, x, np))) pe = 0.f;
        wp[k] = pe;
        float r = 0.f;
        if (resid) {
            float qe = rows::unnorm(lq[k], sq.zmax, P.ilog);
            if (x >= V || !(qall || rows::in_nucleus(qe, x, nq))) qe = 0.f;
            r = rows::resid_weight(pe, ip, qe, iq);
        }
        wr[k] = r;
    }
}

// The thread whose bounds [lo, hi) hold target writes the token: the first of
// its ids where the running sum from lo passes the target (or its last
// positive weight when rounding leaves none).  Returns whether it won.
__device__ __forceinline__ bool locate_in_thread(const SelectParams& P, size_t out_at, int x0, const float (&w)[EPT],
                                                 double lo, double hi, double target, int last_pos) {
    if (!(lo <= target && target < hi)) return false;
    double run = lo;
    int y = -1;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        run += (double)w[k];
        if (y < 0 && run > target) y = x0 + k;
    }
    P.out_tokens[out_at] = (y >= 0) ? y : last_pos;
    return true;
}

template <bool SAMPLING>
__device__ __forceinline__ void select_block(const SelectParams& P, int s, int b) {
    __shared__ SelectShared sh;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    if (tid < kWave) decide(P, b, s == 0, sh);
    __syncthreads();
    if (!sh.live) return;
    const size_t base = (size_t)b * P.T;
    if (!SAMPLING) {
        if (tid == 0) P.out_tokens[base + sh.dstar] = sh.sp.argmax;
        return;
    }
    const bool keep = P.slice_pre != nullptr && P.S <= kSelectKeepSlices;

    // this slice's totals (and the threads' prefixes) are published; the
    // stores are agent-scope atomics (written through, read past a stale L2
    // copy), all complete (vmcnt 0) before the barrier that precedes the
    // arrival count, so no device-wide fence is needed
    float wr[EPT], wp[EPT];
    slice_weights(P, b, s, sh, wr, wp);
    double mine[2] = {0.0, 0.0};
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        mine[0] += (double)wr[k];
        mine[1] += (double)wp[k];
    }
    double incl[2], excl[2], tot[2];
    block_scan2(mine, incl, excl, tot, sh, 0);
    if (P.S == 1) {
        // one slice holds the whole row: this workgroup draws at once
        const size_t out_at = base + sh.dstar;
        const bool use_resid = (sh.c0 >= 0) && (tot[0] > 0.0);
        const int col = use_resid ? 0 : 1;
        const double target = (double)P.u_final[b] * tot[col];
        float w[EPT];
        int last_pos = -1;
        const int x0 = EPT * tid;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            w[k] = use_resid ? wr[k] : wp[k];
            if (w[k] > 0.f) last_pos = x0 + k;
        }
        if (tid == 0) { sh.winner = 0; sh.found = -1; }
        __syncthreads();
        if (locate_in_thread(P, out_at, x0, w, excl[col], incl[col], target, last_pos)) sh.winner = 1;
        atomicMax(&sh.found, last_pos);
        __syncthreads();
        if (tid == 0 && !sh.winner) P.out_tokens[out_at] = sh.found;   // rounding left no winner
        return;
    }
    if (keep) {
        double* pre = (double*)(P.slice_pre + ((size_t)b * P.S + s) * ST + tid);
        __hip_atomic_store(pre, excl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pre + 1, excl[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
        double* slot = (double*)(P.slice_tot + (size_t)b * P.S + s);
        __hip_atomic_store(slot, tot[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 1, tot[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        sh.is_last = arrive_last(P.arrive + b, P.S);
    }
    __syncthreads();
    if (!sh.is_last) return;
    const size_t out_at = base + sh.dstar;

    if (keep) {
        // wave 0: prefix over the slice totals in slice order and the slice
        // s* holding the target: the first whose running prefix exceeds it
        // (rounding at the very end: the last slice with weight)
        if (tid < kWave) {
            double v0 = 0.0, v1 = 0.0;
            if (lane < P.S) {
                const double* src = (const double*)(P.slice_tot + (size_t)b * P.S + lane);
                v0 = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                v1 = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const double i0 = wave_scan_d(v0), i1 = wave_scan_d(v1);
            const double t0 = __shfl(i0, kWave - 1, kWave), t1 = __shfl(i1, kWave - 1, kWave);
            const bool use_resid = (sh.c0 >= 0) && (t0 > 0.0);
            const double target = (double)P.u_final[b] * (use_resid ? t0 : t1);
            const double inc = use_resid ? i0 : i1, val = use_resid ? v0 : v1;
            double exc = __shfl_up(inc, 1, kWave);   // bitwise the previous slice's inclusive prefix
            if (lane == 0) exc = 0.0;
            const unsigned long long past = __ballot(lane < P.S && inc > target);
            const unsigned long long pos = __ballot(lane < P.S && val > 0.0);
            const int sstar = past ? __builtin_ctzll(past) : (pos ? 63 - __builtin_clzll(pos) : -1);
            const int src = sstar >= 0 ? sstar : 0;
            const double cum = __shfl(exc, src, kWave), send = __shfl(inc, src, kWave);
            if (lane == 0) {
                sh.sstar = sstar;
                sh.col = use_resid ? 0 : 1;
                sh.cum = cum;
                sh.send = send;
                sh.target = target;
                sh.winner = 0;
                sh.found = -1;
            }
        }
        __syncthreads();
        const int sstar = sh.sstar;
        if (sstar < 0) {   // no weight at all: cannot happen, p always has mass
            if (tid == 0) P.out_tokens[out_at] = -1;
            return;
        }
        // this thread's bounds in slice s*: [cum + excl_t, cum + excl_t+1),
        // the last thread's ending at the slice's inclusive prefix
        const int col = sh.col;
        const double cum = sh.cum, target = sh.target;
        const double* pre = (const double*)(P.slice_pre + ((size_t)b * P.S + sstar) * ST);
        const double e_lo = __hip_atomic_load(pre + 2 * tid + col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        double e_hi = 0.0;
        if (tid + 1 < ST) e_hi = __hip_atomic_load(pre + 2 * (tid + 1) + col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        slice_weights(P, b, sstar, sh, wr, wp);
        float w[EPT];
        int last_pos = -1;
        const int x0 = sstar * kSelectSlice + EPT * tid;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            w[k] = col == 0 ? wr[k] : wp[k];
            if (w[k] > 0.f) last_pos = x0 + k;
        }
        const double lo = cum + e_lo;
        const double hi = tid + 1 < ST ? cum + e_hi : sh.send;
        if (locate_in_thread(P, out_at, x0, w, lo, hi, target, last_pos)) sh.winner = 1;
        atomicMax(&sh.found, last_pos);
        __syncthreads();
        if (tid == 0 && !sh.winner) P.out_tokens[out_at] = sh.found;   // rounding left no winner
        return;
    }

    // more slices than kept prefixes: prefix over the slice totals by the
    // whole workgroup, then slice s* weighed and scanned again
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
    if (tid == 0) { sh.winner = INT_MAX; sh.found = -1; }
    double sincl[2], sexcl[2], stot[2];
    block_scan2(st_mine, sincl, sexcl, stot, sh, 1);
    const bool use_resid = (sh.c0 >= 0) && (stot[0] > 0.0);
    const int col = use_resid ? 0 : 1;
    const double target = (double)P.u_final[b] * stot[col];
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
    if (sstar == INT_MAX) sstar = sh.found;
    if (sstar < 0) {
        if (tid == 0) P.out_tokens[out_at] = -1;
        return;
    }
    if (tid == sstar / SPT) {
        double run = sexcl[col];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            if (tid * SPT + k == sstar) sh.cum = run;
            run += st_vals[k][col];
        }
    }
    __syncthreads();
    const double cum = sh.cum;
    if (tid == 0) { sh.winner = 0; sh.found = -1; }
    slice_weights(P, b, sstar, sh, wr, wp);
    double m2[2] = {0.0, 0.0};
    float w[EPT];
    int last_pos = -1;
    const int x0 = sstar * kSelectSlice + EPT * tid;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        w[k] = use_resid ? wr[k] : wp[k];
        m2[0] += (double)wr[k];
        m2[1] += (double)wp[k];
        if (w[k] > 0.f) last_pos = x0 + k;
    }
    block_scan2(m2, incl, excl, tot, sh, 0);
    if (locate_in_thread(P, out_at, x0, w, cum + excl[col], cum + incl[col], target, last_pos)) sh.winner = 1;
    atomicMax(&sh.found, last_pos);
    __syncthreads();
    if (tid == 0 && !sh.winner) P.out_tokens[out_at] = sh.found;
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
