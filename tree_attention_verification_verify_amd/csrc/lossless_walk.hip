// Lossless multi-candidate tree sampling: the sibling walk.
//
// Tree acceptance with one independent test per node keeps the target's
// output law only when every node has at most one drafted child.  The walk
// below keeps it for any tree ("投机解码的五条路线", section 4, separates
// lossless verification from typical acceptance; the rejection step and its
// residual are those of the featured article on the founding
// speculative-decoding paper, section 2.1, applied once per sibling):
//
//   start at the root with r = p_root;
//   at node v, try its children c in increasing node id:
//       accept c when u_c < r(x_c) / q_c(x_c): emit x_c, move to c, r = p_c;
//       otherwise r <- norm([r - q_c]_+) (kept if that is all zero) and try
//       the next child;
//   when v has no untried child, draw the final token from r with u_final
//   (inverse CDF in token-id order).
//
// A chain gives exactly the independent rule: the first rejection ends the
// walk, and its residual is computed with the same arithmetic.
//
// Three kernels take the same walk (the host picks one per launch):
//  * more than 4096 ids: the ids of each sequence split over workgroups of
//    4096 that meet at a barrier after every pass (lossless_walk_coop_kernel),
//    while the grid fits twice per CU (at 32000 ids, 8 workgroups per
//    sequence walk about 10% faster than one);
//  * otherwise, up to 32768 ids: one 1024-thread workgroup per sequence with
//    r in registers (lossless_walk_resident_kernel);
//  * otherwise one 1024-thread workgroup per sequence that streams the rows
//    chunk by chunk (lossless_walk_kernel below): wave 0 checks the tree and
//    sets the status bits; each test is a gather by thread 0; each rejection
//    is one chunked pass over the vocabulary that writes the unnormalised
//    residual to one of two workspace rows of the sequence (so a residual
//    that vanishes leaves the previous one intact) and sums it in fp64 in a
//    fixed order.

#include "row_block.h"

namespace sv {
namespace {

using namespace rows;

struct WalkShared {
    unsigned long long kids_of[64];   // children of every node, as a node bitmask
    unsigned long long kids;          // untried children of v
    double W;                         // total of the workspace residual (when r_ws)
    int v, depth, r_ws, cur, accept, live, c;
};

__device__ __forceinline__ float walk_prob(const float* row, const RowStat& st, int x, float ilog) {
    const float e = unnorm(row[x], st.zmax, ilog);
    const Nucleus nu{st.thr, st.cutoff};
    return in_nucleus(e, x, nu) ? (float)((double)e / st.Z) : 0.f;
}

// Unnormalised weights of the current r over one chunk: p_v in its nucleus
// (from the logits), or the workspace residual.
__device__ __forceinline__ void r_weights(const SelectParams& P, int b, const WalkShared& ws, int cb, float4 (&w)[VPT4]) {
    const int T = P.T, V = P.V;
    if (ws.r_ws) {
        const float* R = P.resid_ws + ((size_t)b * 2 + ws.cur) * V;
        load_chunk(R, V, cb, (((uintptr_t)R) & 15) == 0, w);   // past V: -inf, a weight of 0 here
#pragma unroll
        for (int j = 0; j < VPT4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) f4set(w[j], e, fmaxf(f4get(w[j], e), 0.f));
    } else {
        const float* zp = P.target + ((size_t)b * T + ws.v) * V;
        load_chunk(zp, V, cb, (((uintptr_t)zp) & 15) == 0, w);
        const RowStat sp = P.stats[(size_t)b * 2 * T + ws.v];
        const Nucleus np{sp.thr, sp.cutoff};
        // past V the logits read -inf: weight 0 (0 also for a row without a finite logit)
        const bool all = keeps_all(np);
#pragma unroll
        for (int j = 0; j < VPT4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pe = unnorm(f4get(w[j], e), sp.zmax, P.ilog);
                f4set(w[j], e, (pe > 0.f && (all || in_nucleus(pe, elem_index(cb, j, e), np))) ? pe : 0.f);
            }
    }
}

__device__ __forceinline__ void store_chunk(float* row, int V, int cb, const float4 (&w)[VPT4]) {
    const bool aligned = (((uintptr_t)row) & 15) == 0;
#pragma unroll
    for (int j = 0; j < VPT4; ++j) {
        const int idx = elem_index(cb, j, 0);
        if (aligned && idx + 3 < V) {
            *(float4*)(row + idx) = w[j];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (idx + e < V) row[idx + e] = f4get(w[j], e);
        }
    }
}

// r <- [r - q_c]_+ over the whole row into the other workspace row; returns its fp64 total.
__device__ __forceinline__ double residual_pass(const SelectParams& P, int b, int c, const WalkShared& ws, Smem& sm) {
    const int T = P.T, V = P.V;
    const RowStat sq = P.stats[(size_t)b * 2 * T + T + c];
    const Nucleus nq{sq.thr, sq.cutoff};
    const bool all = keeps_all(nq);
    const float iq = (float)(1.0 / sq.Z);
    const float ir = ws.r_ws ? (float)(1.0 / ws.W) : (float)(1.0 / P.stats[(size_t)b * 2 * T + ws.v].Z);
    const float* zq = P.draft + ((size_t)b * T + c) * V;
    const bool aq = (((uintptr_t)zq) & 15) == 0;
    float* out = P.resid_ws + ((size_t)b * 2 + (ws.cur ^ 1)) * V;
    double W = 0.0;
    for (int cb = 0; cb < V; cb += CHUNK) {
        float4 r[VPT4], q[VPT4];
        r_weights(P, b, ws, cb, r);
        load_chunk(zq, V, cb, aq, q);
        // past V both weights are 0, so is the residual
#pragma unroll
        for (int j = 0; j < VPT4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float qe = unnorm(f4get(q[j], e), sq.zmax, P.ilog);
                if (!(all || in_nucleus(qe, elem_index(cb, j, e), nq))) qe = 0.f;
                f4set(q[j], e, resid_weight(f4get(r[j], e), ir, qe, iq));
            }
        store_chunk(out, V, cb, q);
        W += slot_totals(q, sm);
    }
    return W;
}

// Inverse-CDF draw from r: y = min{k : u * W < C_k} in token-id order.
__device__ __forceinline__ int draw_from_r(const SelectParams& P, int b, const WalkShared& ws, double u, Smem& sm) {
    const int V = P.V;
    float4 w[VPT4];
    if (V <= CHUNK) {
        r_weights(P, b, ws, 0, w);
        const double W = slot_totals(w, sm);
        int y = locate_in_chunk(w, 0, V, 0.0, u * W, sm);
        if (y < 0) {
            int last = -1;
#pragma unroll
            for (int j = 0; j < VPT4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (f4get(w[j], e) > 0.f) last = max(last, elem_index(0, j, e));
            y = block_max_int(last, sm);
        }
        return y;
    }
    // streamed: chunk totals, then the chunk holding the draw again
    double W = 0.0;
    int nc = 0;
    for (int cb = 0; cb < V; cb += CHUNK, ++nc) {
        r_weights(P, b, ws, cb, w);
        const double S = slot_totals(w, sm);
        if (threadIdx.x == 0) sm.chunk_sum[nc] = S;
        W += S;
    }
    __syncthreads();
    const double target = u * W;
    double cum = 0.0;
    int cstar = -1;
    for (int k = 0; k < nc; ++k) {
        if (cum + sm.chunk_sum[k] > target) { cstar = k; break; }
        cum += sm.chunk_sum[k];
    }
    if (cstar < 0) {   // rounding: the last chunk with weight
        for (int k = nc - 1; k >= 0; --k)
            if (sm.chunk_sum[k] > 0.0) { cstar = k; break; }
        if (cstar < 0) return -1;
        cum = 0.0;
        for (int k = 0; k < cstar; ++k) cum += sm.chunk_sum[k];
    }
    const int cb = cstar * CHUNK;
    r_weights(P, b, ws, cb, w);
    (void)slot_totals(w, sm);
    int y = locate_in_chunk(w, cb, V, cum, target, sm);
    if (y < 0) {
        int last = -1;
#pragma unroll
        for (int j = 0; j < VPT4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (f4get(w[j], e) > 0.f) last = max(last, elem_index(cb, j, e));
        y = block_max_int(last, sm);
    }
    return y;
}

__global__ __launch_bounds__(NT) void lossless_walk_kernel(SelectParams P) {
    __shared__ Smem sm;
    __shared__ WalkShared ws;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int T = P.T, V = P.V;
    const size_t base = (size_t)b * T;
    const RowStat* st = P.stats + (size_t)b * 2 * T;

    if (tid < kWave) {
        const int lane = tid;
        const bool live = lane < T;
        bool bad_parent;
        (void)ancestor_mask(P.parent + base, T, &bad_parent);
        const int tok = live ? P.tokens[base + lane] : 0;
        const bool bad_token = __any(live && lane >= 1 && (tok < 0 || tok >= V));
        const int L = P.kv_len[b];
        bool bad_kv = (L < 0) || (L > P.Lcap - T);
        bad_kv = bad_kv || __any(page_entries_bad(P.pt, b, L + T, lane, kWave));   // paged: L + T <= Lcap here
        int status = (bad_parent ? 1 : 0) | (bad_token ? 2 : 0) | (bad_kv ? 8 : 0);
        if (live) P.row_token[base + lane] = st[lane].argmax;
        if (live) {
            P.node_accept[base + lane] = (lane == 0) ? 1 : 0;
            P.node_p[base + lane] = 0.f;
            P.node_q[base + lane] = 0.f;
            P.path[base + lane] = (lane == 0 && !bad_parent && !bad_token) ? 0 : -1;
            P.out_tokens[base + lane] = -1;
        }
        if (bad_parent || bad_token) {
            if (lane == 0) {
                P.accept_len[b] = 0;
                P.final_node[b] = -1;
                P.final_from_residual[b] = 0;
                P.status[b] = status;
                ws.live = 0;
            }
        } else {
            const int par = live ? P.parent[base + lane] : -1;
            // status bit 4: some supplied draft gives its own token probability 0
            const bool zero_q = live && lane >= 1 && !(walk_prob(P.draft + (base + lane) * V, st[T + lane], tok,
                                                                 P.ilog) > 0.f);
            if (__any(zero_q)) status |= 4;
            for (int n = 0; n < T; ++n) {
                const unsigned long long k = __ballot(live && lane >= 1 && par == n);
                if (lane == 0) ws.kids_of[n] = k;
            }
            if (lane == 0) {
                P.status[b] = status;
                ws.live = 1;
                ws.v = 0;
                ws.depth = 0;
                ws.r_ws = 0;
                ws.cur = 0;
                ws.W = 0.0;
                ws.kids = ws.kids_of[0];
            }
        }
    }
    __syncthreads();
    if (!ws.live) return;

    // every round tests one child (accepting it or not) or ends the walk: at most 2T rounds
    for (int round = 0; round < 2 * 64 + 1; ++round) {
        const unsigned long long kids = ws.kids;
        __syncthreads();   // every wave has read the state before thread 0 changes it
        if (kids == 0ull) break;
        if (tid == 0) {
            const int c = __builtin_ctzll(kids);
            const int x = P.tokens[base + c];
            const float rx = ws.r_ws ? (float)((double)P.resid_ws[((size_t)b * 2 + ws.cur) * V + x] / ws.W)
                                     : walk_prob(P.target + (base + ws.v) * V, st[ws.v], x, P.ilog);
            const float qx = walk_prob(P.draft + (base + c) * V, st[T + c], x, P.ilog);
            P.node_p[base + c] = rx;
            P.node_q[base + c] = qx;
            const bool acc = (qx > 0.f) && (P.u_accept[base + c] < rx / qx);
            ws.accept = acc ? 1 : 0;
            ws.c = c;
            if (acc) {
                P.node_accept[base + c] = 1;
                P.out_tokens[base + ws.depth] = x;
                ws.depth += 1;
                P.path[base + ws.depth] = c;
                ws.v = c;
                ws.r_ws = 0;
                ws.kids = ws.kids_of[c];
            } else {
                ws.kids &= ~(1ull << c);
            }
        }
        __syncthreads();
        if (ws.accept) continue;   // the next round's barrier follows this read
        const double W = residual_pass(P, b, ws.c, ws, sm);
        __syncthreads();
        if (tid == 0 && W > 0.0) {   // a vanishing residual keeps r
            ws.r_ws = 1;
            ws.cur ^= 1;
            ws.W = W;
        }
        __syncthreads();
    }

    const int y = draw_from_r(P, b, ws, (double)P.u_final[b], sm);
    if (tid == 0) {
        P.out_tokens[base + ws.depth] = y;
        P.accept_len[b] = ws.depth;
        P.final_node[b] = ws.v;
        P.final_from_residual[b] = ws.kids_of[ws.v] != 0ull ? 1 : 0;
    }
}

// ---------------------------------------------------------------------------
// Vocabularies of one chunk (V <= 32768): r stays in the workgroup's
// registers.  Wave 0 first computes every first test of the walk (p of the
// parent and q of the child at the child's token, as the independent rule
// does), so a test needs no global load: p_parent(x_c) while r is still p_v,
// else r(x_c) / W, which the thread holding x_c records during the residual
// pass that produced r.  A rejection is then one read of q_c's row (and of
// p_v's row at the first rejection under v) plus one fixed-order sum.

struct WalkRes {
    unsigned long long kids_of[64];
    float pv0[64];              // p_parent(c)(x_c)
    float qv[64];               // q_c(x_c)
    float u[64];                // u_accept
    int tok[64];
    float qzmax[64];            // statistics of the draft row of each node
    uint32_t qthr[64];
    int qcut[64];
    double qZ[64];
    float rx[2][2];             // per pass (alternating): r_new and r_old at the next child's token
    double wsum[2][NW];         // per pass (alternating): wave totals of the residual
    int live;
};

// Total of w over the workgroup in a fixed order (one barrier): per thread in
// slot order, per wave by the butterfly, then the wave totals in wave order.
// Consecutive calls must alternate `buf`.
__device__ __forceinline__ double block_total(const float4 (&w)[VPT4], double (&wsum)[2][NW], int buf) {
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < VPT4; ++j) t += ((double)w[j].x + (double)w[j].y) + ((double)w[j].z + (double)w[j].w);
    t = wave_sum_d(t);
    if (lane_() == 0) wsum[buf][wave_()] = t;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int k = 0; k < NW; ++k) tot += wsum[buf][k];
    return tot;
}

__device__ __forceinline__ RowStat shfl_row_stat(const RowStat& s, int src) {
    RowStat o;
    o.zmax = __shfl(s.zmax, src, kWave);
    o.argmax = __shfl(s.argmax, src, kWave);
    o.thr = (uint32_t)__shfl((int)s.thr, src, kWave);
    o.cutoff = __shfl(s.cutoff, src, kWave);
    o.Z = __shfl(s.Z, src, kWave);
    return o;
}

// w at slot (j, e) of this thread; j and e are the same in every lane
__device__ __forceinline__ float pick(const float4 (&w)[VPT4], int j, int e) {
    float r = 0.f;
#pragma unroll
    for (int jj = 0; jj < VPT4; ++jj)
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) r = (jj == j && ee == e) ? f4get(w[jj], ee) : r;
    return r;
}

__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

// p_v's weights (unnormalised, in v's nucleus) over the single chunk; past V
// the logits read as -inf and weigh 0 (a row without a finite logit weighs 0
// everywhere)
__device__ __forceinline__ void p_weights(const SelectParams& P, int b, int v, const RowStat& sp, float4 (&w)[VPT4]) {
    const float* zp = P.target + ((size_t)b * P.T + v) * P.V;
    load_chunk(zp, P.V, 0, (((uintptr_t)zp) & 15) == 0, w);
    const Nucleus np{sp.thr, sp.cutoff};
    const bool all = keeps_all(np);
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float pe = unnorm(f4get(w[j], e), sp.zmax, P.ilog);
            f4set(w[j], e, (pe > 0.f && (all || in_nucleus(pe, elem_index(0, j, e), np))) ? pe : 0.f);
        }
}

__global__ __launch_bounds__(NT) void lossless_walk_resident_kernel(SelectParams P) {
    __shared__ Smem sm;
    __shared__ WalkRes ws;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int T = P.T, V = P.V;
    const size_t base = (size_t)b * T;
    const RowStat* st = P.stats + (size_t)b * 2 * T;

    if (tid < kWave) {
        const int lane = tid;
        const bool live = lane < T;
        const int par_in = live ? P.parent[base + lane] : -1;
        const int tok = live ? P.tokens[base + lane] : 0;
        RowStat sl{0.f, 0, 0u, 0, 1.0};
        RowStat sq{0.f, 0, 0u, 0, 1.0};
        float u = 0.f;
        if (live) sl = st[lane];
        if (live && lane >= 1) {
            sq = st[T + lane];
            u = P.u_accept[base + lane];
        }
        const int L = P.kv_len[b];
        bool bad_parent;
        (void)ancestor_mask_of(par_in, T, &bad_parent);
        const bool bad_token = __any(live && lane >= 1 && (tok < 0 || tok >= V));
        bool bad_kv = (L < 0) || (L > P.Lcap - T);
        bad_kv = bad_kv || __any(page_entries_bad(P.pt, b, L + T, lane, kWave));   // paged: L + T <= Lcap here
        int status = (bad_parent ? 1 : 0) | (bad_token ? 2 : 0) | (bad_kv ? 8 : 0);
        if (live) {
            P.row_token[base + lane] = sl.argmax;
            P.node_accept[base + lane] = (lane == 0) ? 1 : 0;
            P.node_p[base + lane] = 0.f;
            P.node_q[base + lane] = 0.f;
            P.path[base + lane] = (lane == 0 && !bad_parent && !bad_token) ? 0 : -1;
            P.out_tokens[base + lane] = -1;
        }
        if (bad_parent || bad_token) {
            if (lane == 0) {
                P.accept_len[b] = 0;
                P.final_node[b] = -1;
                P.final_from_residual[b] = 0;
                P.status[b] = status;
                ws.live = 0;
            }
        } else {
            const int par = par_in;   // valid: parent < node for every node >= 1
            const RowStat spar = shfl_row_stat(sl, par >= 0 ? par : 0);
            float pv = 0.f, qv = 0.f;
            if (live && lane >= 1) {
                const float zt = P.target[(base + par) * V + tok];
                const float zd = P.draft[(base + lane) * V + tok];
                const float et = unnorm(zt, spar.zmax, P.ilog), ed = unnorm(zd, sq.zmax, P.ilog);
                const Nucleus nt{spar.thr, spar.cutoff}, nd{sq.thr, sq.cutoff};
                pv = in_nucleus(et, tok, nt) ? (float)((double)et / spar.Z) : 0.f;
                qv = in_nucleus(ed, tok, nd) ? (float)((double)ed / sq.Z) : 0.f;
            }
            // status bit 4: some supplied draft gives its own token probability 0
            if (__any(live && lane >= 1 && !(qv > 0.f))) status |= 4;
            for (int n = 0; n < T; ++n) {
                const unsigned long long k = __ballot(live && lane >= 1 && par == n);
                if (lane == 0) ws.kids_of[n] = k;
            }
            ws.pv0[lane] = pv;
            ws.qv[lane] = qv;
            ws.u[lane] = u;
            ws.tok[lane] = tok;
            ws.qzmax[lane] = sq.zmax;
            ws.qthr[lane] = sq.thr;
            ws.qcut[lane] = sq.cutoff;
            ws.qZ[lane] = sq.Z;
            if (lane == 0) {
                P.status[b] = status;
                ws.live = 1;
            }
        }
    }
    __syncthreads();
    if (!ws.live) return;

    // walk state, the same in every thread (kept in scalar registers)
    int v = 0, depth = 0, pass = 0;
    unsigned long long kids = uniform_u64(ws.kids_of[0]);
    bool fresh = true;     // r = p_v
    bool have_r = false;   // rr holds r's weights
    double W = 0.0;        // total of r when it is a residual
    float rx_next = 0.f;   // r(x) / W for the next child when r is a residual
    float4 rr[VPT4];
    for (int round = 0; round < 2 * 64 + 1; ++round) {
        int c = -1;
        if (kids != 0ull) {
            c = __builtin_ctzll(kids);
            const float rx = fresh ? ws.pv0[c] : rx_next;
            const float qx = ws.qv[c];
            const bool acc = (qx > 0.f) && (ws.u[c] < rx / qx);
            if (tid == 0) {
                P.node_p[base + c] = rx;
                P.node_q[base + c] = qx;
            }
            if (acc) {
                if (tid == 0) {
                    P.node_accept[base + c] = 1;
                    P.out_tokens[base + depth] = ws.tok[c];
                    P.path[base + depth + 1] = c;
                }
                depth += 1;
                v = c;
                kids = uniform_u64(ws.kids_of[c]);
                fresh = true;
                have_r = false;
                continue;
            }
            kids &= ~(1ull << c);
        }
        // a rejection, or the end of the walk: both need r's weights
        if (!have_r) {
            p_weights(P, b, v, st[v], rr);
            have_r = true;
        }
        if (c < 0) break;
        // r <- [r - q_c]_+ in registers
        float4 q[VPT4];
        const float* zq = P.draft + (base + c) * V;
        load_chunk(zq, V, 0, (((uintptr_t)zq) & 15) == 0, q);
        const Nucleus nq{ws.qthr[c], ws.qcut[c]};
        const float qzmax = ws.qzmax[c];
        const float iq = (float)(1.0 / ws.qZ[c]);
        const float ir = fresh ? (float)(1.0 / st[v].Z) : (float)(1.0 / W);
        // the next child's token x2 sits in slot (j2, e2) of thread t2
        const int c2 = kids ? __builtin_ctzll(kids) : -1;
        const int x2 = __builtin_amdgcn_readfirstlane(c2 >= 0 ? ws.tok[c2] : 0);
        const int t2 = (x2 >> 2) & (NT - 1), j2 = x2 / (4 * NT), e2 = x2 & 3;
        const int buf = pass & 1;
        if (c2 >= 0 && tid == t2) ws.rx[buf][1] = pick(rr, j2, e2);   // r kept
        // past V both weights are 0, so is the residual
#pragma unroll
        for (int j = 0; j < VPT4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) f4set(q[j], e, unnorm(f4get(q[j], e), qzmax, P.ilog));
        if (!keeps_all(nq)) {
#pragma unroll
            for (int j = 0; j < VPT4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!in_nucleus(f4get(q[j], e), elem_index(0, j, e), nq)) f4set(q[j], e, 0.f);
        }
#pragma unroll
        for (int j = 0; j < VPT4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) f4set(q[j], e, resid_weight(f4get(rr[j], e), ir, f4get(q[j], e), iq));
        if (c2 >= 0 && tid == t2) ws.rx[buf][0] = pick(q, j2, e2);    // r new
        const double Wn = block_total(q, ws.wsum, buf);   // its barrier also publishes rx
        if (Wn > 0.0) {
#pragma unroll
            for (int j = 0; j < VPT4; ++j) rr[j] = q[j];
            W = Wn;
            fresh = false;
            if (c2 >= 0) rx_next = (float)((double)ws.rx[buf][0] / W);
        } else if (!fresh && c2 >= 0) {   // a vanishing residual keeps r
            rx_next = (float)((double)ws.rx[buf][1] / W);
        }
        ++pass;
    }

    // the final draw from r: y = min{k : u * W < C_k} in token-id order
    const double Wd = slot_totals(rr, sm);
    int y = locate_in_chunk(rr, 0, V, 0.0, (double)P.u_final[b] * Wd, sm);
    if (y < 0) {
        int last = -1;
#pragma unroll
        for (int j = 0; j < VPT4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (f4get(rr[j], e) > 0.f) last = max(last, elem_index(0, j, e));
        y = block_max_int(last, sm);
    }
    if (tid == 0) {
        P.out_tokens[base + depth] = y;
        P.accept_len[b] = depth;
        P.final_node[b] = v;
        P.final_from_residual[b] = ws.kids_of[v] != 0ull ? 1 : 0;
    }
}

// ---------------------------------------------------------------------------
// The walk spread over K = ceil(V / 4096) workgroups per sequence: workgroup s
// holds token ids 4096 s .. 4096 s + 4095 of r in registers (256 threads x 16).
// Every workgroup takes the same decisions from the same values: the first
// tests as above, and after each residual pass the sequence's K slice totals
// (summed in slice order) and r at the next child's token, published by the
// workgroup holding it.  A pass ends with a barrier of the K workgroups:
// each, once its other stores of the pass have landed (`vmcnt(0)`), stores
// its total tagged with the pass as an agent-scope atomic, and reads the K
// slots until all carry the pass's tag (a bounded wait: running out sets the
// status bit SPEC_VERIFY_STATUS_WALK_TIMEOUT and goes on, so every wave
// ends).  The draw takes r's slice totals from the last pass when r is that
// pass's residual (else from one more synchronised pass), and the workgroup
// holding the slice where u * W falls locates the token.  The last workgroup
// to finish clears the slots and counters for the next step.

constexpr int CT = kWalkThreads;
constexpr int CW = CT / kWave;
constexpr int CV4 = kWalkSlice / (4 * CT);   // float4 per thread

struct CoopShared {
    unsigned long long kids_of[64];
    float pv0[64], qv[64], u[64];
    int tok[64];
    float qzmax[64];
    uint32_t qthr[64];
    int qcut[64];
    double qZ[64];
    double wsum[2][CW];          // wave totals of the block sums (alternating)
    double slot_part[CW][CV4];
    double slot_tot[CV4];
    double W, cum, send;         // after a pass: the total; for the draw: prefixes around slice s*
    float rx_new, rx_old;
    int sstar, winner, found, live, status, last, timed_out;
};

__device__ __forceinline__ int cidx(int first, int j, int e) { return first + 4 * (threadIdx.x + CT * j) + e; }

// Slice [first, first + kWalkSlice) of a row into registers; past V: -inf.
// One lane offset, a resource per slot based at the slot: reads past V
// return 0 without touching memory.
__device__ __forceinline__ void coop_load(const float* row, int V, int first, float4 (&x)[CV4]) {
    const uint64_t a = rows::uniform_addr(row);
    const int f0 = __builtin_amdgcn_readfirstlane(first);
    const int vo = 16 * threadIdx.x;
    const bool aligned = ((a & 15ull) == 0) && ((V & 3) == 0);
    if (aligned) {
#pragma unroll
        for (int j = 0; j < CV4; ++j)
            x[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rows::tail_rsrc(a, V, f0 + 4 * CT * j), vo, 0, 0));
    } else {
#pragma unroll
        for (int j = 0; j < CV4; ++j) {
            const __amdgpu_buffer_rsrc_t rs = rows::tail_rsrc(a, V, f0 + 4 * CT * j);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f4set(x[j], e, __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 4 * e, 0, 0)));
        }
    }
    if (f0 + kWalkSlice > V) {
#pragma unroll
        for (int j = 0; j < CV4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (cidx(f0, j, e) >= V) f4set(x[j], e, -INFINITY);
    }
}

__device__ __forceinline__ float coop_pick(const float4 (&w)[CV4], int j, int e) {
    float r = 0.f;
#pragma unroll
    for (int jj = 0; jj < CV4; ++jj)
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) r = (jj == j && ee == e) ? f4get(w[jj], ee) : r;
    return r;
}

// Workgroup total of w (one barrier; consecutive calls alternate buf).
__device__ __forceinline__ double coop_total(const float4 (&w)[CV4], CoopShared& cs, int buf) {
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < CV4; ++j) t += ((double)w[j].x + (double)w[j].y) + ((double)w[j].z + (double)w[j].w);
    t = wave_sum_d(t);
    if ((threadIdx.x & (kWave - 1)) == 0) cs.wsum[buf][threadIdx.x >> 6] = t;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int k = 0; k < CW; ++k) tot += cs.wsum[buf][k];
    return tot;
}

// Pass totals are published as tagged slots: the low 3 bits of a slice
// total (a nonnegative double) are replaced by 1 + (pass & 3), so a slot
// names the pass it belongs to (slots alternate by pass parity, and 0 is the
// reset state).  Readers strip the tag: every workgroup sees the same totals,
// each within 2^-49 (relative) of the one summed.
__device__ __forceinline__ unsigned long long tag_total(double t, int pass) {
    return (__double_as_longlong(t) & ~7ull) | (unsigned long long)(1 + (pass & 3));
}
__device__ __forceinline__ double untag_total(unsigned long long raw) {
    return __longlong_as_double((long long)(raw & ~7ull));
}

// Barrier of the sequence's K workgroups for pass `pass`, then wave 0 scans
// the K totals in slice order.  With `publish` this workgroup first stores
// its total t in its slot (after its other stores of the pass have landed);
// wave 0 then reads the K slots until each carries this pass's tag (the read
// that sees the tag is the value read: no separate arrival count).  With
// `draw` it also finds the slice s* whose running total first exceeds
// u_final * W (rounding: the last slice with weight) and the prefixes before
// and through it.  Results in cs (after a barrier).
__device__ __forceinline__ void coop_sync_scan(const SelectParams& P, int b, int pass, bool want_rx, double u_final,
                                               bool draw, CoopShared& cs, bool publish, double t) {
    const int K = P.walk_k;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    unsigned long long* part = (unsigned long long*)(P.walk_part + (size_t)(b * 2 + (pass & 1)) * K);
    const unsigned long long want = (unsigned long long)(1 + (pass & 3));
    if (publish) {
        __builtin_amdgcn_s_waitcnt(0);   // this workgroup's other stores of the pass have landed
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(part + (blockIdx.x % K), tag_total(t, pass), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid < kWave) {
        bool late = cs.timed_out != 0;   // after one wait has run out, later ones do not wait
        int it = 0;
        double run = 0.0;        // prefix of the earlier rounds of 64 slices
        int sstar = -1, lastpos = -1;
        double cum = 0.0, send = 0.0, lastcum = 0.0, lastend = 0.0;
        // the target needs the total first: with a draw, two sweeps
        double W = 0.0;
        for (int sweep = 0; sweep < (draw ? 2 : 1); ++sweep) {
            run = 0.0;
            const double target = sweep == 1 ? u_final * W : -1.0;
            for (int k0 = 0; k0 < K; k0 += kWave) {
                const int k = k0 + lane;
                unsigned long long raw = 0ull;
                bool ok = k >= K;
                while (true) {
                    if (!ok) {
                        raw = __hip_atomic_load(part + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ok = (raw & 7ull) == want;
                    }
                    if (__all(ok) || late) break;
                    if (++it > P.walk_spin) late = true;   // a workgroup never arrived: go on, flag it
                    else __builtin_amdgcn_s_sleep(1);
                }
                const double v = untag_total(raw);
                double inc = v;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const double y = __shfl_up(inc, o, kWave);
                    if (lane >= o) inc += y;
                }
                inc += run;
                double exc = __shfl_up(inc, 1, kWave);
                if (lane == 0) exc = run;
                if (sweep == 1) {
                    const unsigned long long past = __ballot(k < K && inc > target);
                    const unsigned long long pos = __ballot(k < K && v > 0.0);
                    if (sstar < 0 && past) {
                        const int l = __builtin_ctzll(past);
                        sstar = k0 + l;
                        cum = __shfl(exc, l, kWave);
                        send = __shfl(inc, l, kWave);
                    }
                    if (pos) {
                        const int l = 63 - __builtin_clzll(pos);
                        lastpos = k0 + l;
                        lastcum = __shfl(exc, l, kWave);
                        lastend = __shfl(inc, l, kWave);
                    }
                }
                run = __shfl(inc, kWave - 1, kWave);
            }
            W = run;
        }
        if (late && lane == 0) {
            __hip_atomic_store(P.walk_sync + 4 * b + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            cs.timed_out = 1;
        }
        if (tid == 0) {
            cs.W = W;
            if (draw) {
                if (sstar < 0) { sstar = lastpos; cum = lastcum; send = lastend; }
                cs.sstar = sstar;
                cs.cum = cum;
                cs.send = send;
            }
            if (want_rx) {
                const float* rx = P.walk_rx + (size_t)(b * 2 + (pass & 1)) * 2;
                cs.rx_new = __hip_atomic_load(rx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                cs.rx_old = __hip_atomic_load(rx + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(CT) void lossless_walk_coop_kernel(SelectParams P) {
    __shared__ CoopShared cs;
    const int K = P.walk_k;
    const int b = blockIdx.x / K, s = blockIdx.x - b * K;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int T = P.T, V = P.V;
    const size_t base = (size_t)b * T;
    const RowStat* st = P.stats + (size_t)b * 2 * T;
    const int first = s * kWalkSlice;   // this workgroup's token ids [first, first + kWalkSlice)
    const bool lead = (s == 0);         // writes the per-node and per-sequence outputs

    if (tid < kWave) {
        const bool live = lane < T;
        const int par_in = live ? P.parent[base + lane] : -1;
        const int tok = live ? P.tokens[base + lane] : 0;
        RowStat sl{0.f, 0, 0u, 0, 1.0};
        RowStat sq{0.f, 0, 0u, 0, 1.0};
        float u = 0.f;
        if (live) sl = st[lane];
        if (live && lane >= 1) {
            sq = st[T + lane];
            u = P.u_accept[base + lane];
        }
        const int L = P.kv_len[b];
        bool bad_parent;
        (void)ancestor_mask_of(par_in, T, &bad_parent);
        const bool bad_token = __any(live && lane >= 1 && (tok < 0 || tok >= V));
        bool bad_kv = (L < 0) || (L > P.Lcap - T);
        bad_kv = bad_kv || (lead && __any(page_entries_bad(P.pt, b, L + T, lane, kWave)));   // paged: L + T <= Lcap here
        int status = (bad_parent ? 1 : 0) | (bad_token ? 2 : 0) | (bad_kv ? 8 : 0);
        // out_tokens: the lead writes the path's drafts and, at the end, -1 past
        // the final position; the final position is written by the workgroup
        // that draws it (stores of different workgroups to one address would
        // not be ordered across XCD caches)
        if (lead && live) {
            P.row_token[base + lane] = sl.argmax;
            P.node_accept[base + lane] = (lane == 0) ? 1 : 0;
            P.node_p[base + lane] = 0.f;
            P.node_q[base + lane] = 0.f;
            P.path[base + lane] = (lane == 0 && !bad_parent && !bad_token) ? 0 : -1;
        }
        if (bad_parent || bad_token) {
            if (lead && live) P.out_tokens[base + lane] = -1;
            if (lane == 0) {
                if (lead) {
                    P.accept_len[b] = 0;
                    P.final_node[b] = -1;
                    P.final_from_residual[b] = 0;
                    P.status[b] = status;
                }
                cs.live = 0;
            }
        } else {
            const int par = par_in;   // valid: parent < node for every node >= 1
            const RowStat spar = shfl_row_stat(sl, par >= 0 ? par : 0);
            float pv = 0.f, qv = 0.f;
            if (live && lane >= 1) {
                const float zt = P.target[(base + par) * V + tok];
                const float zd = P.draft[(base + lane) * V + tok];
                const float et = unnorm(zt, spar.zmax, P.ilog), ed = unnorm(zd, sq.zmax, P.ilog);
                const Nucleus nt{spar.thr, spar.cutoff}, nd{sq.thr, sq.cutoff};
                pv = in_nucleus(et, tok, nt) ? (float)((double)et / spar.Z) : 0.f;
                qv = in_nucleus(ed, tok, nd) ? (float)((double)ed / sq.Z) : 0.f;
            }
            // status bit 4: some supplied draft gives its own token probability 0
            if (__any(live && lane >= 1 && !(qv > 0.f))) status |= 4;
            for (int n = 0; n < T; ++n) {
                const unsigned long long k = __ballot(live && lane >= 1 && par == n);
                if (lane == 0) cs.kids_of[n] = k;
            }
            cs.pv0[lane] = pv;
            cs.qv[lane] = qv;
            cs.u[lane] = u;
            cs.tok[lane] = tok;
            cs.qzmax[lane] = sq.zmax;
            cs.qthr[lane] = sq.thr;
            cs.qcut[lane] = sq.cutoff;
            cs.qZ[lane] = sq.Z;
            if (lane == 0) {
                cs.status = status;
                cs.live = 1;
                cs.timed_out = 0;
            }
        }
    }
    __syncthreads();
    if (!cs.live) return;   // the same in every workgroup of the sequence: none waits

    // walk state, the same in every workgroup of the sequence
    int v = 0, depth = 0, pass = 0;
    unsigned long long kids = uniform_u64(cs.kids_of[0]);
    bool fresh = true;     // r = p_v
    bool have_r = false;   // rr holds this workgroup's slice of r
    double W = 0.0;        // total of r when it is a residual
    float rx_next = 0.f;   // r(x) / W for the next child when r is a residual
    bool last_kept = false;   // r is the residual the last pass produced
    float4 rr[CV4];
    for (int round = 0; round < 2 * 64 + 1; ++round) {
        int c = -1;
        if (kids != 0ull) {
            last_kept = false;
            c = __builtin_ctzll(kids);
            const float rx = fresh ? cs.pv0[c] : rx_next;
            const float qx = cs.qv[c];
            const bool acc = (qx > 0.f) && (cs.u[c] < rx / qx);
            if (lead && tid == 0) {
                P.node_p[base + c] = rx;
                P.node_q[base + c] = qx;
            }
            if (acc) {
                if (lead && tid == 0) {
                    P.node_accept[base + c] = 1;
                    P.out_tokens[base + depth] = cs.tok[c];
                    P.path[base + depth + 1] = c;
                }
                depth += 1;
                v = c;
                kids = uniform_u64(cs.kids_of[c]);
                fresh = true;
                have_r = false;
                continue;
            }
            kids &= ~(1ull << c);
        }
        // a rejection, or the end of the walk: both need r's weights
        const RowStat sp = st[v];
        if (!have_r) {
            coop_load(P.target + (base + v) * V, V, first, rr);
            const Nucleus np{sp.thr, sp.cutoff};
            const bool all = keeps_all(np);
#pragma unroll
            for (int j = 0; j < CV4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pe = unnorm(f4get(rr[j], e), sp.zmax, P.ilog);
                    f4set(rr[j], e, (pe > 0.f && (all || in_nucleus(pe, cidx(first, j, e), np))) ? pe : 0.f);
                }
            have_r = true;
        }
        if (c < 0) break;
        // r <- [r - q_c]_+ on this slice
        float4 q[CV4];
        coop_load(P.draft + (base + c) * V, V, first, q);
        const Nucleus nq{cs.qthr[c], cs.qcut[c]};
        const float qzmax = cs.qzmax[c];
        const float iq = (float)(1.0 / cs.qZ[c]);
        const float ir = fresh ? (float)(1.0 / sp.Z) : (float)(1.0 / W);
        // the next child's token x2: slice s2, slot (j2, e2) of thread t2
        const int c2 = kids ? __builtin_ctzll(kids) : -1;
        const int x2 = __builtin_amdgcn_readfirstlane(c2 >= 0 ? cs.tok[c2] : 0);
        const int s2 = x2 / kWalkSlice, loc2 = x2 - s2 * kWalkSlice;
        const int t2 = (loc2 >> 2) & (CT - 1), j2 = loc2 / (4 * CT), e2 = loc2 & 3;
        const bool owner = c2 >= 0 && s == s2 && tid == t2;
        float* rxp = P.walk_rx + (size_t)(b * 2 + (pass & 1)) * 2;
        if (owner) __hip_atomic_store(rxp + 1, coop_pick(rr, j2, e2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < CV4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) f4set(q[j], e, unnorm(f4get(q[j], e), qzmax, P.ilog));
        if (!keeps_all(nq)) {
#pragma unroll
            for (int j = 0; j < CV4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!in_nucleus(f4get(q[j], e), cidx(first, j, e), nq)) f4set(q[j], e, 0.f);
        }
#pragma unroll
        for (int j = 0; j < CV4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) f4set(q[j], e, resid_weight(f4get(rr[j], e), ir, f4get(q[j], e), iq));
        if (owner) __hip_atomic_store(rxp, coop_pick(q, j2, e2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const double t = coop_total(q, cs, pass & 1);
        coop_sync_scan(P, b, pass, c2 >= 0, 0.0, false, cs, true, t);
        const double Wn = cs.W;
        if (Wn > 0.0) {
#pragma unroll
            for (int j = 0; j < CV4; ++j) rr[j] = q[j];
            W = Wn;
            fresh = false;
            last_kept = true;
            if (c2 >= 0) rx_next = (float)((double)cs.rx_new / W);
        } else if (!fresh && c2 >= 0) {   // a vanishing residual keeps r
            rx_next = (float)((double)cs.rx_old / W);
        }
        ++pass;
    }

    // the final draw from r: y = min{k : u * W < C_k} in token-id order.  The
    // slice totals in slice order give s*; the workgroup holding it locates y.
    // When r is the residual of the last pass, that pass's totals are r's.
    if (last_kept) {
        coop_sync_scan(P, b, pass - 1, false, (double)P.u_final[b], true, cs, false, 0.0);
    } else {
        const double t = coop_total(rr, cs, pass & 1);
        coop_sync_scan(P, b, pass, false, (double)P.u_final[b], true, cs, true, t);
    }
    const int sstar = cs.sstar;
    const double target = (double)P.u_final[b] * cs.W;
    const int draw_buf = last_kept ? (pass & 1) : ((pass + 1) & 1);   // not the last block sum's buffer
    if (s == sstar) {
        // slot totals of this slice (slot j: ids first + 1024 j ..), then the slot
        // holding the target, then the thread, then the id
        double sj[CV4];
#pragma unroll
        for (int j = 0; j < CV4; ++j)
            sj[j] = wave_sum_d(((double)rr[j].x + (double)rr[j].y) + ((double)rr[j].z + (double)rr[j].w));
        if (lane == 0)
#pragma unroll
            for (int j = 0; j < CV4; ++j) cs.slot_part[tid >> 6][j] = sj[j];
        if (tid == 0) { cs.winner = 0; cs.found = -1; }
        __syncthreads();
        double cum = cs.cum;
        int jstar = -1;
#pragma unroll
        for (int j = 0; j < CV4; ++j) {
            double S = 0.0;
#pragma unroll
            for (int w2 = 0; w2 < CW; ++w2) S += cs.slot_part[w2][j];
            if (jstar < 0) {
                if (cum + S > target) jstar = j;
                else cum += S;
            }
        }
        float4 wv = rr[0];
        int last_pos = -1;
#pragma unroll
        for (int j = 0; j < CV4; ++j) {
            const bool hit = j == jstar;
            wv.x = hit ? rr[j].x : wv.x;
            wv.y = hit ? rr[j].y : wv.y;
            wv.z = hit ? rr[j].z : wv.z;
            wv.w = hit ? rr[j].w : wv.w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (f4get(rr[j], e) > 0.f) last_pos = max(last_pos, cidx(first, j, e));
        }
        const size_t out_at = base + depth;
        if (jstar >= 0) {
            // scan over the threads of slot j*: lane sums, wave offsets in order
            const double mine = ((double)wv.x + (double)wv.y) + ((double)wv.z + (double)wv.w);
            double x = mine;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const double y = __shfl_up(x, o, kWave);
                if (lane >= o) x += y;
            }
            if (lane == kWave - 1) cs.wsum[draw_buf][tid >> 6] = x;
            double prev = __shfl_up(x, 1, kWave);
            if (lane == 0) prev = 0.0;
            __syncthreads();
            double wb = 0.0;
#pragma unroll
            for (int w2 = 0; w2 < CW; ++w2) wb += (w2 < (tid >> 6)) ? cs.wsum[draw_buf][w2] : 0.0;
            const double lo = cum + (wb + prev), hi = cum + (wb + x);
            if (lo <= target && target < hi) {
                double run = lo;
                int y = -1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    run += (double)f4get(wv, e);
                    if (y < 0 && run > target) y = cidx(first, jstar, e);
                }
                int lp = -1;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (f4get(wv, e) > 0.f) lp = cidx(first, jstar, e);
                P.out_tokens[out_at] = (y >= 0) ? y : lp;
                cs.winner = 1;
            }
        }
        atomicMax(&cs.found, last_pos);
        __syncthreads();
        if (tid == 0 && !cs.winner) P.out_tokens[out_at] = cs.found;   // rounding left no winner
    }
    if (lead && tid < kWave && tid > depth && tid < T) P.out_tokens[base + tid] = -1;
    if (lead && tid == 0) {
        if (sstar < 0) P.out_tokens[base + depth] = -1;   // no weight at all
        P.accept_len[b] = depth;
        P.final_node[b] = v;
        P.final_from_residual[b] = cs.kids_of[v] != 0ull ? 1 : 0;
        // agent-scope store: the last workgroup to finish may add the time-out bit below
        const int late = __hip_atomic_load(P.walk_sync + 4 * b + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(P.status + b, cs.status | (late ? 16 : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the last workgroup of the sequence to finish (every workgroup has read
    // its last slots by then) clears the slots and the counters for the next
    // launch
    int32_t* sync = P.walk_sync + 4 * b;
    if (tid == 0) {
        __builtin_amdgcn_s_waitcnt(0);
        cs.last = arrive_last(sync + 1, K);
    }
    __syncthreads();
    if (cs.last) {
        unsigned long long* slots = (unsigned long long*)(P.walk_part + (size_t)b * 2 * K);
        for (int i = tid; i < 2 * K; i += CT) __hip_atomic_store(slots + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) {
            // a wait that ran out after the lead wrote the status (the drawing
            // workgroup's, say) still marks the sequence
            if (__hip_atomic_load(sync + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                __hip_atomic_fetch_or(P.status + b, 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + 2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

hipError_t walk_coop_blocks_per_cu(int* blocks) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, lossless_walk_coop_kernel, CT, 0);
}

const char* lossless_walk_kernel_name(const SelectParams& p) {
    if (p.walk_coop && p.V > kWalkSlice) return "lossless_walk_coop_kernel";
    return p.V <= CHUNK ? "lossless_walk_resident_kernel" : "lossless_walk_kernel";
}

hipError_t launch_lossless_walk(const SelectParams& p, hipStream_t s) {
    if (p.walk_coop && p.V > kWalkSlice)
        hipLaunchKernelGGL(lossless_walk_coop_kernel, dim3(p.B * p.walk_k), dim3(CT), 0, s, p);
    else if (p.V <= CHUNK)
        hipLaunchKernelGGL(lossless_walk_resident_kernel, dim3(p.B), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL(lossless_walk_kernel, dim3(p.B), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
