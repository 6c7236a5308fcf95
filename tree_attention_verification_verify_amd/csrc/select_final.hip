// Acceptance decisions, longest accepted root path and the final token, one
// 1024-thread workgroup per sequence.
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
// Phase 1 (wave 0, lane = node): probabilities at the drafted tokens from the
// row statistics and one gathered logit each, decisions, path.  With the
// ancestor sets anc*(i) as 64-bit masks, "whole root path accepted" is
// (anc*(i) & ~accepted) == 0 and depth(i) = popcount(anc*(i)) - 1.
// Phase 2 (all waves): the inverse-CDF draw over row v* (and the draft row of
// its first child), re-read from HBM, in token-id order.

#include "row_block.h"

namespace sv {
namespace {

using namespace rows;

struct SelectShared {
    int vstar, c0, dstar, live;
};

__device__ __forceinline__ float prob_at(const float* row, const RowStat& st, int x, float ilog) {
    const float e = unnorm(row[x], st.zmax, ilog);
    const Nucleus nu{st.thr, st.cutoff};
    return in_nucleus(e, x, nu) ? (float)((double)e / st.Z) : 0.f;
}

// Weights of the final draw for one chunk: residual max(0, p - q) or p alone,
// both restricted to their nuclei.  zq holds the draft logits on entry (when
// resid) and the weights on return.
__device__ void final_weights(const float4 (&zp)[VPT4], float4 (&zq)[VPT4], int cb, int V,
                              const RowStat& sp, const RowStat& sq, bool resid, float ilog) {
    const Nucleus np{sp.thr, sp.cutoff}, nq{sq.thr, sq.cutoff};
    const float ip = (float)(1.0 / sp.Z);
    const float iq = resid ? (float)(1.0 / sq.Z) : 0.f;
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = elem_index(cb, j, c);
            float pe = unnorm(f4get(zp[j], c), sp.zmax, ilog);
            if (!in_nucleus(pe, idx, np)) pe = 0.f;
            float v = pe;
            if (resid) {
                float qe = unnorm(f4get(zq[j], c), sq.zmax, ilog);
                if (!in_nucleus(qe, idx, nq)) qe = 0.f;
                v = resid_weight(pe, ip, qe, iq);
            }
            f4set(zq[j], c, idx < V ? v : 0.f);
        }
}

// Inverse-CDF draw over row v* (residual against draft row c0 when resid).
// ONE_CHUNK: the rows (V <= 32768) stay in registers between the passes.
template <bool ONE_CHUNK>
__device__ int final_draw(const SelectParams& P, int b, int v, int c0, bool resid, Smem& sm) {
    const int V = P.V, T = P.T;
    const float ilog = P.ilog;
    const RowStat sp = P.stats[(size_t)b * 2 * T + v];
    const RowStat sq = resid ? P.stats[(size_t)b * 2 * T + T + c0] : sp;
    const float* zp = P.target + ((size_t)b * T + v) * V;
    const float* zq = resid ? P.draft + ((size_t)b * T + c0) * V : zp;
    const bool ap = (((uintptr_t)zp) & 15) == 0, aq = (((uintptr_t)zq) & 15) == 0;
    const double u = (double)P.u_final[b];
    float4 xp[VPT4], xq[VPT4];   // target logits; draft logits, then the draw weights

    for (int attempt = 0; attempt < 2; ++attempt) {
        const bool use_resid = resid && attempt == 0;
        if constexpr (ONE_CHUNK) {
            // both rows stay in registers: residual weights first, p alone if they vanish
            load_chunk(zp, V, 0, ap, xp);
            bool with_resid = resid;
            double W = 0.0;
            if (resid) {
                load_chunk(zq, V, 0, aq, xq);
                final_weights(xp, xq, 0, V, sp, sq, true, ilog);
                W = slot_totals(xq, sm);
                with_resid = W > 0.0;
            }
            if (!with_resid) {
                final_weights(xp, xq, 0, V, sp, sq, false, ilog);
                W = slot_totals(xq, sm);
            }
            int y = locate_in_chunk(xq, 0, V, 0.0, u * W, sm);
            if (y < 0) {
                int last = -1;
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (f4get(xq[j], c) > 0.f) last = max(last, elem_index(0, j, c));
                y = block_max_int(last, sm);
            }
            return y;
        } else {
        // streamed rows: chunk totals, then re-read the chunk holding the draw
        double W = 0.0;
        int ci = 0;
        for (int cb = 0; cb < V; cb += CHUNK, ++ci) {
            load_chunk(zp, V, cb, ap, xp);
            if (use_resid) load_chunk(zq, V, cb, aq, xq);
            final_weights(xp, xq, cb, V, sp, sq, use_resid, ilog);
            const double S = slot_totals(xq, sm);
            if (threadIdx.x == 0) sm.chunk_sum[ci] = S;
            W += S;
        }
        __syncthreads();
        if (!(W > 0.0)) continue;
        const double target = u * W;
        double cum = 0.0;
        int cstar = -1;
        for (int k = 0; k < ci; ++k) {
            if (cum + sm.chunk_sum[k] > target) { cstar = k; break; }
            cum += sm.chunk_sum[k];
        }
        if (cstar < 0) {   // rounding: the last chunk with weight
            for (int k = ci - 1; k >= 0; --k)
                if (sm.chunk_sum[k] > 0.0) { cstar = k; break; }
            cum = 0.0;
            for (int k = 0; k < cstar; ++k) cum += sm.chunk_sum[k];
        }
        const int cb = cstar * CHUNK;
        load_chunk(zp, V, cb, ap, xp);
        if (use_resid) load_chunk(zq, V, cb, aq, xq);
        final_weights(xp, xq, cb, V, sp, sq, use_resid, ilog);
        (void)slot_totals(xq, sm);
        int y = locate_in_chunk(xq, cb, V, cum, target, sm);
        if (y < 0) {
            int last = -1;
#pragma unroll
            for (int j = 0; j < VPT4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (f4get(xq[j], c) > 0.f) last = max(last, elem_index(cb, j, c));
            y = block_max_int(last, sm);
        }
        return y;
        }
    }
    return -1;   // unreachable: p always has mass
}

template <bool ONE_CHUNK>
__global__ __launch_bounds__(NT) void select_kernel(SelectParams P) {
    __shared__ Smem sm;
    __shared__ SelectShared sh;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int T = P.T, V = P.V;
    const size_t base = (size_t)b * T;
    const int nrows = P.sampling ? 2 * T : T;
    const RowStat* st = P.stats + (size_t)b * nrows;

    if (tid < kWave) {
        const int lane = tid;
        const bool live = lane < T;
        bool bad_parent;
        const unsigned long long anc = ancestor_mask(P.parent + base, T, &bad_parent);
        const int tok = live ? P.tokens[base + lane] : 0;
        const bool bad_token = __any(live && lane >= 1 && (tok < 0 || tok >= V));
        const int L = P.kv_len[b];
        const bool bad_kv = (L < 0) || (L > P.Lcap - T);
        int status = (bad_parent ? 1 : 0) | (bad_token ? 2 : 0) | (bad_kv ? 8 : 0);
        if (live) P.row_token[base + lane] = st[lane].argmax;

        if (bad_parent || bad_token) {
            if (live) {
                P.path[base + lane] = -1;
                P.out_tokens[base + lane] = -1;
                P.node_accept[base + lane] = 0;
                P.node_p[base + lane] = 0.f;
                P.node_q[base + lane] = 0.f;
            }
            if (lane == 0) {
                P.accept_len[b] = 0;
                P.final_node[b] = -1;
                P.final_from_residual[b] = 0;
                P.status[b] = status;
                sh.live = 0;
            }
        } else {
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
            if (live) {
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
                P.accept_len[b] = dstar;
                P.final_node[b] = vstar;
                P.final_from_residual[b] = (P.sampling && kids) ? 1 : 0;
                P.status[b] = status;
                sh.live = 1;
                sh.vstar = vstar;
                sh.dstar = dstar;
                sh.c0 = kids ? __builtin_ctzll(kids) : -1;
            }
        }
    }
    __syncthreads();
    if (!sh.live) return;
    const int vstar = sh.vstar;
    int y;
    if (!P.sampling) y = st[vstar].argmax;
    else y = final_draw<ONE_CHUNK>(P, b, vstar, sh.c0, sh.c0 >= 0, sm);
    if (tid == 0) P.out_tokens[base + sh.dstar] = y;
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
    if (p.V <= CHUNK) hipLaunchKernelGGL(select_kernel<true>, dim3(p.B), dim3(NT), 0, s, p);
    else hipLaunchKernelGGL(select_kernel<false>, dim3(p.B), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
