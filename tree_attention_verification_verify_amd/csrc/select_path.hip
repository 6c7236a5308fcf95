// Acceptance decisions and longest accepted root path, one wave per sequence.
//
// Node i (>= 1) passes its test when u_i < p_parent(i)(x_i) / q_i(x_i)
// (sampling: featured article on the founding speculative-decoding paper,
// section 2.1; "推测解码技术详解：加速LLM推理的关键" section "数学保证：无损输出质量"
// compares a uniform with the ratio) or when x_i is the target's best token
// after its parent (greedy: "大模型推理加速：推测解码与MTP核心原理与工程实践"
// section 3.1 item 3).  Only a prefix accepted consecutively from the root
// counts and the deepest such node v* is kept (first page, section 2.3;
// "投机解码的五条路线" figure 3); ties between equally deep nodes go to the
// smallest node id.  The emitted tokens are the path's drafts followed by the
// candidate final token of row v* (residual or bonus, from the vocab pass).
//
// With the ancestor sets anc*(i) as 64-bit masks, "whole root path accepted"
// is (anc*(i) & ~accepted) == 0 and depth(i) = popcount(anc*(i)) - 1.

#include "device_common.h"
#include "kernels.h"

namespace sv {
namespace {

__global__ __launch_bounds__(64) void select_kernel(SelectParams P) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int T = P.T;
    const size_t base = (size_t)b * T;
    const bool live = lane < T;

    bool bad_parent;
    const unsigned long long anc = ancestor_mask(P.parent + base, T, &bad_parent);
    const int tok = live ? P.tokens[base + lane] : 0;
    const bool bad_token = __any(live && lane >= 1 && (tok < 0 || tok >= P.V));
    const int L = P.kv_len[b];
    const bool bad_kv = (L < 0) || (L > P.Lcap - T);
    int status = (bad_parent ? 1 : 0) | (bad_token ? 2 : 0) | (bad_kv ? 8 : 0);

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
        }
        return;
    }

    const int par = live ? P.parent[base + lane] : -1;
    bool a = (lane == 0);
    bool zero_q = false;
    if (live && lane >= 1) {
        if (P.sampling) {
            const float p = P.node_p[base + lane];
            const float q = P.node_q[base + lane];
            if (q > 0.f) a = P.u_accept[base + lane] < p / q;
            else zero_q = true;
        } else {
            a = (tok == P.row_token[base + par]);
        }
    }
    if (__any(zero_q)) status |= 4;
    const unsigned long long accepted = __ballot(live && a);
    const bool path_ok = live && ((anc & ~accepted) == 0ull);
    const int depth = live ? (__popcll(anc) - 1) : -1;
    // deepest fully accepted node, smallest id on ties
    int key = path_ok ? (depth * 64 + (63 - lane)) : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, kWave));
    const int vstar = 63 - (key & 63);
    const int dstar = key >> 6;
    const unsigned long long on_path = __shfl(anc, vstar, kWave);
    const bool has_child = __any(live && lane >= 1 && par == vstar);

    if (live) {
        P.node_accept[base + lane] = a ? 1 : 0;
        if (!P.sampling || lane == 0) {  // the root is never tested
            P.node_p[base + lane] = 0.f;
            P.node_q[base + lane] = 0.f;
        }
        const bool mine = (on_path >> lane) & 1ull;
        // path[depth] = node; out_tokens[depth-1] = its token; the rest -1
        if (lane > dstar) P.path[base + lane] = -1;
        if (mine) P.path[base + depth] = lane;
        if (mine && lane != 0) P.out_tokens[base + depth - 1] = tok;
        if (lane > dstar) P.out_tokens[base + lane] = -1;
        if (lane == vstar) P.out_tokens[base + dstar] = P.row_token[base + vstar];
    }
    if (lane == 0) {
        P.accept_len[b] = dstar;
        P.final_node[b] = vstar;
        P.final_from_residual[b] = (P.sampling && has_child) ? 1 : 0;
        P.status[b] = status;
    }
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
    hipLaunchKernelGGL(select_kernel, dim3(p.B), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
