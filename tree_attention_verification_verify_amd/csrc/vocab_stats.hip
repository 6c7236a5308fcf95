// Per-row statistics of the target and draft logits: one read of every row.
//
// For every target row v (the distribution after node v) and every draft row
// i >= 1 (the distribution node i was drafted from) this kernel records the
// largest logit, its smallest token id, and the normaliser Z of the effective
// distribution exp((z - zmax)/temperature), restricted to the top-p nucleus
// when top-p is on.  The acceptance test and the final draw then need only a
// gather per drafted token and one re-read of the selected row.  Using the
// effective (temperature, top-p) distributions follows "投机解码的五条路线",
// section on exact verification.
//
// Without top-p each row is streamed once by a 256-thread workgroup with an
// online max / fp64 sum per thread (rescaled by fp64 exp2 when the running
// max grows), merged in a fixed order.  With top-p the cut needs every
// probability relative to the final max: the row (V <= 32768) is held in the
// registers of a 1024-thread workgroup and cut by a 3-level radix select on
// the fp32 bit patterns with integer mass histograms.

#include "row_block.h"

namespace sv {
namespace {

constexpr int ST = kStatsThreads;
constexpr int SW = ST / kWave;

struct StatsSmem {
    float m[SW];
    double s[SW];
    float bv[SW];
    int bi[SW];
};

// row id within the batch -> pointer (nullptr for the unused draft row of the root)
__device__ __forceinline__ const float* row_ptr(const StatsParams& P, int b, int r) {
    if (r < P.T) return P.target + ((size_t)b * P.T + r) * P.V;
    if (r == P.T) return nullptr;
    return P.draft + ((size_t)b * P.T + (r - P.T)) * P.V;
}

// WITH_Z = false (greedy mode): only the largest logit and its id are needed.
// The row streams in batches of U float4 per thread; the next batch's loads
// are in flight while the current one is folded in.  Per logit: one max3
// half-step, one fma and one exp2 (Z); the argmax is located only when a
// batch raises the thread's best value (first batch, then rarely), by the
// first position holding the batch maximum (positions are in id order).
template <bool WITH_Z>
__global__ __launch_bounds__(ST) void row_stats_stream_kernel(StatsParams P) {
    constexpr int U = kStatsUnroll / 2;
    __shared__ StatsSmem sm;
    const int nrows = P.sampling ? 2 * P.T : P.T;
    const int b = blockIdx.x / nrows, r = blockIdx.x - b * nrows;
    if (r == P.T) return;   // no draft row for the root
    const float* row = r < P.T ? P.target + ((size_t)b * P.T + r) * P.V
                               : P.draft + ((size_t)b * P.T + (r - P.T)) * P.V;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int V = P.V;
    const float ilog = P.ilog;
    const bool aligned = (((uintptr_t)row) & 15) == 0;
    const int nv4 = aligned ? (V >> 2) : 0;

    float m = -INFINITY;     // running max of this thread's logits
    double s = 0.0;          // sum of exp2((z - m) * ilog) over this thread's logits
    float bv = -INFINITY;    // best logit and its smallest id
    int bi = INT_MAX;

    // fold n logits with increasing ids (id_of(k)) into the thread's running statistics
    auto absorb = [&](const float* x, int n, auto id_of) {
        float lm = -INFINITY;
        for (int k = 0; k + 1 < n; k += 2) lm = __builtin_fmaxf(lm, __builtin_fmaxf(x[k], x[k + 1]));
        if (n & 1) lm = fmaxf(lm, x[n - 1]);
        if (lm > bv) {   // the first position holding lm has the smallest id
            int at = -1;
            for (int k = n - 1; k >= 0; --k) at = (x[k] == lm) ? k : at;
            bv = lm;
            bi = id_of(at);
        }
        if (!WITH_Z) return;
        if (lm > m) {
            if (m != -INFINITY) s *= exp2((double)(m - lm) * (double)ilog);
            m = lm;
        }
        if (m == -INFINITY) return;
        const float off = -m * ilog;
        float part = 0.f;
        for (int k = 0; k < n; ++k) part += __builtin_amdgcn_exp2f(fmaf(x[k], ilog, off));
        s += (double)part;
    };

    auto load = [&](int base4, float (&x)[4 * U]) {
        const bool full = base4 + U * ST <= nv4;   // every load of the batch in range: no guards
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i4 = base4 + u * ST + tid;
            float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (full || i4 < nv4) v = *(const float4*)(row + 4 * i4);
            x[4 * u] = v.x; x[4 * u + 1] = v.y; x[4 * u + 2] = v.z; x[4 * u + 3] = v.w;
        }
    };
    if (nv4 > 0) {   // two register batches in turn (unrolled by two: no copies)
        float xa[4 * U], xb[4 * U];
        load(0, xa);
        for (int base4 = 0; base4 < nv4; base4 += 2 * U * ST) {
            const int b1 = base4 + U * ST, b2 = base4 + 2 * U * ST;
            if (b1 < nv4) load(b1, xb);
            absorb(xa, 4 * U, [&](int k) { return 4 * (base4 + (k >> 2) * ST + tid) + (k & 3); });
            if (b1 >= nv4) break;
            if (b2 < nv4) load(b2, xa);
            absorb(xb, 4 * U, [&](int k) { return 4 * (b1 + (k >> 2) * ST + tid) + (k & 3); });
        }
    }
    for (int i = 4 * nv4 + tid; i < V; i += ST) {   // unaligned rows and the tail
        const float x[1] = {row[i]};
        absorb(x, 1, [&](int) { return i; });
    }

    // merge: max, then the sums rescaled to it, then the argmax (fixed order)
    if (!WITH_Z) m = bv;
    float wm = wave_max(m);
    if (lane == 0) sm.m[wave] = wm;
    __syncthreads();
    float M = sm.m[0];
#pragma unroll
    for (int w = 1; w < SW; ++w) M = fmaxf(M, sm.m[w]);
    double mine = (!WITH_Z || m == -INFINITY) ? 0.0 : s * exp2((double)(m - M) * (double)ilog);
    mine = wave_sum_d(mine);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rows::argmax_step(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
    if (lane == 0) {
        sm.s[wave] = mine;
        sm.bv[wave] = bv;
        sm.bi[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        double Z = 0.0;
        float best = sm.bv[0];
        int besti = sm.bi[0];
        for (int w = 0; w < SW; ++w) Z += sm.s[w];
        for (int w = 1; w < SW; ++w) rows::argmax_step(best, besti, sm.bv[w], sm.bi[w]);
        RowStat st;
        st.zmax = M;
        st.argmax = besti;
        st.thr = 0u;
        st.cutoff = INT_MAX;
        st.Z = Z;
        P.stats[(size_t)b * nrows + r] = st;
    }
}

// Top-p rows: the whole row in registers, cut, then the nucleus normaliser.
__global__ __launch_bounds__(rows::NT) void row_stats_topp_kernel(StatsParams P) {
    using namespace rows;
    __shared__ Smem sm;
    const int nrows = 2 * P.T;
    const int b = blockIdx.x / nrows, r = blockIdx.x - b * nrows;
    const float* row = row_ptr(P, b, r);
    if (!row) return;
    const int V = P.V;
    const float ilog = P.ilog;
    const bool aligned = (((uintptr_t)row) & 15) == 0;
    float4 e[VPT4];
    load_chunk(row, V, 0, aligned, e);
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = elem_index(0, j, c);
            const float v = f4get(e[j], c);
            if (idx < V && (v > bv || (v == bv && idx < bi))) { bv = v; bi = idx; }
        }
    const int best = block_argmax(bv, bi, sm);
    const float M = block_max(thread_max(e), sm);
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) f4set(e[j], c, unnorm(f4get(e[j], c), M, ilog));
    const Nucleus nu = find_nucleus(e, 0, V, P.top_p, sm);
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float v = f4get(e[j], c);
            if (in_nucleus(v, elem_index(0, j, c), nu)) s += (double)v;
        }
    const double Z = block_sum_d(s, sm);
    if (threadIdx.x == 0) {
        RowStat st;
        st.zmax = M;
        st.argmax = best;
        st.thr = nu.thr;
        st.cutoff = nu.cutoff;
        st.Z = Z;
        P.stats[(size_t)b * nrows + r] = st;
    }
}

}  // namespace

hipError_t launch_row_stats(const StatsParams& p, hipStream_t s) {
    const int nrows = p.sampling ? 2 * p.T : p.T;
    dim3 grid((unsigned)(p.B * nrows));
    if (p.sampling && p.top_p < 1.f)
        hipLaunchKernelGGL(row_stats_topp_kernel, grid, dim3(rows::NT), 0, s, p);
    else if (p.sampling)
        hipLaunchKernelGGL(row_stats_stream_kernel<true>, grid, dim3(ST), 0, s, p);
    else
        hipLaunchKernelGGL(row_stats_stream_kernel<false>, grid, dim3(ST), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
