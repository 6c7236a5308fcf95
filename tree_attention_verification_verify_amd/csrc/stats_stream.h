// Row statistics of one logits row without top-p, streamed once by one
// 256-thread workgroup (the body of the streaming row-statistics kernel; the
// attention launch of small grids also runs it in workgroups of its own, see
// launch_attention_mfma).  Internal to the library.
#pragma once

#include "row_block.h"

namespace sv {

constexpr int kStatsWaves = kStatsThreads / kWave;

struct StatsSmem {
    float m[kStatsWaves];
    double s[kStatsWaves];
    float bv[kStatsWaves];
    int bi[kStatsWaves];
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
//
// One group of kStatsThreads threads (t = 0..kStatsThreads-1 within the
// group, sm its own) takes row blk.  An inactive group (a row that needs no
// statistics, or none at all) reads nothing and writes nothing but passes the
// same two barriers, so two groups can share a workgroup.
template <bool WITH_Z>
__device__ __forceinline__ void row_stats_stream_group(const StatsParams& P, int blk, int t, bool active, StatsSmem& sm) {
    constexpr int U = kStatsUnroll / 2;
    const int nrows = P.sampling ? 2 * P.T : P.T;
    const int b = blk / nrows, r = blk - b * nrows;
    const float* row = !active ? P.target
                     : r < P.T ? P.target + ((size_t)b * P.T + r) * P.V
                               : P.draft + ((size_t)b * P.T + (r - P.T)) * P.V;
    const int tid = t, lane = tid & 63, wave = tid >> 6;
    const int V = active ? P.V : 0;
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

    // buffer loads (tracked in order, so a batch's loads stay in flight while
    // the previous batch is folded in), each based at its slot with the lane
    // offset alone checked against what is left of the row: reads past the
    // row return 0 without touching memory.  A batch that reaches past the
    // aligned part is masked to -inf only when it is folded in, after the
    // next batch's loads have been issued.
    const uint64_t row_a = rows::uniform_addr(row);
    auto load = [&](int base4, float (&x)[4 * U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float4 v = __builtin_bit_cast(
                float4, __builtin_amdgcn_raw_buffer_load_b128(rows::tail_rsrc(row_a, V, 4 * (base4 + u * kStatsThreads)), 16 * tid, 0,
                                                               kStreamPolicy));
            x[4 * u] = v.x; x[4 * u + 1] = v.y; x[4 * u + 2] = v.z; x[4 * u + 3] = v.w;
        }
    };
    auto mask_tail = [&](int base4, float (&x)[4 * U]) {
        if (base4 + U * kStatsThreads <= nv4) return;   // the whole batch is in range
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base4 + u * kStatsThreads + tid >= nv4) x[4 * u] = x[4 * u + 1] = x[4 * u + 2] = x[4 * u + 3] = -INFINITY;
    };
    if (nv4 > 0) {   // two register batches in turn (unrolled by two: no copies)
        // the next batch is loaded unconditionally (past the row the loads
        // return 0 and are unused): a conditional load would leave the waits
        // after it counting as if it had not been issued
        float xa[4 * U], xb[4 * U];
        load(0, xa);
        for (int base4 = 0; base4 < nv4; base4 += 2 * U * kStatsThreads) {
            const int b1 = base4 + U * kStatsThreads, b2 = base4 + 2 * U * kStatsThreads;
            load(b1, xb);
            mask_tail(base4, xa);
            absorb(xa, 4 * U, [&](int k) { return 4 * (base4 + (k >> 2) * kStatsThreads + tid) + (k & 3); });
            if (b1 >= nv4) break;
            load(b2, xa);
            mask_tail(b1, xb);
            absorb(xb, 4 * U, [&](int k) { return 4 * (b1 + (k >> 2) * kStatsThreads + tid) + (k & 3); });
        }
    }
    for (int i = 4 * nv4 + tid; i < V; i += kStatsThreads) {   // unaligned rows and the tail
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
    for (int w = 1; w < kStatsWaves; ++w) M = fmaxf(M, sm.m[w]);
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
    if (tid == 0 && active) {
        double Z = 0.0;
        float best = sm.bv[0];
        int besti = sm.bi[0];
        for (int w = 0; w < kStatsWaves; ++w) Z += sm.s[w];
        for (int w = 1; w < kStatsWaves; ++w) rows::argmax_step(best, besti, sm.bv[w], sm.bi[w]);
        RowStat st;
        st.zmax = M;
        st.argmax = besti;
        st.thr = 0u;
        st.cutoff = INT_MAX;
        st.Z = Z;
        P.stats[(size_t)b * nrows + r] = st;
    }
}

// Row blk by a workgroup of kStatsThreads threads (the root's draft row has
// no statistics: the whole workgroup leaves).
template <bool WITH_Z>
__device__ __forceinline__ void row_stats_stream_block(const StatsParams& P, int blk) {
    __shared__ StatsSmem sm;
    const int nrows = P.sampling ? 2 * P.T : P.T;
    if (blk % nrows == P.T) return;
    row_stats_stream_group<WITH_Z>(P, blk, threadIdx.x, true, sm);
}

// Rows 2 blk2 and 2 blk2 + 1 by the two halves of a workgroup of
// 2 kStatsThreads threads, each half with exactly the arithmetic of
// row_stats_stream_block (so the statistics are the same bits).
template <bool WITH_Z>
__device__ __forceinline__ void row_stats_stream_pair(const StatsParams& P, int blk2) {
    __shared__ StatsSmem sm2[2];
    const int nrows = P.sampling ? 2 * P.T : P.T;
    const int half = threadIdx.x / kStatsThreads;
    const int blk = 2 * blk2 + half;
    const bool active = blk < P.B * nrows && blk % nrows != P.T;
    row_stats_stream_group<WITH_Z>(P, blk, (int)threadIdx.x - half * kStatsThreads, active, sm2[half]);
}

}  // namespace sv
