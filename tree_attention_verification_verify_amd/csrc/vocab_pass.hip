// Vocabulary pass of the verify step: per-row temperature softmax statistics,
// the probabilities the acceptance test needs, and the candidate final token
// of every row, in one read of the logits.
//
// Rules followed: effective distributions (temperature, top-p) are the ones
// used for acceptance ("投机解码的五条路线", section on exact verification); on
// rejection the correction is drawn from norm([p - q]_+), and after a fully
// accepted path a bonus token is drawn from the target's next distribution
// (featured article on the founding speculative-decoding paper, sections 2.1
// and 2.2); greedy mode uses the target's best token ("大模型推理加速：推测解码与
// MTP核心原理与工程实践" section 3.1 item 3).
//
// Job layout (ours): one 1024-thread workgroup per job.
//   greedy:   job v (< T)       : argmax of target row v.
//   sampling: job v (< T)       : target row v and, if v has children, the
//                                 draft row of its first child c0; writes
//                                 p_v(x_c) for every child c, q_c0(x_c0), and
//                                 the candidate final token of row v (residual
//                                 against q_c0, or bonus from p_v for a leaf).
//             job T + i (i >= 1): draft row of node i when i is not the first
//                                 child of its parent; writes q_i(x_i).
// The selection kernel then only gathers: the final token is the candidate of
// the selected row.  Every logits row is read once when V <= 32768 (the row
// stays in registers); longer rows are streamed in 32768-element chunks.
//
// Precision: exp in fp32, sums in fp64 in a fixed order (deterministic).  The
// top-p cut is a radix select on the fp32 bit patterns of the unnormalised
// probabilities with fixed-point integer mass histograms (exact, order-free);
// ties at the cut keep the smallest token ids.  Sampling is the inverse CDF in
// token-id order: the smallest k with u * W < C_k.

#include <limits.h>

#include "device_common.h"
#include "kernels.h"

namespace sv {
namespace {

constexpr int NT = kVocabThreads;
constexpr int NW = NT / kWave;
constexpr int VPT4 = 8;                     // float4 per thread per chunk
constexpr int CHUNK = NT * VPT4 * 4;
static_assert(CHUNK == kVocabChunk, "chunk size");
constexpr int MAX_CHUNKS = 128;
constexpr float kFix = 1099511627776.0f;    // 2^40: fixed-point scale of top-p masses

struct Smem {
    float f[NW];
    double d[NW];
    unsigned long long u[NW];
    int i[NW];
    double dpre[NW + 1];
    unsigned long long upre[NW + 1];
    float fr;
    double dr;
    unsigned long long ur;
    int ir;
    unsigned long long hist[1024];
    double chunk_sum[MAX_CHUNKS];
    int winner;
    int found;
};

__device__ __forceinline__ int tid_() { return threadIdx.x; }
__device__ __forceinline__ int lane_() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_() { return threadIdx.x >> 6; }

// element index of (slot j, component e) for this thread in chunk cb
__device__ __forceinline__ int elem_index(int cb, int j, int e) { return cb + 4 * (tid_() + NT * j) + e; }

__device__ __forceinline__ float f4get(const float4& v, int e) {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}
__device__ __forceinline__ void f4set(float4& v, int e, float x) {
    if (e == 0) v.x = x; else if (e == 1) v.y = x; else if (e == 2) v.z = x; else v.w = x;
}

// Block reductions: each wave reduces, wave 0 reduces the wave results in a
// fixed order and broadcasts one value (deterministic, two barriers).
__device__ float block_max(float v, Smem& sm) {
    v = wave_max(v);
    if (lane_() == 0) sm.f[wave_()] = v;
    __syncthreads();
    if (wave_() == 0) {
        float x = wave_max(lane_() < NW ? sm.f[lane_()] : -INFINITY);
        if (lane_() == 0) sm.fr = x;
    }
    __syncthreads();
    return sm.fr;
}

__device__ double block_sum_d(double v, Smem& sm) {
    v = wave_sum_d(v);
    if (lane_() == 0) sm.d[wave_()] = v;
    __syncthreads();
    if (wave_() == 0) {
        double x = wave_sum_d(lane_() < NW ? sm.d[lane_()] : 0.0);
        if (lane_() == 0) sm.dr = x;
    }
    __syncthreads();
    return sm.dr;
}

__device__ unsigned long long block_sum_u64(unsigned long long v, Smem& sm) {
    v = wave_sum_u64(v);
    if (lane_() == 0) sm.u[wave_()] = v;
    __syncthreads();
    if (wave_() == 0) {
        unsigned long long x = wave_sum_u64(lane_() < NW ? sm.u[lane_()] : 0ull);
        if (lane_() == 0) sm.ur = x;
    }
    __syncthreads();
    return sm.ur;
}

__device__ int block_max_int(int v, Smem& sm) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    if (lane_() == 0) sm.i[wave_()] = v;
    __syncthreads();
    if (wave_() == 0) {
        int x = lane_() < NW ? sm.i[lane_()] : INT_MIN;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, kWave));
        if (lane_() == 0) sm.ir = x;
    }
    __syncthreads();
    return sm.ir;
}

__device__ __forceinline__ void argmax_step(float& v, int& idx, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < idx)) { v = v2; idx = i2; }
}

// (value, index) max with the smallest index among equal values.
__device__ int block_argmax(float v, int idx, Smem& sm) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) argmax_step(v, idx, __shfl_xor(v, o, kWave), __shfl_xor(idx, o, kWave));
    if (lane_() == 0) { sm.f[wave_()] = v; sm.i[wave_()] = idx; }
    __syncthreads();
    if (wave_() == 0) {
        float x = lane_() < NW ? sm.f[lane_()] : -INFINITY;
        int xi = lane_() < NW ? sm.i[lane_()] : INT_MAX;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) argmax_step(x, xi, __shfl_xor(x, o, kWave), __shfl_xor(xi, o, kWave));
        if (lane_() == 0) sm.ir = xi;
    }
    __syncthreads();
    return sm.ir;
}

// Inclusive scan of v over thread order; *excl receives the exclusive prefix.
// Adjacent threads' bounds are bitwise equal (incl_t == excl_{t+1}): wave
// offsets are accumulated sequentially from the waves' last inclusive values.
__device__ unsigned long long block_scan_u64(unsigned long long v, unsigned long long* excl, Smem& sm) {
    unsigned long long x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const unsigned long long y = __shfl_up(x, o, kWave);
        if (lane_() >= o) x += y;
    }
    if (lane_() == kWave - 1) sm.u[wave_()] = x;
    unsigned long long prev = __shfl_up(x, 1, kWave);
    if (lane_() == 0) prev = 0;
    __syncthreads();
    if (tid_() == 0) {
        unsigned long long acc = 0;
        for (int w = 0; w < NW; ++w) { sm.upre[w] = acc; acc += sm.u[w]; }
    }
    __syncthreads();
    const unsigned long long base = sm.upre[wave_()];
    *excl = base + prev;
    return base + x;
}

__device__ double block_scan_d(double v, double* excl, Smem& sm) {
    double x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(x, o, kWave);
        if (lane_() >= o) x += y;
    }
    if (lane_() == kWave - 1) sm.d[wave_()] = x;
    double prev = __shfl_up(x, 1, kWave);
    if (lane_() == 0) prev = 0.0;
    __syncthreads();
    if (tid_() == 0) {
        double acc = 0.0;
        for (int w = 0; w < NW; ++w) { sm.dpre[w] = acc; acc += sm.d[w]; }
    }
    __syncthreads();
    const double base = sm.dpre[wave_()];
    *excl = base + prev;
    return base + x;
}

// Load chunk cb of a row: out-of-range entries become -inf.
__device__ void load_chunk(const float* row, int V, int cb, bool aligned, float4 (&x)[VPT4]) {
#pragma unroll
    for (int j = 0; j < VPT4; ++j) {
        const int idx = elem_index(cb, j, 0);
        if (aligned && idx + 3 < V) {
            x[j] = *(const float4*)(row + idx);
        } else {
            float4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) f4set(v, e, (idx + e < V) ? row[idx + e] : -INFINITY);
            x[j] = v;
        }
    }
}

__device__ float thread_max(const float4 (&x)[VPT4]) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPT4; ++j) m = fmaxf(fmaxf(fmaxf(m, x[j].x), fmaxf(x[j].y, x[j].z)), x[j].w);
    return m;
}

// Unnormalised probability of a logit: exp((z - zmax) / temperature).
__device__ __forceinline__ float unnorm(float z, float zmax, float ilog) { return exp2f((z - zmax) * ilog); }

// max(0, p - q) from unnormalised values and inverse normalisers.  Both
// products are rounded before the subtraction (contraction into a fused
// multiply-add is switched off here), so identical distributions give
// exactly zero.
__device__ __forceinline__ float resid_weight(float ep, float ip, float eq, float iq) {
#pragma clang fp contract(off)
    const float p = ep * ip;
    const float q = eq * iq;
    return fmaxf(p - q, 0.f);
}

// Top-p cut of a register-resident row of unnormalised probabilities e.
struct Nucleus {
    uint32_t thr;   // bit pattern of the cut value
    int cutoff;     // ties at thr are kept for token ids < cutoff
};

__device__ __forceinline__ bool in_nucleus(float e, int idx, const Nucleus& nu) {
    const uint32_t bits = __float_as_uint(e);
    return bits > nu.thr || (bits == nu.thr && idx < nu.cutoff);
}

__device__ __forceinline__ unsigned long long fixmass(float e) { return (unsigned long long)__float2ull_rn(e * kFix); }

// One radix level: histogram (by `shift`/`width` bits) of the mass of the
// elements whose bits above the level equal `prefix`, then the bucket where
// the mass counted from the top first reaches `need`.  Returns the bucket;
// *above receives the mass of the larger buckets.
__device__ int radix_level(const float4 (&e)[VPT4], int cb, int V, int shift, uint32_t prefix, int prefix_shift,
                           double need, unsigned long long* above, Smem& sm) {
    const int tid = tid_();
    sm.hist[tid] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < VPT4; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = elem_index(cb, j, c);
            if (idx < V) {
                const float v = f4get(e[j], c);
                const uint32_t bits = __float_as_uint(v);
                if ((bits >> prefix_shift) == prefix) {
                    const int bucket = (bits >> shift) & 1023;
                    atomicAdd(&sm.hist[bucket], fixmass(v));
                }
            }
        }
    }
    __syncthreads();
    // thread t holds bucket 1023 - t: scanning thread order = descending value
    unsigned long long excl;
    const unsigned long long incl = block_scan_u64(sm.hist[1023 - tid], &excl, sm);
    if (tid == 0) sm.found = -1;
    __syncthreads();
    if ((double)excl < need && need <= (double)incl) atomicMax(&sm.found, tid);
    __syncthreads();
    int t = sm.found;
    if (t < 0) t = NT - 1;   // need above every bucket: cannot happen for need <= total
    if (tid == t) sm.u[0] = excl;
    __syncthreads();
    *above = sm.u[0];
    __syncthreads();
    return 1023 - t;
}

__device__ Nucleus find_nucleus(const float4 (&e)[VPT4], int cb, int V, float top_p, Smem& sm) {
    unsigned long long mine = 0;
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (elem_index(cb, j, c) < V) mine += fixmass(f4get(e[j], c));
    const unsigned long long total = block_sum_u64(mine, sm);
    const double need = (double)top_p * (double)total;
    unsigned long long a1, a2, a3;
    const int b1 = radix_level(e, cb, V, 20, 0u, 31, need, &a1, sm);
    const int b2 = radix_level(e, cb, V, 10, (uint32_t)b1, 20, need - (double)a1, &a2, sm);
    const int b3 = radix_level(e, cb, V, 0, ((uint32_t)b1 << 10) | (uint32_t)b2, 10, need - (double)a1 - (double)a2,
                               &a3, sm);
    Nucleus nu;
    nu.thr = ((uint32_t)b1 << 20) | ((uint32_t)b2 << 10) | (uint32_t)b3;
    nu.cutoff = INT_MAX;
    const unsigned long long above = a1 + a2 + a3;
    const unsigned long long tie_mass = fixmass(__uint_as_float(nu.thr));
    int ties = 0;
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (elem_index(cb, j, c) < V && __float_as_uint(f4get(e[j], c)) == nu.thr) ++ties;
    ties = (int)block_sum_u64((unsigned long long)ties, sm);
    if (ties > 1 && tie_mass > 0) {
        const double rest = need - (double)above;
        long long k = (long long)ceil(rest / (double)tie_mass);
        if (k < 1) k = 1;
        if (k < ties) {
            // smallest cutoff c with #ties(idx < c) >= k, by bisection on the token id
            int lo = 0, hi = V;
            while (lo < hi) {
                const int mid = lo + (hi - lo) / 2;
                int cnt = 0;
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int idx = elem_index(cb, j, c);
                        if (idx < V && idx <= mid && __float_as_uint(f4get(e[j], c)) == nu.thr) ++cnt;
                    }
                cnt = (int)block_sum_u64((unsigned long long)cnt, sm);
                if (cnt >= k) hi = mid; else lo = mid + 1;
            }
            nu.cutoff = lo + 1;
        }
    }
    return nu;
}

// Sum of w over a chunk (fp64, fixed order).
__device__ double chunk_total(const float4 (&w)[VPT4], Smem& sm) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
        s += ((double)w[j].x + (double)w[j].y) + ((double)w[j].z + (double)w[j].w);
    return block_sum_d(s, sm);
}

// Smallest token id k of this chunk with base + C_k > target (C = prefix sums
// of w in id order within the chunk), or -1 if the chunk does not reach it.
__device__ int locate_in_chunk(const float4 (&w)[VPT4], int cb, int V, double base, double target, Smem& sm) {
    double cum = base;
    int jstar = -1;
#pragma unroll
    for (int j = 0; j < VPT4; ++j) {
        const double sj = ((double)w[j].x + (double)w[j].y) + ((double)w[j].z + (double)w[j].w);
        const double S = block_sum_d(sj, sm);
        if (jstar < 0) {
            if (cum + S > target) jstar = j;
            else cum += S;
        }
    }
    if (jstar < 0) return -1;
    float4 wv = w[0];
#pragma unroll
    for (int j = 1; j < VPT4; ++j)
        if (j == jstar) wv = w[j];
    const double mysum = ((double)wv.x + (double)wv.y) + ((double)wv.z + (double)wv.w);
    double excl;
    double incl = block_scan_d(mysum, &excl, sm);
    excl += cum;
    incl += cum;
    if (tid_() == 0) { sm.winner = INT_MAX; sm.found = -1; }
    __syncthreads();
    if (excl <= target && target < incl) atomicMin(&sm.winner, tid_());
    __syncthreads();
    int last_pos = -1;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (f4get(wv, c) > 0.f) last_pos = elem_index(cb, jstar, c);
    if (tid_() == sm.winner) {
        double run = excl;
        int y = -1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            run += (double)f4get(wv, c);
            if (y < 0 && run > target) y = elem_index(cb, jstar, c);
        }
        sm.found = (y >= 0) ? y : last_pos;
    }
    __syncthreads();
    int y = sm.found;
    __syncthreads();
    if (y < 0) {  // rounding left no winner: last positive weight of the slot
        y = block_max_int(last_pos, sm);
    }
    return y;
}

// ---------------------------------------------------------------- kernel

// KIND 0: greedy; 1: sampling with rows held in registers (V <= CHUNK);
// 2: sampling with rows streamed in chunks.
template <int KIND>
__global__ __launch_bounds__(NT) void vocab_kernel(VocabParams P) {
    __shared__ Smem sm;
    __shared__ int kids_s[64];
    __shared__ int nkids_s;
    const int T = P.T, V = P.V;
    const int jobs = P.sampling ? 2 * T : T;
    const int b = blockIdx.x / jobs;
    const int job = blockIdx.x - b * jobs;
    const int tid = tid_();
    const int32_t* par_row = P.parent + (size_t)b * T;
    const int32_t* tok_row = P.tokens + (size_t)b * T;

    // ---- greedy: argmax of target row `job`
    if constexpr (KIND == 0) {
        const float* row = P.target + ((size_t)b * T + job) * V;
        const bool aligned = (((uintptr_t)row) & 15) == 0;
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int cb = 0; cb < V; cb += CHUNK) {
            float4 x[VPT4];
            load_chunk(row, V, cb, aligned, x);
#pragma unroll
            for (int j = 0; j < VPT4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float v = f4get(x[j], c);
                    const int idx = elem_index(cb, j, c);
                    if (idx < V && (v > bv || (v == bv && idx < bi))) { bv = v; bi = idx; }
                }
        }
        const int best = block_argmax(bv, bi, sm);
        if (tid == 0) P.row_token[(size_t)b * T + job] = best;
        return;
    } else {

    // ---- sampling: which rows does this job own?
    int v = -1, c0 = -1, di = -1;  // target row, its first child (draft row), lone draft row
    if (tid < kWave) {
        const int lane = tid;
        const int p = (lane < T) ? par_row[lane] : -2;
        if (job < T) {
            const unsigned long long kids = __ballot(lane >= 1 && lane < T && p == job);
            if (lane == 0) {
                int n = 0;
                unsigned long long k = kids;
                while (k) { const int c = __builtin_ctzll(k); kids_s[n++] = c; k &= k - 1; }
                nkids_s = n;
            }
        } else {
            // node i's draft row is read here only when i is not its parent's first child
            const int i = job - T;
            const int pi = __shfl(p, i < T ? i : 0, kWave);
            const bool valid = i >= 1 && pi >= 0 && pi < i;
            const unsigned long long earlier = __ballot(lane >= 1 && lane < i && p == pi);
            if (lane == 0) nkids_s = (valid && earlier != 0ull) ? 0 : -1;
        }
    }
    __syncthreads();
    if (job < T) {
        v = job;
        c0 = nkids_s > 0 ? kids_s[0] : -1;
    } else {
        if (nkids_s < 0) return;   // first child (handled with its parent's row) or invalid
        di = job - T;
    }
    const int nkids = (job < T) ? nkids_s : 0;

    constexpr bool one_chunk = (KIND == 1);
    const float ilog = P.ilog;
    const bool topp = P.top_p < 1.0f;
    const float* zp = (v >= 0) ? P.target + ((size_t)b * T + v) * V : nullptr;
    const int qrow = (v >= 0) ? c0 : di;
    const float* zq = (qrow >= 0) ? P.draft + ((size_t)b * T + qrow) * V : nullptr;
    const bool ap = zp && ((((uintptr_t)zp) & 15) == 0);
    const bool aq = zq && ((((uintptr_t)zq) & 15) == 0);

    float Mp = 0.f, Mq = 0.f;
    double Zp = 1.0, Zq = 1.0;
    Nucleus np{0u, INT_MAX}, nq{0u, INT_MAX};
    float4 ep[VPT4], eq[VPT4];

    if constexpr (one_chunk) {
        // the whole row stays in registers
        if (zp) {
            load_chunk(zp, V, 0, ap, ep);
            Mp = block_max(thread_max(ep), sm);
            double s = 0.0;
#pragma unroll
            for (int j = 0; j < VPT4; ++j) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float e = unnorm(f4get(ep[j], c), Mp, ilog);
                    f4set(ep[j], c, e);
                }
                s += ((double)ep[j].x + (double)ep[j].y) + ((double)ep[j].z + (double)ep[j].w);
            }
            if (topp) {
                np = find_nucleus(ep, 0, V, P.top_p, sm);
                s = 0.0;
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float e = f4get(ep[j], c);
                        if (!in_nucleus(e, elem_index(0, j, c), np)) f4set(ep[j], c, 0.f);
                    }
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
                    s += ((double)ep[j].x + (double)ep[j].y) + ((double)ep[j].z + (double)ep[j].w);
            }
            Zp = block_sum_d(s, sm);
        }
        if (zq) {
            load_chunk(zq, V, 0, aq, eq);
            Mq = block_max(thread_max(eq), sm);
            double s = 0.0;
#pragma unroll
            for (int j = 0; j < VPT4; ++j) {
#pragma unroll
                for (int c = 0; c < 4; ++c) f4set(eq[j], c, unnorm(f4get(eq[j], c), Mq, ilog));
                s += ((double)eq[j].x + (double)eq[j].y) + ((double)eq[j].z + (double)eq[j].w);
            }
            if (topp) {
                nq = find_nucleus(eq, 0, V, P.top_p, sm);
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (!in_nucleus(f4get(eq[j], c), elem_index(0, j, c), nq)) f4set(eq[j], c, 0.f);
                s = 0.0;
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
                    s += ((double)eq[j].x + (double)eq[j].y) + ((double)eq[j].z + (double)eq[j].w);
            }
            Zq = block_sum_d(s, sm);
        }
    } else {
        // streamed rows: online max / sum per thread, merged at the end
        float mp = -INFINITY, mq = -INFINITY;
        double sp = 0.0, sq = 0.0;
        for (int cb = 0; cb < V; cb += CHUNK) {
            if (zp) {
                load_chunk(zp, V, cb, ap, ep);
                const float lm = thread_max(ep);
                if (lm > mp) {
                    if (mp != -INFINITY) sp *= (double)exp2f((mp - lm) * ilog);
                    mp = lm;
                }
                if (mp != -INFINITY)
#pragma unroll
                    for (int j = 0; j < VPT4; ++j)
                        sp += ((double)unnorm(ep[j].x, mp, ilog) + (double)unnorm(ep[j].y, mp, ilog)) +
                              ((double)unnorm(ep[j].z, mp, ilog) + (double)unnorm(ep[j].w, mp, ilog));
            }
            if (zq) {
                load_chunk(zq, V, cb, aq, eq);
                const float lm = thread_max(eq);
                if (lm > mq) {
                    if (mq != -INFINITY) sq *= (double)exp2f((mq - lm) * ilog);
                    mq = lm;
                }
                if (mq != -INFINITY)
#pragma unroll
                    for (int j = 0; j < VPT4; ++j)
                        sq += ((double)unnorm(eq[j].x, mq, ilog) + (double)unnorm(eq[j].y, mq, ilog)) +
                              ((double)unnorm(eq[j].z, mq, ilog) + (double)unnorm(eq[j].w, mq, ilog));
            }
        }
        if (zp) {
            Mp = block_max(mp, sm);
            Zp = block_sum_d(mp == -INFINITY ? 0.0 : sp * (double)exp2f((mp - Mp) * ilog), sm);
        }
        if (zq) {
            Mq = block_max(mq, sm);
            Zq = block_sum_d(mq == -INFINITY ? 0.0 : sq * (double)exp2f((mq - Mq) * ilog), sm);
        }
    }

    // ---- probabilities at the drafted tokens
    if (zp && tid < nkids) {
        const int c = kids_s[tid];
        const int x = tok_row[c];
        float pv = 0.f;
        if (x >= 0 && x < V) {
            const float e = unnorm(zp[x], Mp, ilog);
            if (!topp || in_nucleus(e, x, np)) pv = (float)((double)e / Zp);
        }
        P.node_p[(size_t)b * T + c] = pv;
    }
    if (zq && tid == 0) {
        const int x = tok_row[qrow];
        float qv = 0.f;
        if (x >= 0 && x < V) {
            const float e = unnorm(zq[x], Mq, ilog);
            if (!topp || in_nucleus(e, x, nq)) qv = (float)((double)e / Zq);
        }
        P.node_q[(size_t)b * T + qrow] = qv;
    }
    if (!zp) return;   // lone draft row: done

    // ---- candidate final token of row v
    const float ip = (float)(1.0 / Zp);
    const float iq = (float)(1.0 / Zq);
    const bool resid = (c0 >= 0);
    const double u = (double)P.u_final[b];
    int y = -1;
    if constexpr (one_chunk) {
        bool use_resid = resid;
        if (resid) {  // residual weights overwrite the draft row in place
#pragma unroll
            for (int j = 0; j < VPT4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    f4set(eq[j], c, resid_weight(f4get(ep[j], c), ip, f4get(eq[j], c), iq));
            const double W = chunk_total(eq, sm);
            if (W > 0.0) y = locate_in_chunk(eq, 0, V, 0.0, u * W, sm);
            else use_resid = false;
        }
        if (!use_resid) {
            const double W = chunk_total(ep, sm);
            y = locate_in_chunk(ep, 0, V, 0.0, u * W, sm);
        }
    } else {
        // pass over the chunks for the CDF totals, then re-read the chunk holding the draw
        bool use_resid = resid;
        for (int attempt = 0; attempt < 2; ++attempt) {
            double W = 0.0;
            int ci = 0;
            for (int cb = 0; cb < V; cb += CHUNK, ++ci) {
                load_chunk(zp, V, cb, ap, ep);
                if (use_resid) load_chunk(zq, V, cb, aq, eq);
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float pe = unnorm(f4get(ep[j], c), Mp, ilog);
                        f4set(ep[j], c, use_resid ? resid_weight(pe, ip, unnorm(f4get(eq[j], c), Mq, ilog), iq) : pe);
                    }
                const double S = chunk_total(ep, sm);
                if (tid == 0) sm.chunk_sum[ci] = S;
                W += S;
            }
            __syncthreads();
            if (use_resid && !(W > 0.0)) { use_resid = false; continue; }
            const double target = u * W;
            double cum = 0.0;
            int cstar = -1;
            for (int k = 0; k < ci; ++k) {
                if (cum + sm.chunk_sum[k] > target) { cstar = k; break; }
                cum += sm.chunk_sum[k];
            }
            if (cstar < 0) {  // rounding: last chunk with weight
                for (int k = ci - 1; k >= 0; --k)
                    if (sm.chunk_sum[k] > 0.0) { cstar = k; break; }
                cum = 0.0;
                for (int k = 0; k < cstar; ++k) cum += sm.chunk_sum[k];
            }
            const int cb = cstar * CHUNK;
            load_chunk(zp, V, cb, ap, ep);
            if (use_resid) load_chunk(zq, V, cb, aq, eq);
#pragma unroll
            for (int j = 0; j < VPT4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float pe = unnorm(f4get(ep[j], c), Mp, ilog);
                    f4set(ep[j], c, use_resid ? resid_weight(pe, ip, unnorm(f4get(eq[j], c), Mq, ilog), iq) : pe);
                }
            y = locate_in_chunk(ep, cb, V, cum, target, sm);
            if (y < 0) {
                int last_pos = -1;
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (f4get(ep[j], c) > 0.f) last_pos = max(last_pos, elem_index(cb, j, c));
                y = block_max_int(last_pos, sm);
            }
            break;
        }
    }
    if (tid == 0) P.row_token[(size_t)b * T + v] = y;
    }
}

}  // namespace

hipError_t launch_vocab(const VocabParams& p, hipStream_t s) {
    const int jobs = p.sampling ? 2 * p.T : p.T;
    dim3 grid((unsigned)(p.B * jobs));
    if (!p.sampling) hipLaunchKernelGGL(vocab_kernel<0>, grid, dim3(NT), 0, s, p);
    else if (p.nchunks == 1) hipLaunchKernelGGL(vocab_kernel<1>, grid, dim3(NT), 0, s, p);
    else hipLaunchKernelGGL(vocab_kernel<2>, grid, dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
