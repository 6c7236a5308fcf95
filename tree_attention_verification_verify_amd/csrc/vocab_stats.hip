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
// probability relative to the final max: a 512-thread workgroup per row
// (two per CU) reads a row of up to 32768 logits into registers once, or
// streams a longer row twice, lists the candidates for the cut in LDS and
// cuts by a 3-level radix select on the fp32 bit patterns with exact integer
// masses (significand sums per bucket, see the kernel).

#include "row_block.h"
#include "stats_stream.h"

namespace sv {
namespace {

constexpr int ST = kStatsThreads;

template <bool WITH_Z>
__global__ __launch_bounds__(ST) void row_stats_stream_kernel(StatsParams P) {
    row_stats_stream_block<WITH_Z>(P, blockIdx.x);
}

constexpr int TNW = rows::NW;

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((unsigned long long)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Top-p rows: exact significand sums.
//
// An unnormalised probability e (normal, at most 1) with exponent field E and
// 24-bit significand s equals s * 2^(E - 150).  The radix buckets keep the
// pattern's top bits, so the elements of a bucket share E and the bucket's
// mass is its significand sum times 2^(E - 150): one 64-bit LDS add of s per
// element, exact for any row length.
//
// Level 1 buckets are pattern bits 29..20 (seven exponent bits, three
// significand bits), in windows of 13 exponents (104 buckets, 8 copies by
// lane & 7, which spreads the adds of one instruction over different
// addresses).  Window 0 holds the candidates, e >= 2^-12: the pass that
// computes the probabilities lists them in LDS (each wave in its own
// segment, no atomics) and sums the others per thread (fp32 within a float4,
// fp64 across them, in a fixed order).  The cut lies among the candidates
// whenever top_p times the row total is at most their mass; at the batch-32
// chain shape the list holds about 5% of a row, and level 1 and the search
// inside the crossing bucket (a ranking of its elements when at most 64,
// else levels 2 and 3) read it instead of the row.  A row whose cut lies
// lower (a flat distribution, or top_p close to 1) takes the next windows
// down, one pass over the row each, until one holds the crossing; a wave
// whose segment overflowed (a flat row) sends the levels to the row as well.
// Each level-1 bucket is converted to units of 2^-48 (exact for E >= 102; a
// bucket of e < 2^-25 is rounded to the nearest unit, below 2^-49 of the
// largest probability; the row total stays below 2^63).  Inside the crossing
// bucket masses are counted in significand units; the nucleus normaliser is
// assembled from the two parts in fp64.
//
// A row of up to rows::CHUNK logits is loaded into registers once (its
// maximum, then its probabilities, from the same registers); a longer row is
// streamed, once for the maximum and once for the probabilities.  Either way
// the row's registers are free once the list is written, which keeps a
// 512-thread row within 128 VGPRs: two rows share a CU, one row's loads and
// barriers overlapping the other's arithmetic.
constexpr int kMassUnitsLog2 = 48;                  // level-1 scan units: 2^-48
constexpr int kExactExp = 150 - kMassUnitsLog2;     // smallest exponent field converted exactly
constexpr uint32_t kCandBits = 115u << 23;          // 2^-12: smallest candidate
constexpr int kWinExps = 13;                        // exponents per level-1 window
constexpr int kWinBuckets = 8 * kWinExps;           // 104
constexpr int kWin0Lo = 8 * (127 - kWinExps + 1);   // smallest level-1 bucket of window 0
constexpr int kH1Copies = 8;
constexpr int kTopBucket = 1016;                    // level-1 bucket of 1.0 (exponent 127)
constexpr int kCandListCap = 8192;                  // listed candidates per row
constexpr int kToppThreads = 512;                   // threads per top-p row
constexpr int kFewB1 = kWave;                       // largest crossing bucket ranked without levels 2 and 3 (a lane per element)

__device__ __forceinline__ uint32_t significand(uint32_t bits) { return (bits & 0x7FFFFFu) | 0x800000u; }

// Level-1 bucket k (exponent field k >> 3) with significand sum h, in 2^-48 units.
__device__ __forceinline__ unsigned long long bucket_units(unsigned long long h, int k) {
    const int sh = (k >> 3) - kExactExp;
    if (sh >= 0) return h << sh;
    if (sh < -40) return 0ull;   // h < 2^40: rounds to 0
    return (h + (1ull << (-sh - 1))) >> -sh;
}

// Maximum of three floats by v_max3_f32 (quiet NaNs are ignored; the
// operands need no quieting first, unlike fmaxf on values loaded from memory).
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Wave maximum / minimum in every lane, by DPP row shifts and broadcasts
// (lanes without a source keep their own value), then lane 63.
__device__ __forceinline__ float wave_max_dpp(float v) {
#define SV_MAXSTEP(CTRL, ROWS) v = max3_f32(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp( \
        __builtin_bit_cast(int, v), __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, false)), v)
    SV_MAXSTEP(0x111, 0xf); SV_MAXSTEP(0x112, 0xf); SV_MAXSTEP(0x114, 0xf); SV_MAXSTEP(0x118, 0xf);
    SV_MAXSTEP(0x142, 0xa); SV_MAXSTEP(0x143, 0xc);
#undef SV_MAXSTEP
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
}
__device__ __forceinline__ int wave_min_dpp(int v) {
#define SV_MINSTEP(CTRL, ROWS) v = min(v, __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false))
    SV_MINSTEP(0x111, 0xf); SV_MINSTEP(0x112, 0xf); SV_MINSTEP(0x114, 0xf); SV_MINSTEP(0x118, 0xf);
    SV_MINSTEP(0x142, 0xa); SV_MINSTEP(0x143, 0xc);
#undef SV_MINSTEP
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

struct NucleusSmem {
    unsigned long long h1[kWinBuckets][kH1Copies];   // level 1, one window: significand sums
    unsigned long long h2[1024];                     // level 2: significand sums
    uint32_t h3[1024];                               // level 3: counts
    unsigned long long wt[4][TNW];
    double wtail[TNW];                               // per wave: fp64 mass of the elements below the candidates
    unsigned long long sel_above[4];
    unsigned long long sel_mass[4];
    int sel_bucket[4];
    int sel_found[4];
    double needv;
    unsigned long long win_total;
    float wmax[TNW];
    int wbest[TNW];
    unsigned long long cnt[2][TNW];
    int overflow;                                    // some wave's list segment overflowed
    uint32_t few[TNW][kFewB1];                       // per wave: its elements in the crossing bucket
    uint32_t nfew[TNW];
    uint32_t few_thr;
    unsigned long long few_above, few_at;
};

// Significand sum of bucket i of the level-1 window whose smallest bucket is
// k_lo.  Buckets of exponent 0 (zeros, subnormals) and above the bucket of
// 1.0 (non-numbers) carry no mass.
__device__ __forceinline__ unsigned long long win_significands(const NucleusSmem& sm, int k_lo, int i) {
    const int k = k_lo + i;
    if (k < 8 || k > kTopBucket) return 0ull;
    unsigned long long s = 0;
#pragma unroll
    for (int c = 0; c < kH1Copies; ++c) s += sm.h1[i][c];
    return s;
}

// Crossing bucket of one level (selection slot S) among NB buckets, bucket
// j = 0 the largest: the bucket where the mass counted from the top, starting
// at `above`, first reaches need; without one (need outside (above, above +
// total]) sel_found[S] = 0 and bucket NB - 1.  units(j) is bucket j's mass.
// With TOTAL need becomes top_p times (total + extra()), extra() being mass
// outside the buckets in the same units (evaluated after the first barrier);
// the total lands in win_total.  Thread t holds buckets K t .. K t + K - 1.
// Returns need, the same in every thread.
template <int S, int NB, bool TOTAL, int TPB, class U, class X>
__device__ __forceinline__ double nucleus_scan(double need, unsigned long long above, float top_p, NucleusSmem& sm,
                                               U&& units, X&& extra) {
    constexpr int K = (NB + TPB - 1) / TPB;
    constexpr int NTS = (NB + K - 1) / K;
    constexpr int NWS = (NTS + kWave - 1) / kWave;
    static_assert(NWS <= TNW, "one scan slot per wave");
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool scanner = tid < NWS * kWave;
    unsigned long long x[K], mine = 0, incl = 0;
    __syncthreads();
    if (scanner) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            x[k] = K * tid + k < NB ? units(K * tid + k) : 0ull;
            mine += x[k];
        }
        incl = wave_scan_u64(mine);
        if (NWS > 1 && lane == kWave - 1) sm.wt[S][wave] = incl;
    }
    if (NWS > 1) __syncthreads();
    if (scanner) {
        unsigned long long total;
        if (NWS > 1) {
            const unsigned long long wsc = wave_scan_u64(lane < NWS ? sm.wt[S][lane] : 0ull);
            const int wv = __builtin_amdgcn_readfirstlane(wave);
            total = readlane_u64(wsc, NWS - 1);
            incl += wv > 0 ? readlane_u64(wsc, wv - 1) : 0ull;
        } else {
            total = readlane_u64(incl, kWave - 1);
        }
        incl += above;
        if (TOTAL) {
            need = (double)top_p * ((double)total + extra());
            if (tid == 0) {
                sm.needv = need;
                sm.win_total = total;
            }
        }
        // the integer bounds, as doubles, tile (above, above + total] without
        // gaps: at most one bucket holds need
        const bool exists = (double)above < need && need <= (double)(above + total);
        unsigned long long lo = incl - mine;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int j = K * tid + k;
            const unsigned long long hi = lo + x[k];
            if (j < NB && (exists ? ((double)lo < need && need <= (double)hi) : j == NB - 1)) {
                sm.sel_bucket[S] = j;
                sm.sel_above[S] = lo;
                sm.sel_mass[S] = x[k];
                sm.sel_found[S] = exists ? 1 : 0;
            }
            lo = hi;
        }
        if (!TOTAL && tid == 0) sm.win_total = total;
    }
    __syncthreads();
    return TOTAL ? sm.needv : need;
}

// One row per workgroup of TPB threads.  RESIDENT: the row (V <= rows::CHUNK)
// is loaded into registers once; otherwise it is streamed in blocks of
// 4 * HB * TPB ids, the next block's loads in flight.  Rarer cases read the
// row again: a cut below the candidates (one pass per lower window, then
// levels 2 and 3 from the row), an overflowed list (level 1 and levels 2 and
// 3 from the row), and tied probabilities straddling the cut (a pass counting
// the ties per chunk of rows::CHUNK ids when the row has several, then a
// bisection on the token id inside the chunk holding the k-th tie).  The
// launch bounds ask for two workgroups per CU.
template <int TPB, bool RESIDENT>
__global__ __launch_bounds__(TPB, 2 * TPB / (4 * kWave)) void row_stats_topp_kernel(StatsParams P) {
    using namespace rows;
    constexpr int NWB = TPB / kWave;
    constexpr int N4 = CHUNK / (4 * TPB);       // float4 per thread holding a chunk
    constexpr int HB = 4;                       // float4 per thread per streamed block
    constexpr int SEG = kCandListCap / NWB;     // list entries per wave
    static_assert(NWB <= TNW && N4 * 4 * TPB == CHUNK, "workgroup shape");
    __shared__ NucleusSmem sm;
    __shared__ uint32_t clist[kCandListCap];    // candidate patterns, a segment per wave
    __shared__ int chunk_ties[MAX_CHUNKS];
    const int nrows = 2 * P.T;
    const int b = blockIdx.x / nrows, r = blockIdx.x - b * nrows;
    const float* row = row_ptr(P, b, r);
    if (!row) return;
    const int V = P.V;
    const float ilog = P.ilog;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool aligned = (((uintptr_t)row) & 15) == 0;
    auto clear_h1 = [&]() {
        for (int k = tid; k < kWinBuckets * kH1Copies; k += TPB) (&sm.h1[0][0])[k] = 0ull;
    };
    // cleared histograms and counts are ordered before their atomics by a later barrier
    auto clear_all = [&]() {
        clear_h1();
        for (int k = tid; k < 1024; k += TPB) {
            sm.h2[k] = 0ull;
            sm.h3[k] = 0u;
        }
        if (tid < MAX_CHUNKS) chunk_ties[tid] = 0;
        if (tid == 0) sm.overflow = 0;
    };

    // the probabilities of one float4: candidates into this wave's list
    // segment (a slot's candidates together, positions from the ballot), the
    // others into the thread's fp64 tail sum.  While the segment has room for
    // five more full slots every lane stores without a branch: a lane without
    // a candidate writes past the slot's last listed entry (a position that
    // a later candidate, stored after it, overwrites, or that is never read),
    // so the logits of a float4 do not wait on each other's control flow.
    uint32_t* const seg = clist + __builtin_amdgcn_readfirstlane(wave) * SEG;
    uint32_t nseg = 0;   // the same in every lane of the wave
    double tail = 0.0;
    auto take4 = [&](const float (&v)[4]) {
        float t4[4];
        auto list = [&](bool checked) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t bits = __float_as_uint(v[c]);
                const bool cand = bits >= kCandBits;
                t4[c] = cand ? 0.f : v[c];
                const unsigned long long mask = __ballot(cand);
                // position among this slot's candidates; the slot's entries
                // start at the (wave-uniform) end of the list
                const uint32_t own = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                const uint32_t cnt = (uint32_t)__popcll(mask);
                if (!checked) {
                    (seg + nseg)[cand ? own : cnt + (uint32_t)lane] = bits;
                } else if (cand && nseg + own < (uint32_t)SEG) {
                    seg[nseg + own] = bits;
                }
                nseg += cnt;
            }
        };
        if (nseg + 5u * kWave <= (uint32_t)SEG) list(false);
        else list(true);
        tail += (double)((t4[0] + t4[1]) + (t4[2] + t4[3]));
        // added where it is made (left to itself the compiler makes every
        // term first and holds them all)
        asm volatile("" : "+v"(tail));
    };

    float M;
    if constexpr (RESIDENT) {
        float4 e[N4];
        issue_chunk<N4, TPB>(row, V, 0, aligned, e);
        clear_all();
        // entries past the row end (read as 0) become -inf; only slots that
        // reach V need the test
#pragma unroll
        for (int j = 0; j < N4; ++j)
            if (4 * TPB * (j + 1) > V)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (elem_index<TPB>(0, j, c) >= V) f4set(e[j], c, -INFINITY);
        // largest logit: thread maximum (two logits per max3), wave, block
        float bv = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4 * N4; k += 2) bv = max3_f32(bv, f4get(e[k / 4], k % 4), f4get(e[k / 4], k % 4 + 1));
        const float wm = wave_max_dpp(bv);
        if (lane == 0) sm.wmax[wave] = wm;
        __syncthreads();
        M = sm.wmax[0];
#pragma unroll
        for (int w = 1; w < NWB; ++w) M = fmaxf(M, sm.wmax[w]);
        // its smallest id: only threads holding M look for their first position
        int bi = INT_MAX;
        if (bv == M) {
#pragma unroll
            for (int j = N4 - 1; j >= 0; --j)
#pragma unroll
                for (int c = 3; c >= 0; --c) {
                    const int idx = elem_index<TPB>(0, j, c);
                    bi = (f4get(e[j], c) == M && idx < V) ? idx : bi;
                }
        }
        bi = wave_min_dpp(bi);
        if (lane == 0) sm.wbest[wave] = bi;   // read after later barriers
#pragma unroll
        for (int j = 0; j < N4; ++j) {
            const float v[4] = {unnorm(e[j].x, M, ilog), unnorm(e[j].y, M, ilog), unnorm(e[j].z, M, ilog),
                                unnorm(e[j].w, M, ilog)};
            take4(v);
        }
    } else {
        clear_all();
        // pass 1: the largest logit and its smallest id: per block the
        // thread's maximum and the first of its positions holding it; blocks
        // come in id order
        float bv = -INFINITY;
        int bi = INT_MAX;
        for_each_chunk<HB, TPB>(row, V, aligned, [&](float4 (&x)[HB], int cb) {
            float m = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4 * HB; k += 2) m = max3_f32(m, f4get(x[k / 4], k % 4), f4get(x[k / 4], k % 4 + 1));
            if (m > bv) {   // the first position holding m has the smallest id of this block
                int loc = INT_MAX;
#pragma unroll
                for (int j = HB - 1; j >= 0; --j)
#pragma unroll
                    for (int c = 3; c >= 0; --c) {
                        const int idx = elem_index<TPB>(cb, j, c);
                        loc = (f4get(x[j], c) == m && idx < V) ? idx : loc;
                    }
                bv = m;
                bi = loc;
            }
        });
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) argmax_step(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
        if (lane == 0) {
            sm.wmax[wave] = bv;
            sm.wbest[wave] = bi;
        }
        __syncthreads();
        M = sm.wmax[0];
#pragma unroll
        for (int w = 1; w < NWB; ++w) M = fmaxf(M, sm.wmax[w]);
        // pass 2: the probabilities
        for_each_chunk<HB, TPB>(row, V, aligned, [&](float4 (&x)[HB], int) {
#pragma unroll
            for (int j = 0; j < HB; ++j) {
                const float v[4] = {unnorm(x[j].x, M, ilog), unnorm(x[j].y, M, ilog), unnorm(x[j].z, M, ilog),
                                    unnorm(x[j].w, M, ilog)};
                take4(v);
            }
        });
    }
    {
        const double wtl = wave_sum_d(tail);
        if (lane == 0) {
            sm.wtail[wave] = wtl;   // read after the scan's first barrier
            if (nseg > (uint32_t)SEG) sm.overflow = 1;
        }
    }
    // f(e) for every probability of the row, read again
    auto each_prob = [&](auto&& f) {
        for_each_chunk<HB, TPB>(row, V, aligned, [&](float4 (&x)[HB], int) {
#pragma unroll
            for (int j = 0; j < HB; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) f(__float_as_uint(unnorm(f4get(x[j], c), M, ilog)));
        });
    };
    unsigned long long* const h1c = &sm.h1[0][lane & (kH1Copies - 1)];
    auto h1_add = [&](uint32_t i, uint32_t bits) { atomicAdd(h1c + i * kH1Copies, (unsigned long long)significand(bits)); };
    // window 0 (non-numbers in its last bucket, which carries no mass)
    auto win0_add = [&](uint32_t bits) { h1_add(min((bits >> 20) - (uint32_t)kWin0Lo, (uint32_t)kWinBuckets - 1), bits); };
    // each wave adds its listed candidates at once; if some wave's list
    // overflowed, window 0 is cleared and taken from the row instead
    if (nseg <= (uint32_t)SEG)
        for (uint32_t i = (uint32_t)lane; i < nseg; i += kWave) win0_add(seg[i]);
    __syncthreads();
    const bool listed = sm.overflow == 0;   // every candidate is in the list
    if (!listed) {
        clear_h1();
        __syncthreads();
        each_prob([&](uint32_t bits) {
            if (bits >= kCandBits) win0_add(bits);
        });
    }
    // scan index t = nb - 1 - i: the largest bucket first
    int k_lo = kWin0Lo;      // the window's smallest bucket
    int nb = kWinBuckets;    // and its bucket count
    auto win_units = [&](int t) -> unsigned long long {
        const int i = nb - 1 - t;
        return i >= 0 ? bucket_units(win_significands(sm, k_lo, i), k_lo + i) : 0ull;
    };
    const double need = nucleus_scan<0, kWinBuckets, true, TPB>(0.0, 0ull, P.top_p, sm, win_units, [&]() {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < NWB; ++w) t += sm.wtail[w];
        return ldexp(t, kMassUnitsLog2);
    });
    unsigned long long above = 0ull;   // mass of the windows above the current one (2^-48 units)
    int found = sm.sel_found[0];
    const bool from_list = listed && found;   // the crossing bucket's elements are listed
    // the cut lies below the candidates: windows further down, one pass each,
    // until one holds the crossing
    for (int E_hi = 127 - kWinExps; !found && need > 0.0 && E_hi >= 1; E_hi -= kWinExps) {
        above += sm.win_total;
        const int E_lo = max(1, E_hi - kWinExps + 1);
        k_lo = 8 * E_lo;
        nb = 8 * (E_hi - E_lo + 1);
        __syncthreads();   // every thread has read the previous window
        clear_h1();
        __syncthreads();
        each_prob([&](uint32_t bits) {
            const uint32_t i = (bits >> 20) - (uint32_t)k_lo;
            if (i < (uint32_t)nb) h1_add(i, bits);
        });
        nucleus_scan<0, kWinBuckets, false, TPB>(need, above, P.top_p, sm, win_units, []() { return 0.0; });
        found = sm.sel_found[0];
    }
    // b1: the crossing level-1 bucket; a1: the mass above it (2^-48 units);
    // without a crossing every nonzero mass is kept
    int b1 = 0;
    unsigned long long a1 = above + sm.win_total, h_b1 = 0ull;
    if (found) {
        const int i = nb - 1 - sm.sel_bucket[0];
        b1 = k_lo + i;
        a1 = sm.sel_above[0];
        h_b1 = win_significands(sm, k_lo, i);
    }
    const int E1 = b1 >> 3;
    // what is left to reach, in significand units of bucket b1 (the level-1
    // conversion of a bucket below 2^-25 rounded: clamp to the bucket's sum)
    double need1 = 0.0;
    if (found && need > 0.0) need1 = fmin(ldexp(need - (double)a1, kExactExp - E1), (double)h_b1);
    // A bucket that carries mass has an exponent field of 1..127 and lies at
    // or below bucket 1016, so matching its pattern bits implies carrying mass.
    const uint32_t b1m = found ? (uint32_t)b1 : 0xFFFFFFFFu;
    // elements whose pattern >> pshift equals prefix go through f: each wave
    // its list segment, or the row read again
    auto each_in = [&](int pshift, uint32_t prefix, auto&& f) {
        if (from_list) {
            for (uint32_t i = (uint32_t)lane; i < nseg; i += kWave) {
                const uint32_t bits = seg[i];
                if ((bits >> pshift) == prefix) f(bits);
            }
        } else {
            each_prob([&](uint32_t bits) {
                if ((bits >> pshift) == prefix) f(bits);
            });
        }
    };
    // thr: the pattern where the mass counted from the top reaches need;
    // inside b1 the mass of the patterns above thr and of all elements at thr
    // (significand units)
    uint32_t thr = 0u;
    unsigned long long above_thr = 0ull, at_thr = 0ull;
    // a listed crossing bucket of at most kFewB1 elements (the usual case: a
    // bucket spans a factor of 2^(1/8)): each wave copies its elements there
    // to a short list; then every wave holds them a lane each, compares them
    // with its share of the others broadcast in turn, and one wave adds the
    // shares up to each element's mass interval in the order of decreasing
    // pattern (ties in list order; the intervals tile (0, h_b1] as the
    // buckets of the radix levels do)
    bool few = false;
    if (from_list) {
        uint32_t nb = 0;
        for (uint32_t i0 = 0; i0 < nseg; i0 += kWave) {
            const uint32_t i = i0 + (uint32_t)lane;
            const uint32_t bits = i < nseg ? seg[i] : 0u;
            const bool m = i < nseg && (bits >> 20) == b1m;
            const unsigned long long mask = __ballot(m);
            if (m) {
                const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)mask, nb));
                if (pos < (uint32_t)kFewB1) sm.few[wave][pos] = bits;
            }
            nb += (uint32_t)__popcll(mask);
        }
        if (lane == 0) sm.nfew[wave] = nb;
        __syncthreads();
        uint32_t tot = 0;
#pragma unroll
        for (int w = 0; w < NWB; ++w) tot += sm.nfew[w];
        few = tot <= (uint32_t)kFewB1;
    }
    if (few) {
        // every wave: lane i holds element i of the waves' lists in order
        uint32_t key = 0u, n = 0;
#pragma unroll
        for (int w = 0; w < NWB; ++w) {
            const uint32_t nw = sm.nfew[w];
            if ((uint32_t)lane >= n && (uint32_t)lane < n + nw) key = sm.few[w][lane - n];
            n += nw;
        }
        // this wave's share of the other elements (j = wave, wave + NWB, ...):
        // gt, the mass of greater patterns; upto, that plus the ties up to
        // and including this element (list order).  Partial sums in the
        // level-2 histogram's storage, which this path does not use.
        static_assert(2 * NWB * kWave <= 1024, "partial sums");
        unsigned long long gt = 0ull, upto = 0ull;
        for (uint32_t j = (uint32_t)wave; j < n; j += NWB) {
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, (int)j);
            const unsigned long long sj = significand(kj);
            if (kj > key) gt += sj;
            if (kj > key || (kj == key && j <= (uint32_t)lane)) upto += sj;
        }
        sm.h2[wave * kWave + lane] = gt;
        sm.h2[(NWB + wave) * kWave + lane] = upto;
        __syncthreads();
        if (wave == 0) {
            gt = 0ull;
            upto = 0ull;
#pragma unroll
            for (int w = 0; w < NWB; ++w) {
                gt += sm.h2[w * kWave + lane];
                upto += sm.h2[(NWB + w) * kWave + lane];
            }
            const bool valid = (uint32_t)lane < n;
            const unsigned long long own = valid ? (unsigned long long)significand(key) : 0ull;
            unsigned long long cross = __ballot(valid && (double)(upto - own) < need1 && need1 <= (double)upto);
            if (!cross) cross = __ballot(valid && upto == h_b1);   // need1 clamped to the bucket's mass
            const int jx = cross ? __builtin_ctzll(cross) : 0;
            const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)key, jx);
            const unsigned long long nt = (unsigned long long)__popcll(__ballot(valid && key == t));
            const unsigned long long g = readlane_u64(gt, jx);
            if (lane == 0) {
                sm.few_thr = t;
                sm.few_at = nt * significand(t);
                sm.few_above = g;
            }
        }
        __syncthreads();
        thr = sm.few_thr;
        above_thr = sm.few_above;
        at_thr = sm.few_at;
    } else {
        // level 2: significand sums of pattern bits 19..10
        each_in(20, b1m, [&](uint32_t bits) { atomicAdd(&sm.h2[(bits >> 10) & 1023u], (unsigned long long)significand(bits)); });
        nucleus_scan<1, 1024, false, TPB>(need1, 0ull, P.top_p, sm, [&](int t) { return sm.h2[1023 - t]; },
                                          []() { return 0.0; });
        const uint32_t b2 = 1023u - (uint32_t)sm.sel_bucket[1];
        const unsigned long long a2 = sm.sel_above[1];
        double need2 = 0.0;
        if (need1 > 0.0) need2 = fmin(need1 - (double)a2, (double)sm.sel_mass[1]);
        // level 3: counts of the exact patterns
        const uint32_t one = 1u;
        const uint32_t p3 = found ? (((uint32_t)b1 << 10) | b2) : 0xFFFFFFFFu;
        each_in(10, p3, [&](uint32_t bits) { atomicAdd(&sm.h3[bits & 1023u], one); });
        nucleus_scan<2, 1024, false, TPB>(need2, 0ull, P.top_p, sm, [&](int t) -> unsigned long long {
            const uint32_t k3 = 1023u - (uint32_t)t;
            return (unsigned long long)sm.h3[k3] * significand((((uint32_t)b1 << 10 | b2) << 10) | k3);
        }, []() { return 0.0; });
        if (found) {
            thr = (((uint32_t)b1 << 10 | b2) << 10) | (1023u - (uint32_t)sm.sel_bucket[2]);
            above_thr = a2 + sm.sel_above[2];
            at_thr = sm.sel_mass[2];
        }
    }
    Nucleus nu;
    nu.thr = thr;
    nu.cutoff = INT_MAX;
    // the kept mass at thr: all of it, or k of the tied elements
    unsigned long long kept = at_thr;
    const unsigned long long tie_mass = found ? significand(thr) : 0ull;
    if (tie_mass > 0 && kept > 0) {
        const unsigned long long ties = kept / tie_mass;
        long long k = (long long)ceil((need1 - (double)above_thr) / (double)tie_mass);
        if (k < 1) k = 1;
        if (ties > 1 && (unsigned long long)k < ties) {
            // ties straddle the cut: the smallest cutoff c with #ties(id < c)
            // >= k, by bisection on the token id inside the chunk holding the
            // k-th tie (ties per chunk first when the row has several; block
            // counts in alternating buffers); exactly k ties then lie below
            const int nchunks = (V + CHUNK - 1) / CHUNK;
            long long before = 0;
            int cstar = 0;
            if (nchunks > 1) {
                for_each_chunk<HB, TPB>(row, V, aligned, [&](float4 (&x)[HB], int cb) {
                    unsigned long long cnt = 0;
#pragma unroll
                    for (int j = 0; j < HB; ++j)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (elem_index<TPB>(cb, j, c) < V && __float_as_uint(unnorm(f4get(x[j], c), M, ilog)) == nu.thr)
                                ++cnt;
                    cnt = wave_sum_u64(cnt);
                    if (lane == 0) atomicAdd(&chunk_ties[cb / CHUNK], (int)cnt);
                });
                __syncthreads();
                cstar = nchunks - 1;
                for (int c = 0; c < nchunks; ++c) {
                    if (before + chunk_ties[c] >= k) { cstar = c; break; }
                    before += chunk_ties[c];
                }
            }
            // the thread's ties in the chunk as a mask over its elements in
            // id order (slot j, component c: bit 4 j + c); the elements with
            // id <= mid are a prefix of that order
            static_assert(4 * N4 <= 64, "tie mask");
            const int cb = cstar * CHUNK;
            unsigned long long tmask = 0ull;
            {
                float4 e[N4];
                load_chunk<N4, TPB>(row, V, cb, aligned, e);
#pragma unroll
                for (int j = 0; j < N4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (__float_as_uint(unnorm(f4get(e[j], c), M, ilog)) == nu.thr && elem_index<TPB>(cb, j, c) < V)
                            tmask |= 1ull << (4 * j + c);
            }
            const int first = cb + 4 * tid;   // id of the thread's element 0
            int lo = cb, hi = min(V, cb + CHUNK) - 1, par = 0;
            while (lo < hi) {
                const int mid = lo + (hi - lo) / 2;
                const int d = mid - first;
                const int n_le = d < 0 ? 0 : min(4 * N4, 4 * (d / (4 * TPB)) + min(d % (4 * TPB), 3) + 1);
                const unsigned long long below = n_le >= 64 ? ~0ull : ((1ull << n_le) - 1ull);
                const unsigned long long cnt = wave_sum_u64((unsigned long long)__popcll(tmask & below));
                if (lane == 0) sm.cnt[par][wave] = cnt;
                __syncthreads();
                unsigned long long tot = (unsigned long long)before;
#pragma unroll
                for (int w = 0; w < NWB; ++w) tot += sm.cnt[par][w];
                par ^= 1;
                if (tot >= (unsigned long long)k) hi = mid; else lo = mid + 1;
            }
            nu.cutoff = lo + 1;
            kept = (unsigned long long)k * tie_mass;
        }
    }
    if (tid == 0) {
        // the smallest id holding the maximum, over the waves whose own
        // maximum it is
        int best = INT_MAX;
#pragma unroll
        for (int w = 0; w < NWB; ++w)
            if (sm.wmax[w] == M) best = min(best, sm.wbest[w]);
        // normaliser of the nucleus: the buckets above b1 (2^-48 units) and
        // the kept part of b1 (significand units, 2^(E1 - 150) each)
        const unsigned long long in_b1 = found ? above_thr + kept : 0ull;
        RowStat st;
        st.zmax = M;
        st.argmax = best;
        st.thr = nu.thr;
        st.cutoff = nu.cutoff;
        st.Z = ldexp((double)a1, -kMassUnitsLog2) + ldexp((double)in_b1, E1 - 150);
        P.stats[(size_t)b * nrows + r] = st;
    }
}

// Debug output: the effective target distribution of every row, p =
// TopP(softmax(z / temperature)), from the row's statistics (same weight,
// nucleus test and fp64 division as the probability the acceptance test
// reads, so probs[b, parent(i), x_i] equals node_p[b, i] bit for bit).  One
// workgroup per (row, slice of kProbSlice ids); consecutive lanes write
// consecutive ids.  HBM-bound: reads and writes 4 bytes per logit.
constexpr int kProbSlice = ST * 8;

__global__ __launch_bounds__(ST) void write_probs_kernel(StatsParams P, float* probs) {
    const int row = blockIdx.x;                 // b * T + i
    const int b = row / P.T, i = row - b * P.T;
    const RowStat st = P.stats[(size_t)b * 2 * P.T + i];
    const rows::Nucleus nu{st.thr, st.cutoff};
    const float* z = P.target + (size_t)row * P.V;
    float* out = probs + (size_t)row * P.V;
    const int first = blockIdx.y * kProbSlice + threadIdx.x;
#pragma unroll
    for (int j = 0; j < kProbSlice / ST; ++j) {
        const int k = first + j * ST;
        if (k < P.V) {
            const float e = rows::unnorm(z[k], st.zmax, P.ilog);
            out[k] = rows::in_nucleus(e, k, nu) ? (float)((double)e / st.Z) : 0.f;
        }
    }
}

}  // namespace

namespace {
// Which row-statistics kernel a launch takes: with top-p (sampling mode) the
// cut needs the row in registers (up to rows::CHUNK ids) or streamed twice;
// otherwise one streaming read.
enum StatsKind { kStatsTopp, kStatsToppChunked, kStatsStream };
StatsKind stats_kind(const StatsParams& p) {
    if (p.sampling && p.top_p < 1.f) return p.V <= rows::CHUNK ? kStatsTopp : kStatsToppChunked;
    return kStatsStream;
}
}  // namespace

bool row_stats_streams(const StatsParams& p) { return stats_kind(p) == kStatsStream; }

const char* row_stats_kernel_name(const StatsParams& p) {
    switch (stats_kind(p)) {
    case kStatsTopp:
    case kStatsToppChunked: return "row_stats_topp_kernel";
    default: return "row_stats_stream_kernel";
    }
}

hipError_t launch_row_stats(const StatsParams& p, hipStream_t s) {
    const int nrows = p.sampling ? 2 * p.T : p.T;
    dim3 grid((unsigned)(p.B * nrows));
    switch (stats_kind(p)) {
    case kStatsTopp:
        hipLaunchKernelGGL((row_stats_topp_kernel<kToppThreads, true>), grid, dim3(kToppThreads), 0, s, p);
        break;
    case kStatsToppChunked:
        hipLaunchKernelGGL((row_stats_topp_kernel<kToppThreads, false>), grid, dim3(kToppThreads), 0, s, p);
        break;
    default:
        if (p.sampling) hipLaunchKernelGGL(row_stats_stream_kernel<true>, grid, dim3(ST), 0, s, p);
        else hipLaunchKernelGGL(row_stats_stream_kernel<false>, grid, dim3(ST), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace sv

namespace sv {

hipError_t launch_write_probs(const StatsParams& p, float* probs, hipStream_t s) {
    const dim3 grid((unsigned)(p.B * p.T), (unsigned)((p.V + kProbSlice - 1) / kProbSlice));
    hipLaunchKernelGGL(write_probs_kernel, grid, dim3(ST), 0, s, p, probs);
    return hipGetLastError();
}

}  // namespace sv
