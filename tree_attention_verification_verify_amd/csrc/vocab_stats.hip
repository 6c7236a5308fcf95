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
// probability relative to the final max: a row of up to 32768 logits is held
// in the registers of a 1024-thread workgroup and cut by a 3-level radix
// select on the fp32 bit patterns with exact integer masses (significand sums
// per bucket, see the kernel); a longer row is streamed twice, its candidates
// for the cut listed on chip.

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
// Top-p rows held on chip (V <= 32768): exact significand sums.
//
// A kept-mass candidate e (an unnormalised probability: normal, at most 1)
// with exponent field E and 24-bit significand s equals s * 2^(E - 150).  The
// radix buckets keep the pattern's top bits, so every element of a bucket
// shares the bits above it: a bucket's significand sum follows exactly from
// its element count n and the sum of its patterns modulo 2^32, as long as
// the bits below the bucket's prefix add up to less than 2^32.  Every LDS
// atomic is therefore a 32-bit add (count, pattern), and the probabilities
// stay in their registers (no 64-bit operand pairs): with at most 64 VGPRs a
// CU holds two rows at once, so one row's loads overlap another's cut and
// 352 rows of 32000 logits run in one wave of workgroups.
//
// Level 1 buckets are pattern bits 29..20 (seven exponent bits, three
// significand bits), in windows of 13 exponents (104 buckets, 8 copies by
// lane & 7 so that each copy holds at most V/8 = 4096 elements and its
// low-20-bit sum stays below 2^32).  Window 0 holds the candidates, e >=
// 2^-12; the others are summed per thread (fp32 within a float4, fp64 across
// them, in a fixed order) and the cut lies among the candidates whenever
// top_p times the row total is at most their mass.  At the batch-32 chain
// shape that leaves about 5% of the logits for the atomics.  A row whose cut
// lies lower (a flat distribution, or top_p close to 1) takes the next
// windows down, one register pass each, until one holds the crossing.  Each
// level-1 bucket is converted to units of 2^-48 (exact for E >= 102; a bucket
// of e < 2^-25 is rounded to the nearest unit, below 2^-49 of the largest
// probability; the row total stays below 2^63).  Levels 2 and 3 lie inside
// the crossing bucket and count significand units; the nucleus normaliser is
// assembled from the two parts in fp64.
constexpr int kMassUnitsLog2 = 48;                  // level-1 scan units: 2^-48
constexpr int kExactExp = 150 - kMassUnitsLog2;     // smallest exponent field converted exactly
constexpr uint32_t kCandBits = 115u << 23;          // 2^-12: smallest candidate
constexpr int kWinExps = 13;                        // exponents per level-1 window
constexpr int kWinBuckets = 8 * kWinExps;           // 104
constexpr int kH1Copies = 8;
constexpr int kTopBucket = 1016;                    // level-1 bucket of 1.0 (exponent 127)
constexpr int kNListCap = 128;                      // per-wave list of the crossing bucket's elements

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
    uint32_t h1[kWinBuckets][kH1Copies][2];   // level 1, one window: (count, pattern sum mod 2^32)
    uint32_t h2[1024][2];                     // level 2: (count, pattern sum mod 2^32)
    uint32_t h3[1024];                        // level 3: counts
    unsigned long long wt[4][TNW];
    double wtail[TNW];                        // per wave: fp64 mass of the elements below the candidates
    unsigned long long sel_above[4];
    unsigned long long sel_mass[4];
    int sel_bucket[4];
    int sel_found[4];
    double needv;
    unsigned long long win_total;
    float wmax[TNW];
    int wbest[TNW];
    unsigned long long cnt[2][TNW];
    uint32_t list[TNW * kNListCap];           // per wave: patterns of its elements in the level-1 crossing bucket
};

// Significand sum of bucket i of the level-1 window whose smallest bucket is
// k_lo: each copy's low 20 bits from its count and pattern sum (below 2^32:
// at most 4096 elements per copy).  Buckets of exponent 0 (zeros,
// subnormals) and above the bucket of 1.0 (non-numbers) carry no mass.
__device__ __forceinline__ unsigned long long win_significands(const NucleusSmem& sm, int k_lo, int i) {
    const int k = k_lo + i;
    if (k < 8 || k > kTopBucket) return 0ull;
    unsigned long long n = 0, low = 0;
    const uint32_t pre = (uint32_t)k << 20;
#pragma unroll
    for (int c = 0; c < kH1Copies; ++c) {
        const uint32_t nc = sm.h1[i][c][0];
        n += nc;
        low += (uint32_t)(sm.h1[i][c][1] - nc * pre);
    }
    return low + n * (0x800000ull | ((unsigned long long)(k & 7) << 20));
}

// Significand sum of level-2 bucket k2 inside level-1 bucket b1: each
// element's low 10 bits from the count and pattern sum (below 2^25).
__device__ __forceinline__ unsigned long long level2_significands(const NucleusSmem& sm, uint32_t b1, uint32_t k2) {
    const uint32_t n = sm.h2[k2][0];
    const uint32_t pre = ((b1 << 10) | k2) << 10;
    return (unsigned long long)(uint32_t)(sm.h2[k2][1] - n * pre) + (unsigned long long)n * (0x800000ull | (pre & 0x7FFFFFu));
}

// Crossing bucket of one level (selection slot S) among NB buckets, bucket
// j = 0 the largest: the bucket where the mass counted from the top, starting
// at `above`, first reaches need; without one (need outside (above, above +
// total]) sel_found[S] = 0 and bucket NB - 1.  units(j) is bucket j's mass.
// With TOTAL need becomes top_p times (total + extra()), extra() being mass
// outside the buckets in the same units (evaluated after the first barrier);
// the total lands in win_total.  Threads 0..NB-1 hold one bucket each.
// Returns need, the same in every thread.
template <int S, int NB, bool TOTAL, int TPB, class U, class X>
__device__ __forceinline__ double nucleus_scan(double need, unsigned long long above, float top_p, NucleusSmem& sm,
                                               U&& units, X&& extra) {
    constexpr int NWS = (NB + kWave - 1) / kWave;
    static_assert(NB <= TPB && NWS <= TNW, "one bucket per thread");
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool scanner = tid < NWS * kWave;
    unsigned long long x = 0, incl = 0;
    __syncthreads();
    if (scanner) {
        x = tid < NB ? units(tid) : 0ull;
        incl = wave_scan_u64(x);
        if (lane == kWave - 1) sm.wt[S][wave] = incl;
    }
    __syncthreads();
    if (scanner) {
        const unsigned long long wsc = wave_scan_u64(lane < NWS ? sm.wt[S][lane] : 0ull);
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const unsigned long long total = readlane_u64(wsc, NWS - 1);
        incl += (wv > 0 ? readlane_u64(wsc, wv - 1) : 0ull) + above;
        const unsigned long long excl = incl - x;
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
        if (exists ? ((double)excl < need && need <= (double)incl) : tid == NB - 1) {
            sm.sel_bucket[S] = tid;
            sm.sel_above[S] = excl;
            sm.sel_mass[S] = x;
            sm.sel_found[S] = exists ? 1 : 0;
            if (!TOTAL && tid == NB - 1) sm.win_total = total;
        }
        if (!TOTAL && tid == 0) sm.win_total = total;
    }
    __syncthreads();
    return TOTAL ? sm.needv : need;
}

// TPB threads per row, N4 = CHUNK / (4 TPB) float4 per thread.
template <int TPB>
__global__ __launch_bounds__(TPB) void row_stats_topp_kernel(StatsParams P) {
    using namespace rows;
    __shared__ NucleusSmem sm;
    const int nrows = 2 * P.T;
    const int b = blockIdx.x / nrows, r = blockIdx.x - b * nrows;
    const float* row = row_ptr(P, b, r);
    if (!row) return;
    const int V = P.V;
    const float ilog = P.ilog;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool aligned = (((uintptr_t)row) & 15) == 0;
    constexpr int N4 = CHUNK / (4 * TPB), NWB = TPB / kWave;
    static_assert(N4 * 4 * TPB <= 8 * 4096, "each level-1 copy holds at most 4096 elements");
    float4 e[N4];
    issue_chunk<N4, TPB>(row, V, 0, aligned, e);
    auto clear_h1 = [&]() {
        for (int k = tid; k < kWinBuckets * kH1Copies * 2; k += TPB) (&sm.h1[0][0][0])[k] = 0u;
    };
    // cleared histograms are ordered before their atomics by the next barrier
    clear_h1();
    for (int k = tid; k < 1024; k += TPB) {
        sm.h2[k][0] = 0u;
        sm.h2[k][1] = 0u;
        sm.h3[k] = 0u;
    }
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
    float M = sm.wmax[0];
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
    if (lane == 0) sm.wbest[wave] = bi;   // read after the next barrier

    // unnormalised probabilities; candidates into level-1 window 0 (anything
    // at or above 2^-12, non-numbers in its last bucket, which carries no
    // mass), the others into an fp64 sum
    uint32_t* const h1c = &sm.h1[0][lane & (kH1Copies - 1)][0];
    const uint32_t one = 1u;
    {
        double tail = 0.0;
#pragma unroll
        for (int j = 0; j < N4; ++j) {
            float t4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float v = unnorm(f4get(e[j], c), M, ilog);
                f4set(e[j], c, v);
                const uint32_t bits = __float_as_uint(v);
                const bool cand = bits >= kCandBits;
                t4[c] = cand ? 0.f : v;
                if (cand) {
                    const uint32_t i = min((bits >> 20) - (uint32_t)(8 * (127 - kWinExps + 1)), (uint32_t)kWinBuckets - 1);
                    atomicAdd(h1c + i * (kH1Copies * 2), one);
                    atomicAdd(h1c + i * (kH1Copies * 2) + 1, bits);
                }
            }
            tail += (double)((t4[0] + t4[1]) + (t4[2] + t4[3]));
            // added where it is made (left to itself the compiler makes every
            // term first and holds them all)
            asm volatile("" : "+v"(tail));
        }
        const double wtl = wave_sum_d(tail);
        if (lane == 0) sm.wtail[wave] = wtl;   // read after the scan's first barrier
    }
    // the probabilities, opaque to the compiler from here on: values it
    // derived from them above (bucket indices) are not kept alive for reuse
#pragma unroll
    for (int j = 0; j < N4; ++j) asm volatile("" : "+v"(e[j].x), "+v"(e[j].y), "+v"(e[j].z), "+v"(e[j].w));
    // significand sum of window bucket i (level-1 bucket k_lo + i): each
    // copy's low 20 bits from its count and pattern sum
    int k_lo = 8 * (127 - kWinExps + 1);   // the window's smallest bucket
    int nb = kWinBuckets;                  // and its bucket count
    auto win_significands = [&](int i) { return sv::win_significands(sm, k_lo, i); };
    // scan index t = nb - 1 - i: the largest bucket first
    auto win_units = [&](int t) -> unsigned long long {
        const int i = nb - 1 - t;
        return i >= 0 ? bucket_units(win_significands(i), k_lo + i) : 0ull;
    };
    const double need = nucleus_scan<0, kWinBuckets, true, TPB>(0.0, 0ull, P.top_p, sm, win_units, [&]() {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < NWB; ++w) t += sm.wtail[w];
        return ldexp(t, kMassUnitsLog2);
    });
    unsigned long long above = 0ull;   // mass of the windows above the current one (2^-48 units)
    int found = sm.sel_found[0];
    // the cut lies below the candidates: windows further down, one register
    // pass each, until one holds the crossing
    for (int E_hi = 127 - kWinExps; !found && need > 0.0 && E_hi >= 1; E_hi -= kWinExps) {
        above += sm.win_total;
        const int E_lo = max(1, E_hi - kWinExps + 1);
        k_lo = 8 * E_lo;
        nb = 8 * (E_hi - E_lo + 1);
        __syncthreads();   // every thread has read the previous window
        clear_h1();
        __syncthreads();
#pragma unroll
        for (int j = 0; j < N4; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t bits = __float_as_uint(f4get(e[j], c));
                const uint32_t i = (bits >> 20) - (uint32_t)k_lo;
                if (i < (uint32_t)nb) {
                    atomicAdd(h1c + i * (kH1Copies * 2), one);
                    atomicAdd(h1c + i * (kH1Copies * 2) + 1, bits);
                }
            }
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
        h_b1 = win_significands(i);
    }
    const int E1 = b1 >> 3;
    // what is left to reach, in significand units of bucket b1 (the level-1
    // conversion of a bucket below 2^-25 rounded: clamp to the bucket's sum)
    double need1 = 0.0;
    if (found && need > 0.0) need1 = fmin(ldexp(need - (double)a1, kExactExp - E1), (double)h_b1);

    // levels 2 and 3 only see bucket b1: each wave lists its elements there
    // (writes and reads of a wave's own list need no barrier) and reads the
    // list, or its registers when the list is too short for them.  A bucket
    // that carries mass has an exponent field of 1..127 and lies at or below
    // bucket 1016, so matching its pattern bits implies carrying mass.
    constexpr int CAP = TNW * kNListCap / NWB;
    uint32_t* const mylist = sm.list + wave * CAP;
    const uint32_t b1m = found ? (uint32_t)b1 : 0xFFFFFFFFu;
    uint32_t nlist = 0;
#pragma unroll
    for (int j = 0; j < N4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t bits = __float_as_uint(f4get(e[j], c));
            const bool m = (bits >> 20) == b1m;
            const unsigned long long mask = __ballot(m);
            if (m) {
                const uint32_t pos = nlist + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                if (pos < (uint32_t)CAP) mylist[pos] = bits;
            }
            nlist += (uint32_t)__popcll(mask);
        }
    const bool listed = nlist <= (uint32_t)CAP;
    // elements whose pattern >> pshift equals prefix go through f (the prefix
    // made opaque to the compiler, so that the register pass does not keep
    // the listing's comparison masks alive to reuse them)
    auto each_in = [&](int pshift, uint32_t prefix, auto&& f) {
        prefix = (uint32_t)__builtin_amdgcn_readfirstlane((int)prefix);
        asm volatile("" : "+s"(prefix));
        if (listed) {
            for (uint32_t i = (uint32_t)lane; i < nlist; i += kWave) {
                const uint32_t bits = mylist[i];
                if ((bits >> pshift) == prefix) f(bits);
            }
        } else {
#pragma unroll
            for (int j = 0; j < N4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t bits = __float_as_uint(f4get(e[j], c));
                    if ((bits >> pshift) == prefix) f(bits);
                }
        }
    };
    // level 2: (count, pattern sum) of pattern bits 19..10; each bucket's low
    // 10 bits add up to below 2^25
    each_in(20, b1m, [&](uint32_t bits) {
        const uint32_t k2 = (bits >> 10) & 1023u;
        atomicAdd(&sm.h2[k2][0], one);
        atomicAdd(&sm.h2[k2][1], bits);
    });
    nucleus_scan<1, 1024, false, TPB>(need1, 0ull, P.top_p, sm, [&](int t) {
        return level2_significands(sm, (uint32_t)b1, 1023u - (uint32_t)t);
    }, []() { return 0.0; });
    const uint32_t b2 = 1023u - (uint32_t)sm.sel_bucket[1];
    const unsigned long long a2 = sm.sel_above[1];
    double need2 = 0.0;
    if (need1 > 0.0) need2 = fmin(need1 - (double)a2, (double)sm.sel_mass[1]);
    // level 3: counts of the exact patterns
    const uint32_t p3 = found ? (((uint32_t)b1 << 10) | b2) : 0xFFFFFFFFu;
    each_in(10, p3, [&](uint32_t bits) { atomicAdd(&sm.h3[bits & 1023u], one); });
    nucleus_scan<2, 1024, false, TPB>(need2, 0ull, P.top_p, sm, [&](int t) -> unsigned long long {
        const uint32_t k3 = 1023u - (uint32_t)t;
        return (unsigned long long)sm.h3[k3] * significand((((uint32_t)b1 << 10 | b2) << 10) | k3);
    }, []() { return 0.0; });
    Nucleus nu;
    nu.thr = found ? ((((uint32_t)b1 << 10 | b2) << 10) | (1023u - (uint32_t)sm.sel_bucket[2])) : 0u;
    nu.cutoff = INT_MAX;
    // significand-unit masses above thr inside b1, and of the elements at thr
    // (all of the last bucket: (number of ties) * (significand of one))
    const unsigned long long a3 = sm.sel_above[2];
    unsigned long long kept = found ? sm.sel_mass[2] : 0ull;
    const unsigned long long tie_mass = found ? significand(nu.thr) : 0ull;
    if (tie_mass > 0 && kept > 0) {
        const unsigned long long ties = kept / tie_mass;
        long long k = (long long)ceil((need2 - (double)a3) / (double)tie_mass);
        if (k < 1) k = 1;
        if (ties > 1 && (unsigned long long)k < ties) {
            // ties straddle the cut: the smallest cutoff c with #ties(id < c) >= k,
            // by bisection on the token id (block counts, alternating buffers);
            // exactly k ties then lie below the cutoff
            int lo = 0, hi = V, par = 0;
            while (lo < hi) {
                const int mid = lo + (hi - lo) / 2;
                unsigned long long cnt = 0;
#pragma unroll
                for (int j = 0; j < N4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int idx = elem_index<TPB>(0, j, c);
                        if (idx < V && idx <= mid && __float_as_uint(f4get(e[j], c)) == nu.thr) ++cnt;
                    }
                cnt = wave_sum_u64(cnt);
                if (lane == 0) sm.cnt[par][wave] = cnt;
                __syncthreads();
                unsigned long long tot = 0;
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
        int best = sm.wbest[0];
#pragma unroll
        for (int w = 1; w < NWB; ++w) best = min(best, sm.wbest[w]);
        // normaliser of the nucleus: the buckets above b1 (2^-48 units) and
        // the kept part of b1 (significand units, 2^(E1 - 150) each)
        const unsigned long long in_b1 = found ? a2 + a3 + kept : 0ull;
        RowStat st;
        st.zmax = M;
        st.argmax = best;
        st.thr = nu.thr;
        st.cutoff = nu.cutoff;
        st.Z = ldexp((double)a1, -kMassUnitsLog2) + ldexp((double)in_b1, E1 - 150);
        P.stats[(size_t)b * nrows + r] = st;
    }
}

// Top-p rows longer than one register chunk (V > 32768): the same cut (the
// same units, windows and levels as the on-chip kernel) with the row
// streamed, each next block's loads in flight.  Pass 1: the maximum and its
// first position.  Pass 2: the unnormalised probabilities; candidates (e >=
// 2^-12) into level-1 window 0 and into a list in LDS (up to kCandListCap
// entries), the others into the fp64 tail sum.  Levels 2 and 3 then read the
// list, so a row is streamed twice.  Rarer cases stream again: a cut below
// the candidates (one pass per lower window, then levels 2 and 3 from the
// stream), a list that overflowed (levels 2 and 3 from the stream), and tied
// probabilities straddling the cut (one pass counting the ties per 32768-id
// chunk, then a bisection inside the chunk that holds the k-th tie).
constexpr int kCandListCap = 8192;

__global__ __launch_bounds__(rows::NT) void row_stats_topp_chunked_kernel(StatsParams P) {
    using namespace rows;
    __shared__ NucleusSmem sm;
    __shared__ uint32_t clist[kCandListCap];   // patterns of the candidates (pass 2)
    __shared__ uint32_t cn;
    __shared__ int chunk_ties[MAX_CHUNKS];
    const int nrows = 2 * P.T;
    const int b = blockIdx.x / nrows, r = blockIdx.x - b * nrows;
    const float* row = row_ptr(P, b, r);
    if (!row) return;
    const int V = P.V;
    const float ilog = P.ilog;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool aligned = (((uintptr_t)row) & 15) == 0;
    constexpr int HB = VPT4 / 2;   // float4 per thread per streamed block (two blocks in flight)
    constexpr int TPB = NT, NWB = TPB / kWave;
    auto clear_h1 = [&]() {
        for (int k = tid; k < kWinBuckets * kH1Copies * 2; k += TPB) (&sm.h1[0][0][0])[k] = 0u;
    };
    // cleared histograms and counts are ordered before their atomics by the next barrier
    clear_h1();
    for (int k = tid; k < 1024; k += TPB) {
        sm.h2[k][0] = 0u;
        sm.h2[k][1] = 0u;
        sm.h3[k] = 0u;
    }
    if (tid < MAX_CHUNKS) chunk_ties[tid] = 0;
    if (tid == 0) cn = 0u;

    // pass 1: the largest logit and its smallest id: per block the thread's
    // maximum and the first of its positions holding it; blocks come in id order
    float bv = -INFINITY;
    int bi = INT_MAX;
    for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int cb) {
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4 * HB; k += 2) m = max3_f32(m, f4get(x[k / 4], k % 4), f4get(x[k / 4], k % 4 + 1));
        if (m > bv) {   // the first position holding m has the smallest id of this block
            int loc = INT_MAX;
#pragma unroll
            for (int j = HB - 1; j >= 0; --j)
#pragma unroll
                for (int c = 3; c >= 0; --c) {
                    const int idx = elem_index(cb, j, c);
                    loc = (f4get(x[j], c) == m && idx < V) ? idx : loc;
                }
            bv = m;
            bi = loc;
        }
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) argmax_step(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
    if (lane == 0) { sm.wmax[wave] = bv; sm.wbest[wave] = bi; }
    __syncthreads();
    float M = sm.wmax[0];
    int best = sm.wbest[0];
#pragma unroll
    for (int w = 1; w < NWB; ++w) argmax_step(M, best, sm.wmax[w], sm.wbest[w]);

    // pass 2: candidates into level-1 window 0 and the list, the others into
    // the tail sum
    uint32_t* const h1c = &sm.h1[0][lane & (kH1Copies - 1)][0];
    const uint32_t one = 1u;
    {
        double tail = 0.0;
        for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int) {
#pragma unroll
            for (int j = 0; j < HB; ++j) {
                float t4[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float v = unnorm(f4get(x[j], c), M, ilog);
                    const uint32_t bits = __float_as_uint(v);
                    const bool cand = bits >= kCandBits;
                    t4[c] = cand ? 0.f : v;
                    const unsigned long long mask = __ballot(cand);
                    if (cand) {
                        const uint32_t i = min((bits >> 20) - (uint32_t)(8 * (127 - kWinExps + 1)), (uint32_t)kWinBuckets - 1);
                        atomicAdd(h1c + i * (kH1Copies * 2), one);
                        atomicAdd(h1c + i * (kH1Copies * 2) + 1, bits);
                    }
                    if (mask) {   // the wave's candidates of this slot go to the list together
                        uint32_t at = 0;
                        if (lane == 0) at = atomicAdd(&cn, (uint32_t)__popcll(mask));
                        at = (uint32_t)__builtin_amdgcn_readfirstlane((int)at);
                        const uint32_t pos = at + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                        if (cand && pos < (uint32_t)kCandListCap) clist[pos] = bits;
                    }
                }
                tail += (double)((t4[0] + t4[1]) + (t4[2] + t4[3]));
            }
        });
        const double wtl = wave_sum_d(tail);
        if (lane == 0) sm.wtail[wave] = wtl;   // read after the scan's first barrier
    }
    int k_lo = 8 * (127 - kWinExps + 1);
    int nb = kWinBuckets;
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
    unsigned long long above = 0ull;
    int found = sm.sel_found[0];
    const bool in_list = found && cn <= (uint32_t)kCandListCap;   // the crossing bucket's elements are listed
    for (int E_hi = 127 - kWinExps; !found && need > 0.0 && E_hi >= 1; E_hi -= kWinExps) {
        above += sm.win_total;
        const int E_lo = max(1, E_hi - kWinExps + 1);
        k_lo = 8 * E_lo;
        nb = 8 * (E_hi - E_lo + 1);
        __syncthreads();   // every thread has read the previous window
        clear_h1();
        __syncthreads();
        for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int) {
#pragma unroll
            for (int j = 0; j < HB; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t bits = __float_as_uint(unnorm(f4get(x[j], c), M, ilog));
                    const uint32_t i = (bits >> 20) - (uint32_t)k_lo;
                    if (i < (uint32_t)nb) {
                        atomicAdd(h1c + i * (kH1Copies * 2), one);
                        atomicAdd(h1c + i * (kH1Copies * 2) + 1, bits);
                    }
                }
        });
        nucleus_scan<0, kWinBuckets, false, TPB>(need, above, P.top_p, sm, win_units, []() { return 0.0; });
        found = sm.sel_found[0];
    }
    int b1 = 0;
    unsigned long long a1 = above + sm.win_total, h_b1 = 0ull;
    if (found) {
        const int i = nb - 1 - sm.sel_bucket[0];
        b1 = k_lo + i;
        a1 = sm.sel_above[0];
        h_b1 = win_significands(sm, k_lo, i);
    }
    const int E1 = b1 >> 3;
    double need1 = 0.0;
    if (found && need > 0.0) need1 = fmin(ldexp(need - (double)a1, kExactExp - E1), (double)h_b1);
    const uint32_t b1m = found ? (uint32_t)b1 : 0xFFFFFFFFu;
    // elements whose pattern >> pshift equals prefix go through f: from the
    // list when it holds the crossing bucket, else from the stream
    auto each_in = [&](int pshift, uint32_t prefix, auto&& f) {
        if (in_list) {
            const uint32_t n = cn;
            for (uint32_t i = (uint32_t)tid; i < n; i += TPB) {
                const uint32_t bits = clist[i];
                if ((bits >> pshift) == prefix) f(bits);
            }
        } else {
            for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int) {
#pragma unroll
                for (int j = 0; j < HB; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t bits = __float_as_uint(unnorm(f4get(x[j], c), M, ilog));
                        if ((bits >> pshift) == prefix) f(bits);
                    }
            });
        }
    };
    each_in(20, b1m, [&](uint32_t bits) {
        const uint32_t k2 = (bits >> 10) & 1023u;
        atomicAdd(&sm.h2[k2][0], one);
        atomicAdd(&sm.h2[k2][1], bits);
    });
    nucleus_scan<1, 1024, false, TPB>(need1, 0ull, P.top_p, sm, [&](int t) {
        return level2_significands(sm, (uint32_t)b1, 1023u - (uint32_t)t);
    }, []() { return 0.0; });
    const uint32_t b2 = 1023u - (uint32_t)sm.sel_bucket[1];
    const unsigned long long a2 = sm.sel_above[1];
    double need2 = 0.0;
    if (need1 > 0.0) need2 = fmin(need1 - (double)a2, (double)sm.sel_mass[1]);
    const uint32_t p3 = found ? (((uint32_t)b1 << 10) | b2) : 0xFFFFFFFFu;
    each_in(10, p3, [&](uint32_t bits) { atomicAdd(&sm.h3[bits & 1023u], one); });
    nucleus_scan<2, 1024, false, TPB>(need2, 0ull, P.top_p, sm, [&](int t) -> unsigned long long {
        const uint32_t k3 = 1023u - (uint32_t)t;
        return (unsigned long long)sm.h3[k3] * significand((((uint32_t)b1 << 10 | b2) << 10) | k3);
    }, []() { return 0.0; });
    Nucleus nu;
    nu.thr = found ? ((((uint32_t)b1 << 10 | b2) << 10) | (1023u - (uint32_t)sm.sel_bucket[2])) : 0u;
    nu.cutoff = INT_MAX;
    const unsigned long long a3 = sm.sel_above[2];
    unsigned long long kept = found ? sm.sel_mass[2] : 0ull;
    const unsigned long long tie_mass = found ? significand(nu.thr) : 0ull;
    if (tie_mass > 0 && kept > 0) {
        const unsigned long long ties = kept / tie_mass;
        long long k = (long long)ceil((need2 - (double)a3) / (double)tie_mass);
        if (k < 1) k = 1;
        if (ties > 1 && (unsigned long long)k < ties) {
            // ties straddle the cut: ties per chunk, then the smallest cutoff c
            // with #ties(id < c) >= k by bisection inside the chunk holding
            // the k-th tie (block counts, alternating buffers)
            for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int cb) {
                unsigned long long cnt = 0;
#pragma unroll
                for (int j = 0; j < HB; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (elem_index(cb, j, c) < V && __float_as_uint(unnorm(f4get(x[j], c), M, ilog)) == nu.thr) ++cnt;
                cnt = wave_sum_u64(cnt);
                if (lane == 0) atomicAdd(&chunk_ties[cb / CHUNK], (int)cnt);
            });
            __syncthreads();
            const int nchunks = (V + CHUNK - 1) / CHUNK;
            long long before = 0;
            int cstar = nchunks - 1;
            for (int c = 0; c < nchunks; ++c) {
                if (before + chunk_ties[c] >= k) { cstar = c; break; }
                before += chunk_ties[c];
            }
            const int cb = cstar * CHUNK;
            float4 e[VPT4];
            load_chunk(row, V, cb, aligned, e);
#pragma unroll
            for (int j = 0; j < VPT4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) f4set(e[j], c, unnorm(f4get(e[j], c), M, ilog));
            int lo = cb, hi = min(V, cb + CHUNK) - 1, par = 0;
            while (lo < hi) {
                const int mid = lo + (hi - lo) / 2;
                unsigned long long cnt = 0;
#pragma unroll
                for (int j = 0; j < VPT4; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int idx = elem_index(cb, j, c);
                        if (idx < V && idx <= mid && __float_as_uint(f4get(e[j], c)) == nu.thr) ++cnt;
                    }
                cnt = wave_sum_u64(cnt);
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
        const unsigned long long in_b1 = found ? a2 + a3 + kept : 0ull;
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
constexpr int kToppThreads = 1024;  // threads per row of the on-chip top-p kernel
// Which row-statistics kernel a launch takes: with top-p (sampling mode) the
// cut needs the row on chip (up to rows::CHUNK ids) or streamed; otherwise
// one streaming read.
enum StatsKind { kStatsTopp, kStatsToppChunked, kStatsStream };
StatsKind stats_kind(const StatsParams& p) {
    if (p.sampling && p.top_p < 1.f) return p.V <= rows::CHUNK ? kStatsTopp : kStatsToppChunked;
    return kStatsStream;
}
}  // namespace

bool row_stats_streams(const StatsParams& p) { return stats_kind(p) == kStatsStream; }

const char* row_stats_kernel_name(const StatsParams& p) {
    switch (stats_kind(p)) {
    case kStatsTopp: return "row_stats_topp_kernel";
    case kStatsToppChunked: return "row_stats_topp_chunked_kernel";
    default: return "row_stats_stream_kernel";
    }
}

hipError_t launch_row_stats(const StatsParams& p, hipStream_t s) {
    const int nrows = p.sampling ? 2 * p.T : p.T;
    dim3 grid((unsigned)(p.B * nrows));
    switch (stats_kind(p)) {
    case kStatsTopp: hipLaunchKernelGGL(row_stats_topp_kernel<kToppThreads>, grid, dim3(kToppThreads), 0, s, p); break;
    case kStatsToppChunked: hipLaunchKernelGGL(row_stats_topp_chunked_kernel, grid, dim3(rows::NT), 0, s, p); break;
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
