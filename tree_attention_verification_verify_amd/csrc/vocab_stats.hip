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
// per bucket, see the kernel); a longer row is streamed once per step of the
// same cut with fixed-point masses.

#include "row_block.h"
#include "stats_stream.h"

namespace sv {
namespace {

constexpr int ST = kStatsThreads;

template <bool WITH_Z>
__global__ __launch_bounds__(ST) void row_stats_stream_kernel(StatsParams P) {
    row_stats_stream_block<WITH_Z>(P, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Top-p cut of the streamed rows (V > 32768): a 3-level radix select (10 bits
// per level, from the top) on the fp32 patterns of the unnormalised
// probabilities, with fixed-point (2^-40) mass histograms.  Each level costs
// three barriers: histogram; scan of the buckets in descending order inside
// each wave; wave offsets read by every thread (integer sums, so any order
// gives the same result) and the crossing bucket published.  The first level
// sees every logit, so its histogram has HK copies (lane & (HK - 1)),
// interleaved per bucket so the copies of one bucket sit in different banks:
// a wave's 64 atomics then collide HK times less on the crowded buckets.
constexpr int HK = 4;
constexpr int TNW = rows::NW;
constexpr int kListCap = 256;   // per-wave list of the elements in the first level's crossing bucket
constexpr uint32_t kZeroMassBits = 0x2B000000u;   // 2^-41: rounds to mass 0 (ties to even)
constexpr uint32_t kOneBits = 0x3F800000u;        // 1.0

struct ToppSmem {
    unsigned long long h1[1024 * HK];   // level 1: copy c of bucket k at k * HK + c
    unsigned long long h2[1024];
    unsigned long long h3[1024];
    unsigned long long wt[3][TNW];      // per level: wave totals of the bucket scan
    unsigned long long sel_above[3];    // per level: mass of the larger buckets
    unsigned long long sel_mass[3];     // per level: mass of the crossing bucket
    int sel_bucket[3];
    float bv[TNW];
    int bi[TNW];
    unsigned long long cnt[2][TNW];
    uint32_t list[TNW][kListCap];       // per wave: patterns of its elements in the first-level bucket
};

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((unsigned long long)hi << 32) | lo;
}

// One level of the cut, in two parts.  Accumulate: elements whose pattern
// above bit PSHIFT equals `prefix` add their mass to bucket
// (bits >> SHIFT) & 1023 (no barrier: a row may take several chunks).  Scan:
// the crossing is the bucket where the mass counted from the largest bucket
// down first reaches need (for level 0 need is top_p times the row total,
// which only the scan knows); without a crossing (need outside (0, total])
// bucket 0.
template <int L, int N = rows::VPT4>
__device__ __forceinline__ void topp_accumulate(const float4 (&e)[N], uint32_t prefix, ToppSmem& sm) {
    using namespace rows;
    constexpr int SHIFT = 20 - 10 * L;
    constexpr int PSHIFT = L == 0 ? 31 : 30 - 10 * L;
    constexpr int HC = L == 0 ? HK : 1;
    unsigned long long* h = L == 0 ? sm.h1 : (L == 1 ? sm.h2 : sm.h3);
    const int copy = L == 0 ? (lane_() & (HK - 1)) : 0;
    // only masses in (0, 2^40] count: entries past the row end (e = 0),
    // probabilities at or below 2^-41 (zero in fixed point) and non-numbers
    // add nothing
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float v = f4get(e[j], c);
            const uint32_t bits = __float_as_uint(v);
            if (bits > kZeroMassBits && bits <= kOneBits && (bits >> PSHIFT) == prefix)
                atomicAdd(&h[((bits >> SHIFT) & 1023) * HC + copy], fixmass(v));
        }
}

// Levels 1 and 2 from a wave's list instead of its registers (the same
// elements: the list holds every one of the wave's nonzero masses in the
// first level's crossing bucket); lanes take entries in turn.
template <int L>
__device__ __forceinline__ void topp_accumulate_list(const uint32_t* list, uint32_t n, uint32_t prefix, ToppSmem& sm) {
    constexpr int SHIFT = 20 - 10 * L;
    constexpr int PSHIFT = 30 - 10 * L;
    static_assert(L == 1 || L == 2, "list levels");
    unsigned long long* h = L == 1 ? sm.h2 : sm.h3;
    for (uint32_t i = (uint32_t)rows::lane_(); i < n; i += kWave) {
        const uint32_t bits = list[i];
        if ((bits >> PSHIFT) == prefix) atomicAdd(&h[(bits >> SHIFT) & 1023], rows::fixmass(__uint_as_float(bits)));
    }
}

// The wave's elements with a nonzero mass in first-level bucket b1, appended
// to its list after the n already there (positions by ballot); returns how
// many there are now (the list holds them when that is at most kListCap).
// The same in every lane.
template <int N = rows::VPT4, int CAP = kListCap>
__device__ __forceinline__ uint32_t topp_compact(const float4 (&e)[N], uint32_t b1, uint32_t* list, uint32_t n = 0) {
    using namespace rows;
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t bits = __float_as_uint(f4get(e[j], c));
            const bool m = bits > kZeroMassBits && bits <= kOneBits && (bits >> 20) == b1;
            const unsigned long long mask = __ballot(m);
            if (m) {
                const uint32_t pos = n + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                if (pos < (uint32_t)CAP) list[pos] = bits;
            }
            n += (uint32_t)__popcll(mask);
        }
    return n;
}

// The crossing bucket lands in sm.sel_*[L].  Returns need (level 0: the one
// it computed).  TPB threads: each takes 1024 / TPB consecutive buckets in
// descending order (thread order = descending bucket).
template <int L, int TPB = rows::NT>
__device__ __forceinline__ double topp_scan(double need, float top_p, ToppSmem& sm) {
    using namespace rows;
    constexpr int HC = L == 0 ? HK : 1;
    constexpr int BPT = 1024 / TPB, NWB = TPB / kWave;
    static_assert(BPT * TPB == 1024 && NWB <= TNW, "buckets per thread");
    unsigned long long* h = L == 0 ? sm.h1 : (L == 1 ? sm.h2 : sm.h3);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    __syncthreads();
    const int bk0 = 1023 - BPT * tid;   // this thread's largest bucket
    unsigned long long xs[BPT];
    unsigned long long x = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        xs[q] = 0;
#pragma unroll
        for (int c = 0; c < HC; ++c) xs[q] += h[(bk0 - q) * HC + c];
        x += xs[q];
    }
    unsigned long long incl = wave_scan_u64(x);
    if (lane == kWave - 1) sm.wt[L][wave] = incl;
    __syncthreads();
    // lanes 0..NWB-1 scan the wave totals; this wave's offset and the total
    // are then read from single lanes
    const unsigned long long wsc = wave_scan_u64(lane < NWB ? sm.wt[L][lane] : 0ull);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const unsigned long long total = readlane_u64(wsc, NWB - 1);
    incl += wv > 0 ? readlane_u64(wsc, wv - 1) : 0ull;
    const unsigned long long excl = incl - x;
    if (L == 0) need = (double)top_p * (double)total;
    // the integer bounds, as doubles, tile (0, (double)total] without gaps, so
    // a crossing exists exactly when need lies in that range, and is unique
    const bool exists = 0.0 < need && need <= (double)total;
    unsigned long long lo = excl;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const unsigned long long hi = lo + xs[q];
        if (exists ? ((double)lo < need && need <= (double)hi) : (tid == TPB - 1 && q == BPT - 1)) {
            sm.sel_bucket[L] = bk0 - q;
            sm.sel_above[L] = lo;
            sm.sel_mass[L] = xs[q];
        }
        lo = hi;
    }
    __syncthreads();
    return need;
}

// ---------------------------------------------------------------------------
// Top-p rows held on chip (V <= 32768): exact significand sums.
//
// A kept-mass candidate e (an unnormalised probability: normal, at most 1)
// with exponent field E and 24-bit significand s equals s * 2^(E - 150), and
// every element of a level-1 bucket (pattern bits 29..20: seven exponent
// bits and three significand bits) shares E.  Level 1 therefore adds, per
// bucket, the u64 value (1 << 48) + pattern: the top bits count the elements
// n and the low 48 bits hold the sum of patterns (below 2^46), from which the
// significand sum is sum - n * ((E - 1) << 23), exact.  The scan converts each
// bucket to units of 2^-48 (exact for E >= 102; a bucket of e < 2^-25 is
// rounded to the nearest unit, an error below 2^-49 of the largest
// probability, and the row total stays below 2^63).  Levels 2 and 3 lie
// inside the crossing bucket and stay in significand units; the nucleus
// normaliser is assembled from the two parts in fp64.
//
// Only candidates (e >= 2^-12) enter the level-1 histogram: the others are
// summed per thread (fp32 within a float4, fp64 across them: a fixed order
// of additions, then fixed-order wave and block sums), and the cut lies among
// the candidates whenever top_p times the row total is at most their mass.
// At the batch-32 chain shape this leaves about 5% of the logits for the LDS
// atomics.  A row whose cut lies lower (a flat distribution, or top_p close
// to 1) adds the others to the histogram too and scans again, with the row
// total taken from the histogram alone.
constexpr int kMassUnitsLog2 = 48;                  // level-1 scan units: 2^-48
constexpr int kExactExp = 150 - kMassUnitsLog2;     // smallest exponent field converted exactly
constexpr uint32_t kCandBits = 115u << 23;          // 2^-12: smallest candidate

__device__ __forceinline__ uint32_t significand(uint32_t bits) { return (bits & 0x7FFFFFu) | 0x800000u; }
constexpr unsigned long long kCountOne = 1ull << 48;   // one element in a level-1 bucket entry
constexpr int kTopBucket = 1016;                        // level-1 bucket of 1.0 (exponent 127)

// Significand sum of level-1 bucket k from its entry (count << 48) + sum of patterns.
__device__ __forceinline__ unsigned long long bucket_significands(unsigned long long entry, int k) {
    const unsigned long long n = entry >> 48, pat = entry & (kCountOne - 1);
    return pat - n * ((unsigned long long)((k >> 3) - 1) << 23);
}

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
    unsigned long long h1[1024 * HK];   // level 1: copy c of bucket k at k * HK + c
    unsigned long long h2[1024];
    unsigned long long h3[1024];
    unsigned long long wt[4][TNW];
    double wtail[TNW];                  // per wave: fp64 mass of the elements below the candidates
    unsigned long long sel_above[4];
    unsigned long long sel_mass[4];
    int sel_bucket[4];
    int sel_found[4];
    double needv[4];
    float wmax[TNW];
    int wbest[TNW];
    unsigned long long cnt[2][TNW];
    uint32_t list[TNW * kListCap];      // per wave: patterns of its elements in the level-1 crossing bucket
};

// Crossing bucket of one level (selection slot S): the bucket where the mass
// counted from the largest bucket down first reaches need; without one (need
// outside (0, total]) bucket 0, with sel_found[S] = 0.  units(k) is bucket
// k's mass.  With TOTAL the level sets need to top_p times (its total +
// extra()), extra() being mass outside the buckets in the same units
// (evaluated after the first barrier).  Returns need, the same in every
// thread.  The first kScanThreads threads scan, 1024 / kScanThreads buckets
// each (with all 1024 threads, one bucket each: the scan is a chain of
// dependent steps, and one bucket per thread measured 26.4 against 28.0 us at
// four buckets per thread on one wave per SIMD).
constexpr int kScanThreads = 1024;
template <int S, bool TOTAL, int TPB, class U, class X>
__device__ __forceinline__ double nucleus_scan(double need, float top_p, NucleusSmem& sm, U&& units, X&& extra) {
    constexpr int SCT = TPB < kScanThreads ? TPB : kScanThreads;
    constexpr int BPT = 1024 / SCT, NWS = SCT / kWave;
    static_assert(BPT * SCT == 1024 && NWS <= TNW, "buckets per thread");
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool scanner = tid < SCT;
    const int bk0 = 1023 - BPT * tid;   // this thread's largest bucket
    unsigned long long xs[BPT];
    unsigned long long x = 0, incl = 0;
    __syncthreads();
    if (scanner) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            xs[q] = units(bk0 - q);
            x += xs[q];
        }
        incl = wave_scan_u64(x);
        if (lane == kWave - 1) sm.wt[S][wave] = incl;
    }
    __syncthreads();
    if (scanner) {
        const unsigned long long wsc = wave_scan_u64(lane < NWS ? sm.wt[S][lane] : 0ull);
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const unsigned long long total = readlane_u64(wsc, NWS - 1);
        incl += wv > 0 ? readlane_u64(wsc, wv - 1) : 0ull;
        const unsigned long long excl = incl - x;
        if (TOTAL) {
            need = (double)top_p * ((double)total + extra());
            if (tid == 0) sm.needv[S] = need;
        }
        const bool exists = 0.0 < need && need <= (double)total;
        // the integer bounds, as doubles, tile (0, total] without gaps: one
        // thread's range holds need, and one of its buckets
        const bool mine = exists ? ((double)excl < need && need <= (double)incl) : tid == SCT - 1;
        if (mine) {
            unsigned long long lo = excl;
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const unsigned long long hi = lo + xs[q];
                if (exists ? ((double)lo < need && need <= (double)hi) : q == BPT - 1) {
                    sm.sel_bucket[S] = bk0 - q;
                    sm.sel_above[S] = lo;
                    sm.sel_mass[S] = xs[q];
                    sm.sel_found[S] = exists ? 1 : 0;
                }
                lo = hi;
            }
        }
    }
    __syncthreads();
    return TOTAL ? sm.needv[S] : need;
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
    float4 e[N4];
    issue_chunk<N4, TPB>(row, V, 0, aligned, e);
    // cleared histograms are ordered before their atomics by the next barrier
    for (int k = tid; k < 1024 * HK; k += TPB) sm.h1[k] = 0ull;
    for (int k = tid; k < 1024; k += TPB) {
        sm.h2[k] = 0ull;
        sm.h3[k] = 0ull;
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

    // unnormalised probabilities; candidates into level 1 ((count, pattern
    // sum) per bucket, HK copies by lane), the others into an fp64 sum
    uint8_t* const h1c = (uint8_t*)sm.h1 + 8 * (lane & (HK - 1));
    auto add_h1 = [&](uint32_t bits) {
        atomicAdd((unsigned long long*)(h1c + ((bits >> 15) & (1023u * 8 * HK))), kCountOne + bits);
    };
    {
        // the others' sum: fp32 within each float4 (four terms below 2^-12,
        // relative error below 2^-22), fp64 across them, in a fixed order
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
                if (cand) add_h1(bits);
            }
            tail += (double)((t4[0] + t4[1]) + (t4[2] + t4[3]));
            // added where it is made (left to itself the compiler makes every
            // term first and holds them all)
            asm volatile("" : "+v"(tail));
        }
        const double wtl = wave_sum_d(tail);
        if (lane == 0) sm.wtail[wave] = wtl;   // read after the scan's first barrier
    }
    // buckets of exponent 0 (zeros, subnormals) and above the bucket of 1.0
    // (non-numbers) carry no mass
    auto h1_significands = [&](int k) -> unsigned long long {
        if (k < 8 || k > kTopBucket) return 0ull;
        unsigned long long s = 0;
#pragma unroll
        for (int c = 0; c < HK; ++c) s += sm.h1[k * HK + c];
        return bucket_significands(s, k);
    };
    auto h1_units = [&](int k) { return bucket_units(h1_significands(k), k); };
    double need = nucleus_scan<0, true, TPB>(0.0, P.top_p, sm, h1_units, [&]() {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < NWB; ++w) t += sm.wtail[w];
        return ldexp(t, kMassUnitsLog2);
    });
    int s1 = 0;   // selection slot of level 1
    if (!sm.sel_found[0]) {
        // the cut lies below the candidates: the others join the histogram
#pragma unroll
        for (int j = 0; j < N4; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t bits = __float_as_uint(f4get(e[j], c));
                if (bits < kCandBits) add_h1(bits);
            }
        need = nucleus_scan<3, true, TPB>(0.0, P.top_p, sm, h1_units, []() { return 0.0; });
        s1 = 3;
    }
    const uint32_t b1 = (uint32_t)sm.sel_bucket[s1];
    const unsigned long long a1 = sm.sel_above[s1];
    const int E1 = (int)(b1 >> 3);
    const unsigned long long h_b1 = h1_significands((int)b1);   // the crossing bucket's significand sum
    // what is left to reach, in significand units of bucket b1 (the level-1
    // conversion of a bucket below 2^-25 rounded: clamp to the bucket's sum)
    double need1 = 0.0;
    if (need > 0.0 && h_b1 > 0) need1 = fmin(ldexp(need - (double)a1, kExactExp - E1), (double)h_b1);

    // levels 2 and 3 only see bucket b1: each wave lists its elements there
    // (writes and reads of a wave's own list need no barrier) and reads the
    // list, or its registers when the list is too short for them.  A bucket
    // that carries mass has an exponent field of 1..127 and lies at or below
    // bucket 1016, so matching its pattern bits implies carrying mass.
    constexpr int CAP = TNW * kListCap / NWB;
    uint32_t* const mylist = sm.list + wave * CAP;
    const uint32_t b1m = h_b1 > 0 ? b1 : 0xFFFFFFFFu;
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
    // prefix of the elements a level counts: pattern >> pshift == prefix
    // (made opaque to the compiler, so that the register pass does not keep
    // the listing's 64 comparison masks alive to reuse them)
    auto accumulate = [&](unsigned long long* h, int shift, int pshift, uint32_t prefix) {
        prefix = (uint32_t)__builtin_amdgcn_readfirstlane((int)prefix);
        asm volatile("" : "+s"(prefix));
        if (listed) {
            for (uint32_t i = (uint32_t)lane; i < nlist; i += kWave) {
                const uint32_t bits = mylist[i];
                if ((bits >> pshift) == prefix) atomicAdd(&h[(bits >> shift) & 1023], (unsigned long long)significand(bits));
            }
        } else {
#pragma unroll
            for (int j = 0; j < N4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t bits = __float_as_uint(f4get(e[j], c));
                    if ((bits >> pshift) == prefix)
                        atomicAdd(&h[(bits >> shift) & 1023], (unsigned long long)significand(bits));
                }
        }
    };
    auto none = []() { return 0.0; };
    accumulate(sm.h2, 10, 20, b1m);
    nucleus_scan<1, false, TPB>(need1, P.top_p, sm, [&](int k) { return sm.h2[k]; }, none);
    const uint32_t b2 = (uint32_t)sm.sel_bucket[1];
    const unsigned long long a2 = sm.sel_above[1];
    double need2 = 0.0;
    if (need1 > 0.0) need2 = fmin(need1 - (double)a2, (double)sm.sel_mass[1]);
    accumulate(sm.h3, 0, 10, h_b1 > 0 ? ((b1 << 10) | b2) : 0xFFFFFFFFu);
    nucleus_scan<2, false, TPB>(need2, P.top_p, sm, [&](int k) { return sm.h3[k]; }, none);
    Nucleus nu;
    nu.thr = (b1 << 20) | (b2 << 10) | (uint32_t)sm.sel_bucket[2];
    nu.cutoff = INT_MAX;
    // significand-unit masses above thr inside b1, and of the elements at thr
    // (all of the last bucket: (number of ties) * (significand of one))
    const unsigned long long a3 = sm.sel_above[2];
    unsigned long long kept = sm.sel_mass[2];
    const unsigned long long tie_mass = h_b1 > 0 ? significand(nu.thr) : 0ull;
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
        RowStat st;
        st.zmax = M;
        st.argmax = best;
        st.thr = nu.thr;
        st.cutoff = nu.cutoff;
        st.Z = ldexp((double)a1, -kMassUnitsLog2) + ldexp((double)(a2 + a3 + kept), E1 - 150);
        P.stats[(size_t)b * nrows + r] = st;
    }
}

// Top-p rows longer than one register chunk (V > 32768).  The same cut, with
// the row streamed chunk by chunk (each next chunk's loads in flight): one
// pass for the maximum and its first position, one each for radix levels 1
// and 2 (level 3 reads the entries of level 1's crossing bucket that the
// level-2 pass listed, unless a wave's list overflowed), and, only when tied
// probabilities straddle the cut, one pass counting the ties per chunk and a
// bisection inside the chunk that holds the k-th tie.
__global__ __launch_bounds__(rows::NT) void row_stats_topp_chunked_kernel(StatsParams P) {
    using namespace rows;
    __shared__ ToppSmem sm;
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
    // cleared histograms and counts are ordered before their atomics by the next barrier
#pragma unroll
    for (int k = 0; k < HK; ++k) sm.h1[k * NT + tid] = 0ull;
    sm.h2[tid] = 0ull;
    sm.h3[tid] = 0ull;
    if (tid < MAX_CHUNKS) chunk_ties[tid] = 0;

    // largest logit and its smallest id: per chunk the thread's maximum and
    // the first of its positions holding it; chunks come in id order
    float bv = -INFINITY;
    int bi = INT_MAX;
    for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int cb) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < HB; ++j) m = fmaxf(fmaxf(m, fmaxf(x[j].x, x[j].y)), fmaxf(x[j].z, x[j].w));
        int loc = INT_MAX;
#pragma unroll
        for (int j = HB - 1; j >= 0; --j)
#pragma unroll
            for (int c = 3; c >= 0; --c) {
                const int idx = elem_index(cb, j, c);
                loc = (f4get(x[j], c) == m && idx < V) ? idx : loc;
            }
        if (m > bv || (m == bv && loc < bi)) { bv = m; bi = loc; }
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) argmax_step(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
    if (lane == 0) { sm.bv[wave] = bv; sm.bi[wave] = bi; }
    __syncthreads();
    float M = sm.bv[0];
    int best = sm.bi[0];
#pragma unroll
    for (int w = 1; w < TNW; ++w) argmax_step(M, best, sm.bv[w], sm.bi[w]);
    auto to_e = [&](auto& x) {
        constexpr int n = (int)(sizeof(x) / sizeof(float4));
#pragma unroll
        for (int j = 0; j < n; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) f4set(x[j], c, unnorm(f4get(x[j], c), M, ilog));
    };

    // the cut: one streamed pass per level
    for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int) { to_e(x); topp_accumulate<0, HB>(x, 0u, sm); });
    const double need = topp_scan<0>(0.0, P.top_p, sm);
    const uint32_t b1 = (uint32_t)sm.sel_bucket[0];
    const unsigned long long a1 = sm.sel_above[0];
    // the level-2 pass also lists each wave's elements in bucket b1; level 3
    // then reads the list, and only a wave whose list overflowed streams its
    // part of the row once more
    uint32_t nlist = 0;
    for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int) {
        to_e(x);
        topp_accumulate<1, HB>(x, b1, sm);
        nlist = topp_compact<HB>(x, b1, sm.list[wave], nlist);
    });
    topp_scan<1>(need - (double)a1, P.top_p, sm);
    const uint32_t b2 = (uint32_t)sm.sel_bucket[1];
    const unsigned long long a2 = sm.sel_above[1];
    const uint32_t p2 = (b1 << 10) | b2;
    if (nlist <= (uint32_t)kListCap)
        topp_accumulate_list<2>(sm.list[wave], nlist, p2, sm);
    else
        for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int) { to_e(x); topp_accumulate<2, HB>(x, p2, sm); });
    topp_scan<2>(need - (double)a1 - (double)a2, P.top_p, sm);
    Nucleus nu;
    nu.thr = (b1 << 20) | (b2 << 10) | (uint32_t)sm.sel_bucket[2];
    nu.cutoff = INT_MAX;
    const unsigned long long above = a1 + a2 + sm.sel_above[2];
    unsigned long long kept = sm.sel_mass[2];
    const unsigned long long tie_mass = fixmass(__uint_as_float(nu.thr));
    if (tie_mass > 0) {
        const unsigned long long ties = kept / tie_mass;
        long long k = (long long)ceil((need - (double)above) / (double)tie_mass);
        if (k < 1) k = 1;
        if (ties > 1 && (unsigned long long)k < ties) {
            // ties straddle the cut: ties per chunk, then the smallest cutoff c
            // with #ties(id < c) >= k by bisection inside the chunk holding
            // the k-th tie (block counts, alternating buffers)
            for_each_chunk<HB>(row, V, aligned, [&](float4 (&x)[HB], int cb) {
                to_e(x);
                unsigned long long cnt = 0;
#pragma unroll
                for (int j = 0; j < HB; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (elem_index(cb, j, c) < V && __float_as_uint(f4get(x[j], c)) == nu.thr) ++cnt;
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
            to_e(e);
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
                for (int w = 0; w < TNW; ++w) tot += sm.cnt[par][w];
                par ^= 1;
                if (tot >= (unsigned long long)k) hi = mid; else lo = mid + 1;
            }
            nu.cutoff = lo + 1;
            kept = (unsigned long long)k * tie_mass;
        }
    }
    if (tid == 0) {
        RowStat st;
        st.zmax = M;
        st.argmax = best;
        st.thr = nu.thr;
        st.cutoff = nu.cutoff;
        st.Z = (double)(above + kept) * (1.0 / (double)kFix);
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
