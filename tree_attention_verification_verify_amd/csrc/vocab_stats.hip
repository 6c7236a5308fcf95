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
// select on the fp32 bit patterns with integer mass histograms (ten barriers
// in all unless tied probabilities straddle the cut); a longer row is
// streamed once per step of the same cut.  The nucleus normaliser is its
// exact integer mass.

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
                float4, __builtin_amdgcn_raw_buffer_load_b128(rows::tail_rsrc(row_a, V, 4 * (base4 + u * ST)), 16 * tid, 0,
                                                               kStreamPolicy));
            x[4 * u] = v.x; x[4 * u + 1] = v.y; x[4 * u + 2] = v.z; x[4 * u + 3] = v.w;
        }
    };
    auto mask_tail = [&](int base4, float (&x)[4 * U]) {
        if (base4 + U * ST <= nv4) return;   // the whole batch is in range
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base4 + u * ST + tid >= nv4) x[4 * u] = x[4 * u + 1] = x[4 * u + 2] = x[4 * u + 3] = -INFINITY;
    };
    if (nv4 > 0) {   // two register batches in turn (unrolled by two: no copies)
        // the next batch is loaded unconditionally (past the row the loads
        // return 0 and are unused): a conditional load would leave the waits
        // after it counting as if it had not been issued
        float xa[4 * U], xb[4 * U];
        load(0, xa);
        for (int base4 = 0; base4 < nv4; base4 += 2 * U * ST) {
            const int b1 = base4 + U * ST, b2 = base4 + 2 * U * ST;
            load(b1, xb);
            mask_tail(base4, xa);
            absorb(xa, 4 * U, [&](int k) { return 4 * (base4 + (k >> 2) * ST + tid) + (k & 3); });
            if (b1 >= nv4) break;
            load(b2, xa);
            mask_tail(b1, xb);
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

// ---------------------------------------------------------------------------
// Top-p rows.  The row stays in registers; the cut is a 3-level radix select
// (10 bits per level, from the top) on the fp32 patterns of the unnormalised
// probabilities, with exact integer mass histograms.  Each level costs three
// barriers: histogram; scan of the buckets in descending order inside each
// wave; wave offsets read by every thread (integer sums, so any order gives
// the same result) and the crossing bucket published.  The first level sees
// every logit, so its histogram has HK copies (lane & (HK - 1)), interleaved
// per bucket so the copies of one bucket sit in different banks: a wave's
// 64 atomics then collide HK times less on the crowded buckets.
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

// TPB threads per row, N4 = CHUNK / (4 TPB) float4 per thread.  (256
// threads, two rows per CU, measured slower at V = 32000: 39 against 34 us
// for 352 rows; each row's passes then take three times as long.)
template <int TPB>
__global__ __launch_bounds__(TPB) void row_stats_topp_kernel(StatsParams P) {
    using namespace rows;
    __shared__ ToppSmem sm;
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
    load_chunk<N4, TPB>(row, V, 0, aligned, e);
    // cleared histograms are ordered before their atomics by the next barrier
    for (int k = tid; k < 1024 * HK; k += TPB) sm.h1[k] = 0ull;
    for (int k = tid; k < 1024; k += TPB) {
        sm.h2[k] = 0ull;
        sm.h3[k] = 0ull;
    }

    // largest logit and its smallest id (the largest logit is zmax): the
    // thread's maximum, then the first of its positions (in id order) holding it
    float bv = -INFINITY;
#pragma unroll
    for (int j = 0; j < N4; ++j) bv = fmaxf(fmaxf(bv, fmaxf(e[j].x, e[j].y)), fmaxf(e[j].z, e[j].w));
    int bi = INT_MAX;
#pragma unroll
    for (int j = N4 - 1; j >= 0; --j)
#pragma unroll
        for (int c = 3; c >= 0; --c) {
            const int idx = elem_index<TPB>(0, j, c);
            bi = (f4get(e[j], c) == bv && idx < V) ? idx : bi;
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) argmax_step(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
    if (lane == 0) { sm.bv[wave] = bv; sm.bi[wave] = bi; }
    __syncthreads();
    float M = sm.bv[0];
    int best = sm.bi[0];
#pragma unroll
    for (int w = 1; w < NWB; ++w) argmax_step(M, best, sm.bv[w], sm.bi[w]);
#pragma unroll
    for (int j = 0; j < N4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) f4set(e[j], c, unnorm(f4get(e[j], c), M, ilog));

    // the cut
    topp_accumulate<0, N4>(e, 0u, sm);
    const double need = topp_scan<0, TPB>(0.0, P.top_p, sm);
    const uint32_t b1 = (uint32_t)sm.sel_bucket[0];
    const unsigned long long a1 = sm.sel_above[0];
    // levels 2 and 3 only see bucket b1: each wave lists its elements there
    // once (writes and reads of a wave's own list need no barrier) and reads
    // the list, or its registers when the list is too short for them
    // the list space of TNW waves shared by the NWB waves of this row
    constexpr int CAP = TNW * kListCap / NWB;
    uint32_t* const mylist = &sm.list[0][0] + wave * CAP;
    const uint32_t nlist = topp_compact<N4, CAP>(e, b1, mylist);
    const bool listed = nlist <= (uint32_t)CAP;
    if (listed) topp_accumulate_list<1>(mylist, nlist, b1, sm);
    else topp_accumulate<1, N4>(e, b1, sm);
    topp_scan<1, TPB>(need - (double)a1, P.top_p, sm);
    const uint32_t b2 = (uint32_t)sm.sel_bucket[1];
    const unsigned long long a2 = sm.sel_above[1];
    if (listed) topp_accumulate_list<2>(mylist, nlist, (b1 << 10) | b2, sm);
    else topp_accumulate<2, N4>(e, (b1 << 10) | b2, sm);
    topp_scan<2, TPB>(need - (double)a1 - (double)a2, P.top_p, sm);
    Nucleus nu;
    nu.thr = (b1 << 20) | (b2 << 10) | (uint32_t)sm.sel_bucket[2];
    nu.cutoff = INT_MAX;
    // masses above thr, and of the elements at thr (all of the last bucket:
    // (number of ties) * (mass of one))
    const unsigned long long above = a1 + a2 + sm.sel_above[2];
    unsigned long long kept = sm.sel_mass[2];
    const unsigned long long tie_mass = fixmass(__uint_as_float(nu.thr));
    if (tie_mass > 0) {
        const unsigned long long ties = kept / tie_mass;
        long long k = (long long)ceil((need - (double)above) / (double)tie_mass);
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
        // normaliser of the nucleus from its exact fixed-point mass: each
        // element is rounded by at most 2^-41 and the sum holds the top
        // element (e = 1), so the relative error is at most V * 2^-41
        RowStat st;
        st.zmax = M;
        st.argmax = best;
        st.thr = nu.thr;
        st.cutoff = nu.cutoff;
        st.Z = (double)(above + kept) * (1.0 / (double)kFix);
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
