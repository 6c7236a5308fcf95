// Device helpers shared by the verify-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace sv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}


// Data-parallel-primitive lane moves (gfx9 DPP controls): lanes without a
// source, and rows outside ROWS, read 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)v), hi = dpp_u32<CTRL, ROWS>((uint32_t)(v >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ double dpp_d(double v) {
    return __builtin_bit_cast(double, dpp_u64<CTRL, ROWS>(__builtin_bit_cast(unsigned long long, v)));
}

// Inclusive scan over the 64 lanes of a wave in VALU: shifts by 1, 2, 4, 8
// inside each row of 16 lanes (row_shr), then the last lane of row 0 into
// row 1 and of row 2 into row 3 (row_bcast:15), then lane 31 into rows 2 and
// 3 (row_bcast:31).  Integer sums: exact in any order.
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long x) {
    x += dpp_u64<0x111>(x);
    x += dpp_u64<0x112>(x);
    x += dpp_u64<0x114>(x);
    x += dpp_u64<0x118>(x);
    x += dpp_u64<0x142, 0xa>(x);
    x += dpp_u64<0x143, 0xc>(x);
    return x;
}

// The same scan of doubles (a fixed order of additions per lane, so the same
// bits on every run).
__device__ __forceinline__ double wave_scan_d(double x) {
    x += dpp_d<0x111>(x);
    x += dpp_d<0x112>(x);
    x += dpp_d<0x114>(x);
    x += dpp_d<0x118>(x);
    x += dpp_d<0x142, 0xa>(x);
    x += dpp_d<0x143, 0xc>(x);
    return x;
}

__device__ __forceinline__ unsigned long long lane63_u64(unsigned long long v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, kWave - 1);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), kWave - 1);
    return ((unsigned long long)hi << 32) | lo;
}

// Wave totals, the same in every lane: the last lane of the scan.
__device__ __forceinline__ double wave_sum_d(double v) {
    return __builtin_bit_cast(double, lane63_u64(__builtin_bit_cast(unsigned long long, wave_scan_d(v))));
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) { return lane63_u64(wave_scan_u64(v)); }

// Cache-policy operand of the buffer loads that stream data read once (K/V
// tiles that no other workgroup reads, logits rows of the row statistics):
// the non-temporal bit.  Measured against the default policy: the steps at
// the long-context and batch-32 chain shapes 9% faster (their attention is
// HBM-bound), the row statistics at the 70B GQA tree shape 11% faster.
constexpr int kStreamPolicy = 2;

// Sequence handled by the workgroups of rank r when a grid is ordered by
// decreasing kv_len (ties by index), so that the longest prefixes start
// first and the shortest fill the tail: with more workgroups than fit on the
// GPU at once, a long prefix started last would otherwise run on alone.  One
// wave ranks up to 64 sequences (each lane one, the others' lengths
// broadcast in turn); larger batches keep the index order.  Returns the
// sequence and its kv_len (one load either way); every wave that calls it
// gets the same answer.
__device__ __forceinline__ int2 seq_by_length(const int* kv_len, int B, int r) {
    if (B <= 1 || B > kWave) return make_int2(r, kv_len[r]);
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane < B ? kv_len[lane] : 0;
    int rank = 0;
    for (int j = 0; j < B; ++j) {
        const int lj = __builtin_amdgcn_readlane(li, j);
        rank += (lj > li || (lj == li && j < lane)) ? 1 : 0;
    }
    const unsigned long long m = __ballot(lane < B && rank == r);
    const int b = m ? __builtin_ctzll(m) : r;
    return make_int2(b, __builtin_amdgcn_readlane(li, b));
}

// Arrival count of a group of G workgroups at a per-group counter: true for
// the G-th arrival.  The increment wraps to 0 in the same atomic (an old
// value >= G-1 becomes 0), so no reset store follows and the counter stays in
// [0, G): every completed group leaves it where it was, and calls that were
// (wrongly) interleaved leave it at 0 again once all their workgroups have
// counted, instead of poisoning every later call.  The caller makes its
// published stores land before it counts (vmcnt(0) and a barrier).
__device__ __forceinline__ bool arrive_last(int32_t* counter, int G) {
    const uint32_t old = __builtin_amdgcn_atomic_inc32((uint32_t*)counter, (uint32_t)(G - 1), __ATOMIC_RELAXED, "agent");
    return old == (uint32_t)(G - 1);
}

// Per-node ancestor bitmasks anc*(i) (bit j set iff node j is on node i's
// root path, i itself included), by pointer jumping over parent[] in one
// wave: after k rounds each node has collected 2^k nodes of its chain, so 6
// rounds cover any depth below 64.  Lane i handles node i (T <= 64).  Nodes
// whose parent entry is invalid (root not -1, or not 0 <= parent[i] < i) get
// only their own bit; *bad is set for the whole wave in that case.
// p_in: parent[lane] as loaded by the caller (ignored for lanes >= T).
__device__ __forceinline__ unsigned long long ancestor_mask_of(int p_in, int T, bool* bad) {
    const int lane = threadIdx.x & (kWave - 1);
    int p = -1;
    bool invalid = false;
    if (lane < T) {
        p = p_in;
        if (lane == 0) invalid = (p != -1);
        else invalid = (p < 0 || p >= lane);
        if (invalid) p = -1;
    }
    unsigned long long a = (lane < T) ? (1ull << lane) : 0ull;
#pragma unroll
    for (int round = 0; round < 6; ++round) {
        const int src = p < 0 ? lane : p;
        unsigned long long pa = __shfl(a, src, kWave);
        int pp = __shfl(p, src, kWave);
        if (p >= 0) {
            a |= pa;
            p = pp;
        }
    }
    *bad = __any(invalid);
    return a;
}

__device__ __forceinline__ unsigned long long ancestor_mask(const int32_t* parent_row, int T, bool* bad) {
    const int lane = threadIdx.x & (kWave - 1);
    return ancestor_mask_of(lane < T ? parent_row[lane] : -1, T, bad);
}

// Paged caches: whether some block-table entry of sequence b's slots
// 0..n_slots-1 lies outside the pool, for the entries j = first, first + step,
// ... this thread checks (the caller combines the threads' answers).  The
// caller has checked n_slots <= width << bs_log2, so the row is not overrun.
// Dense caches (no table): false.
__device__ __forceinline__ bool page_entries_bad(const PageTable& pt, int b, int n_slots, int first, int step) {
    if (!pt.table) return false;
    const int used = (n_slots + (1 << pt.bs_log2) - 1) >> pt.bs_log2;
    const int32_t* row = pt.table + (size_t)b * pt.width;
    bool bad = false;
#pragma unroll 8
    for (int j = first; j < used; j += step) {
        const int e = row[j];
        bad |= (e < 0) | (e >= pt.num_blocks);
    }
    return bad;
}

}  // namespace sv
