// Block-wide helpers for the row kernels (wave64, gfx950; 1024 threads unless
// a helper takes the workgroup size): deterministic reductions and scans,
// register-resident logits chunks, the top-p membership test and the
// inverse-CDF search.  Internal to the library.
//
// Element layout of a chunk: thread t holds float4 slots j = 0..VPT4-1 at
// token ids cb + 4*(t + NT*j) + e, so (j, t, e) order is token-id order and
// every slot is one coalesced 16 KB read by the workgroup.
#pragma once

#include <limits.h>

#include "device_common.h"
#include "kernels.h"

namespace sv {
namespace rows {

constexpr int NT = kVocabThreads;
constexpr int NW = NT / kWave;
constexpr int VPT4 = 8;                     // float4 per thread per chunk
constexpr int CHUNK = NT * VPT4 * 4;
static_assert(CHUNK == kVocabChunk, "chunk size");
constexpr int MAX_CHUNKS = 128;

struct Smem {
    double d[NW];
    int i[NW];
    double dpre[NW + 1];
    int ir;
    double chunk_sum[MAX_CHUNKS];
    double slot_part[NW][VPT4];
    double slot_tot[VPT4];
    int winner;
    int found;
};

__device__ __forceinline__ int tid_() { return threadIdx.x; }
__device__ __forceinline__ int lane_() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_() { return threadIdx.x >> 6; }

// element index of (slot j, component e) for this thread in chunk cb
// (TPB threads per workgroup)
template <int TPB = NT>
__device__ __forceinline__ int elem_index(int cb, int j, int e) { return cb + 4 * (tid_() + TPB * j) + e; }

__device__ __forceinline__ float f4get(const float4& v, int e) {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}
__device__ __forceinline__ void f4set(float4& v, int e, float x) {
    if (e == 0) v.x = x; else if (e == 1) v.y = x; else if (e == 2) v.z = x; else v.w = x;
}

// Block maximum: each wave reduces, wave 0 reduces the wave results and
// broadcasts (two barriers).
__device__ __forceinline__ int block_max_int(int v, Smem& sm) {
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

// Inclusive scan of v over thread order; *excl receives the exclusive prefix.
// Adjacent threads' bounds are bitwise equal (incl_t == excl_{t+1}): wave
// offsets are accumulated sequentially from the waves' last inclusive values.
__device__ __forceinline__ double block_scan_d(double v, double* excl, Smem& sm) {
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

// Row pointer and chunk base in scalar registers (they are the same in every
// lane), so the per-slot resources below are built by scalar arithmetic.
__device__ __forceinline__ uint64_t uniform_addr(const float* row) {
    const uint64_t a = (uint64_t)(uintptr_t)row;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Buffer resource for floats first..V-1 of the row at scalar address a (none
// left past the end).  Loads through it use only a lane offset and the
// immediate offset, the parts the hardware checks against the resource size:
// a read at or past V returns 0 without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tail_rsrc(uint64_t a, int V, int first) {
    const int bytes = V > first ? (V - first) * 4 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a + 4ull * (uint64_t)(uint32_t)first), 0, bytes, 0x00020000);
}

// Issue the loads of chunk cb of a row: whole float4s when the row is
// 16-byte aligned and V is a multiple of 4 (the choice is the same for the
// whole workgroup), else single floats.  Each slot j has a resource based at
// its first float (cb + 4 NT j), so one lane offset serves every load and
// reads past the row return 0 (mask_chunk replaces them): a chunk past the
// end may be loaded too.  There is no branch between the loads: all of them
// are in flight before the first is used.
template <int N = VPT4, int TPB = NT>
__device__ __forceinline__ void issue_chunk(const float* row, int V, int cb, bool aligned, float4 (&x)[N]) {
    const uint64_t a = uniform_addr(row);
    const int c0 = __builtin_amdgcn_readfirstlane(cb);
    const int vo = 16 * tid_();
    if (aligned && (V & 3) == 0) {
#pragma unroll
        for (int j = 0; j < N; ++j)
            x[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(tail_rsrc(a, V, c0 + 4 * TPB * j), vo, 0, 0));
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const __amdgpu_buffer_rsrc_t rs = tail_rsrc(a, V, c0 + 4 * TPB * j);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f4set(x[j], e, __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 4 * e, 0, 0)));
        }
    }
}

// Entries of the block at cb past V become -inf (nothing to do for a full block).
template <int N = VPT4, int TPB = NT>
__device__ __forceinline__ void mask_chunk(int V, int cb, float4 (&x)[N]) {
    if (cb + TPB * N * 4 <= V) return;
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (elem_index<TPB>(cb, j, e) >= V) f4set(x[j], e, -INFINITY);
}

// Load chunk cb of a row (N float4 per thread, TPB threads): out-of-range entries become -inf.
template <int N = VPT4, int TPB = NT>
__device__ __forceinline__ void load_chunk(const float* row, int V, int cb, bool aligned, float4 (&x)[N]) {
    issue_chunk<N, TPB>(row, V, cb, aligned, x);
    mask_chunk<N, TPB>(V, cb, x);
}

// f(x, cb) for every block of N float4 per thread (4 N TPB ids at cb) of a
// row in order, each next block's loads in flight while f runs (loaded
// unconditionally: a conditional load would make the compiler's later waits
// count as if it had not been issued).
template <int N = VPT4, int TPB = NT, class F>
__device__ __forceinline__ void for_each_chunk(const float* row, int V, bool aligned, F&& f) {
    constexpr int STEP = 4 * TPB * N;
    float4 xa[N], xb[N];
    issue_chunk<N, TPB>(row, V, 0, aligned, xa);
    for (int cb = 0; cb < V; cb += 2 * STEP) {
        issue_chunk<N, TPB>(row, V, cb + STEP, aligned, xb);
        mask_chunk<N, TPB>(V, cb, xa);
        f(xa, cb);
        if (cb + STEP >= V) break;
        issue_chunk<N, TPB>(row, V, cb + 2 * STEP, aligned, xa);
        mask_chunk<N, TPB>(V, cb + STEP, xb);
        f(xb, cb + STEP);
    }
}

// Unnormalised probability of a logit: exp((z - zmax) / temperature), by the
// hardware base-2 exponential (results below 2^-126, far under any weight a
// decision can resolve, may flush to zero).  Every kernel computes it here.
__device__ __forceinline__ float unnorm(float z, float zmax, float ilog) {
    return __builtin_amdgcn_exp2f((z - zmax) * ilog);
}

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

// Without top-p the cut keeps every token (thr 0, no tie cutoff): the
// membership test can be skipped.
__device__ __forceinline__ bool keeps_all(const Nucleus& nu) { return nu.thr == 0u && nu.cutoff == INT_MAX; }


// Totals of the weights of every slot j (token ids cb + 4*(t + NT*j) + e over
// all threads t), all slots in one reduction: stored in sm.slot_tot[j]; the
// chunk total (fp64, fixed order) is returned.
__device__ __forceinline__ double slot_totals(const float4 (&w)[VPT4], Smem& sm) {
    double sj[VPT4];
#pragma unroll
    for (int j = 0; j < VPT4; ++j)
        sj[j] = wave_sum_d(((double)w[j].x + (double)w[j].y) + ((double)w[j].z + (double)w[j].w));
    if (lane_() == 0)
#pragma unroll
        for (int j = 0; j < VPT4; ++j) sm.slot_part[wave_()][j] = sj[j];
    __syncthreads();
    if (tid_() < VPT4) {
        double t = 0.0;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) t += sm.slot_part[w2][tid_()];
        sm.slot_tot[tid_()] = t;
    }
    __syncthreads();
    double total = 0.0;
#pragma unroll
    for (int j = 0; j < VPT4; ++j) total += sm.slot_tot[j];
    return total;
}

// Smallest token id k of this chunk with base + C_k > target (C = prefix sums
// of w in id order within the chunk), or -1 if the chunk does not reach it.
// Needs sm.slot_tot from slot_totals(w) on the same weights.
__device__ __forceinline__ int locate_in_chunk(const float4 (&w)[VPT4], int cb, int V, double base, double target, Smem& sm) {
    double cum = base;
    int jstar = -1;
#pragma unroll
    for (int j = 0; j < VPT4; ++j) {
        const double S = sm.slot_tot[j];
        if (jstar < 0) {
            if (cum + S > target) jstar = j;
            else cum += S;
        }
    }
    if (jstar < 0) return -1;
    // component-wise selects keep w in registers (a copy of w[jstar] would
    // need a pointer to a runtime slot, i.e. the array in scratch memory)
    float4 wv = w[0];
#pragma unroll
    for (int j = 1; j < VPT4; ++j) {
        const bool hit = j == jstar;
        wv.x = hit ? w[j].x : wv.x;
        wv.y = hit ? w[j].y : wv.y;
        wv.z = hit ? w[j].z : wv.z;
        wv.w = hit ? w[j].w : wv.w;
    }
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

}  // namespace rows
}  // namespace sv
