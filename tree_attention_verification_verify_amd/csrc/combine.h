// Merge of split-prefix attention partials (internal to libspecverify).
//
// A row's splits s hold O_s (unnormalised), m_s (running max, log2 units) and
// l_s (row sum); the merged row is sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s over splits that saw a key (the usual log-sum-exp merge).
// One thread per 8 consecutive head-dim columns of a row (two float4 reads
// per split, one 16-byte store of bf16 or two of fp32): D/8 threads per row,
// 256/(D/8) rows per 256-thread block.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace sv {

template <int D>
constexpr int combine_rows_per_block() { return 256 / (D / 8); }

// Up to this many splits a thread loads all of its partials at once.
constexpr int kCombineMaxSplits = 8;

// Merge of NS splits of one row slice: every split's (m, l) and columns are
// loaded before any is used (one round trip to memory instead of one per
// split); a split that saw no key holds no columns and is skipped.
template <int NS, int D>
__device__ __forceinline__ void combine_fixed(const AttnParams& P, int pair, int r, int d0, float& lsum, floatx4_t& a0,
                                              floatx4_t& a1) {
    float2 ml[NS];
    floatx4_t o0[NS], o1[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const size_t prow = ((size_t)pair * NS + s) * P.Rpad + r;
        ml[s] = P.part_ml[prow];
        const floatx4_t* src = (const floatx4_t*)(P.part_o + prow * D + d0);
        o0[s] = src[0];
        o1[s] = src[1];
    }
    float mmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (ml[s].y > 0.f) mmax = fmaxf(mmax, ml[s].x);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (ml[s].y > 0.f) {
            const float w = exp2f(ml[s].x - mmax);
            lsum += ml[s].y * w;
            a0 += w * o0[s];
            a1 += w * o1[s];
        }
    }
}

// Merge block `blk` run by 256 threads, t = 0..255 this thread's index among them.
template <bool BF16, int D>
__device__ __forceinline__ void combine_block(const AttnParams& P, long blk, int t) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int TPR = D / 8;
    constexpr int RPB = 256 / TPR;
    const long row = (long)blk * RPB + t / TPR;
    const int d0 = (t % TPR) * 8;
    const long pairs = (long)P.B * P.Hkv;
    if (row >= pairs * P.R) return;
    const int pair = (int)(row / P.R), r = (int)(row - (long)pair * P.R);
    const int b = pair / P.Hkv, kvh = pair - b * P.Hkv;
    const int node = r / P.g, head = kvh * P.g + (r - node * P.g);

    float lsum = 0.f;
    floatx4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    if (P.nsplit <= kCombineMaxSplits) {
        switch (P.nsplit) {
            case 1: combine_fixed<1, D>(P, pair, r, d0, lsum, a0, a1); break;
            case 2: combine_fixed<2, D>(P, pair, r, d0, lsum, a0, a1); break;
            case 3: combine_fixed<3, D>(P, pair, r, d0, lsum, a0, a1); break;
            case 4: combine_fixed<4, D>(P, pair, r, d0, lsum, a0, a1); break;
            case 5: combine_fixed<5, D>(P, pair, r, d0, lsum, a0, a1); break;
            case 6: combine_fixed<6, D>(P, pair, r, d0, lsum, a0, a1); break;
            case 7: combine_fixed<7, D>(P, pair, r, d0, lsum, a0, a1); break;
            default: combine_fixed<8, D>(P, pair, r, d0, lsum, a0, a1); break;
        }
    } else {
        float mmax = -INFINITY;
        for (int s = 0; s < P.nsplit; ++s) {
            const float2 ml = P.part_ml[((size_t)pair * P.nsplit + s) * P.Rpad + r];
            if (ml.y > 0.f) mmax = fmaxf(mmax, ml.x);
        }
        for (int s = 0; s < P.nsplit; ++s) {
            const size_t prow = ((size_t)pair * P.nsplit + s) * P.Rpad + r;
            const float2 ml = P.part_ml[prow];
            if (!(ml.y > 0.f)) continue;
            const float w = exp2f(ml.x - mmax);
            lsum += ml.y * w;
            const floatx4_t* src = (const floatx4_t*)(P.part_o + prow * D + d0);
            a0 += w * src[0];
            a1 += w * src[1];
        }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    a0 *= inv;
    a1 *= inv;
    const size_t obase = ((size_t)(b * P.T + node) * P.Hq + head) * D + d0;
    if constexpr (BF16) {
        const u32x4_t w = {pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]), pack_bf16x2(a1[0], a1[1]),
                           pack_bf16x2(a1[2], a1[3])};
        *(u32x4_t*)((uint16_t*)P.out + obase) = w;
    } else {
        floatx4_t* dst = (floatx4_t*)((float*)P.out + obase);
        dst[0] = a0;
        dst[1] = a1;
    }
}

}  // namespace sv
