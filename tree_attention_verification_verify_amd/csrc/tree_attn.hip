// Tree-masked attention of the T candidate nodes over the shared KV prefix.
//
// What is computed (flattened tree with a root-path mask: "大模型推理加速：推测
// 解码与MTP核心原理与工程实践" section 3.2; mask: "推测解码技术详解：加速LLM推理的关键"
// section "Tree Attention验证"; no sibling visibility: "投机解码的五条路线"
// section 4): for sequence b, query head h, node i, KV head kv = h / g,
//   keys S = {0..L_b-1} U {L_b + j : j on node i's root path, i included}
//   O[b,i,h] = softmax_S(scale * Q[b,i,h] . K[b,kv,S]) V[b,kv,S]
//
// Work decomposition (ours, for gfx950): one workgroup per (sequence, KV
// head, prefix split, row block).  All g*T query rows that share a KV head
// sit in the same workgroup family, so a K/V tile read from HBM is used by
// every tree node and every query head of the group.  The tree mask is a
// per-node 64-bit ancestor set built in registers from parent[]; only tiles
// that reach slot L_b pay for masking.  Online softmax runs in the log2
// domain; splits are merged by attn_combine_kernel.
//
// MFMA path (bf16, >= 16 rows per KV head): S^T = K Q^T and O^T = V^T P^T
// with v_mfma_f32_32x32x16_bf16, so the query index is the MFMA column and a
// lane owns one query: the softmax rescale of O never leaves the lane.  Keys
// are permuted inside each 32-key sub-tile (bits 2 and 3 of the row index
// swapped) so that the S^T accumulator registers of a lane are exactly the
// P^T operand the PV product needs, and V^T is staged transposed in LDS.
//
// VALU path (fp32, or fewer than 16 rows per KV head): one wave per block;
// QK^T with one lane per key (bf16 dot2 or fp32 FMA), PV with one lane per
// head-dim column; these shapes are HBM-bound, not contraction-bound.

#include "device_common.h"
#include "kernels.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swap_bits_2_3(int x) {
    return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Chunk swizzle of V rows: the 4 consecutive keys one transposed read touches
// land in 4 disjoint quarters of the row's chunk range.
template <int CH>
__device__ __forceinline__ int v_swizzle(int key) { return (key & 3) * (CH / 4); }

// ---------------------------------------------------------------- MFMA path

template <int D, int WAVES, int NSUB>
__global__ __launch_bounds__(WAVES * 64, NSUB == 1 ? 3 : 2) void attn_mfma_kernel(AttnParams P) {
    constexpr int KT = 32 * NSUB;           // keys per tile (NSUB sub-tiles of 32)
    constexpr int CH = D / 8;               // 16-byte chunks per K/V row
    constexpr int KSTEPS = D / 16;          // k-steps of the QK^T product
    constexpr int DT = D / 32;              // 32-row tiles of O^T
    static_assert((KT * D * 2 / 1024) % WAVES == 0, "whole 1 KB blocks per wave");

    __shared__ __align__(16) uint8_t k_lds[2 * KT * D * 2];     // two buffers
    __shared__ __align__(16) uint8_t v_lds[2 * KT * D * 2];
    __shared__ unsigned long long anc_lds[64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int group, rb;
    if (P.rowblocks == 1) {
        group = blockIdx.x;
        rb = 0;
    } else {  // row blocks of one (pair, split) go to the same XCD, back to back
        const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
        rb = local % P.rowblocks;
        group = (local / P.rowblocks) * 8 + xcd;
    }
    if (group >= P.B * P.Hkv * P.nsplit) return;
    const int pair = group / P.nsplit, split = group - pair * P.nsplit;
    const int b = pair / P.Hkv, kvh = pair - b * P.Hkv;
    const int T = P.T, g = P.g;
    const int L = P.kv_len[b];
    const bool kv_ok = (L >= 0) && (L <= P.Lcap - T);
    const int N = L + T;
    const int k0 = split * P.chunk;
    const int k1 = min(N, k0 + P.chunk);
    const int qcol = lane & 31, half = lane >> 5;
    const int r = rb * (WAVES * 32) + wave * 32 + qcol;
    const bool row_ok = r < P.R;
    const int node = row_ok ? r / g : 0;
    const int head = kvh * g + (row_ok ? r - node * g : 0);
    const size_t part_row = (size_t)group * P.Rpad + r;

    if (!kv_ok || k0 >= k1) {
        if (P.nsplit == 1) {
            if (row_ok) {
                uint16_t* o = (uint16_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * D;
                for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) o[d] = 0;
            }
        } else if (row_ok && half == 0) {
            P.part_ml[part_row] = make_float2(-INFINITY, 0.f);
        }
        return;
    }

    if (wave == 0) {
        bool bad;
        unsigned long long a = ancestor_mask(P.parent + (size_t)b * T, T, &bad);
        anc_lds[lane] = a;
    }

    // Q^T operand: lane holds Q[row r][16*ks + 8*half .. +7] for every k-step.
    bf16x8_t qb[KSTEPS];
    {
        const uint16_t* qrow = (const uint16_t*)P.q + ((size_t)(b * T + node) * P.Hq + head) * D;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4*)(qrow + 16 * ks + 8 * half);
            qb[ks] = as_bf16x8(v);
        }
    }
    const uint16_t* kbase = (const uint16_t*)P.k + (size_t)(b * P.Hkv + kvh) * P.Lcap * D;
    const uint16_t* vbase = (const uint16_t*)P.v + (size_t)(b * P.Hkv + kvh) * P.Lcap * D;

    __syncthreads();
    const unsigned long long anc_row = anc_lds[node];

    floatx16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const floatx16_t zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int krow = swap_bits_2_3(qcol);   // key (within a 32-key sub-tile) fed to MFMA row qcol

    // Tile staging, software-pipelined, straight from HBM into LDS: buffer
    // loads with the LDS as destination (each lane's 16 bytes land at the LDS
    // base + 16 * lane) fill the other LDS buffer with tile t+1 while tile t is
    // computed.  The chunk swizzles of the LDS layout (K: chunk ^ key%CH for
    // the MFMA operand reads, V: chunk ^ v_swizzle(key) for the transposed
    // reads) are applied on the global side: lane i of a 1 KB block loads the
    // logical chunk that belongs at its slot.  The buffer resources end at key
    // k1, so loads past the split read zeros (and those keys are masked).
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, k1 * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, k1 * D * 2, 0x00020000);
    constexpr int BLOCKS = KT * D * 2 / 1024;          // 1 KB blocks per tile
    constexpr int ROWS_PER_BLOCK = 1024 / (D * 2);
    auto issue_k = [&](int t, int buf) {
#pragma unroll
        for (int j = 0; j < BLOCKS / WAVES; ++j) {
            const int blk = j * WAVES + wave;
            const int row = blk * ROWS_PER_BLOCK + lane / CH;
            const int kc = (lane % CH) ^ (row & (CH - 1));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                krs, (__attribute__((address_space(3))) void*)(k_lds + buf * (KT * D * 2) + blk * 1024), 16,
                (t + row) * (D * 2) + kc * 16, 0, 0, 0);
        }
    };
    auto issue_v = [&](int t, int buf) {
#pragma unroll
        for (int j = 0; j < BLOCKS / WAVES; ++j) {
            const int blk = j * WAVES + wave;
            const int row = blk * ROWS_PER_BLOCK + lane / CH;
            const int vc = (lane % CH) ^ v_swizzle<CH>(row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vrs, (__attribute__((address_space(3))) void*)(v_lds + buf * (KT * D * 2) + blk * 1024), 16,
                (t + row) * (D * 2) + vc * 16, 0, 0, 0);
        }
    };

    // PV operand by transposed LDS reads (ds_read_b64_tr_b16): within each
    // 16-lane group, source lane s addresses 4 columns (4*(s&3)..+3) of key row
    // s>>2 of a 4-key block, and output lane j receives column j of all 4 keys.
    // Lane l = (G = l>>4, s = l&15) therefore reads key 8*(G>>1) + 4*h + (s>>2)
    // of the 16-key step and columns 32*dt + 16*(G&1) + 4*(s&3); it gets the
    // column 32*dt + (l&31) for keys 8*(l>>5) + 4*h + 0..3: with h = 0, 1 these
    // are the 8 k-slots the P^T operand of the lane holds.
    const int tr_key = 8 * (lane >> 5) + (((lane & 15) >> 2));
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // S^T[KT keys x 32 queries] of one tile (NSUB 32-key sub-tiles).
    auto qk = [&](int kbuf, floatx16_t (&s)[NSUB]) {
        const uint8_t* kl = k_lds + kbuf * (KT * D * 2);
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) {
            const int kk = sub * 32 + krow;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const int c = 2 * ks + half;
                const u32x4 a = *(const u32x4*)(kl + kk * (D * 2) + ((c ^ (kk & (CH - 1))) << 4));
                s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qb[ks], ks == 0 ? zero16 : s[sub],
                                                                 0, 0, 0);
            }
        }
    };

    // Online softmax (log2 domain) of one tile's scores and O^T += V^T P^T.
    // need_mask (wave-uniform): the tile reaches the tree slots or the end of the split.
    auto softmax_pv = [&](int t, int vbuf, floatx16_t (&s)[NSUB], bool need_mask) {
        const uint8_t* vl = v_lds + vbuf * (KT * D * 2);
        // accumulator element e of lane (qcol, half) holds key 16*(e>>3) + 8*half + (e&7) of its sub-tile
        if (need_mask) {
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = t + sub * 32 + 16 * (e >> 3) + 8 * half + (e & 7);
                    const unsigned rel = (unsigned)(key - L);
                    const bool tree_vis = (key < k1) && ((anc_row >> (rel & 63u)) & 1ull);
                    const bool vis = (key < L) | (key >= L && tree_vis);
                    s[sub][e] = vis ? s[sub][e] : -INFINITY;
                }
        }
        float m16[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) m16[e] = NSUB == 1 ? s[0][e] : fmaxf(s[0][e], s[NSUB - 1][e]);
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int e = 0; e < w; ++e) m16[e] = fmaxf(m16[e], m16[e + w]);
        float mx = fmaxf(m16[0], __shfl_xor(m16[0], 32, kWave));
        const float m_new = fmaxf(m_run, mx * P.c);
        if (__any(m_new > m_run)) {       // rescale only when some running max grows
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
            m_run = m_new;
        }
        const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
        float psum = 0.f;
        bf16x8_t pb[NSUB][2];
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                float p[8];
#pragma unroll
                for (int w = 0; w < 8; ++w) p[w] = __builtin_amdgcn_exp2f(fmaf(s[sub][8 * h2 + w], P.c, neg_m));
                psum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                bf16x2_t q0 = __builtin_convertvector((floatx2_t){p[0], p[1]}, bf16x2_t);
                bf16x2_t q1 = __builtin_convertvector((floatx2_t){p[2], p[3]}, bf16x2_t);
                bf16x2_t q2 = __builtin_convertvector((floatx2_t){p[4], p[5]}, bf16x2_t);
                bf16x2_t q3 = __builtin_convertvector((floatx2_t){p[6], p[7]}, bf16x2_t);
                pb[sub][h2] = bf16x8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
            }
        }
        l_run += psum;

        // O^T[d x q] += V^T[d x keys] P^T[keys x q]
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int col = 32 * dt + tr_col;
                    const int key0 = sub * 32 + 16 * h2 + tr_key;
                    const int key1 = key0 + 4;
                    const int c = col >> 3;
                    const uint8_t* p0 = vl + key0 * (D * 2) + ((c ^ v_swizzle<CH>(key0)) << 4) + (col & 7) * 2;
                    const uint8_t* p1 = vl + key1 * (D * 2) + ((c ^ v_swizzle<CH>(key1)) << 4) + (col & 7) * 2;
                    const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
                    const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p1);
                    const v8s a = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), pb[sub][h2],
                                                                    o[dt], 0, 0, 0);
                }
            }
        }
    };

    // Double-buffered: tile t+1 streams into the other LDS buffers while tile t
    // is computed; one barrier per tile.
    floatx16_t s_cur[NSUB];
    issue_k(k0, 0);
    issue_v(k0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int it = 0;
    for (int t = k0; t < k1; t += KT, ++it) {
        const int cur = it & 1;
        if (t + KT < k1) {
            issue_k(t + KT, cur ^ 1);
            issue_v(t + KT, cur ^ 1);
        }
        qk(cur, s_cur);
        softmax_pv(t, cur, s_cur, t + KT > L || t + KT > k1);
        __builtin_amdgcn_s_waitcnt(0);    // tile t+1 has landed
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    if (!row_ok) return;
    // O^T element e of tile dt: column d = 32*dt + 8*(e>>2) + 4*half + (e&3)
    if (P.nsplit == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = (uint16_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int d = 32 * dt + 8 * e4 + 4 * half;
                u32x2 w = {pack_bf16x2(o[dt][4 * e4] * inv, o[dt][4 * e4 + 1] * inv),
                           pack_bf16x2(o[dt][4 * e4 + 2] * inv, o[dt][4 * e4 + 3] * inv)};
                *(u32x2*)(orow + d) = w;
            }
        }
    } else {
        float* prow = P.part_o + part_row * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int d = 32 * dt + 8 * e4 + 4 * half;
                *(floatx4_t*)(prow + d) = floatx4_t{o[dt][4 * e4], o[dt][4 * e4 + 1], o[dt][4 * e4 + 2],
                                                    o[dt][4 * e4 + 3]};
            }
        }
        if (half == 0) P.part_ml[part_row] = make_float2(m_run, l_tot);
    }
}

// ---------------------------------------------------------------- VALU path

template <bool BF16, int D, int MAXR>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnParams P) {
    constexpr int KT = 64;
    constexpr int EB = BF16 ? 2 : 4;
    constexpr int ROWB = D * EB;
    constexpr int CH = ROWB / 16;
    constexpr int DPL = D / 64;             // head-dim columns per lane in PV

    __shared__ __align__(16) uint8_t q_lds[MAXR * ROWB];
    __shared__ __align__(16) uint8_t k_lds[KT * ROWB];
    __shared__ __align__(16) float p_lds[KT * MAXR];
    __shared__ unsigned long long anc_lds[64];

    const int lane = threadIdx.x;
    const int rb = blockIdx.x % P.rowblocks;
    const int group = blockIdx.x / P.rowblocks;
    const int pair = group / P.nsplit, split = group - pair * P.nsplit;
    const int b = pair / P.Hkv, kvh = pair - b * P.Hkv;
    const int T = P.T, g = P.g;
    const int L = P.kv_len[b];
    const bool kv_ok = (L >= 0) && (L <= P.Lcap - T);
    const int N = L + T;
    const int k0 = split * P.chunk;
    const int k1 = min(N, k0 + P.chunk);
    const int rbase = rb * MAXR;

    if (!kv_ok || k0 >= k1) {
        for (int j = 0; j < MAXR; ++j) {
            const int r = rbase + j;
            if (r >= P.R) break;
            const int node = r / g, head = kvh * g + (r - node * g);
            if (P.nsplit == 1) {
                uint8_t* o = (uint8_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * ROWB;
                for (int x = lane; x < ROWB / 4; x += 64) ((uint32_t*)o)[x] = 0u;
            } else if (lane == 0) {
                P.part_ml[(size_t)group * P.Rpad + r] = make_float2(-INFINITY, 0.f);
            }
        }
        return;
    }

    {
        bool bad;
        anc_lds[lane] = ancestor_mask(P.parent + (size_t)b * T, T, &bad);
    }
    for (int idx = lane; idx < MAXR * CH; idx += 64) {
        const int j = idx / CH, c = idx - j * CH;
        const int r = rbase + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < P.R) {
            const int node = r / g, head = kvh * g + (r - node * g);
            v = *(const u32x4*)((const uint8_t*)P.q + ((size_t)(b * T + node) * P.Hq + head) * ROWB + c * 16);
        }
        *(u32x4*)(q_lds + j * ROWB + c * 16) = v;
    }
    __syncthreads();
    unsigned long long anc_r[MAXR];
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        const int r = rbase + j;
        anc_r[j] = anc_lds[r < P.R ? r / g : 0];
    }

    const uint8_t* kbase = (const uint8_t*)P.k + (size_t)(b * P.Hkv + kvh) * P.Lcap * ROWB;
    const uint8_t* vbase = (const uint8_t*)P.v + (size_t)(b * P.Hkv + kvh) * P.Lcap * ROWB;

    float m_run[MAXR], l_run[MAXR], o[MAXR][DPL];
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int x = 0; x < DPL; ++x) o[j][x] = 0.f;
    }

    for (int t = k0; t < k1; t += KT) {
        for (int idx = lane; idx < KT * CH; idx += 64) {
            const int key = idx / CH, c = idx - key * CH;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t + key < k1) v = *(const u32x4*)(kbase + (size_t)(t + key) * ROWB + c * 16);
            *(u32x4*)(k_lds + key * ROWB + ((c ^ (key & (CH - 1))) << 4)) = v;
        }
        __syncthreads();

        // scores: lane = key
        float s[MAXR];
#pragma unroll
        for (int j = 0; j < MAXR; ++j) s[j] = 0.f;
        for (int c = 0; c < CH; ++c) {
            const u32x4 kc = *(const u32x4*)(k_lds + lane * ROWB + ((c ^ (lane & (CH - 1))) << 4));
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {
                const u32x4 qc = *(const u32x4*)(q_lds + j * ROWB + c * 16);
                if constexpr (BF16) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        // copy the lanes out of the vectors first: a bit_cast of a vector
                        // element is lowered as a cast of element 0 by this compiler
                        const uint32_t qw = qc[w], kw = kc[w];
                        s[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw),
                                                               __builtin_bit_cast(bf16x2_t, kw), s[j], false);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) s[j] = fmaf(__uint_as_float(qc[w]), __uint_as_float(kc[w]), s[j]);
                }
            }
        }

        const int key = t + lane;
        const bool tail = key >= L;
#pragma unroll
        for (int j = 0; j < MAXR; ++j) {
            float val = s[j] * P.c;
            const bool vis = key < k1 && (!tail || ((anc_r[j] >> (key - L)) & 1ull));
            if (!vis) val = -INFINITY;
            const float mx = wave_max(val);
            const float m_new = fmaxf(m_run[j], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run[j] - m_use);
            const float p = exp2f(val - m_use);
            m_run[j] = m_new;
            l_run[j] = l_run[j] * alpha + p;
#pragma unroll
            for (int x = 0; x < DPL; ++x) o[j][x] *= alpha;
            p_lds[lane * MAXR + j] = p;
        }
        __syncthreads();

        // PV: lane owns head-dim columns lane*DPL .. +DPL-1
        const int nk = min(KT, k1 - t);
        for (int kk = 0; kk < nk; ++kk) {
            float v[DPL];
            const uint8_t* vrow = vbase + (size_t)(t + kk) * ROWB;
            if constexpr (BF16) {
                if constexpr (DPL == 2) {
                    const uint32_t w = *(const uint32_t*)(vrow + lane * 4);
                    v[0] = bf16_lo(w);
                    v[1] = bf16_hi(w);
                } else {
                    v[0] = __uint_as_float(((uint32_t) * (const uint16_t*)(vrow + lane * 2)) << 16);
                }
            } else {
#pragma unroll
                for (int x = 0; x < DPL; ++x) v[x] = *(const float*)(vrow + (lane * DPL + x) * 4);
            }
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {
                const float p = p_lds[kk * MAXR + j];
#pragma unroll
                for (int x = 0; x < DPL; ++x) o[j][x] = fmaf(p, v[x], o[j][x]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        const float l_tot = wave_sum(l_run[j]);
        const int r = rbase + j;
        if (r >= P.R) continue;
        const int node = r / g, head = kvh * g + (r - node * g);
        if (P.nsplit == 1) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            uint8_t* orow = (uint8_t*)P.out + ((size_t)(b * T + node) * P.Hq + head) * ROWB;
#pragma unroll
            for (int x = 0; x < DPL; ++x) {
                const int d = lane * DPL + x;
                if constexpr (BF16)
                    ((uint16_t*)orow)[d] = (uint16_t)f32_to_bf16_bits(o[j][x] * inv);
                else
                    ((float*)orow)[d] = o[j][x] * inv;
            }
        } else {
            const size_t prow = (size_t)group * P.Rpad + r;
#pragma unroll
            for (int x = 0; x < DPL; ++x) P.part_o[prow * D + lane * DPL + x] = o[j][x];
            if (lane == 0) P.part_ml[prow] = make_float2(m_run[j], l_tot);
        }
    }
}

// ---------------------------------------------------------------- split merge

template <bool BF16, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams P) {
    constexpr int DPL = D / 64;
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long pairs = (long)P.B * P.Hkv;
    if (row >= pairs * P.R) return;
    const int pair = (int)(row / P.R), r = (int)(row - (long)pair * P.R);
    const int b = pair / P.Hkv, kvh = pair - b * P.Hkv;
    const int node = r / P.g, head = kvh * P.g + (r - node * P.g);

    float mmax = -INFINITY;
    for (int s = 0; s < P.nsplit; ++s) {
        const float2 ml = P.part_ml[((size_t)pair * P.nsplit + s) * P.Rpad + r];
        if (ml.y > 0.f) mmax = fmaxf(mmax, ml.x);
    }
    float lsum = 0.f, acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
    for (int s = 0; s < P.nsplit; ++s) {
        const size_t prow = ((size_t)pair * P.nsplit + s) * P.Rpad + r;
        const float2 ml = P.part_ml[prow];
        if (!(ml.y > 0.f)) continue;
        const float w = exp2f(ml.x - mmax);
        lsum += ml.y * w;
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[x] = fmaf(P.part_o[prow * D + lane * DPL + x], w, acc[x]);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const size_t obase = ((size_t)(b * P.T + node) * P.Hq + head) * D + lane * DPL;
#pragma unroll
    for (int x = 0; x < DPL; ++x) {
        if constexpr (BF16)
            ((uint16_t*)P.out)[obase + x] = (uint16_t)f32_to_bf16_bits(acc[x] * inv);
        else
            ((float*)P.out)[obase + x] = acc[x] * inv;
    }
}

template <bool BF16, int D>
hipError_t launch_valu_rows(const AttnParams& p, int maxr, dim3 grid, hipStream_t s) {
    switch (maxr) {
        case 2: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 2>), grid, dim3(64), 0, s, p); break;
        case 4: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 4>), grid, dim3(64), 0, s, p); break;
        case 6: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 6>), grid, dim3(64), 0, s, p); break;
        case 8: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 8>), grid, dim3(64), 0, s, p); break;
        case 12: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 12>), grid, dim3(64), 0, s, p); break;
        default: hipLaunchKernelGGL((attn_valu_kernel<BF16, D, 16>), grid, dim3(64), 0, s, p); break;
    }
    return hipGetLastError();
}

}  // namespace

int valu_rows_for(int R) {
    if (R <= 2) return 2;
    if (R <= 4) return 4;
    if (R <= 6) return 6;
    if (R <= 8) return 8;
    if (R <= 12) return 12;
    return kValuRows;
}

hipError_t launch_attention_mfma(const AttnParams& p, int waves, hipStream_t s) {
    const int groups = p.B * p.Hkv * p.nsplit;
    int blocks;
    if (p.rowblocks == 1) blocks = groups;
    else blocks = ((groups + 7) / 8) * 8 * p.rowblocks;
    dim3 grid(blocks);
    constexpr int S = kAttnSubTiles;
    if (p.D == 128) {
        if (waves == 4) hipLaunchKernelGGL((attn_mfma_kernel<128, 4, S>), grid, dim3(256), 0, s, p);
        else if (waves == 2) hipLaunchKernelGGL((attn_mfma_kernel<128, 2, S>), grid, dim3(128), 0, s, p);
        else hipLaunchKernelGGL((attn_mfma_kernel<128, 1, S>), grid, dim3(64), 0, s, p);
    } else {
        if (waves == 4) hipLaunchKernelGGL((attn_mfma_kernel<64, 4, S>), grid, dim3(256), 0, s, p);
        else if (waves == 2) hipLaunchKernelGGL((attn_mfma_kernel<64, 2, S>), grid, dim3(128), 0, s, p);
        else hipLaunchKernelGGL((attn_mfma_kernel<64, 1, S>), grid, dim3(64), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_attention_valu(const AttnParams& p, bool bf16, hipStream_t s) {
    dim3 grid(p.B * p.Hkv * p.nsplit * p.rowblocks);
    const int maxr = p.Rpad / p.rowblocks;
    if (bf16) return p.D == 128 ? launch_valu_rows<true, 128>(p, maxr, grid, s)
                                : launch_valu_rows<true, 64>(p, maxr, grid, s);
    return p.D == 128 ? launch_valu_rows<false, 128>(p, maxr, grid, s)
                      : launch_valu_rows<false, 64>(p, maxr, grid, s);
}

hipError_t launch_attention_combine(const AttnParams& p, bool bf16, hipStream_t s) {
    const long rows = (long)p.B * p.Hkv * p.R;
    dim3 grid((unsigned)((rows + 3) / 4));
    if (bf16) {
        if (p.D == 128) hipLaunchKernelGGL((attn_combine_kernel<true, 128>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((attn_combine_kernel<true, 64>), grid, dim3(256), 0, s, p);
    } else {
        if (p.D == 128) hipLaunchKernelGGL((attn_combine_kernel<false, 128>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((attn_combine_kernel<false, 64>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace sv
