// Tree-masked attention on the vector ALU for few query rows per KV head.
//
// What is computed is the same as in tree_attn.hip (flattened candidate tree
// with a root-path mask: "大模型推理加速：推测解码与MTP核心原理与工程实践" section 3.2;
// "推测解码技术详解：加速LLM推理的关键" section "Tree Attention验证"; no sibling
// visibility: "投机解码的五条路线" section 4).  This kernel serves shapes with at
// most 8 query rows per KV head (chains, or trees without grouped heads) whose
// K/V rows are at most 256 bytes: too thin a contraction for the matrix cores,
// so the work is HBM-bound and the kernel is built to keep tile loads in
// flight.
//
// Work decomposition (ours, for gfx950): one workgroup of 4 waves per
// (sequence, KV head, prefix split).  64-key K and V tiles are staged into LDS
// by buffer loads with an LDS destination, double-buffered one tile ahead;
// wave w takes keys 16w..16w+15 of every tile.  QK^T: lane = 4 * key + quarter,
// each lane holds its quarter of every query row in registers and reduces the
// four quarters by two lane exchanges; softmax is online per wave with a
// lazily raised reference (raised only when a score exceeds it by more than
// 2^8 in the exp2 domain); PV: lane = D/64 head-dim columns, weights read back
// from LDS.  The four waves' (O, m, l) merge through LDS at the end; prefix
// splits are merged by the finishing launch (combine.h).

#include "device_common.h"
#include "kernels.h"
#include "stats_stream.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int VW = 4;            // waves per workgroup
constexpr int VKT = 64;          // keys per tile
constexpr int VKW = VKT / VW;    // keys per wave per tile
constexpr float kLazyRef = 8.f;  // log2 headroom of the lazily raised reference

// STREAM: non-temporal K/V tile loads.  FUSE: workgroups from attn_blocks on
// compute the streaming row statistics of S instead (one per logits row).
template <bool BF16, int D, int MAXR, bool PAGED, bool STREAM, bool FUSE = false>
__global__ __launch_bounds__(VW * 64, 2) void attn_valu_tiled_kernel(AttnParams P, StatsParams S, int attn_blocks) {
    if constexpr (FUSE) {
        static_assert(VW * 64 == kStatsThreads, "row statistics workgroups of 256 threads");
        if ((int)blockIdx.x >= attn_blocks) {
            if (S.sampling) row_stats_stream_block<true>(S, (int)blockIdx.x - attn_blocks);
            else row_stats_stream_block<false>(S, (int)blockIdx.x - attn_blocks);
            return;
        }
    }
    constexpr int EB = BF16 ? 2 : 4;
    constexpr int ROWB = D * EB;              // bytes per K/V row
    static_assert(ROWB == 128 || ROWB == 256, "K/V rows of 128 or 256 bytes");
    constexpr int CH = ROWB / 16;             // 16-byte chunks per row
    constexpr int QCH = CH / 4;               // chunks of a quarter row (QK operand per lane)
    constexpr int TILEB = VKT * ROWB;         // bytes per K or V tile
    constexpr int RPB = 1024 / ROWB;          // rows per 1 KB staging block
    constexpr int LPW = TILEB / 1024 / VW;    // blocks per wave per operand and tile
    constexpr int CPB = ROWB / 64;            // bytes of a V row per lane in PV
    constexpr int CPL = CPB / EB;             // head-dim columns per lane in PV

    __shared__ __align__(16) uint8_t k_lds0[TILEB];
    __shared__ __align__(16) uint8_t k_lds1[TILEB];
    __shared__ __align__(16) uint8_t v_lds0[TILEB];
    __shared__ __align__(16) uint8_t v_lds1[TILEB];
    __shared__ __align__(16) float p_lds[VW][VKW][MAXR];   // each wave's weights, [key][row]
    __shared__ unsigned long long anc_lds[64];
    __shared__ float2 ml_lds[VW][MAXR];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroups in order of decreasing prefix length (longest first); group
    // is the (sequence, KV head, split) slot of the partial results
    const int pair0 = blockIdx.x / P.nsplit, split = blockIdx.x - pair0 * P.nsplit;
    const int rank = pair0 / P.Hkv, kvh = pair0 - rank * P.Hkv;
    const int2 bl = seq_by_length(P.kv_len, P.B, rank);
    const int b = bl.x, L = bl.y;
    const int pair = b * P.Hkv + kvh;
    const int group = pair * P.nsplit + split;
    const int T = P.T, g = P.g, R = P.R;
    bool kv_ok = (L >= 0) && (L <= P.Lcap - T);
    const int N = L + T;
    if constexpr (PAGED) {
        const bool bad = kv_ok && page_entries_bad(P.pt, b, N, tid, VW * 64);
        kv_ok = kv_ok && !__syncthreads_or(bad);
    }
    const int k0 = split * P.chunk;
    const int k1 = min(N, k0 + P.chunk);
    auto out_row = [&](int r) -> size_t {   // element offset of query row r's output
        const int node = r / g;
        return ((size_t)(b * T + node) * P.Hq + kvh * g + (r - node * g)) * D;
    };

    if (!kv_ok || k0 >= k1) {
        if (P.nsplit == 1) {
            for (int x = tid; x < R * (ROWB / 4); x += VW * 64) {
                const int r = x / (ROWB / 4), w = x - r * (ROWB / 4);
                ((uint32_t*)((uint8_t*)P.out + out_row(r) * EB))[w] = 0u;
            }
        } else if (tid < R) {
            P.part_ml[(size_t)group * P.Rpad + tid] = make_float2(-INFINITY, 0.f);
        }
        return;
    }
    if (tid < kWave) {
        bool bad;
        anc_lds[lane] = ancestor_mask(P.parent + (size_t)b * T, T, &bad);
    }

    // Staging: block load l of a tile (l < LPW: K, else V); lane i of a 1 KB
    // block fills LDS slot i.  K rows carry a chunk swizzle (slot c of row r
    // holds chunk c ^ (r % CH)) so the quarter-row reads of QK^T spread over
    // the banks; V rows are stored as they are.  The resources end at key k1:
    // rows past the split read zeros.
    constexpr uint32_t kRsrcFlags = 0x00020000;
    const size_t head_off = PAGED ? (size_t)kvh * ((size_t)ROWB << P.pt.bs_log2)
                                  : (size_t)(b * P.Hkv + kvh) * P.Lcap * ROWB;
    const uint8_t* kbase = (const uint8_t*)P.k + head_off;
    const uint8_t* vbase = (const uint8_t*)P.v + head_off;
    // paged: one resource per pool, based at this KV head's slice of page 0;
    // a block wholly inside a page and the split is read through it with the
    // page's offset as the scalar offset (when the pool spans < 4 GiB)
    const int page_bytes = PAGED ? P.Hkv * (ROWB << P.pt.bs_log2) : 0;
    const bool pool_small = PAGED && (uint64_t)P.pt.num_blocks * (uint64_t)page_bytes < (1ull << 32);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, PAGED ? -1 : k1 * ROWB, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, PAGED ? -1 : k1 * ROWB, kRsrcFlags);
    const int32_t* trow = PAGED ? P.pt.table + (size_t)b * P.pt.width : nullptr;
    // paged caches: lane l of the result holds the page entry of block load l
    // of the tile at key t (-1 past the split); fetched one step ahead
    auto load_pages = [&](int t) -> int {
        int e = -1;
        if (PAGED && lane < 2 * LPW) {
            const int blk = (lane < LPW ? lane : lane - LPW) * VW + wave;
            const int key0 = t + blk * RPB;
            if (key0 < k1) e = trow[key0 >> P.pt.bs_log2];
        }
        return e;
    };
    auto issue_load = [&](int l, int t, uint8_t* kdst, uint8_t* vdst, int page) {
        const bool isk = l < LPW;
        const int blk = (isk ? l : l - LPW) * VW + wave;
        const int row = blk * RPB + lane / CH;
        const int c = (lane % CH) ^ (isk ? (row & (CH - 1)) : 0);
        auto* dst = (__attribute__((address_space(3))) void*)((isk ? kdst : vdst) + blk * 1024);
        if constexpr (PAGED) {
            const int key0 = t + blk * RPB;   // first slot of the block (wave-uniform)
            const int in_page = key0 & ((1 << P.pt.bs_log2) - 1);
            if (pool_small && page >= 0 && key0 + RPB <= k1) {   // wave-uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? krs : vrs, dst, 16, (in_page + lane / CH) * ROWB + c * 16,
                                                         (uint32_t)page * (uint32_t)page_bytes, 0, STREAM ? kStreamPolicy : 0);
                return;
            }
            const int room = min(max(k1 - (key0 - in_page), 0), 1 << P.pt.bs_log2);
            const uint64_t addr = (uint64_t)((isk ? kbase : vbase) +
                                             (size_t)max(page, 0) * P.Hkv * ((size_t)ROWB << P.pt.bs_log2));
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
            const int bytes = __builtin_amdgcn_readfirstlane(page >= 0 ? room * ROWB : 0);
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, bytes, kRsrcFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (in_page + lane / CH) * ROWB + c * 16, 0, 0,
                                                     STREAM ? kStreamPolicy : 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? krs : vrs, dst, 16, (t + row) * ROWB + c * 16, 0, 0,
                                                     STREAM ? kStreamPolicy : 0);
        }
    };

    // Query rows: lane (kk, qd) = (lane / 4, lane % 4) holds quarter qd of every row.
    const int kk = lane >> 2, qd = lane & 3;
    u32x4 qv[MAXR][QCH];
#pragma unroll
    for (int j = 0; j < MAXR; ++j)
#pragma unroll
        for (int i = 0; i < QCH; ++i) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (j < R) v = *(const u32x4*)((const uint8_t*)P.q + out_row(j) * EB + (qd * QCH + i) * 16);
            qv[j][i] = v;
        }

    int pga = -1, pgb = -1;
    if constexpr (PAGED) {
        const int p0 = load_pages(k0);
        pga = load_pages(k0 + VKT);   // the first step's loads
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int l = 0; l < 2 * LPW; ++l) issue_load(l, k0, k_lds0, v_lds0, __builtin_amdgcn_readlane(p0, l));
    } else {
#pragma unroll
        for (int l = 0; l < 2 * LPW; ++l) issue_load(l, k0, k_lds0, v_lds0, -1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    unsigned long long anc_r[MAXR];
#pragma unroll
    for (int j = 0; j < MAXR; ++j) anc_r[j] = anc_lds[j < R ? j / g : 0];

    float o[MAXR][CPL], m_run[MAXR], l_part[MAXR];
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        m_run[j] = -INFINITY;
        l_part[j] = 0.f;
#pragma unroll
        for (int x = 0; x < CPL; ++x) o[j][x] = 0.f;
    }

    auto step = [&](int t, const uint8_t* kl, const uint8_t* vl, uint8_t* k_fill, uint8_t* v_fill, int pg_cur,
                    int& pg_next) {
        if (t + VKT < k1) {
            int pages[2 * LPW];
#pragma unroll
            for (int l = 0; l < 2 * LPW; ++l) pages[l] = PAGED ? __builtin_amdgcn_readlane(pg_cur, l) : -1;
            if constexpr (PAGED) pg_next = load_pages(t + 2 * VKT);
#pragma unroll
            for (int l = 0; l < 2 * LPW; ++l) issue_load(l, t + VKT, k_fill, v_fill, pages[l]);
        }
        // QK^T for this lane's key and quarter, then the sum of the four quarters
        const int krow = VKW * wave + kk;
        u32x4 kc[QCH];
#pragma unroll
        for (int i = 0; i < QCH; ++i)
            kc[i] = *(const u32x4*)(kl + krow * ROWB + (((qd * QCH + i) ^ (krow & (CH - 1))) << 4));
        float s[MAXR];
#pragma unroll
        for (int j = 0; j < MAXR; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < QCH; ++i)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t qw = qv[j][i][w], kw = kc[i][w];
                    if constexpr (BF16)
                        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw),
                                                              __builtin_bit_cast(bf16x2_t, kw), acc, false);
                    else
                        acc = fmaf(__uint_as_float(qw), __uint_as_float(kw), acc);
                }
            s[j] = acc;
        }
#pragma unroll
        for (int j = 0; j < MAXR; ++j) s[j] += __shfl_xor(s[j], 1, kWave);
#pragma unroll
        for (int j = 0; j < MAXR; ++j) s[j] += __shfl_xor(s[j], 2, kWave);

        // scores in the exp2 domain, masked: keys past the split, and tree keys off the row's root path
        const int key = t + krow;
        const bool tail = (t + VKT > L) || (t + VKT > k1);
        bool raise = false;
#pragma unroll
        for (int j = 0; j < MAXR; ++j) {
            float val = s[j] * P.c;
            if (tail) {
                const bool vis = key < k1 && (key < L || ((anc_r[j] >> ((unsigned)(key - L) & 63u)) & 1ull));
                val = vis ? val : -INFINITY;
            }
            s[j] = val;
            raise |= val > m_run[j] + kLazyRef;
        }
        if (__any(raise)) {   // raise the reference of every row to the tile maximum where it grew
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {
                const float tmax = wave_max(s[j]);
                if (tmax > m_run[j] + kLazyRef) {
                    const float alpha = m_run[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[j] - tmax);
                    l_part[j] *= alpha;
#pragma unroll
                    for (int x = 0; x < CPL; ++x) o[j][x] *= alpha;
                    m_run[j] = tmax;
                }
            }
        }
        float w[MAXR];
#pragma unroll
        for (int j = 0; j < MAXR; ++j) {
            w[j] = __builtin_amdgcn_exp2f(s[j] - (m_run[j] == -INFINITY ? 0.f : m_run[j]));
            l_part[j] += qd == 0 ? w[j] : 0.f;
        }
        if (qd == 0) {
#pragma unroll
            for (int j = 0; j < MAXR; ++j) p_lds[wave][kk][j] = w[j];
        }
        __builtin_amdgcn_wave_barrier();

        // PV: lane owns head-dim columns lane * CPL .. + CPL - 1
#pragma unroll 4
        for (int k2 = 0; k2 < VKW; ++k2) {
            const uint8_t* vrow = vl + (VKW * wave + k2) * ROWB + lane * CPB;
            float v[CPL];
            if constexpr (BF16) {
                if constexpr (CPL == 2) {
                    const uint32_t x = *(const uint32_t*)vrow;
                    v[0] = bf16_lo(x);
                    v[1] = bf16_hi(x);
                } else {
                    v[0] = __uint_as_float(((uint32_t) * (const uint16_t*)vrow) << 16);
                }
            } else {
#pragma unroll
                for (int x = 0; x < CPL; ++x) v[x] = ((const float*)vrow)[x];
            }
#pragma unroll
            for (int j = 0; j < MAXR; ++j) {
                const float pw = p_lds[wave][k2][j];
#pragma unroll
                for (int x = 0; x < CPL; ++x) o[j][x] = fmaf(pw, v[x], o[j][x]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // the next tile has landed
        __syncthreads();                 // every wave is done with this one
    };
    for (int t = k0; t < k1; t += 2 * VKT) {
        step(t, k_lds0, v_lds0, k_lds1, v_lds1, pga, pgb);
        if (t + VKT >= k1) break;
        step(t + VKT, k_lds1, v_lds1, k_lds0, v_lds0, pgb, pga);
    }

    // merge the four waves: (m, l) and O through the idle tile buffers
    float* xo = (float*)k_lds0;   // [wave][row][column], VW * MAXR * D floats
    static_assert(VW * MAXR * D * 4 <= TILEB, "exchange fits one K buffer");
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        const float lw = wave_sum(l_part[j]);
        if (lane == 0) ml_lds[wave][j] = make_float2(m_run[j], lw);
#pragma unroll
        for (int x = 0; x < CPL; ++x) xo[(wave * MAXR + j) * D + lane * CPL + x] = o[j][x];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
        if (j >= R) break;
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < VW; ++w2) {
            const float2 ml = ml_lds[w2][j];
            if (ml.y > 0.f) M = fmaxf(M, ml.x);
        }
        float acc[CPL], lsum = 0.f;
#pragma unroll
        for (int x = 0; x < CPL; ++x) acc[x] = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < VW; ++w2) {
            const float2 ml = ml_lds[w2][j];
            if (!(ml.y > 0.f)) continue;
            const float f = __builtin_amdgcn_exp2f(ml.x - M);
            lsum += f * ml.y;
#pragma unroll
            for (int x = 0; x < CPL; ++x) acc[x] += f * xo[(w2 * MAXR + j) * D + lane * CPL + x];
        }
        if (P.nsplit == 1) {
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            uint8_t* orow = (uint8_t*)P.out + out_row(j) * EB;
#pragma unroll
            for (int x = 0; x < CPL; ++x) {
                const int d = lane * CPL + x;
                if constexpr (BF16)
                    ((uint16_t*)orow)[d] = (uint16_t)f32_to_bf16_bits(acc[x] * inv);
                else
                    ((float*)orow)[d] = acc[x] * inv;
            }
        } else {
            const size_t prow = (size_t)group * P.Rpad + j;
#pragma unroll
            for (int x = 0; x < CPL; ++x) P.part_o[prow * D + lane * CPL + x] = acc[x];
            if (lane == 0) P.part_ml[prow] = make_float2(M, lsum);
        }
    }
}

template <bool BF16, int D, bool PAGED, bool STREAM, bool FUSE>
void launch_tiled_rows_f(const AttnParams& p, int maxr, dim3 grid, hipStream_t s, const StatsParams& S) {
    const int blocks = (int)grid.x;
    const dim3 g(blocks + (FUSE ? S.B * (S.sampling ? 2 * S.T : S.T) : 0));
    switch (maxr) {
        case 2: hipLaunchKernelGGL((attn_valu_tiled_kernel<BF16, D, 2, PAGED, STREAM, FUSE>), g, dim3(VW * 64), 0, s, p, S, blocks); break;
        case 4: hipLaunchKernelGGL((attn_valu_tiled_kernel<BF16, D, 4, PAGED, STREAM, FUSE>), g, dim3(VW * 64), 0, s, p, S, blocks); break;
        case 6: hipLaunchKernelGGL((attn_valu_tiled_kernel<BF16, D, 6, PAGED, STREAM, FUSE>), g, dim3(VW * 64), 0, s, p, S, blocks); break;
        default: hipLaunchKernelGGL((attn_valu_tiled_kernel<BF16, D, 8, PAGED, STREAM, FUSE>), g, dim3(VW * 64), 0, s, p, S, blocks); break;
    }
}

template <bool BF16, int D, bool PAGED, bool STREAM>
void launch_tiled_rows(const AttnParams& p, int maxr, dim3 grid, hipStream_t s, const StatsParams* fused) {
    if (fused) launch_tiled_rows_f<BF16, D, PAGED, STREAM, true>(p, maxr, grid, s, *fused);
    else launch_tiled_rows_f<BF16, D, PAGED, STREAM, false>(p, maxr, grid, s, StatsParams{});
}

template <bool BF16, int D>
void launch_tiled(const AttnParams& p, int maxr, dim3 grid, hipStream_t s, const StatsParams* fused) {
    if (p.pt.table) {   // paged caches: no fused row statistics
        if (p.stream) launch_tiled_rows<BF16, D, true, true>(p, maxr, grid, s, nullptr);
        else launch_tiled_rows<BF16, D, true, false>(p, maxr, grid, s, nullptr);
    } else {
        if (p.stream) launch_tiled_rows<BF16, D, false, true>(p, maxr, grid, s, fused);
        else launch_tiled_rows<BF16, D, false, false>(p, maxr, grid, s, fused);
    }
}

}  // namespace

bool valu_tiled_supported(bool bf16, int D, int R) {
    const int rowb = D * (bf16 ? 2 : 4);
    return R <= 8 && (rowb == 128 || rowb == 256);
}

hipError_t launch_attention_valu_tiled(const AttnParams& p, bool bf16, hipStream_t s, const StatsParams* fused) {
    const dim3 grid(p.B * p.Hkv * p.nsplit);
    const int maxr = p.Rpad;
    if (bf16) {
        if (p.D == 128) launch_tiled<true, 128>(p, maxr, grid, s, fused);
        else launch_tiled<true, 64>(p, maxr, grid, s, fused);
    } else {
        launch_tiled<false, 64>(p, maxr, grid, s, fused);   // fp32 rows of 256 bytes
    }
    return hipGetLastError();
}

}  // namespace sv
