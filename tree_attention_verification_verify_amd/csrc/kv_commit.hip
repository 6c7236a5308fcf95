// KV commit of the accepted path.
//
// After verification a sequence's cache holds the prefix at slots 0..L-1 and
// tree node i's key/value at slot L+i.  Keeping the accepted path makes its
// nodes contiguous after the prefix: slot L+k receives node path[k] for
// k = 1..accept_len, and the valid length becomes L + accept_len + 1 (the root
// and the accepted drafts).  The cache is preallocated per sequence, so
// whatever lies past the new length is dropped by the length alone (featured
// article on the founding speculative-decoding paper, section 4.3;
// "大模型推理加速：推测解码与MTP核心原理与工程实践", section 3.1 item 4 and
// section 6.3).  Void sequences, lengths out of range and paths that are not
// root paths (path[0] = 0, k <= path[k] < T) are left unchanged.
//
// One workgroup per (sequence, KV head): heads touch disjoint memory.  Every
// 16-byte chunk of the head's moved rows (K and V) is loaded into registers
// before any is stored, since a destination slot may be the source of an
// earlier row; rows already in place are skipped.  The new length is written
// by the last workgroup of the sequence to finish (a per-sequence counter),
// so no workgroup can read a length already updated.
//
// Paged caches: slot s lives in row s % bs of page table[s / bs]; a dense
// cache is addressed the same way as one page of Lcap slots per sequence
// (page b).  A sequence whose used table entries leave the pool is skipped.

#include "device_common.h"
#include "kernels.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CT = 256;                         // threads per workgroup
constexpr int MAXC = (2 * 63 * 32 + CT - 1) / CT;   // chunks per thread: K and V, 63 rows, 32 chunks a row

__global__ __launch_bounds__(CT) void kv_commit_kernel(CommitParams P) {
    __shared__ int src[64];
    __shared__ size_t off_src[64], off_dst[64];   // byte offset of row k's source / destination slot, head 0
    __shared__ int sL, sA, sok;
    const int b = blockIdx.x / P.Hkv, h = blockIdx.x - b * P.Hkv, tid = threadIdx.x;
    const int T = P.T;
    if (tid < kWave) {
        const int lane = tid;
        const int L = P.kv_len[b], A = P.accept_len[b];
        const int p = (lane < T) ? P.path[(size_t)b * T + lane] : -1;
        bool ok = P.final_node[b] >= 0 && L >= 0 && L <= P.Lcap - T && A >= 0 && A < T;
        const bool bad = (lane == 0 && p != 0) || (lane >= 1 && lane <= A && !(lane <= p && p < T));
        ok = ok && !__any(bad);
        ok = ok && !__any(page_entries_bad(P.pt, b, L + T, lane, kWave));
        src[lane] = p;
        if (ok && lane >= 1 && lane <= A) {
            auto slot_off = [&](int slot) -> size_t {
                if (!P.pt.table) return ((size_t)b * P.Hkv * P.Lcap + slot) * P.row_bytes;
                const int page = P.pt.table[(size_t)b * P.pt.width + (slot >> P.pt.bs_log2)];
                return (((size_t)page * P.Hkv << P.pt.bs_log2) + (slot & ((1 << P.pt.bs_log2) - 1))) *
                       P.row_bytes;
            };
            off_src[lane] = slot_off(L + p);
            off_dst[lane] = slot_off(L + lane);
        }
        if (lane == 0) {
            sL = L;
            sA = A;
            sok = ok ? 1 : 0;
        }
    }
    __syncthreads();
    if (!sok) return;
    const int L = sL, A = sA;
    const int cpr = P.row_bytes / 16;             // chunks per row
    const int total = 2 * A * cpr;                 // K and V chunks of rows 1..A
    const size_t head_stride = (size_t)(P.pt.table ? (1 << P.pt.bs_log2) : P.Lcap) * P.row_bytes;
    {
        const size_t head = (size_t)h * head_stride;
        u32x4 reg[MAXC];
#pragma unroll
        for (int m = 0; m < MAXC; ++m) {
            const int idx = m * CT + tid;
            if (idx < total) {
                const int kv = idx / (A * cpr), rest = idx - kv * (A * cpr);
                const int k = 1 + rest / cpr, c = rest - (k - 1) * cpr;
                if (src[k] != k) {
                    const uint8_t* base = (const uint8_t*)(kv ? P.v : P.k);
                    reg[m] = *(const u32x4*)(base + head + off_src[k] + c * 16);
                }
            }
        }
        __syncthreads();   // every source of this head is read before any destination is written
#pragma unroll
        for (int m = 0; m < MAXC; ++m) {
            const int idx = m * CT + tid;
            if (idx < total) {
                const int kv = idx / (A * cpr), rest = idx - kv * (A * cpr);
                const int k = 1 + rest / cpr, c = rest - (k - 1) * cpr;
                if (src[k] != k) {
                    uint8_t* base = (uint8_t*)(kv ? P.v : P.k);
                    *(u32x4*)(base + head + off_dst[k] + c * 16) = reg[m];
                }
            }
        }
    }
    // every workgroup of the sequence has read the old length before it counts
    // itself; a skipped sequence (the same decision in all of them) counts nothing
    if (tid == 0) {
        if (arrive_last(P.arrive + b, P.Hkv)) P.kv_len_out[b] = L + A + 1;
    }
}

}  // namespace

hipError_t launch_kv_commit(const CommitParams& p, hipStream_t s) {
    hipLaunchKernelGGL(kv_commit_kernel, dim3(p.B * p.Hkv), dim3(CT), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
