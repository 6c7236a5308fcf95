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
// One workgroup per sequence.  For each KV head every 16-byte chunk of the
// moved rows (K and V) is loaded into registers before any is stored, since a
// destination slot may be the source of an earlier row; rows already in
// place are skipped.

#include "device_common.h"
#include "kernels.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CT = 256;                         // threads per workgroup
constexpr int MAXC = (2 * 63 * 32 + CT - 1) / CT;   // chunks per thread: K and V, 63 rows, 32 chunks a row

__global__ __launch_bounds__(CT) void kv_commit_kernel(CommitParams P) {
    __shared__ int src[64];
    __shared__ int sL, sA, sok;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int T = P.T;
    if (tid < kWave) {
        const int lane = tid;
        const int L = P.kv_len[b], A = P.accept_len[b];
        const int p = (lane < T) ? P.path[(size_t)b * T + lane] : -1;
        bool ok = P.final_node[b] >= 0 && L >= 0 && L <= P.Lcap - T && A >= 0 && A < T;
        const bool bad = (lane == 0 && p != 0) || (lane >= 1 && lane <= A && !(lane <= p && p < T));
        ok = ok && !__any(bad);
        src[lane] = p;
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
    for (int h = 0; h < P.Hkv; ++h) {
        const size_t head = ((size_t)b * P.Hkv + h) * P.Lcap;
        u32x4 reg[MAXC];
#pragma unroll
        for (int m = 0; m < MAXC; ++m) {
            const int idx = m * CT + tid;
            if (idx < total) {
                const int kv = idx / (A * cpr), rest = idx - kv * (A * cpr);
                const int k = 1 + rest / cpr, c = rest - (k - 1) * cpr;
                if (src[k] != k) {
                    const uint8_t* base = (const uint8_t*)(kv ? P.v : P.k);
                    reg[m] = *(const u32x4*)(base + (head + L + src[k]) * P.row_bytes + c * 16);
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
                    *(u32x4*)(base + (head + L + k) * P.row_bytes + c * 16) = reg[m];
                }
            }
        }
    }
    if (tid == 0) P.kv_len_out[b] = L + A + 1;
}

}  // namespace

hipError_t launch_kv_commit(const CommitParams& p, hipStream_t s) {
    hipLaunchKernelGGL(kv_commit_kernel, dim3(p.B), dim3(CT), 0, s, p);
    return hipGetLastError();
}

}  // namespace sv
