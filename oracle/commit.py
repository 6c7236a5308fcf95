"""KV commit of the accepted path (oracle; test infrastructure only).

After verification the caches of a sequence hold the prefix at slots
0..L-1 and tree node i's key/value at slot L+i.  Keeping the accepted path
means making its nodes contiguous after the prefix and moving the valid
length; everything past it is dropped by the length alone, since the cache
is preallocated per sequence ("大模型推理加速：推测解码与MTP核心原理与工程实践",
section 3.1 item 4 on rolling back and continuing, section 6.3 on releasing
rejected paths; the featured article on the founding speculative-decoding
paper, section 4.3: with a preallocated cache, rolling back only changes the
valid length).

Reading: slot L+k receives node path[k] for k = 1..accept_len (the root,
node 0, already sits at slot L), and the new length is L + accept_len + 1 (the
root and the accepted drafts; the final token is the next step's root).
A sequence is left unchanged when it is void (final_node < 0), its kv_len is
out of range, or its path is not a root path of length accept_len + 1 with
k <= path[k] < T.
"""
from __future__ import annotations

import numpy as np


def commit_kv(k_cache: np.ndarray, v_cache: np.ndarray, kv_len: np.ndarray, path: np.ndarray,
              accept_len: np.ndarray, final_node: np.ndarray, nodes: int):
    """Returns (k, v, kv_len) after the commit; inputs are not modified.

    k_cache, v_cache: [B, Hkv, Lcap, D] (any dtype); kv_len [B]; path [B, T];
    accept_len, final_node [B].
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    new_len = np.array(kv_len, copy=True)
    B, _, Lcap, _ = k.shape
    T = nodes
    for b in range(B):
        L, A = int(kv_len[b]), int(accept_len[b])
        if final_node[b] < 0 or L < 0 or L + T > Lcap or A < 0 or A >= T:
            continue
        p = [int(x) for x in path[b, :A + 1]]
        if p[0] != 0 or any(not (kk <= p[kk] < T) for kk in range(1, A + 1)):
            continue
        src_k = k_cache[b][:, [L + x for x in p], :]      # read every source before any write
        src_v = v_cache[b][:, [L + x for x in p], :]
        k[b][:, L:L + A + 1, :] = src_k
        v[b][:, L:L + A + 1, :] = src_v
        new_len[b] = L + A + 1
    return k, v, new_len
