// KV-cache commit after a verify step: the accepted path's K/V rows move next to the root's,
// the rejected branches' rows are dropped.
//
// [SD-review] §4 (limitations): the cache entries written for rejected drafts have to be rolled
// back; [SD-EAGLE] "Tree Attention Verification": a tree is verified with a few extra KV-cache
// entries, one per node, at ctx_len + node.  After the walk accepted nodes n_1 < ... < n_a (one
// per depth, n_d at depth d, so n_d >= d), the committed sequence is the context, the root and
// that path: row ctx_len + n_d moves to ctx_len + d and the new context length is
// ctx_len + 1 + a.
//
// In place.  A destination ctx_len + d can be the source of a shallower node (n_d' = d with
// d' < d) but never of a deeper one (n_d' >= d' > d), so depths are moved in increasing chunks,
// each chunk read completely before any of it is written.  Rows already in place (n_d == d, e.g.
// every row of a chain) are neither read nor written.

#include "common.h"
#include "kernels.h"

namespace specv {
namespace {

constexpr int kCommitThreads = 256;
constexpr int kChunkRows = 64;                                  // depths per read-then-write round
constexpr int kMaxRowVec = 32;                                  // 16-byte vectors per row (D 128 fp32)
constexpr int kPerThread = kChunkRows * kMaxRowVec / kCommitThreads;

// One workgroup per (sequence, KV head, K or V).
__global__ void __launch_bounds__(kCommitThreads)
kv_commit_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc, const int32_t* __restrict__ ctx_len,
                 const int32_t* __restrict__ accept_len, const int32_t* __restrict__ out_nodes, int n1,
                 int Hkv, int Lmax, int nvec, int32_t* __restrict__ new_ctx_len) {
    __shared__ int32_t s_node[kMaxNodes];
    __shared__ int s_bad;
    const int t = threadIdx.x;
    const int which = blockIdx.x & 1;
    const int unit = blockIdx.x >> 1;
    const int kv = unit % Hkv, b = unit / Hkv;
    const int L = ctx_len[b], a = accept_len[b];
    const int32_t* nodes = out_nodes + static_cast<int64_t>(b) * n1;

    if (t == 0) s_bad = 0;
    __syncthreads();
    // a sequence is committed only if its context fits with the whole tree and its accepted
    // path is a valid path of depths 1..a: n_d in [d, n1) and increasing
    bool ok = a >= 0 && a <= n1 - 1 && L >= 0 && L <= Lmax - n1;
    if (ok) {
        for (int d = 1 + t; d <= a; d += kCommitThreads) {
            const int nd = nodes[d - 1];
            s_node[SPECV_CHK(d, kMaxNodes, kSiteCommitNode)] = nd;
            if (nd < d || nd >= n1 || (d > 1 && nodes[d - 2] >= nd)) s_bad = 1;
        }
    }
    __syncthreads();
    ok = ok && !s_bad;
    if (which == 0 && kv == 0 && t == 0) new_ctx_len[b] = ok ? L + 1 + a : -1;
    if (!ok) return;     // (workgroup-uniform)

    uint4* base = (which ? vc : kc) + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * nvec;
    for (int d0 = 1; d0 <= a; d0 += kChunkRows) {
        const int nv = (min(a + 1, d0 + kChunkRows) - d0) * nvec;
        uint4 buf[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int i = t + j * kCommitThreads;
            if (i < nv) {
                const int d = d0 + i / nvec, e = i % nvec, nd = s_node[d];
                if (nd != d) buf[j] = base[static_cast<int64_t>(SPECV_CHK(L + nd, Lmax, kSiteCommitSrc)) * nvec + e];
            }
        }
        __syncthreads();    // (waits for the loads: the whole chunk is read before it is written)
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int i = t + j * kCommitThreads;
            if (i < nv) {
                const int d = d0 + i / nvec, e = i % nvec, nd = s_node[d];
                if (nd != d) base[static_cast<int64_t>(SPECV_CHK(L + d, Lmax, kSiteCommitDst)) * nvec + e] = buf[j];
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_kv_commit(const KvCommitArgs& a, hipStream_t stream) {
    const int nvec = a.D * (a.bf16 ? 2 : 4) / 16;
    hipLaunchKernelGGL(kv_commit_kernel, dim3(a.B * a.Hkv * 2), dim3(kCommitThreads), 0, stream,
                       static_cast<uint4*>(a.k_cache), static_cast<uint4*>(a.v_cache), a.ctx_len,
                       a.accept_len, a.out_nodes, a.n1, a.Hkv, a.Lmax, nvec, a.new_ctx_len);
    return hipGetLastError();
}

}  // namespace specv
