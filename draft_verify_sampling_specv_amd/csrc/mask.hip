// Ancestor mask and depth from a parent array ([SD-EAGLE] "Tree Attention Verification": every
// node attends to its ancestors and itself; [PTD] Method 1, "Attention Masking").
//
// One workgroup per sequence.  The parent array is staged in LDS and validated first (the
// smallest bad index wins, via an LDS atomic min).  Each thread then owns (row, word) pairs and
// builds the word in a register by walking the row's ancestor chain, so every mask word is
// written exactly once with coalesced stores.  Work per sequence is O((K+1) * W * depth); the
// kernel is launch-latency bound at every practical size.

#include "common.h"
#include "kernels.h"

namespace specv {

__global__ void __launch_bounds__(256) build_tree_mask_kernel(const int32_t* __restrict__ parent,
                                                              int n1, uint32_t* __restrict__ mask,
                                                              int32_t* __restrict__ depth,
                                                              int32_t* __restrict__ tree_status) {
    __shared__ int32_t par[kMaxNodes];
    __shared__ int bad;
    const int b = blockIdx.x;
    const int words = (n1 + 31) >> 5;
    const int32_t* pb = parent + static_cast<int64_t>(b) * n1;
    uint32_t* mb = mask + static_cast<int64_t>(b) * n1 * words;
    int32_t* db = depth + static_cast<int64_t>(b) * n1;

    if (threadIdx.x == 0) bad = n1;
    __syncthreads();
    for (int i = threadIdx.x; i < n1; i += blockDim.x) {
        int p = pb[i];
        par[i] = p;
        bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
        if (!ok) atomicMin(&bad, i);
    }
    __syncthreads();
    const bool valid = (bad == n1);
    if (threadIdx.x == 0) tree_status[b] = valid ? 0 : bad + 1;

    for (int e = threadIdx.x; e < n1 * words; e += blockDim.x) {
        const int i = e / words, w = e - i * words;
        uint32_t word = 0;
        int d = -1;
        if (valid) {
            // walk i, parent(i), ..., root; parent indices strictly decrease, so this ends
            int j = i;
            d = 0;
            while (true) {
                if ((j >> 5) == w) word |= 1u << (j & 31);
                int p = par[SPECV_CHK(j, n1, kSiteMaskWalk)];
                if (p < 0) break;
                j = p;
                ++d;
            }
        }
        mb[e] = word;
        if (w == 0) db[i] = d;
    }
}

hipError_t launch_build_tree_mask(const int32_t* parent, int B, int n1, uint32_t* mask,
                                  int32_t* depth, int32_t* tree_status, hipStream_t stream) {
    hipLaunchKernelGGL(build_tree_mask_kernel, dim3(B), dim3(256), 0, stream, parent, n1, mask,
                       depth, tree_status);
    return hipGetLastError();
}

}  // namespace specv
