// Streaming-read probe: the read ceiling the HBM-bound kernels are compared with (a measurement
// aid for benchmarks, not part of the method).  Each workgroup reads one contiguous slice of the
// buffer with 16-byte non-temporal loads, kProbeLoads per lane in flight -- the load form the
// statistics and attention streams use -- and stores one word per workgroup, so that the reads
// cannot be optimised away.  A sweep of this form over 256-8192 workgroups of 256-1024 threads and
// 4-16 loads per lane peaked at 512 workgroups of 256 threads with 4 loads in flight.

#include "common.h"
#include "kernels.h"

namespace specv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 4;
constexpr int kProbeBlocks = 512;

__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const uint4* __restrict__ src, int64_t per_block, int64_t nvec, uint32_t* __restrict__ sink) {
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per_block;
    const int64_t hi = lo + per_block < nvec ? lo + per_block : nvec;
    uint32_t acc = 0;
    for (int64_t base = lo + threadIdx.x; base < hi; base += static_cast<int64_t>(kProbeThreads) * kProbeLoads) {
        uint4 v[kProbeLoads];
#pragma unroll
        for (int j = 0; j < kProbeLoads; ++j) {
            const int64_t i = base + static_cast<int64_t>(j) * kProbeThreads;
            v[j] = i < hi ? load_nt(src + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kProbeLoads; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    // one word per workgroup: the lanes' words folded together
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o));
    __shared__ uint32_t red[kProbeThreads / kWave];
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < kProbeThreads / kWave; ++w) x ^= red[w];
        sink[blockIdx.x] = x;
    }
}

}  // namespace

int read_probe_blocks() { return kProbeBlocks; }

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t nvec = static_cast<int64_t>(bytes / 16);
    const int64_t per = (nvec + kProbeBlocks - 1) / kProbeBlocks;
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(buf), per, nvec, sink);
    return hipGetLastError();
}

}  // namespace specv
