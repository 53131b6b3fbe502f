// One target-model layer over the draft nodes: the forward pass that produces the verified rows.
// [SD-EAGLE] "Two-Model Setup" (step 2: one parallel target pass over all K + 1 positions);
// [PTD] Method 4, "Verification" (every tree node in one pass, with the tree mask and the matching
// position encoding).  The layer is a pre-norm decoder block:
//   h = rms(x) g1;  [q k v] = h Wqkv^T;  q, k rotated at ctx_len + depth;  k, v -> cache at ctx_len + i;
//   a = tree_attention(q, cache, mask);  y = x + a Wo^T;  h2 = rms(y) g2;  [g u] = h2 Wgu^T;
//   out = y + (silu(g) u) Wdown^T
// bf16 storage for every activation and weight, fp32 accumulation.
//
// The projections are skinny: T = B (K + 1) rows (192 on the chain workload) against weight
// matrices of tens to hundreds of MB, so they are bound by streaming the weights from HBM, not by
// MFMA throughput.  gemm_kernel streams every weight row exactly once:
//   * a workgroup owns 128 weight rows (4 waves x 32) and one K range (split-K, so a few hundred
//     workgroups cover the chip); the weight rows go straight from HBM into MFMA A-operand
//     registers, four 64-column steps in flight per wave;
//   * the T activation rows of the current 64-column step sit in LDS (double-buffered), read as
//     B operands by all four waves; the contraction order inside a step is permuted identically
//     on both operands so that each lane's weight bytes are contiguous (64 B per row per lane);
//   * partial sums go to a workspace [split][T][N] in fp32; a small per-row epilogue kernel adds
//     the splits and applies what follows the product (rotary encoding and the cache append, the
//     residual add and norm, silu(g) u, the final residual add).

#include <cmath>

#include "attn_common.h"
#include "kernels.h"

namespace specv {
namespace {

using attn::as_bf16x8;
using attn::bf16x8_t;
using attn::f32x16_t;

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 32;
constexpr int kMW = 4;                        // multiplying waves per workgroup
constexpr int kLW = 4;                        // activation-staging waves per workgroup
constexpr int kGemmThreads = (kMW + kLW) * kWave;
constexpr int kTileRows = kMW * kRowsPerWave; // weight rows per workgroup
constexpr int kStep = 64;                     // contraction columns per pipeline step
constexpr int kInFlight = 4;                  // weight steps in flight per wave (even: LDS parity)
constexpr int kXSets = 4;                     // activation chunks in flight per staging wave (divides kInFlight)
constexpr int kXStride = kStep + 8;           // LDS row stride (bf16): conflict-free 16-byte reads
constexpr int kMaxMB = 8;                     // activation rows per launch: 32 kMaxMB

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return static_cast<uint16_t>(attn::pack_bf16x2(f, 0.f) & 0xffffu);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < static_cast<int>(blockDim.x) / kWave; ++i) t += red[i];
    return t;
}

// P[split][m][n] = sum over the split's K range of X[m][k] W[n][k].  X: [M][K] bf16 (M <= 32 MB),
// W: [N][K] bf16; K a multiple of 64, N a multiple of 4.  Grid (ceil(N / 128), splits), 8 waves:
//   waves 0-3 multiply: each streams its 32 weight rows into registers kInFlight steps ahead and
//     runs the MFMAs of a step against the activation chunk in LDS;
//   waves 4-7 stage the activation chunks: kXSets chunks in flight in registers, step s + 1 going
//     to LDS while the MFMAs of step s run.
// The roles sit in separate waves because a wave's loads complete (for s_waitcnt) in issue order:
// a wave that waited for its next activation chunk would also wait for every weight load issued
// before it, which would cut the weight prefetch to one step.
//
// kGateUp: W is the [2 N][K] gate/up matrix and the workgroup's 128 rows are gate rows
// 64 t .. 64 t + 63 (waves 0, 1) and the matching up rows N + 64 t .. (waves 2, 3); with one split
// the kernel finishes the MLP activation itself, act[m][n] = silu(gate) up in bf16 (no partials).
//
// kPacked: W is in the tile order of pack_weights_kernel (rows a multiple of 32), so each weight
// load instruction of a wave reads 1 KB contiguous -- 8 whole 128-byte lines -- instead of 32 bytes
// of 32 different rows' lines; the vector L1 then tracks a quarter of the line requests per byte.
template <int MB, bool kGateUp, bool kPacked>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                               const uint16_t* __restrict__ W, int N,
                                                               int steps_per_split, float* __restrict__ P,
                                                               uint16_t* __restrict__ act) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][MB * 32 * kXStride];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int st0 = blockIdx.y * steps_per_split;
    const int nsteps = min(steps_per_split, K / kStep - st0);
    const int64_t k0 = static_cast<int64_t>(st0) * kStep;
    const int padded = (nsteps + kInFlight - 1) / kInFlight * kInFlight;

    if (wv < kMW) {
        const int r = lane & 31, h = lane >> 5;
        // output column block of this wave and the weight row behind this lane (clamped past N:
        // loaded, never stored)
        constexpr int kHalf = kMW / 2;                 // gate waves (the rest hold the matching up rows)
        const int nw = kGateUp ? (blockIdx.x * kHalf + wv % kHalf) * kRowsPerWave : blockIdx.x * kTileRows + wv * kRowsPerWave;
        const int64_t wrow = kGateUp ? min(nw + r, N - 1) + (wv >= kHalf ? N : 0) : min(nw + r, N - 1);
        // row-major: the 32 columns 32 h .. 32 h + 31 of each step, slice j at 8 j; packed: the
        // wave's 32-row block (clamped past N like the rows), 1 KB per (step, slice) from its
        // first step, lane l at 16 l
        const int rb = kGateUp ? min(nw, N - 1) / kRowsPerWave + (wv >= kHalf ? N / kRowsPerWave : 0)
                               : min(nw, N - 1) / kRowsPerWave;
        const uint4* wp = kPacked
            ? reinterpret_cast<const uint4*>(W) + ((static_cast<int64_t>(rb) * (K / kStep) + st0) * 4) * kWave + lane
            : reinterpret_cast<const uint4*>(W + wrow * K + k0 + 32 * h);
        auto wload = [&](int s, int j) { return kPacked ? wp[(s * 4 + j) * kWave] : wp[s * (kStep / 8) + j]; };
        uint4 wr[kInFlight][4];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int s = min(u, nsteps - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) wr[u][j] = wload(s, j);
        }
        f32x16_t acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16_t{};
        __syncthreads();                               // chunk 0 staged
        for (int sb = 0; sb < padded; sb += kInFlight) {
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int s = sb + u;
                const bool live = s < nsteps;          // the padding steps multiply zeros
                const uint16_t* xb = xs[u & 1] + r * kXStride + 32 * h;
                // 4 MFMA k-slices; slice j takes columns 32 h + 8 j .. + 8 of both operands.  Each
                // activation operand is read from LDS just before its MFMA and the compiler
                // interleaves the reads with the MFMAs (reading slice j + 1's operands ahead into a
                // second register set measured 3-4% slower and used 24 more registers).
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8_t a = as_bf16x8(live ? wr[u][j] : make_uint4(0, 0, 0, 0));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const uint4 bx = *reinterpret_cast<const uint4*>(xb + mb * 32 * kXStride + 8 * j);
                        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(bx), acc[mb], 0, 0, 0);
                    }
                }
                // refill this ring slot with the step kInFlight ahead
                const int sw = min(s + kInFlight, nsteps - 1);
#pragma unroll
                for (int j = 0; j < 4; ++j) wr[u][j] = wload(sw, j);
                __syncthreads();                       // chunk s read by all; chunk s + 1 staged
            }
        }
        // acc[mb][i]: weight row 8 (i / 4) + 4 h + i % 4 of the wave's 32, activation row mb 32 + r
        if constexpr (kGateUp) {
            float* up = reinterpret_cast<float*>(&xs[0][0]);    // [2][MB][16][64] up values
            if (wv >= kHalf) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) up[(((wv - kHalf) * MB + mb) * 16 + i) * kWave + lane] = acc[mb][i];
            }
            __syncthreads();
            if (wv < kHalf) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int m = mb * 32 + r;
                    if (m >= M) continue;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = nw + 8 * g + 4 * h;
                        if (n >= N) continue;
                        float o[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float gv = acc[mb][4 * g + e];
                            o[e] = gv / (1.f + __expf(-gv)) * up[((wv * MB + mb) * 16 + 4 * g + e) * kWave + lane];
                        }
                        *reinterpret_cast<uint2*>(act + static_cast<int64_t>(m) * N + n) =
                            make_uint2(attn::pack_bf16x2(o[0], o[1]), attn::pack_bf16x2(o[2], o[3]));
                    }
                }
            }
        } else {
            float* pp = P + static_cast<int64_t>(blockIdx.y) * M * N;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = mb * 32 + r;
                if (m >= M) continue;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = nw + 8 * g + 4 * h;
                    if (n < N)
                        *reinterpret_cast<float4*>(pp + static_cast<int64_t>(m) * N + n) =
                            make_float4(acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]);
                }
            }
        }
    } else {
        // activation chunks: 16 bytes each, kPer per thread, row c / 8, column 8 (c % 8) of the step;
        // rows past M are staged as zeros
        const int xt = threadIdx.x - kMW * kWave;
        constexpr int kPer = MB * 4 / kLW;             // 16-byte chunks per thread and step
        const uint4* xp[kPer];
        int xo[kPer];
        bool xok[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = xt + kLW * kWave * i;
            const int row = c >> 3, col = c & 7;
            xok[i] = row < M;
            xp[i] = reinterpret_cast<const uint4*>(X + static_cast<int64_t>(min(row, M - 1)) * K + k0 + 8 * col);
            xo[i] = row * kXStride + 8 * col;
        }
        uint4 xr[kXSets][kPer];                          // chunk t in set t % kXSets
#pragma unroll
        for (int c = 0; c < kXSets; ++c)
#pragma unroll
            for (int i = 0; i < kPer; ++i) xr[c][i] = xp[i][min(c, nsteps - 1) * (kStep / 8)];
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            *reinterpret_cast<uint4*>(&xs[0][xo[i]]) = xok[i] ? xr[0][i] : make_uint4(0, 0, 0, 0);
        __syncthreads();                               // chunk 0 staged
        for (int sb = 0; sb < padded; sb += kInFlight) {
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int s = sb + u;
                // chunk s + 1 to the LDS buffer that chunk s - 1 used (the wait leaves the chunks
                // after it in flight)
#pragma unroll
                for (int i = 0; i < kPer; ++i)
                    *reinterpret_cast<uint4*>(&xs[(u + 1) & 1][xo[i]]) =
                        xok[i] ? xr[(u + 1) % kXSets][i] : make_uint4(0, 0, 0, 0);
                // the set that held chunk s (in LDS since the last step) takes chunk s + kXSets
                const int sx = min(s + kXSets, nsteps - 1);
#pragma unroll
                for (int i = 0; i < kPer; ++i) xr[u % kXSets][i] = xp[i][sx * (kStep / 8)];
                __syncthreads();
            }
        }
        if constexpr (kGateUp) __syncthreads();        // matches the up-value exchange
    }
}

// The tile order of a weight matrix W [N][K] bf16 (N a multiple of 32, K of 64) for gemm_kernel:
// 16-byte unit ((rb * (K / 64) + s) * 4 + j) * 64 + l holds W[32 rb + l % 32][64 s + 32 (l / 32)
// + 8 j .. + 8]: the A operand of MFMA slice j of step s for lane l of the wave that owns rows
// 32 rb .. 32 rb + 31.  One thread per output unit (coalesced stores).
__global__ __launch_bounds__(kThreads) void pack_weights_kernel(const uint4* __restrict__ W, int N, int K,
                                                                uint4* __restrict__ Pk) {
    const int64_t u = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int ks = K / kStep;
    if (u >= static_cast<int64_t>(N) * K / 8) return;
    const int l = static_cast<int>(u % kWave), j = static_cast<int>((u / kWave) % 4);
    const int64_t t = u / (4 * kWave);
    const int s = static_cast<int>(t % ks);
    const int64_t rb = t / ks;
    const int64_t row = rb * kRowsPerWave + l % 32;
    Pk[u] = W[(row * K + static_cast<int64_t>(s) * kStep + 32 * (l / 32) + 8 * j) / 8];
}

constexpr int kMaxSplits = 16;

// sum over the splits of the four consecutive partials at idx (all loads issued first)
__device__ __forceinline__ float4 split_sum4(const float* __restrict__ P, int splits, int64_t plane, int64_t idx) {
    float4 v[kMaxSplits];
#pragma unroll
    for (int i = 0; i < kMaxSplits; ++i)
        if (i < splits) v[i] = *reinterpret_cast<const float4*>(P + i * plane + idx);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kMaxSplits; ++i)
        if (i < splits) {
            s.x += v[i].x;
            s.y += v[i].y;
            s.z += v[i].z;
            s.w += v[i].w;
        }
    return s;
}

__device__ __forceinline__ void load_bf16x4(const uint16_t* p, float* f) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    f[0] = bf16_lo(w.x);
    f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y);
    f[3] = bf16_hi(w.y);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, const float* f) {
    *reinterpret_cast<uint2*>(p) = make_uint2(attn::pack_bf16x2(f[0], f[1]), attn::pack_bf16x2(f[2], f[3]));
}

// The row-wise kernels (norms) run one 1024-thread workgroup per row and keep the first
// 4 kNormThreads kNormPasses columns of the row in registers between the sum of squares and the
// scaling, so the row is read once; columns past that (rows wider than 8192) are read again.
constexpr int kNormThreads = 1024;
constexpr int kNormPasses = 2;

// bf16 rounding of v, back in fp32 (the value a bf16 store and reload would give)
__device__ __forceinline__ float round_bf16(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// h[t] = rms(x[t]) g.  Also the rotary (cos, sin) of row t's position ctx_len + depth for every
// frequency j < D/2, with the angle formed in fp64: once per row here instead of once per head in
// the q/k/v epilogue.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ g, int hd, float eps,
                                                               uint16_t* __restrict__ h, int n1, int D,
                                                               const int32_t* __restrict__ ctx_len,
                                                               const int32_t* __restrict__ depth, float theta,
                                                               float2* __restrict__ rot) {
    __shared__ float red[kNormThreads / kWave];
    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + row * hd;
    float xv[kNormPasses][4], gv[kNormPasses][4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kNormPasses; ++i) {
        const int c = 4 * (threadIdx.x + i * kNormThreads);
        if (c < hd) {
            load_bf16x4(xr + c, xv[i]);
            load_bf16x4(g + c, gv[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < kNormPasses; ++i)
        if (4 * (threadIdx.x + i * kNormThreads) < hd)
            ss += xv[i][0] * xv[i][0] + xv[i][1] * xv[i][1] + xv[i][2] * xv[i][2] + xv[i][3] * xv[i][3];
    for (int c = 4 * (threadIdx.x + kNormPasses * kNormThreads); c < hd; c += 4 * kNormThreads) {
        float f[4];
        load_bf16x4(xr + c, f);
        ss += f[0] * f[0] + f[1] * f[1] + f[2] * f[2] + f[3] * f[3];
    }
    const float inv = 1.f / sqrtf(block_sum(ss, red) / hd + eps);
#pragma unroll
    for (int i = 0; i < kNormPasses; ++i) {
        const int c = 4 * (threadIdx.x + i * kNormThreads);
        if (c < hd) {
            float f[4];
            for (int e = 0; e < 4; ++e) f[e] = xv[i][e] * inv * gv[i][e];
            store_bf16x4(h + row * hd + c, f);
        }
    }
    for (int c = 4 * (threadIdx.x + kNormPasses * kNormThreads); c < hd; c += 4 * kNormThreads) {
        float f[4], gg[4];
        load_bf16x4(xr + c, f);
        load_bf16x4(g + c, gg);
        for (int e = 0; e < 4; ++e) f[e] = f[e] * inv * gg[e];
        store_bf16x4(h + row * hd + c, f);
    }
    const int j = threadIdx.x;
    if (j < D / 2) {
        const int b = static_cast<int>(row) / n1;
        const double ang = (static_cast<double>(ctx_len[b]) + static_cast<double>(depth[row])) * pow(static_cast<double>(theta), -2.0 * j / D);
        rot[row * (D / 2) + j] = make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
    }
}

// q/k/v of row t = m0 + blockIdx.y, head blockIdx.x (query heads, then key, then value heads),
// one rotary pair (j, j + D/2) per thread: add the splits, rotate q and k at ctx_len + depth (the
// (cos, sin) table of rmsnorm_kernel), write
// q to qrot[t] and k, v to the cache at ctx_len + node.  A row of an invalid sequence (a bad tree,
// or no room in the cache) writes NaN queries (its attention output is NaN) and nothing else.
__global__ __launch_bounds__(64) void qkv_epilogue_kernel(
    const float* __restrict__ P, int splits, int Mc, int m0, int n1, int Hq, int Hkv, int D, int Lmax,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ depth, const float2* __restrict__ rot,
    uint16_t* __restrict__ qrot, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
    const int head = blockIdx.x, mloc = blockIdx.y, j = threadIdx.x;
    const int half = D / 2;
    if (j >= half) return;
    const int t = m0 + mloc;
    const int b = t / n1, i = t - b * n1;
    const int L = ctx_len[b], d = depth[t];
    const bool ok = d >= 0 && L >= 0 && L <= Lmax - n1;
    const int N = (Hq + 2 * Hkv) * D;
    const int64_t plane = static_cast<int64_t>(Mc) * N;
    const float* pr = P + static_cast<int64_t>(mloc) * N + head * D + j;
    const float2 cs = head < Hq + Hkv ? rot[static_cast<int64_t>(t) * half + j] : make_float2(1.f, 0.f);
    float lo = 0.f, hi = 0.f;
    {
        float va[kMaxSplits], vb[kMaxSplits];
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s)
            if (s < splits) {
                va[s] = pr[s * plane];
                vb[s] = pr[s * plane + half];
            }
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s)
            if (s < splits) {
                lo += va[s];
                hi += vb[s];
            }
    }
    if (head < Hq + Hkv) {
        // angle (ctx_len + depth) theta^(-2j/D), from the row's table
        const float c = cs.x, sn = cs.y;
        const float a = lo;
        lo = a * c - hi * sn;
        hi = hi * c + a * sn;
    }
    if (head < Hq) {
        uint16_t* qr = qrot + (static_cast<int64_t>(t) * Hq + head) * D;
        qr[j] = ok ? f32_to_bf16(lo) : 0x7fc0;
        qr[j + half] = ok ? f32_to_bf16(hi) : 0x7fc0;
    } else if (ok) {
        const int kvh = head < Hq + Hkv ? head - Hq : head - Hq - Hkv;
        uint16_t* dst = (head < Hq + Hkv ? kc : vc) +
                        ((static_cast<int64_t>(b) * Hkv + kvh) * Lmax + SPECV_CHK(L + i, Lmax, kSiteLayerCache)) * D;
        dst[j] = f32_to_bf16(lo);
        dst[j + half] = f32_to_bf16(hi);
    }
}

// y[t] = x[t] + sum of splits (stored bf16), h2[t] = rms(y[t]) g; the rounded y stays in registers
// for the scaling (columns past the cached ones read it back)
__global__ __launch_bounds__(kNormThreads) void residual_norm_kernel(const float* __restrict__ P, int splits, int Mc,
                                                                     int m0, int hd, const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ g, float eps,
                                                                     uint16_t* __restrict__ y, uint16_t* __restrict__ h2) {
    __shared__ float red[kNormThreads / kWave];
    const int mloc = blockIdx.x;
    const int64_t t = m0 + mloc;
    const int64_t plane = static_cast<int64_t>(Mc) * hd;
    const float* pr = P + static_cast<int64_t>(mloc) * hd;
    float yv[kNormPasses][4], gv[kNormPasses][4];
#pragma unroll
    for (int i = 0; i < kNormPasses; ++i) {
        const int c = 4 * (threadIdx.x + i * kNormThreads);
        if (c < hd) {
            load_bf16x4(x + t * hd + c, yv[i]);
            load_bf16x4(g + c, gv[i]);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kNormPasses; ++i) {
        const int c = 4 * (threadIdx.x + i * kNormThreads);
        if (c < hd) {
            const float4 s = split_sum4(pr, splits, plane, c);
            yv[i][0] += s.x;
            yv[i][1] += s.y;
            yv[i][2] += s.z;
            yv[i][3] += s.w;
            store_bf16x4(y + t * hd + c, yv[i]);
            for (int e = 0; e < 4; ++e) {
                yv[i][e] = round_bf16(yv[i][e]);          // the stored residual stream
                ss += yv[i][e] * yv[i][e];
            }
        }
    }
    for (int c = 4 * (threadIdx.x + kNormPasses * kNormThreads); c < hd; c += 4 * kNormThreads) {
        const float4 s = split_sum4(pr, splits, plane, c);
        float f[4];
        load_bf16x4(x + t * hd + c, f);
        f[0] += s.x;
        f[1] += s.y;
        f[2] += s.z;
        f[3] += s.w;
        store_bf16x4(y + t * hd + c, f);
        for (int e = 0; e < 4; ++e) {
            f[e] = round_bf16(f[e]);
            ss += f[e] * f[e];
        }
    }
    const float inv = 1.f / sqrtf(block_sum(ss, red) / hd + eps);
#pragma unroll
    for (int i = 0; i < kNormPasses; ++i) {
        const int c = 4 * (threadIdx.x + i * kNormThreads);
        if (c < hd) {
            float f[4];
            for (int e = 0; e < 4; ++e) f[e] = yv[i][e] * inv * gv[i][e];
            store_bf16x4(h2 + t * hd + c, f);
        }
    }
    for (int c = 4 * (threadIdx.x + kNormPasses * kNormThreads); c < hd; c += 4 * kNormThreads) {
        float f[4], gg[4];
        load_bf16x4(y + t * hd + c, f);
        load_bf16x4(g + c, gg);
        for (int e = 0; e < 4; ++e) f[e] = f[e] * inv * gg[e];
        store_bf16x4(h2 + t * hd + c, f);
    }
}

// act[t][j] = silu(g) u with g, u the split sums of columns j and I + j (products with more than
// one split; one split finishes in gemm_kernel<., true>)
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(const float* __restrict__ P, int splits, int Mc, int m0,
                                                            int inter, uint16_t* __restrict__ act) {
    const int mloc = blockIdx.y;
    const int64_t t = m0 + mloc;
    const int j = 4 * (blockIdx.x * kThreads + threadIdx.x);
    if (j >= inter) return;
    const int64_t plane = static_cast<int64_t>(Mc) * 2 * inter;
    const float* pr = P + static_cast<int64_t>(mloc) * 2 * inter;
    const float4 gv = split_sum4(pr, splits, plane, j), uv = split_sum4(pr, splits, plane, inter + j);
    float f[4] = {gv.x / (1.f + __expf(-gv.x)) * uv.x, gv.y / (1.f + __expf(-gv.y)) * uv.y,
                  gv.z / (1.f + __expf(-gv.z)) * uv.z, gv.w / (1.f + __expf(-gv.w)) * uv.w};
    store_bf16x4(act + t * inter + j, f);
}

// out[t] = y[t] + sum of splits
__global__ __launch_bounds__(kThreads) void residual_kernel(const float* __restrict__ P, int splits, int Mc, int m0,
                                                            int hd, const uint16_t* __restrict__ y,
                                                            uint16_t* __restrict__ out) {
    const int mloc = blockIdx.y;
    const int64_t t = m0 + mloc;
    const int c = 4 * (blockIdx.x * kThreads + threadIdx.x);
    if (c >= hd) return;
    const int64_t plane = static_cast<int64_t>(Mc) * hd;
    const float4 s = split_sum4(P + static_cast<int64_t>(mloc) * hd, splits, plane, c);
    float f[4];
    load_bf16x4(y + t * hd + c, f);
    f[0] += s.x;
    f[1] += s.y;
    f[2] += s.z;
    f[3] += s.w;
    store_bf16x4(out + t * hd + c, f);
}

// ---------------------------------------------------------------------------------- host side

// Split count for a product with `tiles` workgroup tiles over K: the most splits that still give
// at most one workgroup per CU (one 8-wave workgroup fills a CU), at least one, at most
// kMaxSplits, and no empty split.
int gemm_splits(int tiles, int K) {
    const int steps = K / kStep;
    const int slots = device_cu_count() * max(1, 8 / (kMW + kLW));   // resident workgroups
    const int s = max(1, min(min(slots / max(tiles, 1), kMaxSplits), steps));
    const int per = (steps + s - 1) / s;
    return (steps + per - 1) / per;
}

int gemm_tiles(int N, bool gate_up) {
    const int rows = gate_up ? kTileRows / 2 : kTileRows;
    return (N + rows - 1) / rows;
}

// gate_up: W is [2 N][K] and act receives silu(gate) up (splits must be 1)
hipError_t launch_gemm(const uint16_t* X, int M, int K, const uint16_t* W, int N, int splits, float* P,
                       uint16_t* act, bool gate_up, bool packed, hipStream_t stream) {
    const int steps = K / kStep;
    const int per = (steps + splits - 1) / splits;
    const dim3 grid(gemm_tiles(N, gate_up), splits);
    const int mb = (M + 31) / 32;
    if (gate_up && splits != 1) return hipErrorInvalidValue;
    switch (mb) {
#define SPECV_GEMM_CASE(n)                                                                              \
        case n:                                                                                         \
            if (packed) {                                                                               \
                if (gate_up) gemm_kernel<n, true, true><<<grid, kGemmThreads, 0, stream>>>(X, M, K, W, N, per, P, act); \
                else gemm_kernel<n, false, true><<<grid, kGemmThreads, 0, stream>>>(X, M, K, W, N, per, P, act); \
            } else {                                                                                    \
                if (gate_up) gemm_kernel<n, true, false><<<grid, kGemmThreads, 0, stream>>>(X, M, K, W, N, per, P, act); \
                else gemm_kernel<n, false, false><<<grid, kGemmThreads, 0, stream>>>(X, M, K, W, N, per, P, act); \
            }                                                                                           \
            break;
        SPECV_GEMM_CASE(1) SPECV_GEMM_CASE(2) SPECV_GEMM_CASE(3) SPECV_GEMM_CASE(4)
        SPECV_GEMM_CASE(5) SPECV_GEMM_CASE(6) SPECV_GEMM_CASE(7) SPECV_GEMM_CASE(8)
#undef SPECV_GEMM_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

struct LayerPlan {
    int T, hd, nqkv, inter;
    int chunk;                       // activation rows per product launch
    int s_qkv, s_o, s_gu, s_down;    // splits per product
    size_t off_h, off_q, off_a, off_y, off_h2, off_act, off_rot, off_p, off_attn, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

LayerPlan plan_layer(int B, int n1, int Hq, int Hkv, int D, int Lmax, int inter) {
    LayerPlan p{};
    p.T = B * n1;
    p.hd = Hq * D;
    p.nqkv = (Hq + 2 * Hkv) * D;
    p.inter = inter;
    p.chunk = min(p.T, 32 * kMaxMB);
    p.s_qkv = gemm_splits(gemm_tiles(p.nqkv, false), p.hd);
    p.s_o = gemm_splits(gemm_tiles(p.hd, false), Hq * D);
    p.s_gu = gemm_splits(gemm_tiles(inter, true), p.hd);
    p.s_down = gemm_splits(gemm_tiles(p.hd, false), inter);
    const size_t T = p.T, e = sizeof(uint16_t);
    size_t o = 0;
    p.off_h = o;   o += align256(T * p.hd * e);
    p.off_q = o;   o += align256(T * Hq * D * e);
    p.off_a = o;   o += align256(T * Hq * D * e);
    p.off_y = o;   o += align256(T * p.hd * e);
    p.off_h2 = o;  o += align256(T * p.hd * e);
    p.off_act = o; o += align256(T * inter * e);
    p.off_rot = o; o += align256(T * (D / 2) * sizeof(float2));
    const size_t pmax = max(max(size_t(p.s_qkv) * p.nqkv, size_t(p.s_o) * p.hd),
                            max(size_t(p.s_gu) * 2 * inter, size_t(p.s_down) * p.hd));
    p.off_p = o;   o += align256(pmax * p.chunk * sizeof(float));
    p.off_attn = o;
    o += align256(attn_workspace_bytes(B, n1, Hq, Hkv, D, Lmax));
    p.total = o;
    return p;
}

}  // namespace

size_t layer_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax, int inter) {
    return plan_layer(B, n1, Hq, Hkv, D, Lmax, inter).total;
}

hipError_t launch_verify_layer(const LayerArgs& a, hipStream_t stream) {
    const LayerPlan p = plan_layer(a.B, a.n1, a.Hq, a.Hkv, a.D, a.Lmax, a.inter);
    char* ws = static_cast<char*>(a.workspace);
    auto bf = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
    uint16_t *h = bf(p.off_h), *q = bf(p.off_q), *att = bf(p.off_a), *y = bf(p.off_y), *h2 = bf(p.off_h2),
             *act = bf(p.off_act);
    float* P = reinterpret_cast<float*>(ws + p.off_p);
    float2* rot = reinterpret_cast<float2*>(ws + p.off_rot);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    uint16_t* out = static_cast<uint16_t*>(a.out);
    hipError_t e;

    rmsnorm_kernel<<<p.T, kNormThreads, 0, stream>>>(x, static_cast<const uint16_t*>(a.attn_norm), p.hd, a.eps, h,
                                                     a.n1, a.D, a.ctx_len, a.depth, a.theta, rot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int heads = a.Hq + 2 * a.Hkv;
    for (int m0 = 0; m0 < p.T; m0 += p.chunk) {
        const int mc = min(p.chunk, p.T - m0);
        if ((e = launch_gemm(h + static_cast<int64_t>(m0) * p.hd, mc, p.hd, static_cast<const uint16_t*>(a.w_qkv),
                             p.nqkv, p.s_qkv, P, nullptr, false, a.packed, stream)) != hipSuccess)
            return e;
        qkv_epilogue_kernel<<<dim3(heads, mc), 64, 0, stream>>>(P, p.s_qkv, mc, m0, a.n1, a.Hq, a.Hkv, a.D, a.Lmax,
                                                                a.ctx_len, a.depth, rot, q,
                                                                static_cast<uint16_t*>(a.k_cache),
                                                                static_cast<uint16_t*>(a.v_cache));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    AttnArgs aa{q, a.k_cache, a.v_cache, a.ctx_len, a.mask, a.B, a.n1, a.Hq, a.Hkv, a.D, a.Lmax,
                1.f / sqrtf(static_cast<float>(a.D)), true, att, nullptr, ws + p.off_attn};
    if ((e = launch_attention(aa, stream)) != hipSuccess) return e;
    const dim3 row_grid_hd((p.hd / 4 + kThreads - 1) / kThreads, 1);
    for (int m0 = 0; m0 < p.T; m0 += p.chunk) {
        const int mc = min(p.chunk, p.T - m0);
        if ((e = launch_gemm(att + static_cast<int64_t>(m0) * p.hd, mc, p.hd, static_cast<const uint16_t*>(a.w_o),
                             p.hd, p.s_o, P, nullptr, false, a.packed, stream)) != hipSuccess)
            return e;
        residual_norm_kernel<<<mc, kNormThreads, 0, stream>>>(P, p.s_o, mc, m0, p.hd, x,
                                                          static_cast<const uint16_t*>(a.mlp_norm), a.eps, y, h2);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    for (int m0 = 0; m0 < p.T; m0 += p.chunk) {
        const int mc = min(p.chunk, p.T - m0);
        const bool fused = p.s_gu == 1;
        if ((e = launch_gemm(h2 + static_cast<int64_t>(m0) * p.hd, mc, p.hd,
                             static_cast<const uint16_t*>(a.w_gate_up), fused ? a.inter : 2 * a.inter, p.s_gu, P,
                             act + static_cast<int64_t>(m0) * a.inter, fused, a.packed, stream)) != hipSuccess)
            return e;
        if (!fused) {
            silu_mul_kernel<<<dim3((a.inter / 4 + kThreads - 1) / kThreads, mc), kThreads, 0, stream>>>(
                P, p.s_gu, mc, m0, a.inter, act);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    for (int m0 = 0; m0 < p.T; m0 += p.chunk) {
        const int mc = min(p.chunk, p.T - m0);
        if ((e = launch_gemm(act + static_cast<int64_t>(m0) * a.inter, mc, a.inter,
                             static_cast<const uint16_t*>(a.w_down), p.hd, p.s_down, P, nullptr, false, a.packed,
                             stream)) !=
            hipSuccess)
            return e;
        residual_kernel<<<dim3(row_grid_hd.x, mc), kThreads, 0, stream>>>(P, p.s_down, mc, m0, p.hd, y, out);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_pack_weights(const void* w, int N, int K, void* packed, hipStream_t stream) {
    const int64_t units = static_cast<int64_t>(N) * K / 8;
    const int64_t blocks = (units + kThreads - 1) / kThreads;
    pack_weights_kernel<<<static_cast<unsigned>(blocks), kThreads, 0, stream>>>(
        static_cast<const uint4*>(w), N, K, static_cast<uint4*>(packed));
    return hipGetLastError();
}

}  // namespace specv
