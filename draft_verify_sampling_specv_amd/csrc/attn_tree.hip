// Tree-attention verify, general case (many query rows per KV head: big trees x GQA groups)
// ([SD-EAGLE] "Tree Attention Verification"; [PTD] Method 4, "Verification").
//   * grid (split, KV head x row group, sequence).  The query rows of one KV head are the
//     G x (K+1) pairs (node, head in group), row r = node * G + g, cut into 32-row blocks; one
//     wave per row block.  The key range ctx_len + K + 1 is cut into 32-key tiles and the tiles
//     into `nsplit` contiguous splits (flash-decoding style), one workgroup per split.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K is the A operand (from LDS), Q^T the B operand
//     (kept in registers), so the 32x32 result puts one query row in each lane column and the
//     row max / row sum need one cross-half shuffle.
//   * O^T += V^T P^T with the same instruction; P stays in registers (the accumulator layout of
//     S^T is reused as the B operand with a matching key permutation), V is staged in LDS
//     transposed ([d][key]) so each lane reads 4 consecutive keys per 8-byte LDS read.
//   * K/V tiles are loaded once per workgroup with coalesced 16-byte global loads, double
//     buffered in LDS (the next tile's loads are in flight while the current one is computed).
//   * The tree mask is applied only on tiles that reach past the context.
//   * Each split writes an unnormalised partial (O, running max, sum); a combine kernel merges the
//     splits (log-sum-exp weights), writes bf16 O and the natural-log LSE.

#include "attn_common.h"
#include "kernels.h"

namespace specv {
namespace {
using namespace attn;

constexpr int kMaxWaves = 8;

template <int D>
struct Smem {
    static constexpr int kRow = D + 8;             // K tile row pitch (bf16): 16 bytes of padding
    static constexpr int kVtRow = kTileKeys + 4;   // V^T tile row pitch (bf16): 8 bytes of padding
    uint16_t k[2][kTileKeys * kRow];
    uint16_t vt[2][D * kVtRow];
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct AttnLayout {
    size_t opart, ml, total;
    AttnLayout(int B, int Hkv, int nsplit, int R, int D) {
        opart = 0;
        ml = align256(sizeof(float) * size_t(B) * Hkv * nsplit * R * D);
        total = align256(ml + sizeof(float2) * size_t(B) * Hkv * nsplit * R);
    }
};

struct Plan {
    int nsplit, nw, groups, rbpg, chunks;
};

template <int D, int NW>
__global__ void __launch_bounds__(NW * kWave)
attn_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                    const uint16_t* __restrict__ vc, const int32_t* __restrict__ ctx_len,
                    const uint32_t* __restrict__ mask, int n1, int Hq, int Hkv, int Lmax,
                    float c2, int nsplit, int groups, int rbpg, float* __restrict__ opart,
                    float2* __restrict__ mlpart) {
    constexpr int kChunksPerRow = D / 8;                  // 16-byte chunks per K/V row
    constexpr int kChunks = kTileKeys * kChunksPerRow;    // per tile, for K and for V
    constexpr int kDB = D / 32;                           // 32-wide d blocks of O^T
    constexpr int kKS = D / 16;                           // k-steps of S^T = K Q^T
    constexpr int kThreads = NW * kWave;
    constexpr int MAXC = (kChunks + kThreads - 1) / kThreads;   // 16-byte chunks per thread
    __shared__ Smem<D> sm;

    const int split = blockIdx.x;
    const int kv = blockIdx.y / groups, grp = blockIdx.y % groups;
    const int b = blockIdx.z;
    const int G = Hq / Hkv, R = G * n1;
    const int RB = (R + 31) / 32;
    constexpr int nthreads = kThreads;
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int h = lane / 32, col = lane % 32;
    const int rb = grp * rbpg + w;
    const bool wave_rows = rb < RB && w < rbpg;
    const int row = rb * 32 + col;
    const bool row_ok = wave_rows && row < R;
    const int words = (n1 + 31) >> 5;

    const int L = ctx_len[b];
    const bool seq_ok = L >= 0 && L + n1 <= Lmax;
    const int Ltot = L + n1;
    const int ntiles = seq_ok ? (Ltot + kTileKeys - 1) / kTileKeys : 0;
    const int tps = (ntiles + nsplit - 1) / nsplit;
    const int t0 = split * tps, t1 = min(ntiles, t0 + tps);
    const int64_t pbase = (static_cast<int64_t>(b) * Hkv + kv) * nsplit + split;

    // query row of this lane: node i, head kv*G + g
    const int node = row_ok ? row / G : 0;
    const int g = row_ok ? row - node * G : 0;
    const uint32_t* mrow = mask + (static_cast<int64_t>(b) * n1 + node) * words;

    bf16x8_t qreg[kKS];
    {
        const uint16_t* qp = q + ((static_cast<int64_t>(b) * n1 + node) * Hq + kv * G + g) * D;
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_ok) v = *reinterpret_cast<const uint4*>(qp + 16 * s + 8 * h);
            qreg[s] = as_bf16x8(v);
        }
    }

    const uint16_t* kbase = kc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;
    const uint16_t* vbase = vc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;

    uint4 kpre[MAXC], vpre[MAXC];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = threadIdx.x + j * nthreads;
            const int key = t * kTileKeys + c / kChunksPerRow;
            const int d0 = (c % kChunksPerRow) * 8;
            kpre[j] = make_uint4(0, 0, 0, 0);
            vpre[j] = make_uint4(0, 0, 0, 0);
            if (c < kChunks && key < Ltot) {
                kpre[j] = *reinterpret_cast<const uint4*>(kbase + static_cast<int64_t>(key) * D + d0);
                vpre[j] = *reinterpret_cast<const uint4*>(vbase + static_cast<int64_t>(key) * D + d0);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = threadIdx.x + j * nthreads;
            if (c < kChunks) {
                const int key = c / kChunksPerRow;
                const int d0 = (c % kChunksPerRow) * 8;
                *reinterpret_cast<uint4*>(&sm.k[buf][key * Smem<D>::kRow + d0]) = kpre[j];
                const uint32_t vw[4] = {vpre[j].x, vpre[j].y, vpre[j].z, vpre[j].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sm.vt[buf][(d0 + e) * Smem<D>::kVtRow + key] =
                        static_cast<uint16_t>((e & 1) ? (vw[e >> 1] >> 16) : (vw[e >> 1] & 0xffffu));
            }
        }
    };

    f32x16_t o[kDB];
#pragma unroll
    for (int i = 0; i < kDB; ++i) o[i] = f32x16_t{};
    float m = -INFINITY;   // running max of scaled (base-2) scores of this lane's row
    float l = 0.f;

    if (t0 < t1) {
        load_tile(t0);
        store_tile(0);
    }
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        if (t + 1 < t1) load_tile(t + 1);
        if (wave_rows) {
            // S^T (keys x rows) = K Q^T
            f32x16_t s = f32x16_t{};
            const uint16_t* kt = sm.k[buf];
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) {
                const uint4 a = *reinterpret_cast<const uint4*>(&kt[col * Smem<D>::kRow + 16 * ks + 8 * h]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qreg[ks], s, 0, 0, 0);
            }
            // s[r] holds key t*32 + 8*(r/4) + 4*h + r%4 of row `row`
            const int kb = t * kTileKeys;
            if (kb + kTileKeys > L) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 8 * (r / 4) + 4 * h + (r % 4);
                    bool vis = key < L;
                    if (!vis && key < Ltot) {
                        const int jj = key - L;
                        vis = (mrow[jj >> 5] >> (jj & 31)) & 1u;
                    }
                    if (!vis) s[r] = -INFINITY;
                }
            }
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m, mx * c2);
            const float mref = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(m - mref);
            float p[16];
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mref));
                rs += p[r];
            }
            rs += __shfl_xor(rs, 32);
            l = l * alpha + rs;
            m = mnew;
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int i = 0; i < kDB; ++i) o[i] *= alpha;
            }
            // O^T (d x rows) += V^T P^T
            const uint16_t* vt = sm.vt[buf];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                uint4 pw;
                pw.x = pack_bf16x2(p[8 * ks + 0], p[8 * ks + 1]);
                pw.y = pack_bf16x2(p[8 * ks + 2], p[8 * ks + 3]);
                pw.z = pack_bf16x2(p[8 * ks + 4], p[8 * ks + 5]);
                pw.w = pack_bf16x2(p[8 * ks + 6], p[8 * ks + 7]);
                const bf16x8_t pb = as_bf16x8(pw);
#pragma unroll
                for (int db = 0; db < kDB; ++db) {
                    const uint16_t* vr = &vt[(db * 32 + col) * Smem<D>::kVtRow + 16 * ks + 4 * h];
                    const uint2 lo = *reinterpret_cast<const uint2*>(vr);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, o[db], 0, 0, 0);
                }
            }
        }
        if (t + 1 < t1) store_tile(buf ^ 1);
        __syncthreads();
    }

    if (row_ok) {
        const int64_t prow = pbase * R + row;
        float* op = opart + prow * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int d0 = db * 32 + 8 * rr + 4 * h;
                *reinterpret_cast<float4*>(op + d0) =
                    make_float4(o[db][4 * rr + 0], o[db][4 * rr + 1], o[db][4 * rr + 2], o[db][4 * rr + 3]);
            }
        if (h == 0) mlpart[prow] = make_float2(m, l);
    }
}

// Merge the splits of one output row: weights 2^(m_s - M) l_s; out = sum w O_s / sum w l_s.
template <typename OutT>
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ opart, const float2* __restrict__ mlpart,
                    const int32_t* __restrict__ ctx_len, int B, int n1, int Hq, int Hkv, int D,
                    int Lmax, int nsplit, OutT* __restrict__ out, float* __restrict__ lse) {
    const int G = Hq / Hkv, R = G * n1;
    const int dv = D / 4;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(B) * n1 * Hq * dv;
    if (gid >= total) return;
    const int d0 = static_cast<int>(gid % dv) * 4;
    const int64_t orow = gid / dv;                  // (b, node, head)
    const int hh = static_cast<int>(orow % Hq);
    const int node = static_cast<int>((orow / Hq) % n1);
    const int b = static_cast<int>(orow / (static_cast<int64_t>(Hq) * n1));
    const int kv = hh / G, g = hh % G;
    const int row = node * G + g;
    const int L = ctx_len[b];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f, M = -INFINITY;
    const bool ok = L >= 0 && L + n1 <= Lmax;
    if (ok) {
        for (int s = 0; s < nsplit; ++s) {
            const float2 ml = mlpart[((static_cast<int64_t>(b) * Hkv + kv) * nsplit + s) * R + row];
            if (ml.y > 0.f) M = fmaxf(M, ml.x);
        }
        for (int s = 0; s < nsplit; ++s) {
            const int64_t prow = ((static_cast<int64_t>(b) * Hkv + kv) * nsplit + s) * R + row;
            const float2 ml = mlpart[prow];
            if (!(ml.y > 0.f)) continue;
            const float wgt = __builtin_amdgcn_exp2f(ml.x - M);
            const float4 v = *reinterpret_cast<const float4*>(opart + prow * D + d0);
            acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
            den += wgt * ml.y;
        }
    }
    const float inv = ok ? 1.f / den : NAN;
    const float r[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    OutT* op = out + orow * D + d0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(OutT) == 2) {
            const uint32_t u = __float_as_uint(r[e]);
            op[e] = (r[e] != r[e]) ? static_cast<uint16_t>(0x7fc0u)
                                   : static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
        } else {
            op[e] = r[e];
        }
    }
    if (lse && d0 == 0) lse[orow] = ok ? (M + log2f(den)) * kLn2 : NAN;
}

Plan make_plan(int B, int n1, int Hq, int Hkv, int D, int Lmax) {
    const int G = Hq / Hkv, R = G * n1;
    const int RB = (R + 31) / 32;
    Plan p;
    p.groups = (RB + kMaxWaves - 1) / kMaxWaves;
    p.rbpg = (RB + p.groups - 1) / p.groups;
    p.nw = 1;
    while (p.nw < p.rbpg) p.nw *= 2;   // 1, 2, 4 or 8 waves; spare waves only help loading
    p.chunks = 0;
    // Splits over the key range: enough workgroups to cover the machine several times over, at
    // least 4 tiles per split.
    const int tiles = (Lmax + kTileKeys - 1) / kTileKeys;
    const int units = B * Hkv * p.groups;
    int ns = 1;
    while ((units * ns < 512 || units * ns * p.nw < 2048) && tiles / (ns * 2) >= 4) ns *= 2;
    p.nsplit = ns;
    return p;
}

template <int D, int NW>
void launch_partial(const AttnArgs& a, const Plan& p, float* opart, float2* ml, hipStream_t stream) {
    const float c2 = a.scale * kLog2e;
    hipLaunchKernelGGL((attn_partial_kernel<D, NW>), dim3(p.nsplit, a.Hkv * p.groups, a.B),
                       dim3(p.nw * kWave), 0, stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k_cache), static_cast<const uint16_t*>(a.v_cache),
                       a.ctx_len, a.mask, a.n1, a.Hq, a.Hkv, a.Lmax, c2, p.nsplit, p.groups, p.rbpg,
                       opart, ml);
}

template <int D>
void dispatch_partial(const AttnArgs& a, const Plan& p, float* opart, float2* ml, hipStream_t stream) {
    switch (p.nw) {
        case 1: launch_partial<D, 1>(a, p, opart, ml, stream); break;
        case 2: launch_partial<D, 2>(a, p, opart, ml, stream); break;
        case 4: launch_partial<D, 4>(a, p, opart, ml, stream); break;
        default: launch_partial<D, 8>(a, p, opart, ml, stream); break;
    }
}

}  // namespace

size_t attn_tree_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax) {
    const Plan p = make_plan(B, n1, Hq, Hkv, D, Lmax);
    return AttnLayout(B, Hkv, p.nsplit, (Hq / Hkv) * n1, D).total;
}

hipError_t launch_attn_tree(const AttnArgs& a, hipStream_t stream) {
    const Plan p = make_plan(a.B, a.n1, a.Hq, a.Hkv, a.D, a.Lmax);
    const AttnLayout lay(a.B, a.Hkv, p.nsplit, (a.Hq / a.Hkv) * a.n1, a.D);
    char* ws = static_cast<char*>(a.workspace);
    float* opart = reinterpret_cast<float*>(ws + lay.opart);
    float2* ml = reinterpret_cast<float2*>(ws + lay.ml);
    if (a.D == 64) dispatch_partial<64>(a, p, opart, ml, stream);
    else dispatch_partial<128>(a, p, opart, ml, stream);
    const int64_t total = static_cast<int64_t>(a.B) * a.n1 * a.Hq * (a.D / 4);
    const int blocks = static_cast<int>((total + 255) / 256);
    hipLaunchKernelGGL((attn_combine_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream, opart, ml,
                       a.ctx_len, a.B, a.n1, a.Hq, a.Hkv, a.D, a.Lmax, p.nsplit,
                       static_cast<uint16_t*>(a.out), a.lse);
    return hipGetLastError();
}

}  // namespace specv
