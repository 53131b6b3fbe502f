// Tree-attention verify ([SD-EAGLE] "Tree Attention Verification"; [PTD] Method 4,
// "Verification"): every draft node's query attends to the whole committed context and to the
// tree entries of its own ancestors (and itself), all nodes in one pass.
//
// bf16 path (MFMA, gfx950):
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
//   * Online softmax in base 2 with the score scale folded into the exponent; rescaling of the
//     accumulators is skipped when no row's running max moved.
//   * Each split writes an unnormalised partial (O, running max, sum); a combine kernel merges the
//     splits (log-sum-exp weights), writes bf16 O and the natural-log LSE.
// fp32 path: a plain VALU kernel, one wave per output row (used for small fp32 cases).

#include "common.h"
#include "kernels.h"

namespace specv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTileKeys = 32;
constexpr int kMaxWaves = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // round-to-nearest-even fp32 -> bf16, two values per word
    uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    a = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
    b = (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
    return a | b;
}

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

// fp32 path: one wave per (sequence, node, head); lanes stride over the visible keys, each with
// its own online softmax state, merged across the wave at the end.
template <int D>
__global__ void __launch_bounds__(kWave)
attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kc,
                const float* __restrict__ vc, const int32_t* __restrict__ ctx_len,
                const uint32_t* __restrict__ mask, int n1, int Hq, int Hkv, int Lmax, float c2,
                float* __restrict__ out, float* __restrict__ lse) {
    const int hh = blockIdx.x % Hq, node = blockIdx.x / Hq, b = blockIdx.y;
    const int G = Hq / Hkv, kv = hh / G;
    const int lane = threadIdx.x;
    const int words = (n1 + 31) >> 5;
    const int L = ctx_len[b];
    const int64_t orow = (static_cast<int64_t>(b) * n1 + node) * Hq + hh;
    if (!(L >= 0 && L + n1 <= Lmax)) {
        for (int d = lane; d < D; d += kWave) out[orow * D + d] = NAN;
        if (lse && lane == 0) lse[orow] = NAN;
        return;
    }
    const uint32_t* mrow = mask + (static_cast<int64_t>(b) * n1 + node) * words;
    const float* qp = q + orow * D;
    const float* kb = kc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;
    const float* vb = vc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;
    float qv[D];
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] = qp[d];
    float acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    float m = -INFINITY, l = 0.f;
    for (int key = lane; key < L + n1; key += kWave) {
        if (key >= L) {
            const int jj = key - L;
            if (!((mrow[jj >> 5] >> (jj & 31)) & 1u)) continue;
        }
        const float* kr = kb + static_cast<int64_t>(key) * D;
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
        s *= c2;
        const float mn = fmaxf(m, s);
        const float a = exp2f(m - mn);
        const float p = exp2f(s - mn);
        const float* vr = vb + static_cast<int64_t>(key) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = acc[d] * a + p * vr[d];
        l = l * a + p;
        m = mn;
    }
    const float M = wave_max(m);
    const float sc = (m == -INFINITY) ? 0.f : exp2f(m - M);
    const float den = wave_sum(l * sc);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const float v = wave_sum(acc[d] * sc);
        if (lane == (d % kWave)) out[orow * D + d] = v / den;
    }
    if (lse && lane == 0) lse[orow] = (M + log2f(den)) * kLn2;
}

// ------------------------------------------------------------------------------------------
// Decode-shaped case (at most two 32-row blocks per KV head, e.g. chains with small G): the
// workgroup owns one (sequence, KV head); its KS waves split the key tiles round-robin, each wave
// computing all RBW row blocks for its tiles, and the waves' partial softmax states are merged
// through LDS at the end, so the final output is written directly (no partials in HBM).
//   * K goes straight from HBM into MFMA A-operand registers (16-byte loads; lane (c, h) reads key
//     c of the tile, features 16 ks + 8 h .. +8).
//   * V^T operands are built without a transpose: the O^T rows (feature index) are permuted so that
//     MFMA block 2 dh holds the even features 64 dh + 2 i and block 2 dh + 1 the odd ones; a lane's
//     4-byte load of V[key][64 dh + 2 c .. +2] then feeds both blocks (low / high halves).
//   * The next tile's K and V words are prefetched into registers while the current tile runs.

template <int D, int KS, int RBW>
__global__ void __launch_bounds__(KS * kWave)
attn_decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                   const uint16_t* __restrict__ vc, const int32_t* __restrict__ ctx_len,
                   const uint32_t* __restrict__ mask, int n1, int Hq, int Hkv, int Lmax, float c2,
                   uint16_t* __restrict__ out, float* __restrict__ lse) {
    constexpr int kKS = D / 16;        // k-steps of S^T = K Q^T
    constexpr int kDH = D / 64;        // 64-feature halves: MFMA blocks 2 dh (even) and 2 dh + 1 (odd)
    constexpr int kDB = D / 32;
    extern __shared__ float xs[];      // merge buffer: (KS / 2) x RBW x kDB x 16 x 64 floats + m, l
    __shared__ uint4 sq[RBW][kKS][kWave];   // Q^T operands of the workgroup's row blocks

    const int kv = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv, R = G * n1;
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int h = lane / 32, col = lane % 32;
    const int words = (n1 + 31) >> 5;
    const int L = ctx_len[b];
    const bool seq_ok = L >= 0 && L + n1 <= Lmax;
    const int Ltot = L + n1;
    const int ntiles = seq_ok ? (Ltot + kTileKeys - 1) / kTileKeys : 0;

    int rows[RBW];
    bool rok[RBW];
    const uint32_t* mrow[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        rows[j] = (blockIdx.x * RBW + j) * 32 + col;
        rok[j] = rows[j] < R;
        const int node = rok[j] ? rows[j] / G : 0;
        mrow[j] = mask + (static_cast<int64_t>(b) * n1 + node) * words;
    }
    // stage Q^T operands: entry (j, s, lane) = Q[row j*32 + col][16 s + 8 h .. +8]
    for (int e = threadIdx.x; e < RBW * kKS * kWave; e += KS * kWave) {
        const int j = e / (kKS * kWave), s2 = (e / kWave) % kKS, ln = e % kWave;
        const int row = (blockIdx.x * RBW + j) * 32 + ln % 32;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < R) {
            const int node = row / G, g = row - node * G;
            v = *reinterpret_cast<const uint4*>(q + ((static_cast<int64_t>(b) * n1 + node) * Hq + kv * G + g) * D +
                                                16 * s2 + 8 * (ln / 32));
        }
        sq[j][s2][ln] = v;
    }
    __syncthreads();

    const uint16_t* kbase = kc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;
    const uint16_t* vbase = vc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;

    uint4 kn[kKS];
    auto load_k = [&](int t) {
        const int kkey = t * kTileKeys + col;
#pragma unroll
        for (int s2 = 0; s2 < kKS; ++s2)
            kn[s2] = (kkey < Ltot) ? *reinterpret_cast<const uint4*>(kbase + static_cast<int64_t>(kkey) * D + 16 * s2 + 8 * h)
                                   : make_uint4(0, 0, 0, 0);
    };

    f32x16_t o[RBW][kDB];
    float m[RBW], l[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int i = 0; i < kDB; ++i) o[j][i] = f32x16_t{};
    }

    if (w < ntiles) load_k(w);
    for (int t = w; t < ntiles; t += KS) {
        const int kb = t * kTileKeys;
        uint4 kcur[kKS];
#pragma unroll
        for (int s2 = 0; s2 < kKS; ++s2) kcur[s2] = kn[s2];
        // this tile's V words (consumed after the softmax), then the next tile's K
        uint32_t vr[2][kDH][8];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = kb + 16 * ks + 8 * (e / 4) + 4 * h + (e % 4);
#pragma unroll
                for (int dh = 0; dh < kDH; ++dh)
                    vr[ks][dh][e] = (key < Ltot)
                        ? *reinterpret_cast<const uint32_t*>(vbase + static_cast<int64_t>(key) * D + 64 * dh + 2 * col)
                        : 0u;
            }
        if (t + KS < ntiles) load_k(t + KS);

        bf16x8_t pb[RBW][2];
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            f32x16_t s = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kcur[ks]), as_bf16x8(sq[j][ks][lane]), s, 0, 0, 0);
            if (kb + kTileKeys > L) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 8 * (r / 4) + 4 * h + (r % 4);
                    bool vis = key < L;
                    if (!vis && key < Ltot) {
                        const int jj = key - L;
                        vis = (mrow[j][jj >> 5] >> (jj & 31)) & 1u;
                    }
                    if (!vis) s[r] = -INFINITY;
                }
            }
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m[j], mx * c2);
            const float mref = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(m[j] - mref);
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mref));
                rs += s[r];
            }
            rs += __shfl_xor(rs, 32);
            l[j] = l[j] * alpha + rs;
            m[j] = mnew;
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int i = 0; i < kDB; ++i) o[j][i] *= alpha;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                uint4 pw;
                pw.x = pack_bf16x2(s[8 * ks + 0], s[8 * ks + 1]);
                pw.y = pack_bf16x2(s[8 * ks + 2], s[8 * ks + 3]);
                pw.z = pack_bf16x2(s[8 * ks + 4], s[8 * ks + 5]);
                pw.w = pack_bf16x2(s[8 * ks + 6], s[8 * ks + 7]);
                pb[j][ks] = as_bf16x8(pw);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int dh = 0; dh < kDH; ++dh) {
                const uint32_t* x = vr[ks][dh];
                uint4 ev, od;
                ev.x = (x[0] & 0xffffu) | (x[1] << 16);
                ev.y = (x[2] & 0xffffu) | (x[3] << 16);
                ev.z = (x[4] & 0xffffu) | (x[5] << 16);
                ev.w = (x[6] & 0xffffu) | (x[7] << 16);
                od.x = (x[0] >> 16) | (x[1] & 0xffff0000u);
                od.y = (x[2] >> 16) | (x[3] & 0xffff0000u);
                od.z = (x[4] >> 16) | (x[5] & 0xffff0000u);
                od.w = (x[6] >> 16) | (x[7] & 0xffff0000u);
#pragma unroll
                for (int j = 0; j < RBW; ++j) {
                    o[j][2 * dh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ev), pb[j][ks], o[j][2 * dh], 0, 0, 0);
                    o[j][2 * dh + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(od), pb[j][ks], o[j][2 * dh + 1], 0, 0, 0);
                }
            }
    }

    // ---- merge the KS waves' states: halving tree through LDS
    constexpr int kRegs = RBW * kDB * 16;
    float* ml = xs + (KS / 2) * kRegs * kWave;
    for (int half = KS / 2; half >= 1; half /= 2) {
        if (w >= half && w < 2 * half) {
            float* dst = xs + (w - half) * kRegs * kWave;
#pragma unroll
            for (int j = 0; j < RBW; ++j) {
#pragma unroll
                for (int i = 0; i < kDB; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((j * kDB + i) * 16 + r) * kWave + lane] = o[j][i][r];
                ml[((w - half) * RBW + j) * 2 * kWave + lane] = m[j];
                ml[((w - half) * RBW + j) * 2 * kWave + kWave + lane] = l[j];
            }
        }
        __syncthreads();
        if (w < half) {
            const float* src = xs + w * kRegs * kWave;
#pragma unroll
            for (int j = 0; j < RBW; ++j) {
                const float m2 = ml[(w * RBW + j) * 2 * kWave + lane];
                const float l2 = ml[(w * RBW + j) * 2 * kWave + kWave + lane];
                const float M = fmaxf(m[j], m2);
                const float a1 = (m[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[j] - M);
                const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
                for (int i = 0; i < kDB; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o[j][i][r] = a1 * o[j][i][r] + a2 * src[((j * kDB + i) * 16 + r) * kWave + lane];
                l[j] = a1 * l[j] + a2 * l2;
                m[j] = M;
            }
        }
        __syncthreads();
    }

    if (w == 0) {
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            if (!rok[j]) continue;
            const int node = rows[j] / G, g = rows[j] - (rows[j] / G) * G;
            const int64_t orow = (static_cast<int64_t>(b) * n1 + node) * Hq + kv * G + g;
            uint16_t* op = out + orow * D;
            const float inv = seq_ok ? 1.f / l[j] : NAN;
#pragma unroll
            for (int dh = 0; dh < kDH; ++dh)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    // registers 4 rr .. 4 rr + 3 hold feature slots i = 8 rr + 4 h + 0..3, i.e.
                    // features 64 dh + 2 i (even block) and 64 dh + 2 i + 1 (odd block)
                    uint4 st;
                    st.x = pack_bf16x2(o[j][2 * dh][4 * rr + 0] * inv, o[j][2 * dh + 1][4 * rr + 0] * inv);
                    st.y = pack_bf16x2(o[j][2 * dh][4 * rr + 1] * inv, o[j][2 * dh + 1][4 * rr + 1] * inv);
                    st.z = pack_bf16x2(o[j][2 * dh][4 * rr + 2] * inv, o[j][2 * dh + 1][4 * rr + 2] * inv);
                    st.w = pack_bf16x2(o[j][2 * dh][4 * rr + 3] * inv, o[j][2 * dh + 1][4 * rr + 3] * inv);
                    *reinterpret_cast<uint4*>(op + 64 * dh + 2 * (8 * rr + 4 * h)) = st;
                }
            if (lse && h == 0) lse[orow] = seq_ok ? (m[j] + log2f(l[j])) * kLn2 : NAN;
        }
    }
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

template <int D, int KS, int RBW>
void launch_decode(const AttnArgs& a, dim3 grid, hipStream_t stream) {
    const size_t lds = sizeof(float) * (size_t(KS / 2) * RBW * (D / 32) * 16 * kWave + size_t(KS / 2) * RBW * 2 * kWave);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_decode_kernel<D, KS, RBW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    (void)attr;
    hipLaunchKernelGGL((attn_decode_kernel<D, KS, RBW>), grid, dim3(KS * kWave), lds, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.ctx_len, a.mask, a.n1, a.Hq, a.Hkv,
                       a.Lmax, a.scale * kLog2e, static_cast<uint16_t*>(a.out), a.lse);
}

}  // namespace

size_t attn_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax) {
    if (((Hq / Hkv) * n1 + 31) / 32 <= 2) return 0;   // decode-shaped: no partials
    const Plan p = make_plan(B, n1, Hq, Hkv, D, Lmax);
    return AttnLayout(B, Hkv, p.nsplit, (Hq / Hkv) * n1, D).total;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
    const float c2 = a.scale * kLog2e;
    if (!a.bf16) {
        const dim3 grid(a.n1 * a.Hq, a.B);
        if (a.D == 64)
            hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(kWave), 0, stream,
                               static_cast<const float*>(a.q), static_cast<const float*>(a.k_cache),
                               static_cast<const float*>(a.v_cache), a.ctx_len, a.mask, a.n1, a.Hq,
                               a.Hkv, a.Lmax, c2, static_cast<float*>(a.out), a.lse);
        else
            hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(kWave), 0, stream,
                               static_cast<const float*>(a.q), static_cast<const float*>(a.k_cache),
                               static_cast<const float*>(a.v_cache), a.ctx_len, a.mask, a.n1, a.Hq,
                               a.Hkv, a.Lmax, c2, static_cast<float*>(a.out), a.lse);
        return hipGetLastError();
    }
    const int RB = ((a.Hq / a.Hkv) * a.n1 + 31) / 32;
    if (RB <= 2) {
        const dim3 grid(1, a.Hkv, a.B);
        if (a.D == 64) {
            if (RB == 1) launch_decode<64, 8, 1>(a, grid, stream);
            else launch_decode<64, 4, 2>(a, grid, stream);
        } else {
            if (RB == 1) launch_decode<128, 8, 1>(a, grid, stream);
            else launch_decode<128, 4, 2>(a, grid, stream);
        }
        return hipGetLastError();
    }
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
