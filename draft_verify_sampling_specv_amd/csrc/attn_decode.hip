// Tree-attention verify, decode-shaped case: at most two 32-row blocks of queries per KV head
// ([SD-EAGLE] "Tree Attention Verification"; [PTD] Method 4, "Verification").  See the comment
// on attn_decode_kernel for the design.

#include "attn_common.h"
#include "kernels.h"

namespace specv {
namespace {
using namespace attn;

// ------------------------------------------------------------------------------------------
// Decode-shaped case (at most two 32-row blocks per KV head, e.g. chains with small G): one
// workgroup owns all RBW row blocks of one (sequence, KV head), so every K/V byte is read into one
// CU once (eight waves for one block; four waves holding both blocks' accumulators, a wave per
// SIMD, for two -- measured on the low-acceptance chain shape, 45 rows per KV head: 68 us against
// 80 us for a workgroup per block sharing the stream through L2, or for two groups of four waves
// reading each tile twice); its KS waves split the key tiles round-robin, each wave computing the
// workgroup's row blocks for its tiles, and the waves' partial softmax states are merged through
// LDS at the end (one round: scaled states published, each wave sums and stores one slice), so the
// final output is written directly (no partials in HBM).
//   * every K/V load is unconditional, its key index clamped to the last valid key (masked in
//     the softmax), so the compiler never waits for the prefetch before it is needed;
//   * each lane keeps its query row's tree-mask words (at most two) in registers.
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
                   int ngroups, int xcd_map, uint16_t* __restrict__ out, float* __restrict__ lse) {
    constexpr int kKS = D / 16;        // k-steps of S^T = K Q^T
    constexpr int kDH = D / 64;        // 64-feature halves: MFMA blocks 2 dh (even) and 2 dh + 1 (odd)
    constexpr int kDB = D / 32;
    extern __shared__ float xs[];      // merge buffer: KS x RBW x kDB x 16 x 64 floats + m, l
    __shared__ uint4 sq[RBW][kKS][kWave];   // Q^T operands of the workgroup's row blocks

    // block id -> (unit = (sequence, KV head), row group of RBW blocks); with xcd_map the row
    // groups of a unit get ids on the same XCD (ids are dealt to the 8 XCDs round-robin), adjacent
    // in its dispatch order, so they share that XCD's L2 for the unit's K/V
    int unit, grp;
    if (xcd_map) {
        const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
        unit = (s / ngroups) * 8 + x;
        grp = s % ngroups;
    } else {
        unit = blockIdx.x / ngroups;
        grp = blockIdx.x % ngroups;
    }
    const int kv = unit % Hkv, b = unit / Hkv;
    const int G = Hq / Hkv, R = G * n1;
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int h = lane / 32, col = lane % 32;
    const int words = (n1 + 31) >> 5;

    const uint16_t* kbase = kc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;
    const uint16_t* vbase = vc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;

    // Loads are unconditional: a key past the sequence reads its last key instead (finite data,
    // masked out by the softmax; key 0 for an invalid sequence, whose output is NaN anyway).
    // With no register loaded under a branch, the compiler's load counting stays exact, so a
    // wait for one load is not a wait for the loads issued after it.
    // The wave's first K tile is the exception: it is clamped to the cache's last row instead, so
    // that its loads need not wait for ctx_len.  Keys it reads past the sequence hold arbitrary
    // cache contents, but K only enters the scores, and the scores of those keys are replaced by
    // -inf with a select before any arithmetic uses them (V, which is multiplied by p = 0, is
    // always clamped to a real key).
    uint4 kn[kKS];
    auto load_k = [&](int t, int kclamp) {
        const int kkey = SPECV_CHK(min(t * kTileKeys + col, kclamp), Lmax, kSiteDecodeKey);
#pragma unroll
        for (int s2 = 0; s2 < kKS; ++s2)
            kn[s2] = *reinterpret_cast<const uint4*>(kbase + static_cast<int64_t>(kkey) * D + 16 * s2 + 8 * h);
    };

    // Issue order: this lane's mask words and Q word, then the wave's first K tile, so the K
    // stream starts before the Q operands are staged (the staging waits only for the Q word).
    // The mask row stays in registers: the decode shape has at most 64 rows per KV head, so at
    // most 64 nodes and two mask words.
    // ctx_len first, as a vector load: read as a scalar load it would be waited for together with
    // the kernel arguments, before any of the loads below were issued; issued first, waiting for
    // it leaves the loads after it in flight
    const int L0 = __hip_atomic_load(ctx_len + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int rows[RBW];
    bool rok[RBW];
    uint64_t mbits[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        rows[j] = (grp * RBW + j) * 32 + col;
        rok[j] = rows[j] < R;
        const int node = rok[j] ? rows[j] / G : 0;
        const uint32_t* mrow = mask + (static_cast<int64_t>(b) * n1 + node) * words;
        const uint32_t w0 = mrow[0], w1 = mrow[words > 1 ? 1 : 0];
        mbits[j] = w0 | (words > 1 ? static_cast<uint64_t>(w1) << 32 : 0ull);
    }
    // Q^T operand entries (j, s, lane) = Q[row j*32 + col][16 s + 8 h .. +8], kQPer per thread
    constexpr int kQE = RBW * kKS * kWave;
    constexpr int kQPer = (kQE + KS * kWave - 1) / (KS * kWave);
    uint64_t q0[kQPer], q1[kQPer];
    // (relaxed atomic loads: the compiler keeps them ahead of the K loads, which it would
    // otherwise be free to issue first, turning the wait for Q into a wait for K)
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
        const int qe = min(static_cast<int>(threadIdx.x) + i * KS * kWave, kQE - 1);
        const int qj = qe / (kKS * kWave), qs = (qe / kWave) % kKS, qln = qe % kWave;
        const int qrc = min((grp * RBW + qj) * 32 + qln % 32, R - 1);
        const int qnode = qrc / G, qg = qrc - qnode * G;
        const uint64_t* qp = reinterpret_cast<const uint64_t*>(
            q + ((static_cast<int64_t>(b) * n1 + qnode) * Hq + kv * G + qg) * D + 16 * qs + 8 * (qln / 32));
        q0[i] = __hip_atomic_load(qp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        q1[i] = __hip_atomic_load(qp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    asm volatile("" ::: "memory");
    load_k(w, Lmax - 1);
    const int L = __builtin_amdgcn_readfirstlane(L0);
    const bool seq_ok = L >= 0 && L <= Lmax - n1;
    const int Ltot = seq_ok ? L + n1 : 0;
    const int ntiles = seq_ok ? (Ltot + kTileKeys - 1) / kTileKeys : 0;
    const int kmax = seq_ok ? Ltot - 1 : 0;
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
        const int qe = static_cast<int>(threadIdx.x) + i * KS * kWave;
        if (qe < kQE) {
            const int qj = qe / (kKS * kWave), qs = (qe / kWave) % kKS, qln = qe % kWave;
            const int qrow = (grp * RBW + qj) * 32 + qln % 32;
            const uint4 qv = make_uint4(static_cast<uint32_t>(q0[i]), static_cast<uint32_t>(q0[i] >> 32),
                                        static_cast<uint32_t>(q1[i]), static_cast<uint32_t>(q1[i] >> 32));
            sq[qj][qs][qln] = qrow < R ? qv : make_uint4(0, 0, 0, 0);
        }
    }
    // LDS-only barrier: the K tile stays in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    f32x16_t o[RBW][kDB];
    float m[RBW], l[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int i = 0; i < kDB; ++i) o[j][i] = f32x16_t{};
    }

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
                const int key = SPECV_CHK(min(kb + 16 * ks + 8 * (e / 4) + 4 * h + (e % 4), kmax), Lmax, kSiteDecodeKey);
#pragma unroll
                for (int dh = 0; dh < kDH; ++dh)
                    vr[ks][dh][e] = load_nt32(vbase + static_cast<int64_t>(key) * D + 64 * dh + 2 * col);
            }
        load_k(min(t + KS, ntiles - 1), kmax);

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
                    const int jj = key - L;    // tree index when 0 <= jj < n1
                    const bool vis = key < L || (key < Ltot && ((mbits[j] >> (jj & 63)) & 1ull));
                    s[r] = vis ? s[r] : -INFINITY;
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

    // ---- merge the KS waves' states in one round through LDS: every wave publishes (m, l), then
    //      its O scaled to the common max; each wave then sums one slice of the registers over the
    //      KS waves and stores that slice of the output (one 16-byte store per lane)
    constexpr int kRegs = RBW * kDB * 16;
    float* ml = xs + KS * kRegs * kWave;                 // [KS][RBW][m, l][lane]
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        ml[((w * RBW + j) * 2) * kWave + lane] = m[j];
        ml[((w * RBW + j) * 2 + 1) * kWave + lane] = l[j];
    }
    __syncthreads();
    float Mx[RBW], Lx[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        float M = -INFINITY;
        for (int q = 0; q < KS; ++q) M = fmaxf(M, ml[((q * RBW + j) * 2) * kWave + lane]);
        float L = 0.f;
        for (int q = 0; q < KS; ++q) {
            const float mq = ml[((q * RBW + j) * 2) * kWave + lane];
            if (mq != -INFINITY) L += __builtin_amdgcn_exp2f(mq - M) * ml[((q * RBW + j) * 2 + 1) * kWave + lane];
        }
        Mx[j] = M;
        Lx[j] = L;
        const float aw = (m[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[j] - M);
        float* dst = xs + w * kRegs * kWave;
#pragma unroll
        for (int i = 0; i < kDB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[((j * kDB + i) * 16 + r) * kWave + lane] = aw * o[j][i][r];
    }
    __syncthreads();
    // slice sl = (j, dh, rr): registers 4 rr .. 4 rr + 3 of blocks 2 dh (even features) and 2 dh + 1
    // (odd), i.e. feature slots i = 8 rr + 4 h + 0..3: features 64 dh + 2 i and 64 dh + 2 i + 1
    for (int sl = w; sl < RBW * kDH * 4; sl += KS) {
        const int j = sl / (kDH * 4), dh = (sl / 4) % kDH, rr = sl % 4;
        float ev[4] = {0.f, 0.f, 0.f, 0.f}, od[4] = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < KS; ++q) {
            const float* src = xs + q * kRegs * kWave;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ev[e] += src[((j * kDB + 2 * dh) * 16 + 4 * rr + e) * kWave + lane];
                od[e] += src[((j * kDB + 2 * dh + 1) * 16 + 4 * rr + e) * kWave + lane];
            }
        }
        const int row = (grp * RBW + j) * 32 + col;
        if (row < R) {
            const int node = row / G, g = row - node * G;
            const int64_t orow = (static_cast<int64_t>(b) * n1 + node) * Hq + kv * G + g;
            const float inv = seq_ok ? 1.f / Lx[j] : NAN;
            uint4 st;
            st.x = pack_bf16x2(ev[0] * inv, od[0] * inv);
            st.y = pack_bf16x2(ev[1] * inv, od[1] * inv);
            st.z = pack_bf16x2(ev[2] * inv, od[2] * inv);
            st.w = pack_bf16x2(ev[3] * inv, od[3] * inv);
            *reinterpret_cast<uint4*>(out + orow * D + 64 * dh + 2 * (8 * rr + 4 * h)) = st;
            if (lse && h == 0 && dh == 0 && rr == 0)
                lse[orow] = seq_ok ? (Mx[j] + log2f(Lx[j])) * kLn2 : NAN;
        }
    }
}

template <int D, int KS, int RBW>
void launch_decode(const AttnArgs& a, int ngroups, hipStream_t stream) {
    const size_t lds = sizeof(float) * (size_t(KS) * RBW * (D / 32) * 16 * kWave + size_t(KS) * RBW * 2 * kWave);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_decode_kernel<D, KS, RBW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    (void)attr;
    const int units = a.B * a.Hkv;
    const int xcd_map = (ngroups > 1 && units % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((attn_decode_kernel<D, KS, RBW>), dim3(units * ngroups), dim3(KS * kWave), lds, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.ctx_len, a.mask, a.n1, a.Hq, a.Hkv,
                       a.Lmax, a.scale * kLog2e, ngroups, xcd_map, static_cast<uint16_t*>(a.out), a.lse);
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t stream) {
    // one workgroup per (sequence, KV head), so every K/V byte enters one CU: one row block with
    // eight waves, two row blocks with four waves of both blocks' accumulators (a wave per SIMD)
    const int RB = ((a.Hq / a.Hkv) * a.n1 + 31) / 32;
    if (RB == 1) {
        if (a.D == 64) launch_decode<64, 8, 1>(a, 1, stream);
        else launch_decode<128, 8, 1>(a, 1, stream);
    } else {
        if (a.D == 64) launch_decode<64, 4, 2>(a, 1, stream);
        else launch_decode<128, 4, 2>(a, 1, stream);
    }
    return hipGetLastError();
}

}  // namespace specv
