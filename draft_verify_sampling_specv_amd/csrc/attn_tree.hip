// Tree-attention verify, general case: many query rows per KV head (big trees x GQA groups)
// ([SD-EAGLE] "Tree Attention Verification"; [PTD] Method 4, "Verification").
//
// The query rows of one KV head are the G x (K+1) pairs (node, head in group), row r = node * G + g,
// cut into 32-row blocks.  These shapes are MFMA-bound (about G (K+1) flops per K/V byte):
//   * a workgroup is 8 waves (two per SIMD) and owns one (sequence, KV head, key split, row
//     group); a row group is up to 8 row blocks, one per wave; a wave keeps its block's Q^T
//     operands and O^T accumulators in registers;
//   * the split's keys go through an LDS ring of 64-key tiles filled by direct global-to-LDS
//     transfers (no registers, no LDS store instructions), one tile in flight while one is
//     computed and the next being issued, one barrier per tile;
//   * K sits in LDS in MFMA operand order, so each S^T = K Q^T operand is one conflict-free
//     16-byte read; S^T is computed on v_mfma_f32_32x32x16_bf16 as two 32-key blocks (two
//     independent accumulation chains), and each lane ends up holding one query row;
//   * O^T += V^T P^T on the same instruction: P stays in registers (the accumulator layout of S^T
//     reused as the B operand under a matching key permutation); the V^T operands come from
//     transposing LDS reads (ds_read_b64_tr_b16) of row-major V, laid out so that the four keys of
//     one read sit in different bank groups and every offset but the lane's own is a constant;
//   * online softmax in base 2 with the scale folded into the exponent and a lazy reference max:
//     p = exp2(s c2 - m) is taken against the row's current reference without a per-tile max, and
//     the reference moves (max, rescale, recompute) only when some lane's p sum would exceed 2^20;
//   * with one key split the workgroup writes the final bf16 output; with several, each split
//     writes its output normalised by its own sum (bf16) and its (max, sum), and a combine kernel
//     merges them;
//   * the workgroups of one (sequence, KV head, split) that differ only in row group are given
//     block ids on the same XCD, adjacent in dispatch order, so their K/V reads share that XCD's
//     L2.

#include <cmath>

#include "attn_common.h"
#include "kernels.h"

namespace specv {
namespace {
using namespace attn;

constexpr int kTreeWaves = 8;             // one 32-row block per wave, two waves per SIMD
constexpr int kTreeThreads = kTreeWaves * kWave;
constexpr int kTreeTile = 64;             // keys per ring stage
constexpr int kNst = kTreeTile / 32;      // 32-key S^T blocks per tile
constexpr int kStages = 3;                // LDS ring depth (tiles)
constexpr float kLazyMax = 1048576.f;     // 2^20: largest p sum a lane may reach before the reference moves

// One ring stage.
//   K in MFMA operand order: 1 KB block (st, ks) holds, for lane l, the 8 features 16 ks + 8 (l / 32)
//   .. of key 32 st + l % 32 -- exactly lane l's A operand of S^T block st at k-step ks.
//   V as kVT transfers of whole key rows: transfer slot u (1 KB + 64 bytes of padding) holds the
//   rows r with r % kVT == u, in order of r / kVT.  The PV step reads 4 consecutive keys at a
//   time with transposing reads; those keys sit in 4 slots 64 bytes apart in bank order, so the
//   reads are conflict-free.
template <int D>
struct TreeTiles {
    static constexpr int kKS = D / 16;                     // k-steps of S^T
    static constexpr int kKT = kNst * kKS;                 // K transfers per tile
    static constexpr int kVT = kTreeTile * 2 * D / 1024;   // V transfers per tile
    static constexpr int kVStride = 1024 + 64;             // bytes per V transfer slot
    uint16_t k[kStages][kTreeTile * D];
    uint16_t v[kStages][kVT * kVStride / 2];
};

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land at lds + 16 i.
// (Issued as inline assembly so that the compiler neither waits for these loads at its own LDS
// reads nor counts them; the tile pipeline waits for them explicitly.)
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "s"(lds) : "memory", "m0");
}

// The same with a wave-uniform 64-bit base and a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct TreePlan {
    int ngroups;    // row groups per (sequence, KV head): up to kTreeWaves row blocks each
    int nsplit;     // key splits per (sequence, KV head)
};

struct TreeLayout {
    size_t opart, ml, total;
    TreeLayout(int B, int Hkv, int nsplit, int R, int D) {
        opart = 0;
        if (nsplit <= 1) {
            ml = total = 0;
            return;
        }
        ml = align256(sizeof(uint16_t) * size_t(B) * Hkv * nsplit * R * D);
        total = align256(ml + sizeof(float2) * size_t(B) * Hkv * nsplit * R);
    }
};

// The state of the row block a wave owns.
template <int D>
struct WaveRow {
    bf16x8_t q[D / 16];             // Q^T operands: row 32 rb + col, features 16 ks + 8 h ..
    f32x16_t o[D / 32];             // O^T accumulators, block c = features 32 c + i
    float m, l;                     // reference max (base 2, scaled) and this half-wave's sum
    const uint32_t* mrow;           // mask row of this lane's node
};

// This wave's transfers of a tile: kKT transfers of K (one per (32-key block, k-step)) and kVT of
// V (1024 / (2 D) whole rows each), dealt to the waves.  Transfer x of wave w is j = w + 8 x.
template <int D>
struct TileTransfers {
    using T = TreeTiles<D>;
    static constexpr int kCpr = D / 8;                             // 16-byte chunks per V row
    static constexpr int kPerWave = (T::kKT + T::kVT) / kTreeWaves;
    static_assert((T::kKT + T::kVT) % kTreeWaves == 0, "whole transfers per wave");
    uint32_t off[kPerWave];     // this lane's byte offset from the tile's first key row

    __device__ __forceinline__ static bool is_v(int j) { return j >= T::kKT; }
    // key row (within the tile) and feature of this lane's 16 bytes in transfer j
    __device__ __forceinline__ static void source(int j, int lane, int& row, int& feat) {
        if (!is_v(j)) {
            row = 32 * (j / T::kKS) + (lane & 31);
            feat = 16 * (j % T::kKS) + 8 * (lane >> 5);
        } else {
            row = (lane / kCpr) * T::kVT + (j - T::kKT);      // rows u, u + kVT, ...
            feat = 8 * (lane % kCpr);
        }
    }
    __device__ __forceinline__ static uint16_t* dest(TreeTiles<D>& sm, int stage, int j) {
        return is_v(j) ? sm.v[stage] + (j - T::kKT) * (T::kVStride / 2) : sm.k[stage] + j * (kWave * 8);
    }
    __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
        for (int x = 0; x < kPerWave; ++x) {
            int row, feat;
            source(w + x * kTreeWaves, lane, row, feat);
            off[x] = static_cast<uint32_t>((row * D + feat) * 2);
        }
    }
    // Issue tile t into ring stage `stage`.  Tiles entirely inside the sequence use the scalar
    // base + lane offset form; the last tile reads, for keys past the sequence, its last key
    // instead (finite data, masked out by the softmax).
    __device__ __forceinline__ void issue(TreeTiles<D>& sm, int stage, const uint16_t* kbase,
                                          const uint16_t* vbase, int t, int Ltot, int w, int lane) const {
#pragma unroll
        for (int x = 0; x < kPerWave; ++x) {
            const int j = w + x * kTreeWaves;
            const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_address(dest(sm, stage, j)));
            const uint16_t* base = is_v(j) ? vbase : kbase;
            if ((t + 1) * kTreeTile <= Ltot) {
                dma16_sbase(base + static_cast<int64_t>(t) * kTreeTile * D, off[x], lds);
            } else {
                int row, feat;
                source(j, lane, row, feat);
                const int key = SPECV_CHK(min(t * kTreeTile + row, Ltot - 1), Ltot, kSiteTreeKey);
                dma16(base + static_cast<int64_t>(key) * D + feat, lds);
            }
        }
    }
};

// One 64-key tile for this wave's row block.
template <int D>
__device__ __forceinline__ void tile_compute(WaveRow<D>& wr, const uint16_t* kt, const uint16_t* vt,
                                             int kb, int L, int Ltot, int lane, float c2) {
    using T = TreeTiles<D>;
    constexpr int kKS = T::kKS;
    constexpr int kF = D / 32;
    const int h = lane >> 5;
    f32x16_t s[kNst];

    // S^T = K Q^T for the two 32-key blocks (interleaved, independent chains)
    auto compute_s = [&]() {
#pragma unroll
        for (int st = 0; st < kNst; ++st) s[st] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int st = 0; st < kNst; ++st) {
                const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(&kt[((st * kKS + ks) * kWave + lane) * 8]));
                s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wr.q[ks], s[st], 0, 0, 0);
            }
        // s[st][r] is key kb + 32 st + 8 (r / 4) + 4 h + r % 4 of this lane's row
        if (kb + kTreeTile > L) {
#pragma unroll
            for (int st = 0; st < kNst; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 32 * st + 8 * (r / 4) + 4 * h + (r % 4);
                    bool vis = key < L;
                    if (!vis && key < Ltot) {
                        const int jj = key - L;
                        vis = (wr.mrow[SPECV_CHK(jj, Ltot - L, kSiteTreeMaskWord) >> 5] >> (jj & 31)) & 1u;
                    }
                    if (!vis) s[st][r] = -INFINITY;
                }
        }
    };
    // s := p = exp2(s c2 - m) against the current reference; returns this lane's p sum
    auto exponentiate = [&]() {
        const float mref = (wr.m == -INFINITY) ? 0.f : wr.m;
        float rs = 0.f;
#pragma unroll
        for (int st = 0; st < kNst; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[st][r] = __builtin_amdgcn_exp2f(fmaf(s[st][r], c2, -mref));
                rs += s[st][r];
            }
        return rs;
    };

    compute_s();
    float rs = exponentiate();
    if (__ballot(!(rs <= kLazyMax) || wr.m == -INFINITY)) {
        // slow path (first tile of a row, or a score far above the reference): the tile's row
        // max over both half-waves becomes the reference where it is higher
        compute_s();
        float mx = s[0][0];
#pragma unroll
        for (int st = 0; st < kNst; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * c2;
        if (mt > wr.m) {
            const float alpha = __builtin_amdgcn_exp2f(wr.m - mt);    // m = -inf gives 0
            wr.m = mt;
            wr.l *= alpha;
#pragma unroll
            for (int c = 0; c < kF; ++c) wr.o[c] *= alpha;
        }
        rs = exponentiate();
    }
    wr.l += rs;

    // P as the B operands of the PV product: k-step (st, ks) covers the keys
    // 32 st + 16 ks + 8 (e / 4) + 4 h + e % 4 (e = 0..7), the order in which S^T holds them
    bf16x8_t pb[kNst][2];
#pragma unroll
    for (int st = 0; st < kNst; ++st)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint4 pw;
            pw.x = pack_bf16x2(s[st][8 * ks + 0], s[st][8 * ks + 1]);
            pw.y = pack_bf16x2(s[st][8 * ks + 2], s[st][8 * ks + 3]);
            pw.z = pack_bf16x2(s[st][8 * ks + 4], s[st][8 * ks + 5]);
            pw.w = pack_bf16x2(s[st][8 * ks + 6], s[st][8 * ks + 7]);
            pb[st][ks] = as_bf16x8(pw);
        }

    // O^T += V^T P^T.  The V^T operand of block c (lane: feature 32 c + col, the 8 keys of the
    // k-step) comes from two transposing reads of 4 keys each: within each group of 16 lanes,
    // lane 16 g + 4 a + b receives element b of the 8 bytes addressed by lanes 16 g + a, +4, +8,
    // +12, so lane x addresses key (.. + x % 16 / 4) at features 32 c + 16 (x / 16 % 2) + 4 (x % 4).
    // Key r = 32 st + 16 ks + 8 half + 4 h + j sits in slot r % kVT at position r / kVT.
    typedef __attribute__((address_space(3))) const char lds_char;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int kj = (lane & 15) >> 2;
    const int fo = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // lane part of key 4 h + j: slot 4 h + j with at least 8 slots, else slot j and position + h
    lds_char* vb = (lds_char*)(vt) + 2 * fo +
                   ((T::kVT >= 8) ? (4 * h + kj) * T::kVStride : kj * T::kVStride + h * (2 * D));
#pragma unroll
    for (int st = 0; st < kNst; ++st)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int c = 0; c < kF; ++c) {
                v4i16 part[2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    constexpr int kVT = T::kVT;
                    const int rc = 32 * st + 16 * ks + 8 * half;    // key less its lane part 4 h + j
                    const int off = (kVT >= 8) ? (rc % kVT) * T::kVStride + (rc / kVT) * (2 * D)
                                               : (rc / 4) * (2 * D);
                    part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + off + 64 * c));
                }
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
                wr.o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st][ks], wr.o[c], 0, 0, 0);
            }
}

// The split's tiles [t0, t1) through the LDS ring: while tile tt is computed, tile tt + 1 is in
// flight and tile tt + 2 is being issued.  The barrier at the top of each tile both publishes
// tile tt (every wave has waited for its own share of it) and frees the stage of tile tt - 1.
template <int D, bool kActive>
__device__ __forceinline__ void run_tiles(WaveRow<D>& wr, TreeTiles<D>& sm, const uint16_t* kbase,
                                          const uint16_t* vbase, int t0, int t1, int L, int Ltot,
                                          int w, int lane, float c2) {
    constexpr int kPerTile = TileTransfers<D>::kPerWave;        // transfers per wave per tile
    if (t0 >= t1) return;                                      // (workgroup-uniform)
    TileTransfers<D> tx;
    tx.init(w, lane);
    // Let the compiler see every earlier load (Q operands, ...) complete here: it cannot count
    // the ring's transfers, so a load it still believed pending inside the loop would make it
    // wait for all of them.
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) tx.issue(sm, i, kbase, vbase, min(t0 + i, t1 - 1), Ltot, w, lane);
    for (int tt = t0; tt < t1; ++tt) {
        const int i = tt - t0;
        wait_vmcnt<(kStages - 2) * kPerTile>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        tx.issue(sm, (i + kStages - 1) % kStages, kbase, vbase, min(tt + kStages - 1, t1 - 1), Ltot, w, lane);
        if constexpr (kActive)
            tile_compute<D>(wr, sm.k[i % kStages], sm.v[i % kStages], tt * kTreeTile, L, Ltot, lane, c2);
    }
    wait_vmcnt<0>();      // the ring's last (redundant) transfers land before the workgroup ends
}

template <int D>
__global__ void __launch_bounds__(kTreeThreads)
attn_tree_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                 const uint16_t* __restrict__ vc, const int32_t* __restrict__ ctx_len,
                 const uint32_t* __restrict__ mask, int n1, int Hq, int Hkv, int Lmax, float c2,
                 int nsplit, int ngroups, int xcd_map, uint16_t* __restrict__ out, float* __restrict__ lse,
                 uint16_t* __restrict__ opart, float2* __restrict__ mlpart) {
    constexpr int kKS = D / 16;
    constexpr int kF = D / 32;
    __shared__ TreeTiles<D> sm;

    // block id -> (unit = (sequence, KV head, split), row group)
    int unit, grp;
    if (xcd_map) {
        // dispatch deals block ids to the 8 XCDs round-robin: keep the row groups of a unit on one
        // XCD and adjacent in that XCD's dispatch order
        const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
        unit = (s / ngroups) * 8 + x;
        grp = s % ngroups;
    } else {
        unit = blockIdx.x / ngroups;
        grp = blockIdx.x % ngroups;
    }
    const int split = unit % nsplit;
    const int kv = (unit / nsplit) % Hkv;
    const int b = unit / (nsplit * Hkv);

    const int G = Hq / Hkv, R = G * n1;
    const int RB = (R + 31) / 32;
    const int rb0 = grp * RB / ngroups, rb1 = (grp + 1) * RB / ngroups;   // this group's row blocks
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int h = lane >> 5, col = lane & 31;
    const bool active = rb0 + w < rb1;                                    // (wave-uniform)
    const int words = (n1 + 31) >> 5;

    const int L = ctx_len[b];
    const bool seq_ok = L >= 0 && L <= Lmax - n1;
    const int Ltot = SPECV_CHK(seq_ok ? L + n1 : 0, int64_t(Lmax) + 1, kSiteTreeKey);   // (the key range read)
    const int ntiles = seq_ok ? (Ltot + kTreeTile - 1) / kTreeTile : 0;
    const int tps = (ntiles + nsplit - 1) / nsplit;
    const int t0 = min(ntiles, split * tps), t1 = min(ntiles, t0 + tps);

    const int row = (rb0 + w) * 32 + col;
    const bool ok = active && row < R;
    const int node = ok ? row / G : 0;
    const int g = ok ? row - node * G : 0;
    WaveRow<D> wr;
    wr.mrow = mask + (static_cast<int64_t>(b) * n1 + node) * words;
    {
        const uint16_t* qp = q + ((static_cast<int64_t>(b) * n1 + node) * Hq + kv * G + g) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
            wr.q[ks] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0));
    }
    wr.m = -INFINITY;
    wr.l = 0.f;
#pragma unroll
    for (int c = 0; c < kF; ++c) wr.o[c] = f32x16_t{};

    const uint16_t* kbase = kc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;
    const uint16_t* vbase = vc + (static_cast<int64_t>(b) * Hkv + kv) * Lmax * D;
    // every wave runs the same tile loop (same transfers and barriers); only active waves compute
    if (active) run_tiles<D, true>(wr, sm, kbase, vbase, t0, t1, L, Ltot, w, lane, c2);
    else run_tiles<D, false>(wr, sm, kbase, vbase, t0, t1, L, Ltot, w, lane, c2);

    // epilogue: lane (col, h) holds, in block c register 4 rr + e, feature 32 c + 8 rr + 4 h + e of
    // its row; l is the sum over this half-wave's keys, the row's is the sum over both halves
    wr.l += __shfl_xor(wr.l, 32);
    if (!ok) return;
    const float l = wr.l;
    uint16_t* op;
    float inv;
    if (nsplit == 1) {
        const int64_t orow = (static_cast<int64_t>(b) * n1 + node) * Hq + kv * G + g;
        op = out + orow * D;
        inv = seq_ok ? 1.f / l : NAN;
        if (lse && h == 0) lse[orow] = seq_ok ? (wr.m + log2f(l)) * kLn2 : NAN;
    } else {
        const int64_t prow = static_cast<int64_t>(unit) * R + row;
        op = opart + prow * D;
        inv = l > 0.f ? 1.f / l : 0.f;
        if (h == 0) mlpart[prow] = make_float2(wr.m, l);
    }
#pragma unroll
    for (int c = 0; c < kF; ++c)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            uint2 st;
            st.x = pack_bf16x2(wr.o[c][4 * rr + 0] * inv, wr.o[c][4 * rr + 1] * inv);
            st.y = pack_bf16x2(wr.o[c][4 * rr + 2] * inv, wr.o[c][4 * rr + 3] * inv);
            *reinterpret_cast<uint2*>(op + 32 * c + 8 * rr + 4 * h) = st;
        }
}

// Merge the key splits of one output row: weights l_s 2^(m_s - M) on the split outputs O_s (each
// already divided by its own l_s): out = sum w_s O_s / sum w_s; lse = M + log2(sum_s l_s 2^(m_s - M)).
__global__ void __launch_bounds__(256)
attn_tree_combine_kernel(const uint16_t* __restrict__ opart, const float2* __restrict__ mlpart,
                         const int32_t* __restrict__ ctx_len, int B, int n1, int Hq, int Hkv, int D,
                         int Lmax, int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int G = Hq / Hkv, R = G * n1;
    const int dv = D / 8;                           // 8 features (16 bytes) per thread
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(B) * n1 * Hq * dv;
    if (gid >= total) return;
    const int d0 = static_cast<int>(gid % dv) * 8;
    const int64_t orow = gid / dv;                  // (b, node, head)
    const int hh = static_cast<int>(orow % Hq);
    const int node = static_cast<int>((orow / Hq) % n1);
    const int b = static_cast<int>(orow / (static_cast<int64_t>(Hq) * n1));
    const int kv = hh / G, g = hh % G;
    const int row = node * G + g;
    // every load of a batch of kCombine splits is issued at once (their (max, sum) words and
    // partial outputs, whatever the context length says), so a thread waits about one round trip
    // per batch; batches merge online (the running sums rescaled to the new maximum)
    constexpr int kCombine = 8;
    const int L = ctx_len[b];
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float den = 0.f, M = -INFINITY;
    const int64_t ubase = (static_cast<int64_t>(b) * Hkv + kv) * nsplit;
    for (int s0 = 0; s0 < nsplit; s0 += kCombine) {
        float2 ml[kCombine];
        uint4 v[kCombine];
#pragma unroll
        for (int i = 0; i < kCombine; ++i) {
            const int64_t prow = (ubase + min(s0 + i, nsplit - 1)) * R + row;
            ml[i] = mlpart[prow];
            v[i] = *reinterpret_cast<const uint4*>(opart + prow * D + d0);
        }
        float Mn = M;
#pragma unroll
        for (int i = 0; i < kCombine; ++i)
            if (s0 + i < nsplit && ml[i].y > 0.f) Mn = fmaxf(Mn, ml[i].x);
        const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        den *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= sc;
        M = Mn;
#pragma unroll
        for (int i = 0; i < kCombine; ++i) {
            const bool use = s0 + i < nsplit && ml[i].y > 0.f;
            const float wgt = use ? ml[i].y * __builtin_amdgcn_exp2f(ml[i].x - M) : 0.f;
            const uint32_t x[4] = {use ? v[i].x : 0u, use ? v[i].y : 0u, use ? v[i].z : 0u, use ? v[i].w : 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += wgt * __uint_as_float(x[e] << 16);
                acc[2 * e + 1] += wgt * __uint_as_float(x[e] & 0xffff0000u);
            }
            den += wgt;
        }
    }
    const bool ok = L >= 0 && L <= Lmax - n1;
    const float inv = ok ? 1.f / den : NAN;
    uint4 st;
    st.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    st.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    st.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
    st.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
    *reinterpret_cast<uint4*>(out + orow * D + d0) = st;
    if (lse && d0 == 0) lse[orow] = ok ? (M + log2f(den)) * kLn2 : NAN;
}

template <int D>
__global__ void __launch_bounds__(kTreeThreads)
attn_tree_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                 const uint16_t* __restrict__ vc, const int32_t* __restrict__ ctx_len,
                 const uint32_t* __restrict__ mask, int n1, int Hq, int Hkv, int Lmax, float c2,
                 int nsplit, int ngroups, int xcd_map, uint16_t* __restrict__ out, float* __restrict__ lse,
                 uint16_t* __restrict__ opart, float2* __restrict__ mlpart);

// Workgroups of the tree kernel one compute unit holds at once (LDS ring and registers).
int tree_blocks_per_cu(int D) {
    static std::atomic<int> cache64[64], cache128[64];
    const void* f = (D == 64) ? reinterpret_cast<const void*>(&attn_tree_kernel<64>)
                              : reinterpret_cast<const void*>(&attn_tree_kernel<128>);
    return cached_per_device(D == 64 ? cache64 : cache128, [f](int) {
        int n = 0;
        return (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kTreeThreads, 0) == hipSuccess && n > 0) ? n : 1;
    });
}

// Row groups of at most kTreeWaves blocks (one per wave), balanced.  Key splits: the time goes as
// rounds of resident workgroups x tiles per split; take the number of splits (a power of two, at
// least 2 tiles each) that minimises that, counting the combine pass as two tiles.
TreePlan make_plan(int B, int n1, int Hq, int Hkv, int D, int Lmax) {
    const int RB = ((Hq / Hkv) * n1 + 31) / 32;
    const int slots = device_cu_count() * tree_blocks_per_cu(D);
    const int tiles = (Lmax + kTreeTile - 1) / kTreeTile;
    TreePlan p;
    p.ngroups = (RB + kTreeWaves - 1) / kTreeWaves;
    p.nsplit = 1;
    const long long wgs1 = static_cast<long long>(B) * Hkv * p.ngroups;
    long long best = -1;
    for (int ns = 1; ns <= 64 && (ns == 1 || tiles / ns >= 2); ns *= 2) {
        const long long rounds = (wgs1 * ns + slots - 1) / slots;
        const long long cost = rounds * ((tiles + ns - 1) / ns) + (ns > 1 ? 2 : 0);
        if (best < 0 || cost < best) {
            best = cost;
            p.nsplit = ns;
        }
    }
    return p;
}

template <int D>
void launch_tree(const AttnArgs& a, const TreePlan& p, uint16_t* opart, float2* ml, hipStream_t stream) {
    const int units = a.B * a.Hkv * p.nsplit;
    const int blocks = units * p.ngroups;
    const int xcd_map = (p.ngroups > 1 && units % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((attn_tree_kernel<D>), dim3(blocks), dim3(kTreeThreads), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.ctx_len, a.mask, a.n1, a.Hq, a.Hkv,
                       a.Lmax, a.scale * kLog2e, p.nsplit, p.ngroups, xcd_map,
                       static_cast<uint16_t*>(a.out), a.lse, opart, ml);
}

}  // namespace

size_t attn_tree_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax) {
    const TreePlan p = make_plan(B, n1, Hq, Hkv, D, Lmax);
    return TreeLayout(B, Hkv, p.nsplit, (Hq / Hkv) * n1, D).total;
}

hipError_t launch_attn_tree(const AttnArgs& a, hipStream_t stream) {
    const TreePlan p = make_plan(a.B, a.n1, a.Hq, a.Hkv, a.D, a.Lmax);
    const TreeLayout lay(a.B, a.Hkv, p.nsplit, (a.Hq / a.Hkv) * a.n1, a.D);
    char* ws = static_cast<char*>(a.workspace);
    uint16_t* opart = p.nsplit > 1 ? reinterpret_cast<uint16_t*>(ws + lay.opart) : nullptr;
    float2* ml = p.nsplit > 1 ? reinterpret_cast<float2*>(ws + lay.ml) : nullptr;
    if (a.D == 64) launch_tree<64>(a, p, opart, ml, stream);
    else launch_tree<128>(a, p, opart, ml, stream);
    if (p.nsplit > 1) {
        const int64_t total = static_cast<int64_t>(a.B) * a.n1 * a.Hq * (a.D / 8);
        const int blocks = static_cast<int>((total + 255) / 256);
        hipLaunchKernelGGL(attn_tree_combine_kernel, dim3(blocks), dim3(256), 0, stream, opart, ml,
                           a.ctx_len, a.B, a.n1, a.Hq, a.Hkv, a.D, a.Lmax, p.nsplit,
                           static_cast<uint16_t*>(a.out), a.lse);
    }
    return hipGetLastError();
}

}  // namespace specv
