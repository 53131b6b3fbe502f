// Device helpers shared by the specv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------------
// Bounds-checked build.  Compiled with -DSPECV_CHECKED (libspecv_checked.so, a debug library),
// every global or LDS access whose index is derived from input data -- parent and token values,
// context lengths, accepted node ids, frontier entries -- goes through SPECV_CHK(i, n, site).  An index
// outside [0, n) is recorded in specv_oob_word (the first one: site in the high half, the index in
// the low half) and replaced by 0, so the access stays inside its buffer and the kernel runs to its
// end.  In the product build SPECV_CHK(i, n, site) is the index expression itself.
enum CheckSite : int {
    kSiteMaskWalk = 1,
    kSiteCommitNode, kSiteCommitSrc, kSiteCommitDst,
    kSiteAcceptGatherRow, kSiteAcceptGatherToken, kSiteAcceptLink, kSiteAcceptPath, kSiteAcceptEnd,
    kSiteAcceptPass, kSiteAcceptOut,
    kSiteDecodeKey, kSiteTreeKey, kSiteTreeMaskWord, kSiteF32Key, kSiteF32MaskWord,
    kSiteExpandFrontier, kSiteExpandNode, kSiteExpandPos, kSiteLayerCache,
};
#ifdef SPECV_CHECKED
extern __device__ unsigned long long specv_oob_word;
template <typename I>
__device__ __forceinline__ I checked_index(I i, int64_t n, int site) {
    if (static_cast<int64_t>(i) >= 0 && static_cast<int64_t>(i) < n) return i;
    atomicCAS(&specv_oob_word, 0ull,
              (static_cast<unsigned long long>(site) << 32) | static_cast<uint32_t>(static_cast<int64_t>(i)));
    return I(0);
}
#define SPECV_CHK(i, n, site) ::specv::checked_index((i), (n), (site))
#else
#define SPECV_CHK(i, n, site) (i)
#endif

// ---------------------------------------------------------------------------------------------
// Streaming loads with the non-temporal cache policy, for data read once (the KV cache, logit
// rows, packed weights).  Plain streaming reads of HBM measured about 15% faster with it on this
// device (16-byte loads over 1 GiB: 6.9-7.1 TB/s against 6.0-6.2 TB/s with the default policy).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCachePolicyNT = 2;      // buffer-load cache-policy operand: non-temporal

__device__ __forceinline__ uint4 load_nt(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_nt32(const void* p) {
    return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}

// ---------------------------------------------------------------------------------------------
// Element loads.  Logits and attention operands arrive as fp32 or bf16; bf16 is widened to fp32
// by placing its 16 bits in the high half of an fp32 word (exact).

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static constexpr int kVec = 4;   // elements per 16-byte load
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void load_vec(const float* p, int64_t i, float* out) {
        float4 v = *reinterpret_cast<const float4*>(p + i);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
};

template <>
struct Elem<uint16_t> {   // bf16 bit patterns
    static constexpr int kVec = 8;
    __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
    __device__ __forceinline__ static void load_vec(const uint16_t* p, int64_t i, float* out) {
        uint4 v = *reinterpret_cast<const uint4*>(p + i);
        out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
        out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
        out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
        out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
    }
};

// ---------------------------------------------------------------------------------------------
// Wave-wide reductions (64 lanes) through cross-lane shuffles.

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
    return x;
}

// Running (max, sum of exp2((x - max) * k)) pairs: merge two partial softmax statistics.
__device__ __forceinline__ void merge_max_sum(float& m, float& s, float m2, float s2, float k) {
    float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;   // both empty
    s = s * __builtin_amdgcn_exp2f((m - mn) * k) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * k);
    m = mn;
}

__device__ __forceinline__ void wave_max_sum(float& m, float& s, float k) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(m, o);
        float s2 = __shfl_xor(s, o);
        merge_max_sum(m, s, m2, s2, k);
    }
}

// (value, index) argmax with the lowest index winning ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o);
        int i2 = __shfl_xor(i, o);
        argmax_merge(v, i, v2, i2);
    }
}

// ---------------------------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11): ten rounds of two 64x64->128-bit products on the even counter words, the high halves
// XORed with the odd words and the round key, the key advanced by two Weyl constants per round.

struct U64x4 { uint64_t w[4]; };

__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                              uint64_t k0, uint64_t k1) {
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += W0; k1 += W1; }
        uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
        uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
        uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    return U64x4{{c0, c1, c2, c3}};
}

// 64-bit word -> odd multiple of 2^-53 in (0, 1), exact in double.
__device__ __forceinline__ double word_to_uniform(uint64_t w) {
    return static_cast<double>(2ull * (w >> 12) + 1ull) * 0x1p-53;
}

}  // namespace specv
