// Tree-attention verify, fp32 inputs: a plain VALU kernel, one wave per (sequence, node, head).
// Used for small fp32 cases (correctness path; no MFMA).

#include "attn_common.h"
#include "kernels.h"

namespace specv {
namespace {
using namespace attn;

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
    if (!(L >= 0 && L <= Lmax - n1)) {
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
            if (!((mrow[SPECV_CHK(jj >> 5, words, kSiteF32MaskWord)] >> (jj & 31)) & 1u)) continue;
        }
        const float* kr = kb + static_cast<int64_t>(SPECV_CHK(key, Lmax, kSiteF32Key)) * D;
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
        s *= c2;
        const float mn = fmaxf(m, s);
        const float a = exp2f(m - mn);
        const float p = exp2f(s - mn);
        const float* vr = vb + static_cast<int64_t>(SPECV_CHK(key, Lmax, kSiteF32Key)) * D;
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

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
    const float c2 = a.scale * kLog2e;
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

}  // namespace specv
