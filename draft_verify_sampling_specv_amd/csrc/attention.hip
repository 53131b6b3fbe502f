// Tree-attention verify: dispatch between the three attention paths.
//   fp32 inputs                      -> attn_f32.hip    (VALU, correctness path)
//   bf16, <= 2 row blocks per KV head -> attn_decode.hip (HBM-bound decode shape, one kernel)
//   bf16, more rows                   -> attn_tree.hip   (MFMA, LDS-shared K/V, split + combine)

#include "kernels.h"

namespace specv {

static bool decode_shaped(int n1, int Hq, int Hkv) { return ((Hq / Hkv) * n1 + 31) / 32 <= 2; }

size_t attn_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax) {
    if (decode_shaped(n1, Hq, Hkv)) return 0;
    return attn_tree_workspace_bytes(B, n1, Hq, Hkv, D, Lmax);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
    if (!a.bf16) return launch_attn_f32(a, stream);
    if (decode_shaped(a.n1, a.Hq, a.Hkv)) return launch_attn_decode(a, stream);
    return launch_attn_tree(a, stream);
}

}  // namespace specv
