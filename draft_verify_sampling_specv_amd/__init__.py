"""Python binding of libspecv: the verify step of speculative decoding on MI355X.

Argument marshalling only.  Every step runs in the HIP kernels of libspecv.so
(see include/specv.h for the C ABI and the contract of each call); PyTorch
provides device memory and the current stream.  There is no fallback: if the
library has not been built this import fails.

  build_tree_mask(parent)                                  -> mask, depth, status
  tree_attn_verify(q, k_cache, v_cache, ctx_len, mask)     -> out, lse
  accept_resample(target, draft, tokens, parent, T, seed, offset) -> AcceptResult
  accept_resample_noalloc(...)   the same through the entry point that allocates nothing
  kv_commit(k_cache, v_cache, ctx_len, accept_len, out_nodes)     -> new_ctx_len
  tree_expand(draft_logits, frontier, tree, k, T, keep)           -> new_frontier (tree updated)
  verify_layer(x, weights, k_cache, v_cache, ctx_len, mask, depth, Hq) -> out (caches written)
  pack_layer_weights(weights) / pack_weights(w)    the layer's matrices in the tile order its
                                                   products read (verify_layer takes either)
"""

from ._lib import (  # noqa: F401
    SpecvError,
    AcceptResult,
    AcceptBuffers,
    AttnBuffers,
    lib,
    library_path,
    debug_bounds,
    read_probe,
    build_tree_mask,
    tree_attn_verify,
    accept_resample,
    accept_resample_noalloc,
    kv_commit,
    DraftTree,
    tree_expand,
    tree_expand_workspace_bytes,
    accept_workspace_bytes,
    attn_workspace_bytes,
    LayerWeights,
    pack_weights,
    pack_layer_weights,
    verify_layer,
    verify_layer_workspace_bytes,
)
