"""ctypes binding of libspecv.so (names follow include/specv.h)."""

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPECV_LIBRARY=libspecv_checked.so selects the bounds-checked debug build (tests); only the two
# library files built next to this module can be named
_LIBRARIES = ("libspecv.so", "libspecv_checked.so")
_name = os.environ.get("SPECV_LIBRARY", "libspecv.so")
if _name not in _LIBRARIES:
    raise ImportError(f"SPECV_LIBRARY={_name!r}: expected one of {_LIBRARIES}")
library_path = os.path.join(_HERE, _name)

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it with `python draft_verify_sampling_specv_amd/build.py` "
        "(the verify step has no CPU fallback)")

lib = ctypes.CDLL(library_path)

SPECV_F32, SPECV_BF16 = 0, 1
_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p

lib.specv_status_string.restype = ctypes.c_char_p
lib.specv_status_string.argtypes = [ctypes.c_int]
lib.specv_last_error.restype = ctypes.c_char_p
lib.specv_last_error.argtypes = []
lib.specv_debug_bounds.restype = ctypes.c_int64
lib.specv_debug_bounds.argtypes = [ctypes.c_int32]
lib.specv_read_probe.restype = ctypes.c_int
lib.specv_read_probe.argtypes = [_vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _vp]
lib.specv_read_probe_sink_words.restype = ctypes.c_int32
lib.specv_read_probe_sink_words.argtypes = []


def read_probe(buf, sink):
    """Stream `buf` (a CUDA tensor, 16-byte aligned, size a multiple of 16 bytes) once with the
    non-temporal 16-byte loads of the streaming kernels, on the current stream (measurement aid)."""
    nbytes = buf.numel() * buf.element_size()
    _check("specv_read_probe", lib.specv_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), _stream()))


def debug_bounds(reset=True):
    """The bounds record of a checked build (0: no index out of range since the last reset), -1 in
    the product build."""
    return int(lib.specv_debug_bounds(1 if reset else 0))

lib.specv_build_tree_mask.restype = ctypes.c_int
lib.specv_build_tree_mask.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp]

lib.specv_attn_workspace_bytes.restype = ctypes.c_size_t
lib.specv_attn_workspace_bytes.argtypes = [ctypes.c_int32] * 6
lib.specv_tree_attn_verify.restype = ctypes.c_int
lib.specv_tree_attn_verify.argtypes = [
    _vp, _vp, _vp, _vp, _vp,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_float, ctypes.c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp]

lib.specv_accept_workspace_bytes.restype = ctypes.c_size_t
lib.specv_accept_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
lib.specv_accept_resample.restype = ctypes.c_int
lib.specv_accept_resample.argtypes = [
    _vp, _vp, ctypes.c_int, _vp, _vp,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
    ctypes.c_uint64, ctypes.c_uint64,
    _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.specv_accept_resample_rule.restype = ctypes.c_int
lib.specv_accept_resample_rule.argtypes = [
    _vp, _vp, ctypes.c_int, _vp, _vp,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int,
    ctypes.c_uint64, ctypes.c_uint64,
    _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.specv_accept_resample_rule_noalloc.restype = ctypes.c_int
lib.specv_accept_resample_rule_noalloc.argtypes = [
    _vp, _vp, ctypes.c_int, _vp, _vp,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int,
    ctypes.c_uint64, ctypes.c_uint64,
    _vp, _vp, _vp, _vp, _vp, _vp]
SIBLING_RULES = {"without_replacement": 0, "iid": 1, "deterministic": 2}

lib.specv_tree_expand_workspace_bytes.restype = ctypes.c_size_t
lib.specv_tree_expand_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
lib.specv_tree_expand.restype = ctypes.c_int
lib.specv_tree_expand.argtypes = [
    _vp, ctypes.c_int, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
    ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]

lib.specv_kv_commit.restype = ctypes.c_int
lib.specv_kv_commit.argtypes = [
    _vp, _vp, _vp, _vp, _vp,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_int, _vp, _vp]

lib.specv_verify_layer_workspace_bytes.restype = ctypes.c_size_t
lib.specv_verify_layer_workspace_bytes.argtypes = [ctypes.c_int32] * 7
lib.specv_verify_layer.restype = ctypes.c_int
lib.specv_verify_layer.argtypes = (
    [_vp] * 7 + [ctypes.c_float, ctypes.c_float] + [_vp] * 5 + [ctypes.c_int32] * 7 + [_vp, _vp, ctypes.c_size_t, _vp])
lib.specv_verify_layer_packed.restype = ctypes.c_int
lib.specv_verify_layer_packed.argtypes = lib.specv_verify_layer.argtypes
lib.specv_pack_weights.restype = ctypes.c_int
lib.specv_pack_weights.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp]


class SpecvError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib.specv_status_string(status).decode()
        detail = lib.specv_last_error().decode()
        super().__init__(f"{fn}: {msg}" + (f" ({detail})" if detail else ""))


def _check(fn, status):
    if status != 0:
        raise SpecvError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SPECV_BF16
    if t.dtype == torch.float32:
        return SPECV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, dtype=None):
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if dtype is not None and t.dtype != dtype:
        t = t.to(dtype)
    return t.contiguous()


# ----------------------------------------------------------------------------- mask

def build_tree_mask(parent, out=None):
    """parent[B][K+1] int32 (device) -> (mask[B][K+1][W] int32 view of uint32, depth, status)."""
    parent = _dev(parent, torch.int32)
    B, n1 = parent.shape
    words = (n1 + 31) // 32
    if out is None:
        mask = torch.empty((B, n1, words), dtype=torch.int32, device=parent.device)
        depth = torch.empty((B, n1), dtype=torch.int32, device=parent.device)
        status = torch.empty((B,), dtype=torch.int32, device=parent.device)
    else:
        mask, depth, status = out
    _check("specv_build_tree_mask",
           lib.specv_build_tree_mask(_ptr(parent), B, n1 - 1, _ptr(mask), _ptr(depth), _ptr(status), _stream()))
    return mask, depth, status


# ----------------------------------------------------------------------------- attention

def attn_workspace_bytes(B, K, Hq, Hkv, D, Lmax):
    return int(lib.specv_attn_workspace_bytes(B, K, Hq, Hkv, D, Lmax))


@dataclass
class AttnBuffers:
    out: torch.Tensor
    lse: torch.Tensor
    workspace: torch.Tensor

    @staticmethod
    def allocate(q, k_cache):
        B, n1, Hq, D = q.shape
        Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
        ws = attn_workspace_bytes(B, n1 - 1, Hq, Hkv, D, Lmax)
        return AttnBuffers(torch.empty_like(q), torch.empty((B, n1, Hq), dtype=torch.float32, device=q.device),
                           torch.empty((max(ws, 1),), dtype=torch.uint8, device=q.device))


def tree_attn_verify(q, k_cache, v_cache, ctx_len, mask, scale=None, buffers=None):
    """One layer's tree-masked attention.  Returns (out[B][K+1][Hq][D], lse[B][K+1][Hq])."""
    q, k_cache, v_cache = _dev(q), _dev(k_cache), _dev(v_cache)
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, k_cache and v_cache must share a dtype")
    ctx_len, mask = _dev(ctx_len, torch.int32), _dev(mask)
    B, n1, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, Hkv, Lmax, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [B][Hkv][Lmax][D] matching q")
    if mask.shape != (B, n1, (n1 + 31) // 32):
        raise ValueError("mask must be [B][K+1][(K+32)//32]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    bufs = buffers or AttnBuffers.allocate(q, k_cache)
    _check("specv_tree_attn_verify", lib.specv_tree_attn_verify(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), _ptr(mask),
        B, n1 - 1, Hq, Hkv, D, Lmax, float(scale), _dtype_code(q),
        _ptr(bufs.out), _ptr(bufs.lse), _ptr(bufs.workspace), bufs.workspace.numel(), _stream()))
    return bufs.out, bufs.lse


# ----------------------------------------------------------------------------- accept

def accept_workspace_bytes(B, K, V, dtype):
    code = SPECV_BF16 if dtype == torch.bfloat16 else SPECV_F32
    return int(lib.specv_accept_workspace_bytes(B, K, V, code))


@dataclass
class AcceptResult:
    accept_len: torch.Tensor     # [B] int32
    out_tokens: torch.Tensor     # [B][K+1] int32
    out_nodes: torch.Tensor      # [B][K+1] int32
    p_tok: torch.Tensor          # [B][K+1] float32
    q_tok: torch.Tensor          # [B][K+1] float32


@dataclass
class AcceptBuffers:
    result: AcceptResult
    workspace: torch.Tensor

    @staticmethod
    def allocate(B, n1, V, dtype, device):
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        res = AcceptResult(torch.empty((B,), **i32), torch.empty((B, n1), **i32), torch.empty((B, n1), **i32),
                           torch.empty((B, n1), **f32), torch.empty((B, n1), **f32))
        ws = accept_workspace_bytes(B, n1 - 1, V, dtype)
        # zero-filled once; the library keeps it valid from call to call
        return AcceptBuffers(res, torch.zeros((max(ws, 1),), dtype=torch.uint8, device=device))


def accept_resample(target_logits, draft_logits, tokens, parent, temperature, seed=0, offset=0,
                    buffers=None, with_probs=True, siblings="without_replacement"):
    """Exact accept / reject / resample.  `siblings` names how the siblings of a node were
    drafted ("without_replacement", "iid" or "deterministic"); draft_logits may be None at
    temperature 0 or for deterministic siblings."""
    target_logits = _dev(target_logits)
    if draft_logits is not None:
        draft_logits = _dev(draft_logits)
        if draft_logits.dtype != target_logits.dtype or draft_logits.shape != target_logits.shape:
            raise TypeError("draft_logits must match target_logits in dtype and shape")
    tokens, parent = _dev(tokens, torch.int32), _dev(parent, torch.int32)
    B, n1, V = target_logits.shape
    if tokens.shape != (B, n1) or parent.shape != (B, n1):
        raise ValueError("tokens and parent must be [B][K+1]")
    bufs = buffers or AcceptBuffers.allocate(B, n1, V, target_logits.dtype, target_logits.device)
    r = bufs.result
    if siblings not in SIBLING_RULES:
        raise ValueError(f"siblings must be one of {sorted(SIBLING_RULES)}")
    _check("specv_accept_resample_rule", lib.specv_accept_resample_rule(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), _ptr(tokens), _ptr(parent),
        B, n1 - 1, V, float(temperature), SIBLING_RULES[siblings], int(seed), int(offset),
        _ptr(r.accept_len), _ptr(r.out_tokens), _ptr(r.out_nodes),
        _ptr(r.p_tok) if with_probs else None, _ptr(r.q_tok) if with_probs else None,
        _ptr(bufs.workspace), bufs.workspace.numel(), _stream()))
    return r


def accept_resample_noalloc(target_logits, draft_logits, tokens, parent, temperature, seed=0, offset=0,
                            result=None, with_probs=True, siblings="without_replacement"):
    """accept_resample through the entry point that allocates nothing (its workspace is built
    into the library, 8 MiB per device); `result` (an AcceptResult) may be preallocated."""
    target_logits = _dev(target_logits)
    if draft_logits is not None:
        draft_logits = _dev(draft_logits)
        if draft_logits.dtype != target_logits.dtype or draft_logits.shape != target_logits.shape:
            raise TypeError("draft_logits must match target_logits in dtype and shape")
    tokens, parent = _dev(tokens, torch.int32), _dev(parent, torch.int32)
    B, n1, V = target_logits.shape
    if tokens.shape != (B, n1) or parent.shape != (B, n1):
        raise ValueError("tokens and parent must be [B][K+1]")
    if siblings not in SIBLING_RULES:
        raise ValueError(f"siblings must be one of {sorted(SIBLING_RULES)}")
    if result is None:
        i32 = dict(dtype=torch.int32, device=target_logits.device)
        f32 = dict(dtype=torch.float32, device=target_logits.device)
        result = AcceptResult(torch.empty((B,), **i32), torch.empty((B, n1), **i32), torch.empty((B, n1), **i32),
                              torch.empty((B, n1), **f32), torch.empty((B, n1), **f32))
    r = result
    _check("specv_accept_resample_rule_noalloc", lib.specv_accept_resample_rule_noalloc(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), _ptr(tokens), _ptr(parent),
        B, n1 - 1, V, float(temperature), SIBLING_RULES[siblings], int(seed), int(offset),
        _ptr(r.accept_len), _ptr(r.out_tokens), _ptr(r.out_nodes),
        _ptr(r.p_tok) if with_probs else None, _ptr(r.q_tok) if with_probs else None, _stream()))
    return r


# ----------------------------------------------------------------------------- KV commit

def kv_commit(k_cache, v_cache, ctx_len, accept_len, out_nodes, out=None):
    """Move the accepted path's K/V rows in place; returns new_ctx_len[B] int32 (-1: invalid)."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor (it is updated in place)")
    if k_cache.dtype != v_cache.dtype or k_cache.shape != v_cache.shape:
        raise TypeError("k_cache and v_cache must match in dtype and shape")
    ctx_len, accept_len = _dev(ctx_len, torch.int32), _dev(accept_len, torch.int32)
    out_nodes = _dev(out_nodes, torch.int32)
    B, Hkv, Lmax, D = k_cache.shape
    n1 = out_nodes.shape[1]
    if ctx_len.shape != (B,) or accept_len.shape != (B,) or out_nodes.shape != (B, n1):
        raise ValueError("ctx_len, accept_len must be [B] and out_nodes [B][K+1]")
    new_ctx = out if out is not None else torch.empty((B,), dtype=torch.int32, device=k_cache.device)
    _check("specv_kv_commit", lib.specv_kv_commit(
        _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), _ptr(accept_len), _ptr(out_nodes),
        B, n1 - 1, Hkv, D, Lmax, _dtype_code(k_cache), _ptr(new_ctx), _stream()))
    return new_ctx


# ----------------------------------------------------------------------------- tree expansion

@dataclass
class DraftTree:
    parent: torch.Tensor         # [B][nmax] int32
    tokens: torch.Tensor         # [B][nmax] int32
    score: torch.Tensor          # [B][nmax] float64, cumulative draft log-probability
    n_nodes: torch.Tensor        # [B] int32

    @staticmethod
    def with_roots(root_tokens, nmax):
        """A tree per sequence holding only its root (node 0, score 0)."""
        root_tokens = _dev(root_tokens, torch.int32)
        B = root_tokens.shape[0]
        dev = root_tokens.device
        parent = torch.full((B, nmax), -1, dtype=torch.int32, device=dev)
        tokens = torch.full((B, nmax), -1, dtype=torch.int32, device=dev)
        tokens[:, 0] = root_tokens
        return DraftTree(parent, tokens, torch.zeros((B, nmax), dtype=torch.float64, device=dev),
                         torch.ones((B,), dtype=torch.int32, device=dev))


def tree_expand_workspace_bytes(B, F):
    return int(lib.specv_tree_expand_workspace_bytes(B, F))


def tree_expand(draft_logits, frontier, tree, k, temperature, keep, new_frontier=None, workspace=None):
    """One level of top-k expansion of `tree` (updated in place); returns new_frontier[B][keep]."""
    draft_logits = _dev(draft_logits)
    frontier = _dev(frontier, torch.int32)
    B, F, V = draft_logits.shape
    nmax = tree.parent.shape[1]
    if frontier.shape != (B, F):
        raise ValueError("frontier must be [B][F] matching draft_logits")
    for name, t, dt in (("parent", tree.parent, torch.int32), ("tokens", tree.tokens, torch.int32),
                        ("score", tree.score, torch.float64)):
        if t.shape != (B, nmax) or t.dtype != dt or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"tree.{name} must be a contiguous [B][nmax] {dt} GPU tensor")
    if new_frontier is None:
        new_frontier = torch.empty((B, keep), dtype=torch.int32, device=draft_logits.device)
    if workspace is None:
        workspace = torch.empty((max(tree_expand_workspace_bytes(B, F), 1),), dtype=torch.uint8,
                                device=draft_logits.device)
    _check("specv_tree_expand", lib.specv_tree_expand(
        _ptr(draft_logits), _dtype_code(draft_logits), _ptr(frontier), B, F, V, int(k), float(temperature),
        int(keep), nmax, _ptr(tree.parent), _ptr(tree.tokens), _ptr(tree.score), _ptr(tree.n_nodes),
        _ptr(new_frontier), _ptr(workspace), workspace.numel(), _stream()))
    return new_frontier


# ----------------------------------------------------------------------------- verify layer

@dataclass
class LayerWeights:
    """bf16 GPU tensors in the [out][in] layout of a linear map (packed: the four matrices in the
    tile order of specv_pack_weights, their shapes unchanged; see pack_layer_weights)."""
    w_qkv: torch.Tensor          # [(Hq + 2 Hkv) D][Hq D]: query, key, value rows
    w_o: torch.Tensor            # [Hq D][Hq D]
    w_gate_up: torch.Tensor      # [2 inter][Hq D]: gate rows, then up rows
    w_down: torch.Tensor         # [Hq D][inter]
    attn_norm: torch.Tensor      # [Hq D]
    mlp_norm: torch.Tensor       # [Hq D]
    packed: bool = False


def pack_weights(w, out=None):
    """w [N][K] bf16 (GPU, contiguous; N a multiple of 32, K of 64) -> a tensor of the same shape
    holding it in the tile order the layer's products read (specv_pack_weights)."""
    if not w.is_cuda or not w.is_contiguous() or w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("w must be a contiguous 2-D bf16 GPU tensor")
    if out is None:
        out = torch.empty_like(w)
    N, K = w.shape
    _check("specv_pack_weights", lib.specv_pack_weights(_ptr(w), N, K, _ptr(out), _stream()))
    return out


def pack_layer_weights(weights):
    """LayerWeights with its four matrices packed (the norm gains are shared, not copied)."""
    if weights.packed:
        return weights
    return LayerWeights(pack_weights(weights.w_qkv), pack_weights(weights.w_o), pack_weights(weights.w_gate_up),
                        pack_weights(weights.w_down), weights.attn_norm, weights.mlp_norm, packed=True)


def verify_layer_workspace_bytes(B, K, Hq, Hkv, D, Lmax, inter):
    return int(lib.specv_verify_layer_workspace_bytes(B, K, Hq, Hkv, D, Lmax, inter))


def verify_layer(x, weights, k_cache, v_cache, ctx_len, mask, depth, Hq, eps=1e-5, theta=10000.0, out=None,
                 workspace=None):
    """One target layer over the draft nodes: x[B][K+1][Hq D] bf16 -> out (same shape); the nodes'
    rotated keys and values are written to the caches at ctx_len + node."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor (it is written in place)")
    x = _dev(x)
    w = weights
    for name in ("w_qkv", "w_o", "w_gate_up", "w_down", "attn_norm", "mlp_norm"):
        t = getattr(w, name)
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"weights.{name} must be a contiguous bf16 GPU tensor")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    ctx_len, mask, depth = _dev(ctx_len, torch.int32), _dev(mask), _dev(depth, torch.int32)
    B, n1, hd = x.shape
    _, Hkv, Lmax, D = k_cache.shape
    inter = w.w_down.shape[1]
    if hd != Hq * D or k_cache.shape != (B, Hkv, Lmax, D) or v_cache.shape != k_cache.shape:
        raise ValueError("x must be [B][K+1][Hq D] and the caches [B][Hkv][Lmax][D]")
    shapes = {"w_qkv": ((Hq + 2 * Hkv) * D, hd), "w_o": (hd, hd), "w_gate_up": (2 * inter, hd),
              "w_down": (hd, inter), "attn_norm": (hd,), "mlp_norm": (hd,)}
    for name, shp in shapes.items():
        if tuple(getattr(w, name).shape) != shp:
            raise ValueError(f"weights.{name} must be {shp}")
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty((max(verify_layer_workspace_bytes(B, n1 - 1, Hq, Hkv, D, Lmax, inter), 1),),
                                dtype=torch.uint8, device=x.device)
    fn = "specv_verify_layer_packed" if w.packed else "specv_verify_layer"
    _check(fn, getattr(lib, fn)(
        _ptr(x), _ptr(w.w_qkv), _ptr(w.w_o), _ptr(w.w_gate_up), _ptr(w.w_down), _ptr(w.attn_norm),
        _ptr(w.mlp_norm), float(eps), float(theta), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), _ptr(mask),
        _ptr(depth), B, n1 - 1, Hq, Hkv, D, Lmax, inter, _ptr(out), _ptr(workspace), workspace.numel(),
        _stream()))
    return out
