"""CPU-side checks of the C ABI: the library loads, exports every function the header declares,
and rejects bad arguments on the host before any launch (no GPU needed for these calls)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specv.h")
LIB = os.path.join(ROOT, "draft_verify_sampling_specv_amd", "libspecv.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libspecv.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(specv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("specv_build_tree_mask", "specv_tree_attn_verify", "specv_accept_resample",
              "specv_accept_workspace_bytes", "specv_attn_workspace_bytes", "specv_status_string",
              "specv_last_error", "specv_kv_commit"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(lib, n), n


@pytest.fixture(scope="module")
def specv():
    import draft_verify_sampling_specv_amd as m
    return m


def test_checked_build_exports_the_same_functions_and_the_product_build_has_no_record():
    """The bounds-checked debug library (SPECV_CHECKED) is built beside the product one and exports
    every declared function; the product library reports that it records nothing (-1)."""
    checked = os.path.join(ROOT, "draft_verify_sampling_specv_amd", "libspecv_checked.so")
    assert os.path.exists(checked), "libspecv_checked.so not built"
    clib = ctypes.CDLL(checked)
    for n in declared_functions():
        assert hasattr(clib, n), f"{n} missing from libspecv_checked.so"
    lib = ctypes.CDLL(LIB)
    lib.specv_debug_bounds.restype = ctypes.c_int64
    lib.specv_debug_bounds.argtypes = [ctypes.c_int32]
    assert lib.specv_debug_bounds(0) == -1


def test_status_strings(specv):
    lib = specv.lib
    assert lib.specv_status_string(0) == b"ok"
    assert b"invalid" in lib.specv_status_string(1)
    assert lib.specv_status_string(99) == b"unknown status"


def _accept(lib, **kw):
    args = dict(t=1, d=1, dtype=1, tok=1, par=1, B=2, K=3, V=100, T=1.0, seed=0, off=0,
                al=1, ot=1, on=1, pt=None, qt=None, ws=1, wsb=1 << 30, stream=None)
    args.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.specv_accept_resample(p(args["t"]), p(args["d"]), args["dtype"], p(args["tok"]), p(args["par"]),
                                     args["B"], args["K"], args["V"], args["T"], args["seed"], args["off"],
                                     p(args["al"]), p(args["ot"]), p(args["on"]), p(args["pt"]), p(args["qt"]),
                                     p(args["ws"]), args["wsb"], args["stream"])


def test_accept_host_validation(specv):
    lib = specv.lib
    assert _accept(lib, B=-1) == 1
    assert _accept(lib, K=-1) == 1
    assert _accept(lib, K=1024) == 1
    assert _accept(lib, V=0) == 1
    assert _accept(lib, V=(1 << 21) + 1) == 1
    assert _accept(lib, T=-0.5) == 1
    assert _accept(lib, T=float("nan")) == 1
    assert _accept(lib, T=float("inf")) == 1
    assert _accept(lib, dtype=7) == 2
    assert _accept(lib, t=None) == 1
    assert _accept(lib, d=None, T=1.0) == 1
    assert _accept(lib, ws=None) == 3
    assert _accept(lib, wsb=16) == 3
    assert b"workspace" in lib.specv_last_error()
    assert _accept(lib, B=0) == 0                      # empty call, no launch
    assert lib.specv_last_error() == b""


def test_workspace_queries(specv):
    assert specv.accept_workspace_bytes(32, 5, 32000, None) > 0
    assert specv.lib.specv_accept_workspace_bytes(0, 5, 100, 0) == 0
    # many query rows per KV head (tree x GQA group) over a long context are split along the
    # keys and need a workspace for the partials; when sequences x KV heads x row groups already
    # cover the device (or the context is short) there is no split; decode-shaped calls (at most
    # 64 rows per KV head) need none
    assert specv.attn_workspace_bytes(4, 64, 64, 8, 128, 32833) > 0
    assert specv.attn_workspace_bytes(16, 60, 64, 8, 128, 4157) == 0
    assert specv.attn_workspace_bytes(32, 5, 32, 8, 128, 2054) == 0
    assert specv.attn_workspace_bytes(32, 5, 32, 8, 96, 2054) == 0
    assert specv.attn_workspace_bytes(32, 5, 30, 8, 128, 2054) == 0


def test_attention_and_mask_host_validation(specv):
    lib = specv.lib
    v = ctypes.c_void_p(1)

    # every call below must be rejected on the host: the pointers are not device memory
    def attn(**kw):
        a = dict(B=4, K=64, Hq=64, Hkv=8, D=128, Lmax=32833, scale=0.1, dtype=1, ws=v, wsb=8)
        a.update(kw)
        return lib.specv_tree_attn_verify(v, v, v, v, v, a["B"], a["K"], a["Hq"], a["Hkv"], a["D"], a["Lmax"],
                                          a["scale"], a["dtype"], v, None, a["ws"], a["wsb"], None)

    assert attn(Hq=7) == 1
    assert attn(Hkv=0) == 1
    assert attn(D=96) == 2
    assert attn(dtype=5) == 2
    assert attn(Lmax=3) == 1
    assert attn(scale=float("nan")) == 1
    assert attn(scale=-1.0) == 1
    assert attn(K=1024) == 1
    assert attn() == 3                                  # workspace too small
    assert attn(ws=None) == 3
    assert attn(B=0) == 0
    assert lib.specv_build_tree_mask(None, 2, 3, None, None, None, None) == 1
    assert lib.specv_build_tree_mask(v, -2, 3, v, v, v, None) == 1
    assert lib.specv_build_tree_mask(v, 2, 1024, v, v, v, None) == 1
    assert lib.specv_build_tree_mask(None, 0, 3, None, None, None, None) == 0


def test_read_probe_host_validation(specv):
    lib = specv.lib
    v = ctypes.c_void_p(16)
    n = lib.specv_read_probe_sink_words()
    assert n > 0
    assert lib.specv_read_probe(v, 0, None, 0, None) == 0                  # no bytes: nothing to do
    assert lib.specv_read_probe(None, 1024, v, n, None) == 1
    assert lib.specv_read_probe(v, 1024, None, n, None) == 1
    assert lib.specv_read_probe(ctypes.c_void_p(24), 1024, v, n, None) == 1   # misaligned buffer
    assert lib.specv_read_probe(v, 1000, v, n, None) == 1                  # size not a multiple of 16
    assert lib.specv_read_probe(v, 1024, v, n - 1, None) == 1              # sink too small
    assert b"sink" in lib.specv_last_error()


def test_kv_commit_host_validation(specv):
    lib = specv.lib
    v = ctypes.c_void_p(16)

    def commit(**kw):
        a = dict(k=v, vv=v, B=2, K=5, Hkv=8, D=128, Lmax=64, dtype=1)
        a.update(kw)
        return lib.specv_kv_commit(a["k"], a["vv"], v, v, v, a["B"], a["K"], a["Hkv"], a["D"], a["Lmax"],
                                   a["dtype"], v, None)

    assert commit(B=-1) == 1
    assert commit(K=-1) == 1
    assert commit(K=1024) == 1
    assert commit(Hkv=0) == 1
    assert commit(Lmax=5) == 1
    assert commit(D=96) == 2
    assert commit(dtype=3) == 2
    assert commit(k=None) == 1
    assert commit(vv=ctypes.c_void_p(24)) == 1          # misaligned
    assert b"aligned" in lib.specv_last_error()
    assert commit(B=0) == 0


def test_accept_rule_host_validation(specv):
    lib = specv.lib
    v = ctypes.c_void_p(16)

    def call(rule, draft=v, T=1.0):
        return lib.specv_accept_resample_rule(v, draft, 1, v, v, 2, 3, 100, T, rule, 0, 0, v, v, v, None, None,
                                              v, 1 << 30, None)

    assert call(3) == 1
    assert call(-1) == 1
    assert b"rule" in lib.specv_last_error()
    assert call(0, draft=None) == 1          # draft needed without replacement at T > 0
    assert call(1, draft=None) == 1          # and for i.i.d. siblings
    assert lib.specv_accept_resample_rule(v, None, 1, v, v, 0, 3, 100, 1.0, 2, 0, 0, v, v, v, None, None,
                                          v, 1 << 30, None) == 0      # B == 0: no launch


def test_tree_expand_host_validation(specv):
    lib = specv.lib
    v = ctypes.c_void_p(16)

    def call(**kw):
        a = dict(B=2, F=4, V=100, k=3, T=1.0, keep=5, nmax=32, dtype=1, ws=v, wsb=1 << 20)
        a.update(kw)
        return lib.specv_tree_expand(v, a["dtype"], v, a["B"], a["F"], a["V"], a["k"], a["T"], a["keep"], a["nmax"],
                                     v, v, v, v, v, a["ws"], a["wsb"], None)

    assert call(k=0) == 1
    assert call(k=17) == 1
    assert call(F=100, k=16) == 1                        # F * k > 1024
    assert call(T=0.0) == 1
    assert call(keep=0) == 1
    assert call(nmax=1025) == 1
    assert call(V=0) == 1
    assert call(dtype=4) == 2
    assert call(ws=None) == 3
    assert call(wsb=8) == 3
    assert call(B=0) == 0
    assert specv.tree_expand_workspace_bytes(2, 4) > 0


def test_verify_layer_host_validation(specv):
    lib = specv.lib
    v = ctypes.c_void_p(256)

    def call(**kw):
        a = dict(x=v, B=2, K=5, Hq=4, Hkv=2, D=64, Lmax=64, inter=128, eps=1e-5, theta=10000.0, ws=v,
                 wsb=1 << 40)
        a.update(kw)
        return lib.specv_verify_layer(a["x"], v, v, v, v, v, v, a["eps"], a["theta"], v, v, v, v, v,
                                      a["B"], a["K"], a["Hq"], a["Hkv"], a["D"], a["Lmax"], a["inter"], v,
                                      a["ws"], a["wsb"], None)

    assert call(B=-1) == 1
    assert call(K=-1) == 1
    assert call(K=1024) == 1
    assert call(Hq=6, Hkv=4) == 1
    assert call(Lmax=5) == 1
    assert call(inter=100) == 1
    assert call(eps=0.0) == 1
    assert call(theta=1.0) == 1
    assert call(theta=float("nan")) == 1
    assert call(D=96) == 2
    assert call(x=None) == 1
    assert call(x=ctypes.c_void_p(264)) == 1            # misaligned
    assert b"aligned" in lib.specv_last_error()
    assert call(ws=None) == 3
    assert call(wsb=16) == 3
    assert call(ws=ctypes.c_void_p(272)) == 3           # workspace not 256-byte aligned
    assert call(B=0) == 0
    assert specv.verify_layer_workspace_bytes(32, 5, 32, 8, 128, 2054, 14336) > 0
    assert specv.verify_layer_workspace_bytes(32, 5, 32, 8, 128, 2054, 100) == 0
    assert "specv_verify_layer" in declared_functions()


def test_packed_layer_host_validation(specv):
    """The packed layer shares every check of specv_verify_layer; packing checks its sizes,
    pointers, alignment and overlap on the host."""
    lib = specv.lib
    v = ctypes.c_void_p(256)

    def layer(**kw):
        a = dict(B=2, K=5, inter=128, ws=v)
        a.update(kw)
        return lib.specv_verify_layer_packed(v, v, v, v, v, v, v, 1e-5, 10000.0, v, v, v, v, v, a["B"], a["K"], 4, 2,
                                             64, 64, a["inter"], v, a["ws"], 1 << 40, None)

    assert layer(B=-1) == 1
    assert layer(inter=100) == 1
    assert layer(ws=None) == 3
    assert layer(B=0) == 0

    def pack(w=256, N=64, K=128, out=1 << 20):
        return lib.specv_pack_weights(ctypes.c_void_p(w) if w else None, N, K,
                                      ctypes.c_void_p(out) if out else None, None)

    assert pack(N=0) == 1
    assert pack(N=48) == 1                  # not a multiple of 32
    assert pack(K=96) == 1                  # not a multiple of 64
    assert pack(N=-32) == 1
    assert pack(w=0) == 1
    assert pack(out=0) == 1
    assert pack(w=264) == 1                 # misaligned
    assert pack(out=256 + 64 * 128) == 1    # overlaps w (64 x 128 bf16 = 16 KiB)
    assert b"overlap" in lib.specv_last_error()
    for n in ("specv_pack_weights", "specv_verify_layer_packed"):
        assert n in declared_functions()
