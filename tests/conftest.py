import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")


def golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def pytest_terminal_summary(terminalreporter):
    """Every GPU parity check's measured error and near-tie count, beside its tolerance."""
    gc = sys.modules.get("gpu_common")
    if gc is None or not getattr(gc, "RESULTS", None):
        return
    tr = terminalreporter
    tr.section("parity measurements (GPU against the oracle)")
    tr.write_line(f"tolerances: attention bf16 {gc.ATTN_BF16_ABS:g} abs, fp32 {gc.ATTN_F32_ABS:g} abs; "
                  f"p_tok / q_tok {gc.P_REL:g} rel; decisions bit-exact outside near ties (< {gc.NEAR_TIE:g})")
    for name, r in gc.RESULTS.items():
        if r.get("kind") == "accept":
            extra = "".join(f", {k} {r[k]:.2e}" for k in ("p_tok_max_rel", "q_tok_max_rel") if k in r)
            tr.write_line(f"  accept {name}: {r['sequences']} sequences, near ties {r['near_ties']}, "
                          f"mismatches {r['mismatches']}{extra}")
        else:
            tr.write_line("  " + name + ": " + ", ".join(
                f"{k} {v:.3e}" if isinstance(v, float) else f"{k} {v}" for k, v in r.items() if k != "kind"))


@pytest.fixture(autouse=True)
def _bounds_record(request):
    """Under the bounds-checked library (SPECV_LIBRARY=libspecv_checked.so) every GPU test must leave
    the bounds record clear: no kernel index derived from input data fell outside its range."""
    yield
    if os.environ.get("SPECV_LIBRARY") != "libspecv_checked.so" or request.node.get_closest_marker("gpu") is None:
        return
    import draft_verify_sampling_specv_amd as specv
    rec = specv.debug_bounds(reset=True)
    assert rec == 0, f"bounds record {rec:#x}: check site {rec >> 32}, index {rec & 0xffffffff}"
