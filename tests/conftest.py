import os
import sys

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
