import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")
    config.addinivalue_line("markers", "slow: full-size CPU case (still part of the default suite)")


def pytest_report_header(config):
    """Name the HIP library the GPU tests load (path and SHA-256 prefix) in the run's header."""
    try:
        import bit_quantized_grouped_amd as bq
        fp = bq.lib_fingerprint()
        return f"moe_q4 library: {fp['path']} sha256 {fp['sha256_16']}"
    except (ImportError, OSError) as e:
        return f"moe_q4 library: not available ({e})"


def golden_lines(name):
    """Non-comment, non-empty lines of a fixture under tests/golden/."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
