import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# The full-size workload tests whose raw errors the summary lists.
_TABLE = ("test_paged_gqa4_bf16_", "test_long_context_bf16_", "test_ragged_fp16_outliers_",
          "test_dense_decode_fp16", "test_smallq_mha_fp16")


def pytest_terminal_summary(terminalreporter):
    """After a run: the largest |gpu - oracle| of each full-size workload
    test's output and LSE checks, next to the bar each was held to."""
    parity = sys.modules.get("tests.parity") or sys.modules.get("parity")
    if parity is None or not parity.RECORDS:
        return
    rows = {}
    for test, what, err, bar in parity.RECORDS:
        name = test.split("::")[-1]
        if not name.startswith(_TABLE):
            continue
        kind = "lse" if what.startswith("lse") else "out"
        key = (name, kind)
        if key not in rows or err > rows[key][0]:
            rows[key] = (err, bar)
    if not rows:
        return
    terminalreporter.write_sep("-", "raw max |gpu - oracle| of the full-size workload tests")
    for (name, kind), (err, bar) in sorted(rows.items()):
        terminalreporter.write_line("%-58s %-3s %.3e  (bar %s)" % (name, kind, err, bar))
