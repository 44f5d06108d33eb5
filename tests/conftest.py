import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, when no GPU is visible, so that
    # `-m "not gpu"` and a plain run on a CPU-only host both stay green.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    # The attention error of every GPU-vs-oracle comparison made in this run, per case:
    # elements compared, max abs error (and the reference value there), max rel error over
    # |ref| >= 0.5. Written as JSON too when PA_PARITY_REPORT names a file.
    mod = sys.modules.get("tests.parity")
    record = getattr(mod, "RECORD", None)
    if not record:
        return
    tr = terminalreporter
    tr.write_sep("-", "attention parity: max abs error (bound 1e-2), max rel error over |ref| >= 0.5 (bound 2e-2)")
    for name, s in sorted(record.items()):
        tr.write_line(f"{name[:58]:58s} n={s['n']:>10d} calls={s['calls']:>3d} max_abs={s['max_abs']:.3e} "
                      f"(ref {s['max_abs_ref']:+.3f}) max_rel={s['max_rel_ref_ge_0.5']:.3e}")
    path = os.environ.get("PA_PARITY_REPORT")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(record, f, indent=1, sort_keys=True)
