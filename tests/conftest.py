import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, when no GPU is visible; the CPU suite
    # is selected with -m "not gpu" anyway.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover - torch missing
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per parity check of the five workloads (and a count of the
    other checks with their tightest margin), so that the error figures and
    the bars they met stay visible in a quiet run."""
    helpers = sys.modules.get("helpers")
    records = getattr(helpers, "PARITY_RECORDS", None)
    if not records:
        return
    from causal_flash_attention_amd.workloads import WORKLOADS
    names = {w.name for w in WORKLOADS}
    tr = terminalreporter
    tr.write_line("parity against the float64 oracle (value / bar):")
    worst = None
    for label, dtype, m, bars in records:
        ratio = max(m[k] / b for k, b in bars.items())
        if label.split(" ")[0] in names:
            cells = " ".join(f"{k}={m[k]:.2e}/{b:.0e}" for k, b in bars.items())
            tr.write_line(f"  {label.split(' ')[0]} [{dtype}] {cells} (worst {ratio:.2f} of bar)")
        elif worst is None or ratio > worst[0]:
            worst = (ratio, label)
    others = sum(1 for r in records if r[0].split(" ")[0] not in names)
    if others:
        tr.write_line(f"  {others} other parity checks; tightest: {worst[1]} at {worst[0]:.2f} of its bar")
