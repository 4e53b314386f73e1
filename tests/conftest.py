import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size configurations")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them loudly rather than fail
    # when someone runs the whole suite on a CPU-only machine without -m.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """With DAB_PARITY_SUMMARY set, write the measured relative-L2 errors of every parity case that ran
    (the worst sequence or head per gate, and the whole-tensor figures) to that path as a markdown table."""
    path = os.environ.get("DAB_PARITY_SUMMARY")
    if not path:
        return
    try:
        from gpu_util import RECORD
    except Exception:
        return
    if not RECORD:
        return
    keys = ["out", "y", "a", "k_row", "v_row", "out_all", "y_all"]
    lines = ["| case | dtype | gate | " + " | ".join(keys) + " | worst / gate |",
             "|---|---|---|" + "---|" * len(keys) + "---|"]
    for label, dtype, errs in RECORD:
        tol = 1e-2 if dtype == "bf16" else 1e-5
        gated = [errs[k] for k in ("out", "y", "a", "k_row", "v_row") if k in errs]
        cells = [f"{errs[k]:.2e}" if k in errs else "-" for k in keys]
        lines.append(f"| {label} | {dtype} | {tol:.0e} | " + " | ".join(cells) +
                     f" | {max(gated) / tol:.3f} |")
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
