import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host work)")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a host without one they are skipped, not failed,
    # unless they were explicitly selected with -m gpu (then they must run).
    import importlib.util
    has_torch = importlib.util.find_spec("torch") is not None
    gpu = False
    if has_torch:
        import torch
        gpu = torch.cuda.is_available()
    markexpr = config.getoption("-m") or ""
    if gpu or "gpu" in markexpr and "not gpu" not in markexpr:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """Totals of the parity comparisons of the run.  Rule 2 (FP8): scale bytes
    checked, those that differ from the oracle's, those accepted only under
    the accumulation allowance (capped per tensor), how many of those needed
    the matrix core's truncation and the outputs' envelopes, and the blocks
    that match once sigmoid factors below FP32's range are taken as 0.
    Rule 1 (BF16): elements accepted only within their accumulation
    envelope."""
    try:
        from parity_util import RULE1_LOG, RULE2_LOG
    except ImportError:
        return
    if RULE1_LOG:
        acc = sum(a for _, a, _ in RULE1_LOG)
        elems = sum(n for _, _, n in RULE1_LOG)
        worst = max(RULE1_LOG, key=lambda x: x[1] / max(x[2], 1))
        terminalreporter.write_line(
            f"rule 1 over {len(RULE1_LOG)} BF16 tensors: {acc} of {elems} elements beyond 1e-2 of their group's "
            f"largest output and within their accumulation envelope (largest share {worst[1]}/{worst[2]} in "
            f"{worst[0]})")
    if not RULE2_LOG:
        return
    blocks = sum(s["scale_blocks"] for _, s in RULE2_LOG)
    mism = sum(s["scale_boundary_mismatch"] for _, s in RULE2_LOG)
    widened = sum(s["scale_acc_allowance"] for _, s in RULE2_LOG)
    trunc = sum(s.get("scale_mfma_truncation", 0) for _, s in RULE2_LOG)
    under = sum(s.get("scale_fp32_underflow", 0) for _, s in RULE2_LOG)
    beyond = sum(s["beyond_1ulp"] for _, s in RULE2_LOG)
    elems = sum(s["elements"] for _, s in RULE2_LOG)
    worst = max(RULE2_LOG, key=lambda x: x[1]["scale_acc_allowance"] / max(x[1]["scale_blocks"], 1))
    terminalreporter.write_line(
        f"rule 2 over {len(RULE2_LOG)} FP8 tensors: {blocks} E8M0 scale bytes, {mism} differ from the oracle's, "
        f"{widened} of them only inside the accumulation allowance "
        f"({trunc} decided with the matrix core's truncation and the outputs' envelopes), {under} matching with "
        f"FP32-underflowed sigmoid factors at 0 "
        f"(largest share {worst[1]['scale_acc_allowance']}/{worst[1]['scale_blocks']} in {worst[0]}); "
        f"{beyond} of {elems} codes beyond one E4M3 ULP")
