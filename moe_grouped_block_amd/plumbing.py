"""Device-memory plumbing around the binding (torch used for allocation only).

``to_device`` uploads host arrays in the library's ABI layouts (the
generator's arrays already are: row-major, scales (rows, K/32));
``empty_outputs`` allocates the output tensors a problem writes.  Neither
computes anything of the method.
"""
from __future__ import annotations

import numpy as np
import torch

_NP2TORCH = {np.dtype(np.uint8): torch.uint8, np.dtype(np.uint16): torch.int16,
             np.dtype(np.int32): torch.int32, np.dtype(np.float32): torch.float32}


def _kplanes(t: torch.Tensor, k: int) -> torch.Tensor:
    """Device (..., rows, K/32) scale tensor -> its K-block planes, laid out by
    the library's moegg_sf_to_kplanes on the current stream."""
    import moe_grouped_block_amd as mg
    rows = int(t.numel() // (k // 32))
    dst = torch.empty(t.numel(), dtype=torch.uint8, device=t.device)
    mg.sf_to_kplanes(t, dst, rows, k)
    return dst


def to_device(arrays: dict, device="cuda", sf_layout: str = "row_major", k: int | None = None) -> dict:
    """numpy arrays -> contiguous device tensors (bf16 bits travel as int16).
    With sf_layout "kplanes" the scale arrays (sfa, sfb) are uploaded
    row-major and laid out as K-block planes on the device (K = `k`)."""
    out = {}
    for key, v in arrays.items():
        v = np.ascontiguousarray(v)
        t = torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v)
        out[key] = t.to(device, non_blocking=False)
        if sf_layout == "kplanes" and key in ("sfa", "sfb") and v.size:
            out[key] = _kplanes(out[key], int(k))
    return out


def discrete_weights(problem: dict, arrays: dict, device="cuda", seed: int = 0, null_empty=None,
                     sf_layout: str = "row_major"):
    """Per-expert allocations for the discrete-weight mode.

    Expert g's weights (N, row units) and, for MX operands, its (N, K/32)
    scales (as K-block planes with sf_layout "kplanes") get allocations of
    their own, made in a
    shuffled expert order with spacers between them, so their addresses are
    neither contiguous nor ascending.  Returns (pointer tensors {"b_ptrs",
    "sfb_ptrs"}, list of tensors to keep alive).  Experts listed in
    `null_empty` get a null pointer (allowed for experts without rows)."""
    L = int(problem["num_groups"])
    mx = problem["ab_dtype"] != "bf16"
    order = np.random.default_rng(seed).permutation(L)
    null_empty = set(null_empty or ())
    keep, bptr, sptr = [], [0] * L, [0] * L
    for g in order:
        keep.append(torch.empty(4096 + 256 * int(g), dtype=torch.uint8, device=device))   # spacer
        if g in null_empty:
            continue
        b = np.ascontiguousarray(arrays["b"][g])
        tb = torch.from_numpy(b.view(np.int16) if b.dtype == np.uint16 else b).to(device)
        keep.append(tb)
        bptr[g] = tb.data_ptr()
        if mx:
            ts = torch.from_numpy(np.ascontiguousarray(arrays["sfb"][g])).to(device)
            if sf_layout == "kplanes":
                ts = _kplanes(ts, int(problem["k"]))
            keep.append(ts)
            sptr[g] = ts.data_ptr()
    ptrs = {"b_ptrs": torch.tensor(bptr, dtype=torch.int64, device=device)}
    if mx:
        ptrs["sfb_ptrs"] = torch.tensor(sptr, dtype=torch.int64, device=device)
    return ptrs, keep


def n_out(problem: dict) -> int:
    n = int(problem["n"])
    return {"none": n, "srelu": n, "swiglu": n // 2, "geglu": n // 2, "dswiglu": 2 * n, "dgeglu": 2 * n,
            "dsrelu": n}[problem["act"]]


def empty_outputs(problem: dict, device="cuda", fill: int | None = None) -> dict:
    """Allocate every output the problem writes.  `fill` (a byte value) pre-fills
    them so a test can see untouched elements; dprob is always zero-filled
    because the library accumulates into it."""
    m, n, L = int(problem["valid_m"]), int(problem["n"]), int(problem["num_groups"])
    no = n_out(problem)
    out = {}

    def mk(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=device)
        if fill is not None:
            t.view(torch.uint8).fill_(fill)
        return t
    if problem["act"] in ("dswiglu", "dsrelu", "dgeglu"):
        out["dprob"] = torch.zeros(m, dtype=torch.float32, device=device)
        if problem["d_dtype"] == "e4m3":
            out["d"] = mk((m, no), torch.uint8)
            out["d_col"] = mk((m, no), torch.uint8)
            out["sfd_row"] = mk((m, no // 32), torch.uint8)
            out["sfd_col"] = mk((no, m // 32), torch.uint8)
        else:
            out["d"] = mk((m, no), torch.int16)
            if problem["ab_dtype"] != "bf16":
                out["amax"] = mk((L, 2) if problem["act"] in ("dswiglu", "dgeglu") else (L,), torch.float32)
        return out
    if problem.get("c_dtype") == "bf16":
        out["c"] = mk((m, n), torch.int16)
    if problem["d_dtype"] == "bf16":
        out["d"] = mk((m, no), torch.int16)
        out["amax"] = mk((L,), torch.float32)
    else:
        out["d"] = mk((m, no), torch.uint8)
        out["d_col"] = mk((m, no), torch.uint8)
        out["sfd_row"] = mk((m, no // 32), torch.uint8)
        out["sfd_col"] = mk((no, m // 32), torch.uint8)
    return out


def inputs_for(problem: dict, dev_arrays: dict, discrete: dict | None = None) -> dict:
    """Select the input tensors the problem uses from an uploaded case;
    `discrete` (pointer tensors from discrete_weights) replaces b and sfb."""
    keys = ["a", "b", "padded_offsets", "alpha", "prob"]
    if problem["ab_dtype"] != "bf16":
        keys += ["sfa", "sfb"]
    if problem["d_dtype"] == "e4m3":
        keys += ["norm_const"]
    if problem["act"] == "dswiglu":
        keys += ["beta", "c_in"]
    if problem["act"] in ("dsrelu", "dgeglu"):
        keys += ["c_in"]
    if discrete is not None:
        keys = [k for k in keys if k not in ("b", "sfb")]
        return {**{k: dev_arrays[k] for k in keys}, **discrete}
    return {k: dev_arrays[k] for k in keys}


def to_host(outputs: dict) -> dict:
    """Device outputs -> numpy (int16 bf16 bits come back as uint16)."""
    res = {}
    for k, t in outputs.items():
        a = t.detach().cpu().numpy()
        res[k] = a.view(np.uint16) if a.dtype == np.int16 else a
    return res
