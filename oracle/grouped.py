"""Plain fp64 CPU oracle of the contiguous grouped block-scaled GEMM + epilogue.

TEST INFRASTRUCTURE ONLY.  See ``oracle/__init__.py``.

The method computes exactly (up to rounding order) a result with a plain
definition, so this module is that definition written out, step by step, in
float64, with numpy's matmul as the only library primitive:

1. dequantise A and B (block scale per 32 K-elements) -- "Grouped GEMM + Quant
   (SM100)", §Equations, Step 1 (the dequantize() of A with SFA and of B with
   SFB) and §Data Types (MXFP8 / FP4 formats, sf_vec_size 32, E8M0 scales);
2. rows m in [padded_offsets[g-1], padded_offsets[g]) use expert g's weight
   B[:, :, g] -- same page, §Equations, Step 1;
3. per-group scale: C = alpha_g * sum_k a*b ("Grouped GEMM + SwiGLU (SM100)",
   §Equations, Step 1); for the dSwiGLU backward R = alpha_g^2 * sum_k a*b
   ("Grouped GEMM + dGLU (SM100)", BF16 contract, equation for R_g);
4. the activation and gating epilogue (each function below cites its page);
5. output formatting: BF16 rounding of C / D / dC, per-group amax, or FP8 row
   and column quantisation with E8M0 scale factors ("Grouped GEMM + Quant
   (SM100)", §Equations, Step 3).

Readings taken where the pages leave a step open (each is listed, with its
reason, in the design notes of the repository):

* SwiGLU / dSwiGLU block order: in each pair of consecutive 32-column blocks
  the first is the linear/input block X and the second the gate block G (the
  SwiGLU page's Step 2 and its diagram [X0|G0|X1|G1|...]; the dGLU page's
  "interleaved input/gate" C and its [ab, dswiglu] = [d_input, d_gate] order).
* E8M0 scale of an output block: the smallest power of two 2^e with
  2^e >= norm_const * amax * rcp_max, byte e+127 clamped to [0, 254]; an
  all-zero block gets byte 0 and zero codes.
* FP8 elements: D * norm_const / 2^e rounded to nearest even E4M3, saturating
  at 448.
* The quantisation *decisions* (amax, scale byte, element code) are taken in
  float32, the precision the sReLU page states the epilogue is evaluated in:
  the fp64 D is rounded once to float32 and every later step is a float32
  operation in the order written above.
* sReLU tanh clamp: t = tanh(relu(C)/s) capped at 1, c = s*t, D = prob*c^2.
* amax is the max |D| (before any output rounding) over the group's rows and
  all output columns; an empty group reports 0.
* sReLU backward: R = alpha_g^2 * acc as for dSwiGLU, the saved forward C is
  read without a beta scale, and dC / dprob follow from the forward equation
  (see dsrelu); with MX operands its dC is formatted like a forward D (bf16 +
  per-group amax of shape (L), or FP8 rows and columns).
* GeGLU (forward) and dGeGLU (backward): blocks in the order the pages give
  for them, gate first ([G_b | U_b], [dgate_b | dup_b]); the forward's clamp
  applies [glu_clamp_min, glu_clamp_max] to both halves, the backward's to the
  gate from above and to up on both sides, as the dGLU page states.
* Block-scaled dSwiGLU with a BF16 dC reports amax of shape (L, 2) (the dGLU
  page's block-scaled outputs): entry 0 is max |d_input| over the group's
  rows and its input blocks, entry 1 max |d_gate| over its gate blocks.  With
  an FP8 dC, dC is quantised by rows and columns exactly like a forward D.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

RCP_MAX_E4M3 = np.float32(1.0) / np.float32(F.E4M3_MAX)   # rcp_max = 1/q_max, in float32


# ---------------------------------------------------------------------------
# step 1: dequantisation
# ---------------------------------------------------------------------------

def dequantize(codes, scales, ab_dtype: str) -> np.ndarray:
    """value[r, k] = dec(code[r, k]) * 2^(scale[r, k // 32] - 127), in float64.

    BF16 operands carry no scales and are decoded as they are.
    """
    if ab_dtype == "bf16":
        return F.decode_bf16(codes)
    if ab_dtype == "e4m3":
        elem = F.decode_e4m3(codes)
    elif ab_dtype == "e5m2":
        elem = F.decode_e5m2(codes)
    elif ab_dtype == "e2m1x2":
        elem = F.decode_e2m1(F.unpack_e2m1x2(codes))
    else:
        raise ValueError(ab_dtype)
    sf = F.decode_e8m0(scales)
    return elem * np.repeat(sf, 32, axis=-1)


# ---------------------------------------------------------------------------
# step 2: row -> expert
# ---------------------------------------------------------------------------

def group_of_rows(padded_offsets, rows) -> np.ndarray:
    """Expert g owns rows [padded_offsets[g-1], padded_offsets[g]); -1 if none."""
    rows = np.asarray(rows)
    grp = np.full(rows.shape, -1, dtype=np.int64)
    lo = 0
    for g, hi in enumerate(np.asarray(padded_offsets).tolist()):
        grp[(rows >= lo) & (rows < hi)] = g
        lo = hi
    return grp


# ---------------------------------------------------------------------------
# step 4: activations (float64)
# ---------------------------------------------------------------------------

def sigmoid(t):
    with np.errstate(over="ignore"):          # exp(-t) = inf for t << 0 gives 0 exactly
        return 1.0 / (1.0 + np.exp(-t))


def swiglu(c, prob):
    """D[:, bG:(b+1)G] = prob * X_b * swish(G_b), G = 32, swish(x) = x*sigmoid(x).

    "Grouped GEMM + SwiGLU (SM100)", §Equations, Step 2: X_b is the first and
    G_b the second 32-column block of pair b.
    """
    r, n = c.shape
    pairs = c.reshape(r, n // 64, 2, 32)
    x, g = pairs[:, :, 0, :], pairs[:, :, 1, :]
    d = prob[:, None, None] * x * (g * sigmoid(g))
    return d.reshape(r, n // 2)


def srelu(c, prob, s: float):
    """D = prob * relu(C)^2, or with the tanh soft clamp s > 0:
    D = prob * (s * min(tanh(relu(C)/s), 1))^2.

    "Grouped GEMM + sReLU (SM100)", §Equations and §Tanh soft clamp.
    """
    r = np.maximum(c, 0.0)
    if s > 0:
        r = s * np.minimum(np.tanh(r / s), 1.0)
    return prob[:, None] * (r * r)


def dswiglu(rmat, x_saved, prob):
    """dSwiGLU backward over interleaved 32-column blocks.

    "Grouped GEMM + dGLU (SM100)", BF16 contract equations and block-scaled
    Step 2: with R the scaled GEMM gradient (width N) and X = beta*C the saved
    forward pre-activation (width 2N, blocks [input_b | gate_b]), s = sigmoid(gate):
      d_input = R * prob * gate * s
      d_gate  = R * prob * input * s * (1 + gate * (1 - s))
      dprob   = sum over all N columns of R * input * gate * s
    and [d_input_b | d_gate_b] are stored interleaved like X.
    """
    r, n = rmat.shape
    xs = x_saved.reshape(r, n // 32, 2, 32)
    inp, gate = xs[:, :, 0, :], xs[:, :, 1, :]
    rr = rmat.reshape(r, n // 32, 32)
    s = sigmoid(gate)
    p = prob[:, None, None]
    d_in = rr * p * (gate * s)
    d_gate = rr * p * inp * s * (1.0 + gate * (1.0 - s))
    dc = np.stack([d_in, d_gate], axis=2).reshape(r, 2 * n)
    dprob = (rr * inp * gate * s).reshape(r, n).sum(axis=1)
    return dc, dprob


def glu_params(problem: dict):
    """GeGLU / dGeGLU constants of a problem: (gamma, alpha, offset, clamp_min,
    clamp_max); the pages' defaults are gamma 1, alpha 1.702, offset 1 and, for
    the backward, clamps -7 / 7."""
    return (float(problem.get("glu_gamma", 1.0)), float(problem.get("geglu_alpha", 1.702)),
            float(problem.get("linear_offset", 1.0)), float(problem.get("glu_clamp_min", -np.inf)),
            float(problem.get("glu_clamp_max", np.inf)))


def geglu(c, prob, gamma, alpha, offset, cmin, cmax):
    """GeGLU over pairs [G_b | U_b] of 32 columns, gate first ("Grouped GEMM +
    GLU + Hadamard", §Equations, GeGLU): both halves clamped to [cmin, cmax]
    (the page's glu_limit) before the activation,
      D_b = gamma * prob * (U_b + offset) * G_b * sigmoid(alpha * G_b)
    (the page's constants: alpha 1.702, offset 1)."""
    r, n = c.shape
    cs = c.reshape(r, n // 64, 2, 32)
    g = np.clip(cs[:, :, 0, :], cmin, cmax)
    u = np.clip(cs[:, :, 1, :], cmin, cmax)
    d = gamma * prob[:, None, None] * (u + offset) * g * sigmoid(alpha * g)
    return d.reshape(r, n // 2)


def dgeglu(rmat, c_saved, prob, alpha, offset, cmin, cmax):
    """dGeGLU backward ("Grouped GEMM + dGLU (SM100)", dGeGLU equations of the
    BF16 and block-scaled contracts): saved C in pairs [gate_b | up_b] (the
    page's [dgate, dup] output order), gate clamped above only, up on both
    sides, masks from the unclamped values (gradient kept at equality):
      dgate = R prob (up_c + offset) s (1 + alpha gate_c (1 - s)) [gate <= cmax]
      dup   = R prob gate_c s [cmin <= up <= cmax]
      dprob = sum R gate_c s (up_c + offset),  s = sigmoid(alpha gate_c)
    """
    r, n = rmat.shape
    xs = c_saved.reshape(r, n // 32, 2, 32)
    gate, up = xs[:, :, 0, :], xs[:, :, 1, :]
    gc = np.minimum(gate, cmax)
    uc = np.clip(up, cmin, cmax)
    s = sigmoid(alpha * gc)
    rr = rmat.reshape(r, n // 32, 32)
    p = prob[:, None, None]
    dgate = rr * p * (uc + offset) * s * (1.0 + alpha * gc * (1.0 - s)) * (gate <= cmax)
    dup = rr * p * gc * s * ((cmin <= up) & (up <= cmax))
    dc = np.stack([dgate, dup], axis=2).reshape(r, 2 * n)
    dprob = (rr * gc * s * (uc + offset)).reshape(r, n).sum(axis=1)
    return dc, dprob


def dsrelu(rmat, c_saved, prob, s: float):
    """sReLU backward (the pair of "Grouped GEMM + sReLU (SM100)"; its own page
    is not among the sources, so the derivative is taken from the forward's
    §Equations / §Tanh soft clamp): with f(C) = (s * tanh(relu(C)/s))^2
    (relu(C)^2 for s = 0) and the forward D = prob * f(C),
      dC    = R * prob * f'(C),  f'(C) = 2 c (1 - t^2) = 2 c sech^2(C/s) for C > 0
              (t = tanh(C/s), c = s t; sech^2 evaluated directly, free of the
              cancellation of 1 - t^2 as t -> 1), 2 relu(C) for s = 0, 0 for C <= 0
      dprob = sum over the N columns of R * f(C)
    """
    r = np.maximum(c_saved, 0.0)
    if s > 0:
        t = np.minimum(np.tanh(r / s), 1.0)
        c = s * t
        # 1 - t^2 = sech^2(r/s), the derivative of tanh, evaluated as such:
        # written as 1 - t*t it cancels to nothing once t rounds to 1
        with np.errstate(over="ignore"):
            fprime = 2.0 * c / np.cosh(r / s) ** 2
    else:
        c = r
        fprime = 2.0 * r
    dc = rmat * prob[:, None] * fprime
    dprob = (rmat * (c * c)).sum(axis=1)
    return dc, dprob


# ---------------------------------------------------------------------------
# step 5: FP8 quantisation with E8M0 block scales (float32 decisions)
# ---------------------------------------------------------------------------

def e8m0_block_scale(amax32, nc32):
    """Byte of the smallest 2^e >= (nc*amax)*rcp_max (float32 products), clamped
    to [0, 254]; 0 for an all-zero block.

    "Grouped GEMM + Quant (SM100)", §Equations, Step 3: SFD = norm_const *
    max|D| * rcp_max, stored as the E8M0 type of SFA.
    """
    amax32 = np.asarray(amax32, dtype=np.float32)
    sf = (np.float32(nc32) * amax32) * RCP_MAX_E4M3
    mant, ex = np.frexp(sf)                       # exact: sf = mant * 2^ex
    e = np.where(mant == 0.5, ex - 1, ex)         # ceil(log2 sf)
    byte = np.clip(e.astype(np.int64) + 127, 0, 254)
    return np.where(sf > 0, byte, 0).astype(np.uint8)


def quantize_block_values(d32, byte, nc32):
    """E4M3 codes of D * norm_const / 2^(byte-127), evaluated in float32.

    "Grouped GEMM + Quant (SM100)", §Equations, Step 3 (D_quantized).
    """
    d32 = np.asarray(d32, dtype=np.float32)
    prod = d32 * np.float32(nc32)                                  # float32
    scaled = np.ldexp(prod, (127 - byte.astype(np.int32)))         # exact power-of-two scaling
    return F.encode_e4m3(scaled.astype(np.float32))


def quantize_rows(d64, nc: float):
    """Row blocks: 32 consecutive output columns of one row."""
    d32 = d64.astype(np.float32)
    r, n = d32.shape
    blk = d32.reshape(r, n // 32, 32)
    byte = e8m0_block_scale(np.abs(blk).max(axis=2), nc)
    codes = quantize_block_values(blk, byte[:, :, None], nc)
    return codes.reshape(r, n), byte


def quantize_cols(d64, nc: float):
    """Column blocks: 32 consecutive rows of one output column.

    Input rows must be whole 32-row blocks.  Returns codes in the same
    (rows, N_out) layout as D and scale bytes as (N_out, rows/32).
    """
    d32 = d64.astype(np.float32)
    r, n = d32.shape
    blk = d32.reshape(r // 32, 32, n)
    byte = e8m0_block_scale(np.abs(blk).max(axis=1), nc)          # (r/32, n)
    codes = quantize_block_values(blk, byte[:, None, :], nc)
    return codes.reshape(r, n), byte.T.copy()


# ---------------------------------------------------------------------------
# the whole path
# ---------------------------------------------------------------------------

def grouped_gemm(problem: dict, arrays: dict, rows=None) -> dict:
    """Evaluate the grouped GEMM + epilogue for the given rows (default: all).

    ``problem`` keys: num_groups, valid_m, n, k, ab_dtype ('e4m3', 'e2m1x2',
    'bf16'), c_dtype (None or 'bf16'), d_dtype ('bf16' or 'e4m3'), act
    ('none', 'swiglu', 'srelu', 'dswiglu'), srelu_tanh_s.
    ``arrays`` holds the host inputs in the library's logical layouts.

    Returns float64 intermediates ('acc', 'c', 'd' or 'dc', 'dprob') and the
    formatted outputs: 'c_bits' (bf16), 'd_bits' (bf16) + 'amax', or
    'd_code', 'sfd_row' and (when rows are whole 32-row blocks) 'd_col_code',
    'sfd_col', 'col_blocks'.  With a row subset, 'amax' covers those rows only.
    """
    L, valid_m = int(problem["num_groups"]), int(problem["valid_m"])
    n, k = int(problem["n"]), int(problem["k"])
    ab, act = problem["ab_dtype"], problem["act"]
    po = np.asarray(arrays["padded_offsets"])
    rows = np.arange(valid_m) if rows is None else np.asarray(rows, dtype=np.int64)
    grp = group_of_rows(po, rows)
    if (grp < 0).any():
        raise ValueError("row outside every group")

    # steps 1-3: dequantise, per-expert GEMM in float64, per-group scale
    a = dequantize(arrays["a"][rows], None if ab == "bf16" else arrays["sfa"][rows], ab)
    acc = np.zeros((len(rows), n), dtype=np.float64)
    for g in np.unique(grp):
        b_g = dequantize(arrays["b"][g], None if ab == "bf16" else arrays["sfb"][g], ab)
        sel = grp == g
        acc[sel] = a[sel] @ b_g.T
    alpha = np.asarray(arrays["alpha"], dtype=np.float64)[grp]
    prob = np.asarray(arrays["prob"], dtype=np.float64)[rows]
    out = {"rows": rows, "group": grp, "acc": acc}

    if act in ("dswiglu", "dsrelu", "dgeglu"):
        # "Grouped GEMM + dGLU (SM100)": R_g = alpha_g^2 A_g B_g^T (BF16 contract;
        # block-scaled Step 1 with dequantised A, B), then Step 2; the sReLU
        # backward takes the same R and the saved forward C as it is
        rmat = (alpha ** 2)[:, None] * acc
        if act == "dswiglu":
            beta = np.asarray(arrays["beta"], dtype=np.float64)[grp]
            x_saved = beta[:, None] * F.decode_bf16(arrays["c_in"][rows])
            dc, dprob = dswiglu(rmat, x_saved, prob)
        elif act == "dsrelu":
            dc, dprob = dsrelu(rmat, F.decode_bf16(arrays["c_in"][rows]), prob,
                               float(problem.get("srelu_tanh_s", 0.0)))
        else:
            _, ga, off, cmin, cmax = glu_params(problem)
            dc, dprob = dgeglu(rmat, F.decode_bf16(arrays["c_in"][rows]), prob, ga, off, cmin, cmax)
        out.update(r=rmat, dc=dc, dprob=dprob, dc_bits=F.encode_bf16(dc))
        if ab == "bf16":
            return out
        # block-scaled backend: output formatting of dC (Step 3)
        d = dc
        if act in ("dswiglu", "dgeglu") and problem["d_dtype"] == "bf16":
            halves = np.abs(dc).reshape(len(rows), -1, 2, 32)
            amax2 = np.zeros((L, 2), dtype=np.float64)
            for g in np.unique(grp):
                sel = halves[grp == g]
                if sel.size:
                    amax2[g] = sel.max(axis=(0, 1, 3))
            out["amax2"] = amax2
            return out
        out["d"] = d
    else:
        c = alpha[:, None] * acc
        out["c"] = c
        if problem.get("c_dtype") == "bf16":
            out["c_bits"] = F.encode_bf16(c)
        if act == "none":
            d = prob[:, None] * c
        elif act == "swiglu":
            d = swiglu(c, prob)
        elif act == "srelu":
            d = srelu(c, prob, float(problem.get("srelu_tanh_s", 0.0)))
        elif act == "geglu":
            gm, ga, off, cmin, cmax = glu_params(problem)
            d = geglu(c, prob, gm, ga, off, cmin, cmax)
        else:
            raise ValueError(act)
        out["d"] = d

    if problem["d_dtype"] == "bf16":
        out["d_bits"] = F.encode_bf16(d)
        amax = np.zeros(L, dtype=np.float64)
        absd = np.abs(d).max(axis=1) if d.shape[1] else np.zeros(len(rows))
        for g in np.unique(grp):
            amax[g] = absd[grp == g].max()
        out["amax"] = amax
    elif problem["d_dtype"] == "e4m3":
        nc = float(np.asarray(arrays["norm_const"]).reshape(-1)[0])
        out["d_code"], out["sfd_row"] = quantize_rows(d, nc)
        whole = (len(rows) % 32 == 0 and
                 np.all(rows.reshape(-1, 32) == rows.reshape(-1, 32)[:, :1] + np.arange(32)) and
                 np.all(rows.reshape(-1, 32)[:, 0] % 32 == 0)) if len(rows) else False
        if whole:
            out["d_col_code"], out["sfd_col"] = quantize_cols(d, nc)
            out["col_blocks"] = rows.reshape(-1, 32)[:, 0] // 32
    else:
        raise ValueError(problem["d_dtype"])
    return out
