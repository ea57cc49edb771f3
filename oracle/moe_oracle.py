"""CPU oracle for the affine-quantized mixture-of-experts FFN step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check in ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, helpers, tables or generators) and it
imports nothing from the package.

What it computes is the plain definition of the step, written out the slow
and obvious way: dequantize every weight fully to fp32, widen to fp64, and do
fp64 matrix-vector products, an fp64 softmax, an explicit top-K with ties
broken towards the lower expert index, SwiGLU, the down projection and the
weighted combine.  This is the "dequantize, then dense fp32/fp64 math"
arbiter that the MLX issue thread uses to judge ``gather_qmm`` (ml-explore/mlx
issue #3856, "Silent numerical corruption in single long forward on quantized
MoE ...", the minimal pure-mlx repro: ``mx.dequantize`` then a dense matmul),
and the CPU-only path that the flash-moe thread used as ground truth
(danveloper/flash-moe issue thread, "Definitive finding": the ``g_metal = NULL``
CPU path matched the MLX gate scores).

Sources, cited by page title and section:

* Affine group quantization, per-tensor bit width, codes packed along the
  input dimension into uint32 words: danveloper/flash-moe issue thread, the
  quantization-config excerpt (``group_size 64, bits 4, mode affine`` with
  8-bit overrides for ``mlp.gate`` and ``mlp.shared_expert_gate``) and the
  ``[512, 512] U32`` gate-shape remark (packed width x codes per word =
  in_dim).
* Dequantized weight = scale * code + bias: flash-moe-inference skill page,
  the ``matvec_4bit_fma`` kernel sketch (the naive form ``(nibble * scale +
  bias) * x`` and the fused ``fma(nibble, scale*x, bias*x)``).
* Router projection, softmax, top-K, per-expert fused gate/up, down,
  accumulate: markbaseengine MOE_ROUTER_WORKS_BREAKTHROUGH, "Forward Pass
  Sequence"; flash-moe-inference skill page, the per-layer pipeline listing
  (CMD2 routing, CPU softmax + topK, CMD3 expert forward + combine).
* SwiGLU ``g / (1 + exp(-g)) * up``: flash-moe-inference skill page, the
  ``swiglu`` kernel sketch.
* Shared expert scaled by a sigmoid gate, fused into the combine:
  flash-moe-inference skill page, ``moe_combine_residual`` ("MoE combine +
  residual + sigmoid gate"), and the 8-bit ``shared_expert_gate`` of the
  flash-moe quantization config.
* RMSNorm before the router, residual added in the combine:
  flash-moe-inference skill page, the per-layer pipeline listing (CMD2:
  o_proj, norm, routing; CMD3: expert forward, combine), the two-pass
  ``rms_norm_pass1/2`` kernel sketches (sum of squares, then scale) and
  ``moe_combine_residual``; danveloper/flash-moe issue thread, "Definitive
  finding" (the CMD2 chain o_proj -> residual_add -> rms_norm -> routing
  gate matvec).
* gather_qmm: row i computes ``x_i @ dequant(W[rhs_indices[i]])^T``
  (``transpose=True``): ml-explore/mlx issue #3856, minimal repro.
* Requantization of 4-bit experts to 2 bits: flash-moe-inference skill page,
  the setup steps (the 4-bit to 2-bit conversion of the packed experts) and
  the repository layout (``repack_experts_2bit.py``).  The page names the
  tool but not its arithmetic; the reading used is below in
  ``requant_2bit``.

The mxfp4 expert mode that the mlx issue thread runs beside affine
(``mode="mxfp4"``, group size 32, its repro table and the per-model list of
mxfp4 experts) is the OCP Microscaling format that mode names: 4-bit E2M1
elements (1 sign, 2 exponent, 1 mantissa bit, exponent bias 1) with one
E8M0 scale byte (a power of two, ``2**(e - 127)``, 255 = NaN) per 32
elements and no bias; the pages give no more than the mode's name.

Readings where the pages are silent (each is listed with its reason in the
design notes): codes sit low bits first inside a word; scales and biases are
bf16; the group parameter is the number of elements per group; renormalized
top-K weights ``p[idx] / sum(p[idx])``; ties go to the lower index; the
combine adds the K experts in slot order; the 2-bit requantization spans each
group's exact minimum to maximum in three equal steps.

Every function here is pinned by the CPU tests (``tests/test_oracle_*.py``)
against hand-packed words, closed forms, invariants and brute force with
exactly rounded sums; none is "parity unpinned".
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "bf16_bits_to_f32",
    "unpack_codes",
    "fp4_e2m1",
    "e8m0_scale",
    "dequantize",
    "expert_slice",
    "qmatvec",
    "softmax",
    "top_k",
    "route",
    "silu",
    "swiglu",
    "moe_experts",
    "moe_layer",
    "rms_norm",
    "moe_block",
    "gather_qmm",
    "bf16_round",
    "requant_2bit",
    "requant_2bit_fast",
    "expert_bytes",
]


# --------------------------------------------------------------------------
# Format: unpack and dequantize
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32.

    bf16 is the upper half of an IEEE float32, so the widening is exact: the
    16 bits move to the top of a 32-bit word and the low half is zero.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def unpack_codes(words, bits: int, cols: int) -> np.ndarray:
    """Unpack uint32 words into integer codes, one code per input column.

    Each word holds ``32 / bits`` codes.  Column ``k`` of a row lives in word
    ``k // (32 / bits)`` at bit offset ``bits * (k % (32 / bits))``: low bits
    first.  For 4-bit this is "8 nibbles per uint32", for 8-bit "4 bytes per
    uint32" (danveloper/flash-moe issue thread, the 8-bit gate diagnosis).
    """
    if bits not in (2, 4, 8):
        raise ValueError(f"bits must be 2, 4 or 8, got {bits}")
    w = np.asarray(words, dtype=np.uint32)
    per_word = 32 // bits
    if w.shape[-1] * per_word != cols:
        raise ValueError(
            f"packed width {w.shape[-1]} x {per_word} codes/word != cols {cols}")
    mask = np.uint32((1 << bits) - 1)
    shifts = np.arange(per_word, dtype=np.uint32) * np.uint32(bits)
    codes = (w[..., :, None] >> shifts) & mask          # [..., words, per_word]
    return codes.reshape(w.shape[:-1] + (cols,)).astype(np.uint8)


def fp4_e2m1(code) -> np.ndarray:
    """Value of 4-bit E2M1 codes: bit 3 the sign, bits 2-1 the exponent e
    (bias 1), bit 0 the mantissa m.  e = 0: m/2 (zero or one half);
    otherwise (1 + m/2) * 2**(e - 1).  So the magnitudes of codes 0..7 are
    0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def e8m0_scale(byte) -> np.ndarray:
    """Value of E8M0 scale bytes: ``2**(byte - 127)``, byte 255 is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def dequantize(qt: dict) -> np.ndarray:
    """Dequantize a quantized matrix (or a stack of them) to float32.

    Affine: ``w = scale * code + bias`` per group of ``group_size``
    consecutive input columns.  The product of a bf16 scale (8 significant
    bits) and a code of at most 8 bits is exact in float32, so the float32
    result is the single rounding of ``scale * code + bias``.

    mxfp4 (``qt["mode"] == "mxfp4"``): ``w = fp4_e2m1(code) * 2**(e - 127)``
    with the group's scale byte e, no bias; the product of a two-bit
    significand and a power of two is exact in float32 (down to its
    subnormals), so the float32 result is exact unless it overflows.
    """
    bits, gs, cols = int(qt["bits"]), int(qt["group_size"]), int(qt["cols"])
    if cols % gs:
        raise ValueError("cols must be a multiple of group_size")
    if qt.get("mode", "affine") == "mxfp4":
        if bits != 4 or gs != 32:
            raise ValueError("mxfp4 is 4-bit with groups of 32")
        codes = unpack_codes(qt["q"], 4, cols)
        sc = np.repeat(e8m0_scale(qt["scales"]), gs, axis=-1)
        if sc.shape != codes.shape:
            raise ValueError(f"scales shape {sc.shape} does not match codes {codes.shape}")
        with np.errstate(over="ignore", invalid="ignore"):
            return (fp4_e2m1(codes) * sc).astype(np.float32)
    codes = unpack_codes(qt["q"], bits, cols).astype(np.float32)
    s = np.repeat(bf16_bits_to_f32(qt["scales"]), gs, axis=-1)
    b = np.repeat(bf16_bits_to_f32(qt["biases"]), gs, axis=-1)
    if s.shape != codes.shape:
        raise ValueError(f"scales shape {s.shape} does not match codes {codes.shape}")
    prod = s * codes                                   # exact in float32
    return (prod + b).astype(np.float32)               # one rounding


def expert_slice(qt: dict, e: int) -> dict:
    """The quantized matrix of expert ``e`` out of a stacked ``[E, rows, ...]``
    tensor.  The arrays may be numpy arrays or lazy stacks indexable by ``e``."""
    out = dict(qt)
    out["q"] = qt["q"][e]
    out["scales"] = qt["scales"][e]
    if qt.get("biases") is not None:       # (mxfp4 tensors have none)
        out["biases"] = qt["biases"][e]
    return out


# --------------------------------------------------------------------------
# Quantized matrix-vector product
# --------------------------------------------------------------------------

def qmatvec(qt: dict, x) -> np.ndarray:
    """``y[m, r] = sum_k deq(W)[r, k] * x[m, k]`` in fp64.

    ``qt`` is one matrix ``[rows, cols]``; ``x`` is ``[M, cols]`` (fp32 or a
    widened bf16; both are exact in fp64).  Returns fp64 ``[M, rows]``.
    """
    w = dequantize(qt).astype(np.float64)
    x64 = np.asarray(x, dtype=np.float64)
    return x64 @ w.T


# --------------------------------------------------------------------------
# Routing: softmax, top-K, renormalization
# --------------------------------------------------------------------------

def softmax(logits) -> np.ndarray:
    """Row-wise softmax in fp64, max-subtracted."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def top_k(scores, k: int):
    """Explicit top-K: K rounds of "take the largest remaining score, the
    lowest index on ties, then remove it".

    Returns ``(idx int32 [M, k], values [M, k])`` in selection order, i.e.
    descending score with ties in ascending index.
    """
    s = np.array(scores, dtype=np.float64, copy=True)
    if s.ndim == 1:
        s = s[None, :]
    m, e = s.shape
    if not 1 <= k <= e:
        raise ValueError(f"top-k {k} outside [1, {e}]")
    idx = np.empty((m, k), dtype=np.int32)
    val = np.empty((m, k), dtype=np.float64)
    rows = np.arange(m)
    for j in range(k):
        a = np.argmax(s, axis=1)          # numpy returns the first maximum
        idx[:, j] = a
        val[:, j] = s[rows, a]
        s[rows, a] = -np.inf
    return idx, val


def route(logits, k: int, renorm: bool = True):
    """Softmax over all experts, explicit top-K, optional renormalization.

    Returns ``(idx int32 [M, K], w fp64 [M, K], p fp64 [M, E])``.  With
    ``renorm`` the weights are ``p[idx] / sum(p[idx])``.
    """
    p = softmax(logits)
    if p.ndim == 1:
        p = p[None, :]
    idx, pv = top_k(p, k)
    w = pv / pv.sum(axis=1, keepdims=True) if renorm else pv
    return idx, w, p


# --------------------------------------------------------------------------
# Expert FFN and combine
# --------------------------------------------------------------------------

def silu(g) -> np.ndarray:
    """``g / (1 + exp(-g))`` (the flash-moe ``swiglu`` kernel sketch)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(g, u) -> np.ndarray:
    return silu(g) * np.asarray(u, dtype=np.float64)


def _deq64(qt: dict, e: int | None = None) -> np.ndarray:
    return dequantize(qt if e is None else expert_slice(qt, e)).astype(np.float64)


def moe_experts(layer: dict, x, idx, w, residual=None) -> np.ndarray:
    """Expert part of the step for given routing.

    ``y[t] = sum_k w[t,k] * down_e(swiglu(gate_e x_t, up_e x_t))`` with
    ``e = idx[t,k]``, plus ``sigmoid(shared_expert_gate . x_t) * FFN_shared(x_t)``
    when the layer has a shared expert, plus ``residual[t]`` when given.

    The per-expert products run over all rows routed to that expert at once
    (fp64 matmuls), which is the same arithmetic per row as a loop over
    tokens.  The K expert outputs of a token are summed in slot order.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    idx = np.asarray(idx)
    w64 = np.asarray(w, dtype=np.float64)
    m, k = idx.shape
    hidden = int(layer["down"]["rows"])
    per_slot = np.zeros((m, k, hidden), dtype=np.float64)
    flat = idx.reshape(-1)
    for e in np.unique(flat):
        pairs = np.nonzero(flat == e)[0]
        toks, slots = pairs // k, pairs % k
        xe = x64[toks]
        g = xe @ _deq64(layer["gate"], int(e)).T
        u = xe @ _deq64(layer["up"], int(e)).T
        h = swiglu(g, u)
        per_slot[toks, slots] = h @ _deq64(layer["down"], int(e)).T
    y = np.zeros((m, hidden), dtype=np.float64)
    for j in range(k):                     # combine in slot order
        y += w64[:, j:j + 1] * per_slot[:, j]
    sh = layer.get("shared")
    if sh is not None:
        sg = qmatvec(sh["expert_gate"], x64)[:, 0]
        gate_scale = 1.0 / (1.0 + np.exp(-sg))
        g = x64 @ _deq64(sh["gate"]).T
        u = x64 @ _deq64(sh["up"]).T
        y_sh = swiglu(g, u) @ _deq64(sh["down"]).T
        y += gate_scale[:, None] * y_sh
    if residual is not None:
        y += np.asarray(residual, dtype=np.float64).reshape(m, hidden)
    return y


def moe_layer(layer: dict, x, k: int, renorm: bool = True, residual=None,
              logits=None):
    """The whole step: router logits (or given logits), route, experts.

    Returns ``(y, idx, w, logits)``.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    if logits is None:
        logits = qmatvec(layer["router"], x64)
    idx, w, _ = route(logits, k, renorm)
    y = moe_experts(layer, x64, idx, w, residual)
    return y, idx, w, np.asarray(logits, dtype=np.float64)


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """``x / sqrt(mean(x^2) + eps) * weight`` per row, in fp64.

    The two passes of the pages' ``rms_norm_pass1/2``: the mean of the
    squares over the row's H elements, then every element scaled by the
    reciprocal square root and by its own weight.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    g = np.asarray(weight, dtype=np.float64).reshape(-1)
    if g.shape[0] != x64.shape[1]:
        raise ValueError("norm weight length must equal the row length")
    ms = np.mean(x64 * x64, axis=1, keepdims=True)
    return x64 / np.sqrt(ms + float(eps)) * g[None, :]


def moe_block(layer: dict, x, norm_weight, eps: float, k: int, renorm: bool = True):
    """The MoE step with its neighbours fused: ``h = rms_norm(x)`` feeds the
    router and the experts, and the residual stream ``x`` itself is added
    in the combine: ``y = x + MoE(h)``.

    Returns ``(y, idx, w, h)``.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    h = rms_norm(x64, norm_weight, eps)
    y, idx, w, _ = moe_layer(layer, h, k, renorm, residual=x64)
    return y, idx, w, h

# --------------------------------------------------------------------------
# gather_qmm: one projection per row, weight matrix picked per row
# --------------------------------------------------------------------------

def gather_qmm(qt_stack: dict, x, rhs_idx) -> np.ndarray:
    """``out[i] = x[i] @ deq(W[rhs_idx[i]])^T`` in fp64 (``transpose=True``).

    ``x`` is ``[n, cols]``, ``rhs_idx`` is ``[n]``; the order of rows does not
    matter (sorted or not gives the same rows).
    """
    x64 = np.asarray(x, dtype=np.float64)
    ridx = np.asarray(rhs_idx).reshape(-1)
    out = np.zeros((x64.shape[0], int(qt_stack["rows"])), dtype=np.float64)
    for e in np.unique(ridx):
        rows = np.nonzero(ridx == e)[0]
        out[rows] = x64[rows] @ _deq64(qt_stack, int(e)).T
    return out


# --------------------------------------------------------------------------
# Requantization to 2 bits
# --------------------------------------------------------------------------

def bf16_round(v) -> int:
    """Bit pattern of the bf16 value nearest to the exact rational ``v``,
    ties to the even significand (IEEE round to nearest even at 8 significant
    bits).  Normal range only (ValueError outside it); zero maps to +0.
    """
    v = Fraction(v)
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < Fraction(2) ** e:          # now 2^e <= a < 2^(e+1)
        e -= 1
    m = round(a / Fraction(2) ** (e - 7))        # in [128, 256]; half to even
    if m == 256:
        m, e = 128, e + 1
    if not -126 <= e <= 127:
        raise ValueError(f"{float(v)!r} is outside bf16's normal range")
    return sign | ((e + 127) << 7) | (m - 128)


def _pack_2bit(codes) -> np.ndarray:
    """Pack 2-bit codes along the last axis, low bits first (16 per word)."""
    c = np.asarray(codes, dtype=np.uint32)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 16, 16))
    words = np.zeros(c.shape[:-1], dtype=np.uint32)
    for j in range(16):
        words |= c[..., j] << np.uint32(2 * j)
    return words


def requant_2bit(qt: dict) -> dict:
    """Requantize a 4- or 8-bit affine tensor to 2 bits, group by group, with
    the group size kept (flash-moe-inference skill page: the 4-bit to 2-bit
    conversion step and ``repack_experts_2bit.py``; the page gives no
    arithmetic, so this is the plainest reading of "requantize to 2 bits").

    For one group with scale ``s``, bias ``b`` and codes ``q_j`` the weights
    are the exact values ``w_j = s*q_j + b``.  With ``lo = min w_j`` and
    ``hi = max w_j`` the 2-bit grid is ``lo + k*step`` for k = 0..3 and
    ``step = (hi - lo) / 3``.  Each weight takes the nearest grid point, ties
    to the even k; a group with ``step == 0`` takes code 0.  The stored scale
    and bias are ``step`` and ``lo`` rounded to bf16 (nearest, ties to even).
    All of it is exact rational arithmetic; only the two stored values round.
    """
    bits, gs, cols = int(qt["bits"]), int(qt["group_size"]), int(qt["cols"])
    if bits not in (4, 8):
        raise ValueError("the source must be 4- or 8-bit")
    if gs not in (64, 128):
        raise ValueError("2-bit groups are 64 or 128 columns")
    codes = unpack_codes(qt["q"], bits, cols)
    lead = codes.shape[:-1]
    ng = cols // gs
    codes = codes.reshape(-1, ng, gs)
    s_in = bf16_bits_to_f32(qt["scales"]).reshape(-1, ng)
    b_in = bf16_bits_to_f32(qt["biases"]).reshape(-1, ng)
    q2 = np.zeros(codes.shape, dtype=np.uint8)
    s2 = np.zeros(s_in.shape, dtype=np.uint16)
    b2 = np.zeros(b_in.shape, dtype=np.uint16)
    for r in range(codes.shape[0]):
        for g in range(ng):
            s, b = Fraction(float(s_in[r, g])), Fraction(float(b_in[r, g]))
            w = [s * int(c) + b for c in codes[r, g]]
            lo, hi = min(w), max(w)
            step = (hi - lo) / 3
            s2[r, g] = bf16_round(step)
            b2[r, g] = bf16_round(lo)
            if step != 0:
                q2[r, g] = [round((wj - lo) / step) for wj in w]
    return {"q": _pack_2bit(q2.reshape(lead + (cols,))),
            "scales": s2.reshape(lead + (ng,)), "biases": b2.reshape(lead + (ng,)),
            "batch": qt.get("batch", 1), "rows": qt["rows"], "cols": cols, "bits": 2,
            "group_size": gs}


def _bf16_bits_of_exact_f64(v) -> np.ndarray:
    """bf16 bit patterns of fp64 values that hold exact results, each rounded
    once to 8 significant bits (nearest, ties to even) from its full fp64
    significand; zero maps to +0 and anything that would leave bf16's normal
    range raises, as in ``bf16_round``."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    u = v.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = ((u + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)) << np.uint64(45)
    rv = r.view(np.float64)
    ra = np.abs(rv)
    nz = v != 0
    if np.any(nz & ((ra < 2.0 ** -126) | (ra > float(np.float32(3.3895314e38))))):
        raise ValueError("a value is outside bf16's normal range")
    bits = (rv.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(nz, bits, np.uint16(0))


def requant_2bit_fast(qt: dict) -> dict:
    """``requant_2bit`` with the same results, reached by integer arithmetic
    on the codes so it can run over whole expert stacks.

    In one group the weights are ``w_j = s*q_j + b``.  For ``s > 0`` the
    smallest weight belongs to the smallest code and for ``s < 0`` to the
    largest; call that code ``q_lo`` and ``D = q_max - q_min``.  Then
    ``lo = s*q_lo + b``, ``step = |s|*D/3`` and the position of ``w_j`` on the
    grid is ``(w_j - lo)/step = 3*|q_j - q_lo|/D``: a ratio of small integers,
    rounded to the nearest integer with ties to even.  A group with ``s == 0``
    or ``D == 0`` has no spread and takes code 0.  The stored scale is
    ``|s|*D/3`` and the stored bias ``lo``, each rounded once to bf16: ``|s|*D``
    and ``s*q_lo`` are exact in fp64 (at most 16 significant bits), the
    division by three is rounded once in fp64 and its binary expansion never
    falls on a bf16 tie; the sum ``s*q_lo + b`` is checked to be exact in fp64
    and any group where it is not is rounded from the exact rational with
    ``bf16_round``.
    """
    bits, gs, cols = int(qt["bits"]), int(qt["group_size"]), int(qt["cols"])
    if bits not in (4, 8):
        raise ValueError("the source must be 4- or 8-bit")
    if gs not in (64, 128):
        raise ValueError("2-bit groups are 64 or 128 columns")
    codes = unpack_codes(qt["q"], bits, cols)
    lead = codes.shape[:-1]
    ng = cols // gs
    codes = codes.reshape(-1, ng, gs).astype(np.int32)
    s_in = bf16_bits_to_f32(qt["scales"]).reshape(-1, ng).astype(np.float64)
    b_in = bf16_bits_to_f32(qt["biases"]).reshape(-1, ng).astype(np.float64)
    qmin = codes.min(axis=-1)
    qmax = codes.max(axis=-1)
    D = qmax - qmin
    q_lo = np.where(s_in < 0, qmax, qmin)
    flat = (s_in == 0) | (D == 0)
    Dd = np.where(D == 0, 1, D)[..., None]
    twice = 6 * np.abs(codes - q_lo[..., None]) + Dd    # 2 * (3 d / D + 1/2) * D
    k = twice // (2 * Dd)                                # round half up ...
    tie = twice % (2 * Dd) == 0
    k = np.where(tie & (k % 2 == 1), k - 1, k)          # ... then ties to even
    k = np.where(flat[..., None], 0, k).astype(np.uint8)
    step = np.abs(s_in) * D / 3.0
    prod = s_in * q_lo
    lo = prod + b_in
    bp = lo - prod                                       # two-sum: lo is exact iff err == 0
    err = (prod - (lo - bp)) + (b_in - bp)
    lo = lo + 0.0                                        # -0 -> +0, as the exact rational
    s2 = _bf16_bits_of_exact_f64(step)
    b2 = _bf16_bits_of_exact_f64(np.where(err == 0, lo, 0.0))
    for r, g in zip(*np.nonzero(err != 0)):
        b2[r, g] = bf16_round(Fraction(float(s_in[r, g])) * int(q_lo[r, g]) + Fraction(float(b_in[r, g])))
    return {"q": _pack_2bit(k.reshape(lead + (cols,))),
            "scales": s2.reshape(lead + (ng,)), "biases": b2.reshape(lead + (ng,)),
            "batch": qt.get("batch", 1), "rows": qt["rows"], "cols": cols, "bits": 2,
            "group_size": gs}


# --------------------------------------------------------------------------
# Byte accounting
# --------------------------------------------------------------------------

def expert_bytes(hidden: int, inter: int, bits: int, group_size: int = 64,
                 scale_bytes: int = 2) -> int:
    """Bytes of one expert (gate, up: ``[inter, hidden]``; down:
    ``[hidden, inter]``): packed codes plus one scale and one bias per group.
    """
    n = 3 * hidden * inter
    return n * bits // 8 + 2 * scale_bytes * (n // group_size)
