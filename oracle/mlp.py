"""Routed-experts SwiGLU MLP with MXFP8 GEMM operands (oracle; test infrastructure).

What is computed, and where it comes from:

* torchtitan PR #12 "Wire the fully-fused grouped-GEMM MXFP8 plan behind
  fusion_plan", section "What it adds": the whole routed-experts MLP runs as
  four ops -- (1) FC1 grouped GEMM + SwiGLU + dual MXFP8 quantization, (2) FC2
  GEMM, (3) fused dSwiGLU backward, (4) wgrad -- over a padded expert-major
  token layout (per-expert segments aligned to pad_multiple 256; the default
  "swiglu" plan uses 128). Parameters stay stock (w1, w3 [E, F, D], w2
  [E, D, F]); the forward packs w1/w3 into a [E, 2F, D] "32-block order".
  Section "Evidence": zero-token experts get exact-zero weight gradients and a
  backward with zero routed tokens works.
* torchtitan PR #2 "[mxfp8 training] fused gated-activation (SwiGLU) + MXFP8
  quantization kernel override", section "Summary": w13 GEMM -> fused SwiGLU +
  dual MXFP8 quantization -> w2 GEMM, never materialising the BF16
  post-activation; section "Numerics and tests": the fused forward is bitwise
  equal to standalone-cast quantization.

Readings of points the pages leave open:

* 32-block order: W13[e, 64j + i] = w1[e, 32j + i], W13[e, 64j + 32 + i] =
  w3[e, 32j + i] for i < 32 -- 32 gate rows then 32 up rows, alternating.
* w1 is the gate (SiLU applied), w3 the up projection: y = w2(silu(w1 x) * w3 x).
* Every GEMM contracts two MXFP8 operands whose 32-groups lie along the
  contraction axis, accumulating exactly (fp64 here).
* Rounding points: the FC1 output is rounded to BF16 (g, u; the tensor saved
  for backward), h = BF16(silu(g) * u) is then quantized in both directions; in
  backward dh = BF16(dY W2) and dG, dU are each rounded to BF16 before the dual
  quantization of dH13 = pack(dG, dU). With these points the fused epilogue is
  by construction equal to the standalone quantizer applied to the BF16 tensor
  it never stores, which is what "bitwise forward parity" requires.
* Straight-through backward: quantization is the identity in the chain rule.
* Pad rows (inside a segment, after the expert's real rows) are read as zero;
  rows at or after offs[E] are neither read nor written.
"""
import numpy as np

from .formats import bf16_bits_to_f64, bf16_round, f64_to_bf16_bits
from .mx import BLOCK, dequantize_rowwise, quantize_colwise, quantize_rowwise


# --------------------------------------------------------------------------- packing

def pack_w13(w1, w3):
    """[E, F, D] gate and up weights -> [E, 2F, D] in 32-block order (any dtype)."""
    w1 = np.asarray(w1)
    w3 = np.asarray(w3)
    e, f, d = w1.shape
    assert w3.shape == w1.shape and f % BLOCK == 0
    out = np.empty((e, 2 * f, d), dtype=w1.dtype)
    v = out.reshape(e, f // BLOCK, 2, BLOCK, d)
    v[:, :, 0] = w1.reshape(e, f // BLOCK, BLOCK, d)
    v[:, :, 1] = w3.reshape(e, f // BLOCK, BLOCK, d)
    return out


def unpack_w13(w13):
    """Inverse of pack_w13: [E, 2F, D] -> (w1, w3), each [E, F, D]."""
    w13 = np.asarray(w13)
    e, f2, d = w13.shape
    f = f2 // 2
    v = w13.reshape(e, f // BLOCK, 2, BLOCK, d)
    return v[:, :, 0].reshape(e, f, d).copy(), v[:, :, 1].reshape(e, f, d).copy()


def split_gu(h13):
    """Packed FC1 output [M, 2F] -> (g, u), each [M, F]; same 32-block order."""
    m, f2 = h13.shape
    f = f2 // 2
    v = h13.reshape(m, f // BLOCK, 2, BLOCK)
    return v[:, :, 0].reshape(m, f), v[:, :, 1].reshape(m, f)


def join_gu(g, u):
    """(g, u) [M, F] -> packed [M, 2F] (inverse of split_gu)."""
    m, f = g.shape
    out = np.empty((m, 2 * f), dtype=g.dtype)
    v = out.reshape(m, f // BLOCK, 2, BLOCK)
    v[:, :, 0] = g.reshape(m, f // BLOCK, BLOCK)
    v[:, :, 1] = u.reshape(m, f // BLOCK, BLOCK)
    return out


# --------------------------------------------------------------------------- SwiGLU

def sigmoid(g):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def swiglu(g, u):
    """silu(g) * u = g * sigmoid(g) * u, fp64."""
    return g * sigmoid(g) * u


def dswiglu(dh, g, u):
    """Gradients of h = silu(g) * u: returns (dG, dU), fp64.

    d silu / dg = s * (1 + g * (1 - s)) with s = sigmoid(g).
    """
    s = sigmoid(g)
    return dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s


# --------------------------------------------------------------------------- layout

def segments(offs):
    """Expert e owns rows [offs[e], offs[e+1])."""
    offs = [int(o) for o in offs]
    return [(offs[e], offs[e + 1]) for e in range(len(offs) - 1)]


def real_rows_mask(offs, counts, m):
    """Boolean [m]: True for rows that carry a routed token (not pad)."""
    mask = np.zeros(m, dtype=bool)
    for e, (a, b) in enumerate(segments(offs)):
        c = (b - a) if counts is None else int(counts[e])
        mask[a:a + c] = True
    return mask


def check_offsets(offs, counts, pad_multiple, m_capacity):
    """True when offs/counts describe a padded expert-major layout.

    torchtitan PR #12, section "What it adds": every expert's token segment is
    hard-aligned to pad_multiple. Written out: offs[0] = 0; offs never
    decreases (a zero-token expert has an empty segment); every offs[e] is a
    multiple of pad_multiple; the layout fits the allocation (offs[E] <=
    m_capacity); and counts[e], when given, lies in [0, offs[e+1] - offs[e]]
    (the real rows precede the pad rows of the segment). Both arrays are read
    as signed integers.
    """
    offs = np.asarray(offs, dtype=np.int64)
    if offs[0] != 0 or np.any(np.diff(offs) < 0) or offs[-1] > m_capacity:
        return False
    if np.any(offs % pad_multiple != 0):
        return False
    if counts is not None:
        counts = np.asarray(counts, dtype=np.int64)
        if np.any(counts < 0) or np.any(counts > np.diff(offs)):
            return False
    return True


# --------------------------------------------------------------------------- quantization policy

class MX:
    """MXFP8 operands and BF16 rounding points (the method)."""
    exact = False

    @staticmethod
    def row(a):
        q, s = quantize_rowwise(a)
        return q, s, dequantize_rowwise(q, s)

    @staticmethod
    def col(a):
        q, s = quantize_colwise(a)
        return q, s, dequantize_rowwise(q, s)

    @staticmethod
    def bf16(x):
        return bf16_round(x)


class Exact:
    """Identity quantization and no rounding: the fp64 function the method approximates."""
    exact = True

    @staticmethod
    def row(a):
        return None, None, np.asarray(a, dtype=np.float64)

    @staticmethod
    def col(a):
        return None, None, np.asarray(a, dtype=np.float64).T.copy()

    @staticmethod
    def bf16(x):
        return x


def _slice_cols(deq_c, a, b):
    return deq_c[:, a:b]


# --------------------------------------------------------------------------- forward / backward

def quantize_weights(w1, w3, w2, policy=MX):
    """FC1/FC2 weight operands in both directions.

    w1, w3 [E, F, D] and w2 [E, D, F] fp64. Returns a dict with, per expert:
      w13q_r/s_r [2F, D]/[2F, D/32] (groups along D, for FC1 forward),
      w13q_c/s_c [D, 2F]/[D, 2F/32] (groups along 2F, for FC1 dgrad),
      w2q_r/s_r  [D, F]/[D, F/32]   (groups along F, for FC2 forward),
      w2q_c/s_c  [F, D]/[F, D/32]   (groups along D, for FC2 dgrad),
    and the dequantized operands w13_r, w13_c, w2_r, w2_c.
    """
    w13 = pack_w13(w1, w3)
    out = {k: [] for k in ("w13q_r", "w13s_r", "w13_r", "w13q_c", "w13s_c", "w13_c",
                           "w2q_r", "w2s_r", "w2_r", "w2q_c", "w2s_c", "w2_c")}
    for e in range(w13.shape[0]):
        for name, mat in (("w13", w13[e]), ("w2", w2[e])):
            q, s, dq = policy.row(mat)
            out[name + "q_r"].append(q)
            out[name + "s_r"].append(s)
            out[name + "_r"].append(dq)
            q, s, dq = policy.col(mat)
            out[name + "q_c"].append(q)
            out[name + "s_c"].append(s)
            out[name + "_c"].append(dq)
    if not policy.exact:
        for k in out:
            out[k] = np.stack(out[k])
    return out


def mlp_forward(x, w1, w3, w2, offs, counts=None, policy=MX):
    """Forward of the routed-experts MLP.

    x [>= offs[E], D] fp64 (rows past offs[E] ignored); w1, w3 [E, F, D], w2
    [E, D, F] fp64; offs [E+1]; counts [E] real rows per expert or None.
    Returns a dict holding every intermediate the GPU path exposes (codes,
    scales, the saved BF16 FC1 output h13, y).
    """
    offs = [int(o) for o in offs]
    m = offs[-1]
    d = w1.shape[2]
    f = w1.shape[1]
    xin = np.array(x[:m], dtype=np.float64)
    xin[~real_rows_mask(offs, counts, m)] = 0.0
    r = {"offs": offs, "counts": counts, "policy": policy}
    r.update(quantize_weights(w1, w3, w2, policy))
    r["xq_r"], r["xs_r"], x_r = policy.row(xin) if m else (None, None, np.zeros((0, d)))
    r["xq_c"], r["xs_c"], x_c = policy.col(xin) if m else (None, None, np.zeros((d, 0)))
    r["x_c"] = x_c
    h13 = np.zeros((m, 2 * f))
    for e, (a, b) in enumerate(segments(offs)):
        if b > a:
            h13[a:b] = x_r[a:b] @ r["w13_r"][e].T
    h13 = policy.bf16(h13)
    r["h13"] = h13
    g, u = split_gu(h13)
    h = policy.bf16(swiglu(g, u))
    r["h"] = h
    r["hq_r"], r["hs_r"], h_r = policy.row(h) if m else (None, None, np.zeros((0, f)))
    r["hq_c"], r["hs_c"], h_c = policy.col(h) if m else (None, None, np.zeros((f, 0)))
    r["h_c"] = h_c
    y = np.zeros((m, d))
    for e, (a, b) in enumerate(segments(offs)):
        if b > a:
            y[a:b] = h_r[a:b] @ r["w2_r"][e].T
    r["y"] = y
    return r


def mlp_backward(fwd, dy):
    """Backward of the routed-experts MLP (straight-through quantization).

    dy [>= offs[E], D] fp64. Returns a dict with dyq/dhq codes and scales, dh,
    dG, dU, the packed dH13, dx [offs[E], D], dw1, dw3 [E, F, D], dw2 [E, D, F].
    """
    policy = fwd["policy"]
    offs = fwd["offs"]
    m = offs[-1]
    ne = len(offs) - 1
    f2 = fwd["h13"].shape[1]
    f = f2 // 2
    d = dy.shape[1]
    dyin = np.array(dy[:m], dtype=np.float64)
    dyin[~real_rows_mask(offs, fwd["counts"], m)] = 0.0
    r = {}
    r["dyq_r"], r["dys_r"], dy_r = policy.row(dyin) if m else (None, None, np.zeros((0, d)))
    r["dyq_c"], r["dys_c"], dy_c = policy.col(dyin) if m else (None, None, np.zeros((d, 0)))
    dh = np.zeros((m, f))
    for e, (a, b) in enumerate(segments(offs)):
        if b > a:
            dh[a:b] = dy_r[a:b] @ fwd["w2_c"][e].T
    dh = policy.bf16(dh)
    g, u = split_gu(fwd["h13"])
    dg, du = dswiglu(dh, g, u)
    dg = policy.bf16(dg)
    du = policy.bf16(du)
    dh13 = join_gu(dg, du)
    r.update(dh=dh, dg=dg, du=du, dh13=dh13)
    r["dhq_r"], r["dhs_r"], dh_r = policy.row(dh13) if m else (None, None, np.zeros((0, f2)))
    r["dhq_c"], r["dhs_c"], dh_c = policy.col(dh13) if m else (None, None, np.zeros((f2, 0)))
    dx = np.zeros((m, d))
    dw2 = np.zeros((ne, d, f))
    dw13 = np.zeros((ne, f2, d))
    for e, (a, b) in enumerate(segments(offs)):
        if b == a:
            continue                       # zero-token expert: exact-zero gradients
        dw2[e] = _slice_cols(dy_c, a, b) @ _slice_cols(fwd["h_c"], a, b).T
        dx[a:b] = dh_r[a:b] @ fwd["w13_c"][e].T
        dw13[e] = _slice_cols(dh_c, a, b) @ _slice_cols(fwd["x_c"], a, b).T
    dw1, dw3 = unpack_w13(dw13)
    r.update(dx=dx, dw2=dw2, dw13=dw13, dw1=dw1, dw3=dw3)
    return r


# --------------------------------------------------------------------------- stage-wise helpers

def gemm_deq(aq, as_, bq, bs):
    """C = deq(A) deq(B)^T, fp64, for K-contiguous MXFP8 operands A [M, K], B [N, K]."""
    return dequantize_rowwise(aq, as_) @ dequantize_rowwise(bq, bs).T


def swiglu_quant_from_h13(h13_bits):
    """FC1 epilogue from the saved BF16 FC1 output: h = BF16(silu(g) u), dual-quantized.

    h13_bits [M, 2F] uint16 (M % 32 == 0). Returns (h_bits, hq_r, hs_r, hq_c, hs_c).
    """
    g, u = split_gu(bf16_bits_to_f64(h13_bits))
    h = bf16_round(swiglu(g, u))
    hq_r, hs_r = quantize_rowwise(h)
    hq_c, hs_c = quantize_colwise(h)
    return f64_to_bf16_bits(h), hq_r, hs_r, hq_c, hs_c


def dswiglu_quant(dh, h13_bits):
    """FC2-dgrad epilogue: dh (fp64 GEMM result) and saved BF16 h13 -> dual-quantized dH13.

    Returns (dh13_bits [M, 2F] uint16, dhq_r, dhs_r, dhq_c, dhs_c).
    """
    g, u = split_gu(bf16_bits_to_f64(h13_bits))
    dhb = bf16_round(dh)
    dg, du = dswiglu(dhb, g, u)
    dh13 = join_gu(bf16_round(dg), bf16_round(du))
    q_r, s_r = quantize_rowwise(dh13)
    q_c, s_c = quantize_colwise(dh13)
    return f64_to_bf16_bits(dh13), q_r, s_r, q_c, s_c
