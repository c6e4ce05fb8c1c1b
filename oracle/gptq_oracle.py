"""Plain float64 CPU oracle of the GPTQ one-shot layer quantizer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or run this module. The HIP
library neither imports it nor shares any code, table or helper with it.

It follows the pages' definitions step by step, in their order and notation,
with no blocking or fusion beyond what the method itself states. Sources
(page title, then section):

* aiqz.cc, "GPTQ：一键量化大模型压缩" -- sections 二阶信息 (Hessian),
  逐层量化 (layer objective), 误差补偿 (OBS compensation δ_F),
  分组方案 (per-group scale/zero), Python 演示 (a small damping term, per
  output-neuron parameters, numpy round).
* astro-blog-cod.pages.dev, LLM quantization techniques survey -- sections
  1.2 量化原理 (x_q = round(x/s + z), dequant s(x_q - z)), 2.2 最优大脑量化
  (OBS update), 2.3 GPTQ 的改进 (fixed column order, blocks of B = 128,
  Cholesky).
* compassingai.com, "GPTQ" concept page -- section 3 技術原理 (objective,
  H = 2XX^T, per-column scale/zero chosen inside the sweep), section 4
  關鍵引數 (bits 3/4/8; group 128 or -1 for "not grouped").
* mcipr.com, "一文读懂GPTQ" -- section 三 (codes packed into 32-bit integer
  arrays).
* ai-papers.xuzou.cn reading card "GPTQ: Accurate Post-Training Quantization
  for Generative Pre-trained Transformers" -- section 方法适配 (same order for
  all rows so the inverse-Hessian information is shared; lazy batches of
  B = 128 with the global update deferred to block end, same total compute;
  Cholesky precomputation of the needed rows with mild damping).

Readings taken where the pages are silent or disagree (each is also listed in
the design notes of the repository):

* H = 2 * sum_t x_t x_t^T, a sum over tokens, not a mean; X is tokens x
  channels, so H = 2 X^T X.
* Damping is relative: lambda = damp * mean(diag H), H_d = H + lambda I.
* The rows of the inverse Hessian that drive the update are the rows of U,
  the upper Cholesky factor of H_d^{-1} (H_d^{-1} = U^T U). Row q of U,
  scaled by U_qq, is row q of the inverse of the not-yet-quantized
  sub-Hessian, so the OBS step reads: err = w_q - what_q, e = err / U_qq,
  w_j -= e * U_qj for j > q, loss += err^2 / (2 U_qq^2).
* Quantizer: asymmetric min-max with an integer zero point, s = (xmax -
  xmin)/(2^b - 1), z = rint(-xmin/s), code = clamp(rint(x/s) + z, 0, 2^b-1),
  dequant = s (code - z); the range always includes 0 and an all-zero group
  uses [-1, 1]. rint is round-half-to-even.
* Symmetric variant (optional): z = 0 on the signed grid [-2^(b-1),
  2^(b-1) - 1] with s = max|x| / (2^(b-1) - 1), stored as the unsigned code
  signed + 2^(b-1) (so the zero point is the fixed code 2^(b-1)).
* Group statistics come from the current (already compensated) values when
  the sweep reaches the group's first column; group_size = -1 is one group
  per row taken from the original row.
* Blocks are exact: after a block, W[:, i2:] -= E U[i1:i2, i2:] applies the
  deferred rank-1 updates, so any block size gives the same numbers up to
  rounding. Grouping needs block % group == 0 or group % block == 0.
* Act-order (the `desc_act` flag of the library configuration the
  mcipr.com page shows, section 四; the page gives no definition): columns
  are quantized in order of descending diag(H) (ties by ascending column
  index, NaN last), which is the method above run on W[:, p] and
  H[p][:, p]; groups are consecutive in that order, so group statistics
  follow the permuted order.
* The greedy order (astro-blog survey, section 2.2, OBQ) is a slow
  reference: per row, repeatedly the free weight with the least
  (w - quant(w))^2 / [H_F^-1]_qq, with the inverse of the free sub-Hessian
  kept by Gaussian elimination; one grid per row from the original row.
* Calibration pipeline (xuzou.cn reading card, section 计算设置: one
  block at a time, the quantized block's outputs are the next block's
  inputs). Layers reading the same input (the q/k/v projections) share
  one Hessian, accumulated over the calibration chunks, and one factor.
  Inside a block each layer's Hessian comes from its input as produced by
  the already-quantized layers before it. The MLP block is
  X1 = relu(X0 What_up^T), X2 = X1 What_down^T (ReLU: the OPT models the
  pages quantize); the layer weights used to run the block are the
  dequantized weights held as fp16 (s (code - z) in fp32, rounded to
  fp16), and the activations between layers are stored as fp16.
* Packing: per row, an LSB-first bitstream along the columns; code j fills
  bits [b j, b j + b) and word k holds bits [32 k, 32 k + 32); rows are
  zero-padded to ceil(d_col b / 32) words.

Every function here is pinned by the ``-m "not gpu"`` tests (brute force on
tiny inputs, closed forms, invariants and hand-computed fixtures); none is
parity-unpinned.
"""

from __future__ import annotations

from typing import Iterable, Optional, Union

import numpy as np

F64 = np.float64


class NotPositiveDefinite(np.linalg.LinAlgError):
    """The damped Hessian has a non-positive Cholesky pivot."""


# --------------------------------------------------------------------------
# Stage 1: Hessian
# --------------------------------------------------------------------------
def hessian(chunks: Union[np.ndarray, Iterable[np.ndarray]], d: Optional[int] = None) -> np.ndarray:
    """H = 2 * sum over tokens of x x^T, in float64.

    aiqz.cc "GPTQ：一键量化大模型压缩", section 二阶信息: H is twice the sum of
    the outer products of the layer's input vectors. compassingai.com
    "GPTQ", section 3: H = 2XX^T with X holding one column per sample; the
    arrays here hold one row per token, so the same matrix is 2 X^T X.

    ``chunks`` is an array [n_tokens, d] or an iterable of such arrays; the
    sum runs over all of them (a matmul per chunk is the library step).
    """
    if isinstance(chunks, np.ndarray):
        chunks = [chunks]
    H = None
    for x in chunks:
        x = np.asarray(x, dtype=F64)
        if H is None:
            H = np.zeros((x.shape[1], x.shape[1]), dtype=F64)
        H += x.T @ x
    if H is None:
        H = np.zeros((d or 0, d or 0), dtype=F64)
    return 2.0 * H


# --------------------------------------------------------------------------
# Stage 2: damping and the inverse-Hessian factor
# --------------------------------------------------------------------------
def damped(H: np.ndarray, damp: float):
    """H_d = H + lambda I with lambda = damp * mean(diag H).

    xuzou.cn reading card, section 方法适配: the Cholesky route is used with
    a mild damping term; aiqz.cc, section Python 演示: a small multiple of the
    identity is added before inversion. The relative form is the reading
    used here.
    """
    H = np.asarray(H, dtype=F64)
    lam = float(damp) * float(np.mean(np.diag(H))) if H.shape[0] else 0.0
    return H + lam * np.eye(H.shape[0]), lam


def _cholesky_lower(A: np.ndarray) -> np.ndarray:
    try:
        L = np.linalg.cholesky(A)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from None
    if not np.all(np.isfinite(L)) or (L.shape[0] and np.min(np.diag(L)) <= 0.0):
        raise NotPositiveDefinite("non-positive pivot")
    return L


def prepare_hinv(H: np.ndarray, damp: float):
    """Return (U, lambda): U upper triangular with H_d^{-1} = U^T U.

    astro-blog survey, section 2.3 item 3, and xuzou.cn section 方法适配:
    the rows of the inverse Hessian that the sweep needs are precomputed
    with a Cholesky factorization of the damped matrix. Taken literally:
    L = chol(H_d); H_d^{-1} = L^{-T} L^{-1}; U = chol(H_d^{-1})^T.
    Raises NotPositiveDefinite if H_d has a non-positive pivot.
    """
    Hd, lam = damped(H, damp)
    d = Hd.shape[0]
    if d == 0:
        return np.zeros((0, 0)), lam
    L = _cholesky_lower(Hd)
    Linv = np.linalg.inv(L)
    Hinv = Linv.T @ Linv
    U = _cholesky_lower(Hinv).T
    return np.triu(U), lam


# --------------------------------------------------------------------------
# Quantizer
# --------------------------------------------------------------------------
def group_params(x: np.ndarray, bits: int, decide=F64, with_margin: bool = False, symmetric: bool = False,
                 flip=None):
    """Per-row min-max scale and integer zero of a group of columns.

    aiqz.cc, section 分组方案: scale = (max - min)/(2^bits - 1) and the zero
    point maps the minimum to code 0; astro-blog survey, section 1.2: the
    zero point z enters as round(x/s + z). The zero is rounded to an integer
    code here. The range is widened to include 0 (so z is a valid code) and
    an all-zero group uses [-1, 1].

    ``x`` is [rows, cols]. Returns (s, z) as float64 arrays [rows]; z holds
    integers. ``decide`` is the precision of the division and rounding
    that fixes z (float64, or float32 to match a float32 implementation).
    With ``with_margin`` it also returns how far -xmin/s lay from the nearest
    rounding boundary, in grid steps (0 = an exact tie, 0.5 = an integer).

    ``symmetric``: the signed grid with z = 0 of astro-blog survey, section
    1.2 (x_q clamped to [-2^(b-1), 2^(b-1) - 1]), with the scale of the
    aiqz.cc demo (section Python 演示): s = max|x| / (2^(b-1) - 1). Stored
    as unsigned codes, the signed value plus 2^(b-1), so the zero point is
    the fixed code 2^(b-1). An all-zero group uses max|x| = 1. The zero is
    not a rounding decision here, so its margin is reported as 0.5.

    ``flip`` (optional boolean [rows]): in the rows it marks, the zero point
    takes the other rounding of -xmin/s, the integer on the other side of
    the nearest rounding boundary. Parity tests use this to follow a row
    whose float32 history crossed a near-tie; it is not part of the method.
    """
    if symmetric:
        qs = (1 << (bits - 1)) - 1
        amax = np.max(np.abs(x), axis=1)
        amax = np.where(amax == 0.0, 1.0, amax)
        if decide == F64:
            s = amax / qs
        else:
            s = (amax.astype(decide) / decide(qs)).astype(F64)
        z = np.full(s.shape, float(1 << (bits - 1)))
        if flip is not None and np.any(flip):
            raise ValueError("the symmetric grid's zero point is fixed, not a rounding decision")
        if with_margin:
            return s.astype(F64), z, np.full(s.shape, 0.5)
        return s.astype(F64), z
    maxq = (1 << bits) - 1
    xmin = np.minimum(np.min(x, axis=1), 0.0)
    xmax = np.maximum(np.max(x, axis=1), 0.0)
    dead = (xmin == 0.0) & (xmax == 0.0)
    xmin = np.where(dead, -1.0, xmin)
    xmax = np.where(dead, 1.0, xmax)
    if decide == F64:
        s = (xmax - xmin) / maxq
        t = -xmin / s
    else:
        s32 = (xmax.astype(decide) - xmin.astype(decide)) / decide(maxq)
        t = ((-xmin.astype(decide)) / s32).astype(F64)
        s = s32.astype(F64)
    z = np.rint(t)
    margin = 0.5 - np.abs(t - z)
    if flip is not None:
        z = np.where(flip, _other_rounding(t, z), z)
    if with_margin:
        return s.astype(F64), z.astype(F64), margin
    return s.astype(F64), z.astype(F64)


def _other_rounding(t, n):
    """The integer on the other side of the rounding boundary nearest to t,
    where n = rint(t): n + 1 if t lies above n, else n - 1."""
    return np.where(t > n, n + 1.0, n - 1.0)


def quantize_codes(w: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int, decide=F64, with_margin: bool = False,
                   flip=None):
    """code = clamp(rint(w/s) + z, 0, 2^b - 1) (astro-blog survey, 1.2).

    With ``with_margin`` it also returns how far w/s lay from the nearest
    rounding boundary, in grid steps (0 = an exact tie). ``flip`` (optional
    boolean, shaped like w) takes the other rounding of w/s where set (see
    ``group_params``; a test device, not part of the method).
    """
    maxq = (1 << bits) - 1
    if decide == F64:
        t = w / s
    else:
        t = (w.astype(decide) / s.astype(decide)).astype(F64)
    q = np.rint(t)
    margin = 0.5 - np.abs(t - q)
    if flip is not None:
        q = np.where(flip, _other_rounding(t, q), q)
    c = np.clip(q + z, 0, maxq)
    if with_margin:
        return c, margin
    return c


def rtn(W: np.ndarray, bits: int, group_size: int, symmetric: bool = False):
    """Round-to-nearest baseline: every weight rounded on its own group grid.

    aiqz.cc, section Python 演示 (the round-only baseline) and xuzou.cn,
    section 证据 (RTN as the comparison). Group statistics come from the
    original weights; there is no error compensation. Written without the
    column loop so that it is an independent check of the sweep at H = I.
    """
    W = np.asarray(W, dtype=F64)
    d_row, d_col = W.shape
    g = d_col if group_size == -1 else group_size
    n_groups = 1 if group_size == -1 else -(-d_col // group_size)
    codes = np.zeros((d_row, d_col), dtype=np.int64)
    scales = np.zeros((d_row, n_groups))
    zeros = np.zeros((d_row, n_groups))
    for k in range(n_groups):
        sl = slice(k * g, min(d_col, (k + 1) * g))
        s, z = group_params(W[:, sl], bits, symmetric=symmetric)
        scales[:, k], zeros[:, k] = s, z
        codes[:, sl] = quantize_codes(W[:, sl], s[:, None], z[:, None], bits)
    return codes.astype(np.uint8), scales, zeros


def dequantize(codes, scales, zeros, group_size: int) -> np.ndarray:
    """what = s (code - z), with the group of column j being j // g."""
    codes = np.asarray(codes, dtype=F64)
    d_col = codes.shape[1]
    if group_size == -1:
        gi = np.zeros(d_col, dtype=np.int64)
    else:
        gi = np.arange(d_col) // group_size
    return np.asarray(scales, F64)[:, gi] * (codes - np.asarray(zeros, F64)[:, gi])


# --------------------------------------------------------------------------
# Stage 3: fixed-order column sweep with OBS compensation and lazy blocks
# --------------------------------------------------------------------------
def quantize_layer(
    W: np.ndarray,
    U: np.ndarray,
    bits: int,
    group_size: int,
    block: int = 128,
    decide=F64,
    symmetric: bool = False,
    flips=(),
):
    """GPTQ sweep of one layer, columns in natural order.

    * aiqz.cc, section 误差补偿: after a column is rounded, the remaining
      columns of the same row absorb the error through the inverse Hessian,
      delta_F = (q - w_q)/[H^-1]_qq [H^-1]_{F,q}.
    * astro-blog survey, section 2.3 items 1-3 and xuzou.cn, section
      方法适配: a fixed order shared by all rows, blocks of B columns whose
      global update waits until the block is done, inverse rows from a
      Cholesky factor (here the rows of U).
    * compassingai.com "GPTQ", section 3: scale and zero are chosen inside
      the sweep, before a column is rounded.

    W is [d_row, d_col] (any float dtype; upcast exactly to float64). U is
    [d_col, d_col] upper triangular. Returns a dict with codes (uint8),
    scales, zeros (float64, integer-valued), Wq (the dequantized weights),
    row_loss and loss (sum over columns of err^2 / (2 U_qq^2)), packed, and
    two diagnostics of how close each decision came to a tie:
    code_margin [d_row, d_col] (distance of w/s from the nearest rounding
    boundary, in grid steps) and zero_margin [d_row, n_groups] (the same for
    -xmin/s when the zero point was chosen).
    ``decide`` is the precision in which each code is decided (float64 by
    default; float32 reproduces the decision of a float32 implementation
    given the same inputs). ``symmetric`` selects the symmetric grid of
    ``group_params``.

    ``flips`` (a test device, empty for the method itself): (row, "code",
    column) or (row, "zero", group) entries; at each, that row's decision
    takes the other rounding, and the sweep continues from there exactly as
    the method does. The margins returned are those of the decisions as
    computed, before any flip.
    """
    W = np.array(W, dtype=F64, copy=True)
    U = np.asarray(U, dtype=F64)
    d_row, d_col = W.shape
    if U.shape != (d_col, d_col):
        raise ValueError("U must be [d_col, d_col]")
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    if block < 1:
        raise ValueError("block must be >= 1")
    if group_size != -1:
        if group_size < 1 or (block % group_size and group_size % block):
            raise ValueError("need block % group == 0 or group % block == 0")
    n_groups = 1 if group_size == -1 else -(-d_col // group_size)
    codes = np.zeros((d_row, d_col), dtype=np.uint8)
    scales = np.zeros((d_row, n_groups))
    zeros = np.zeros((d_row, n_groups))
    Wq = np.zeros((d_row, d_col))
    row_loss = np.zeros(d_row)
    code_margin = np.zeros((d_row, d_col))
    zero_margin = np.zeros((d_row, n_groups))
    code_flip, zero_flip = {}, {}
    for r, kind, idx in flips:
        if not (0 <= r < d_row):
            raise ValueError(f"flip row {r} out of range")
        if kind == "code" and 0 <= idx < d_col:
            code_flip.setdefault(idx, np.zeros(d_row, dtype=bool))[r] = True
        elif kind == "zero" and 0 <= idx < n_groups:
            zero_flip.setdefault(idx, np.zeros(d_row, dtype=bool))[r] = True
        else:
            raise ValueError(f"bad flip {(r, kind, idx)}")

    if group_size == -1 and d_col:
        s, z, zm = group_params(W, bits, decide, with_margin=True, symmetric=symmetric, flip=zero_flip.get(0))
        scales[:, 0], zeros[:, 0], zero_margin[:, 0] = s, z, zm

    for i1 in range(0, d_col, block):
        i2 = min(i1 + block, d_col)
        E = np.zeros((d_row, i2 - i1))
        for q in range(i1, i2):
            if group_size != -1 and q % group_size == 0:
                k = q // group_size
                s, z, zm = group_params(
                    W[:, q : min(q + group_size, d_col)], bits, decide, with_margin=True, symmetric=symmetric,
                    flip=zero_flip.get(k),
                )
                scales[:, k], zeros[:, k], zero_margin[:, k] = s, z, zm
            w = W[:, q]
            c, code_margin[:, q] = quantize_codes(w, s, z, bits, decide, with_margin=True, flip=code_flip.get(q))
            what = s * (c - z)
            err = w - what
            d = U[q, q]
            row_loss += err * err / (2.0 * d * d)
            e = err / d
            W[:, q + 1 : i2] -= np.outer(e, U[q, q + 1 : i2])
            E[:, q - i1] = e
            codes[:, q] = c.astype(np.uint8)
            Wq[:, q] = what
        if i2 < d_col:
            W[:, i2:] -= E @ U[i1:i2, i2:]

    return dict(
        codes=codes,
        scales=scales,
        zeros=zeros,
        Wq=Wq,
        row_loss=row_loss,
        loss=float(np.sum(row_loss)),
        packed=pack(codes, bits),
        code_margin=code_margin,
        zero_margin=zero_margin,
    )


# --------------------------------------------------------------------------
# Column orders: act-order, and the greedy order of OBQ (slow reference)
# --------------------------------------------------------------------------
def act_order_perm(H: np.ndarray) -> np.ndarray:
    """Column order by descending diag(H): p[q] is the original column taken
    q-th. Equal values keep ascending column order; NaN values come last (in
    ascending column order); -0 equals +0.

    mcipr.com "一文读懂GPTQ", section 四 (the `desc_act` flag of the library
    configuration); the order itself is the reading stated in this module's
    header.
    """
    h = np.diag(np.asarray(H, dtype=F64))

    def key(i):
        v = h[i]
        return (1, 0.0, i) if np.isnan(v) else (0, -v, i)

    return np.array(sorted(range(h.shape[0]), key=key), dtype=np.int64)


def inverse_perm(p: np.ndarray) -> np.ndarray:
    """inv[p[q]] = q."""
    p = np.asarray(p, dtype=np.int64)
    inv = np.empty_like(p)
    inv[p] = np.arange(p.shape[0])
    return inv


def quantize_layer_act_order(
    W: np.ndarray,
    H: np.ndarray,
    bits: int,
    group_size: int,
    block: int = 128,
    damp: float = 0.01,
    decide=F64,
    symmetric: bool = False,
):
    """The layer quantized in act-order: the fixed-order method on the
    columns of W taken in the order p = act_order_perm(H), with the
    Hessian's rows and columns taken in the same order. Returns the dict of
    ``quantize_layer`` (codes, scales, zeros, Wq, packed, ... all in the
    permuted column order, groups consecutive in that order) plus ``perm``,
    ``lam``, ``U`` (the factor of the permuted Hessian), ``Wq_orig`` (the
    dequantized weights back in the original column order) and ``g_idx``
    (group of each original column).
    """
    H = np.asarray(H, dtype=F64)
    p = act_order_perm(H)
    U, lam = prepare_hinv(H[np.ix_(p, p)], damp)
    r = quantize_layer(np.asarray(W)[:, p], U, bits, group_size, block, decide, symmetric)
    inv = inverse_perm(p)
    r.update(
        perm=p,
        lam=lam,
        U=U,
        Wq_orig=r["Wq"][:, inv],
        g_idx=np.zeros(p.shape[0], dtype=np.int64) if group_size == -1 else inv // group_size,
    )
    return r


def obq_greedy(W: np.ndarray, H: np.ndarray, bits: int, damp: float = 0.01, decide=F64, order=None):
    """OBQ, one row at a time (astro-blog survey, section 2.2): among the
    free weights F of the row, quantize the one with the least
    (w_q - quant(w_q))^2 / [H_F^-1]_qq, then correct the free weights by the
    OBS step w_F -= (w_q - quant(w_q)) / [H_F^-1]_qq * [H_F^-1]_{F,q} and
    drop q from the inverse by one Gaussian elimination step,
    H_F'^-1 = H_F^-1 - H_F^-1[:, q] H_F^-1[q, :] / [H_F^-1]_qq. Ties go to
    the lowest column index. ``order`` (optional) fixes the order instead of
    the greedy choice. The grid is one per row from the original row
    (``group_params``), the Hessian is damped as in ``damped``.

    Returns codes, Wq, row_loss, loss (sum of err^2 / (2 [H_F^-1]_qq)) and
    the order taken per row [d_row, d_col].
    """
    W = np.asarray(W, dtype=F64)
    d_row, d_col = W.shape
    H_d, _ = damped(np.asarray(H, dtype=F64), damp)
    Hinv0 = np.linalg.inv(H_d)
    codes = np.zeros((d_row, d_col), dtype=np.uint8)
    Wq = np.zeros((d_row, d_col))
    row_loss = np.zeros(d_row)
    taken = np.zeros((d_row, d_col), dtype=np.int64)
    for r in range(d_row):
        s, z = group_params(W[r : r + 1], bits, decide)
        w = W[r].copy()
        Hinv = Hinv0.copy()
        free = np.ones(d_col, dtype=bool)
        for step in range(d_col):
            if order is None:
                idx = np.flatnonzero(free)
                c = quantize_codes(w[idx], np.full(idx.shape, s[0]), np.full(idx.shape, z[0]), bits, decide)
                cost = (w[idx] - s[0] * (c - z[0])) ** 2 / np.diag(Hinv)[idx]
                q = int(idx[int(np.argmin(cost))])
            else:
                q = int(order[step])
            c = quantize_codes(w[q : q + 1], s, z, bits, decide)[0]
            what = s[0] * (c - z[0])
            err = w[q] - what
            dq = Hinv[q, q]
            row_loss[r] += err * err / (2.0 * dq)
            w[free] -= (err / dq) * Hinv[free, q]
            Hinv = Hinv - np.outer(Hinv[:, q], Hinv[q, :]) / dq
            free[q] = False
            w[q] = what
            codes[r, q] = c
            Wq[r, q] = what
            taken[r, step] = q
    return dict(codes=codes, Wq=Wq, row_loss=row_loss, loss=float(np.sum(row_loss)), order=taken)


# --------------------------------------------------------------------------
# Calibration pipeline: layers sharing an input, and a block quantized
# layer by layer with the quantized layers' outputs as the next inputs
# --------------------------------------------------------------------------
def quantize_shared_input(chunks, Ws, bits: int, group_size: int, block: int = 128, damp: float = 0.01,
                          decide=F64, symmetric: bool = False):
    """Layers that read the same input (xuzou.cn reading card, section
    计算设置; the q/k/v projections of a block): one Hessian summed over the
    calibration chunks, one damped factor, and each layer's rows swept with
    it (section 方法适配: every row uses the same inverse-Hessian
    information). Returns dict(H, U, lam, layers=[quantize_layer dict per W]).
    """
    H = hessian(chunks)
    U, lam = prepare_hinv(H, damp)
    layers = [quantize_layer(W, U, bits, group_size, block, decide, symmetric) for W in Ws]
    return dict(H=H, U=U, lam=lam, layers=layers)


def model_weight_f16(codes, scales, zeros, group_size: int) -> np.ndarray:
    """The dequantized weights as the layer holds them to run: s (code - z)
    with the product rounded to float32, then to float16 (astro-blog
    survey, section 1.2)."""
    codes = np.asarray(codes)
    d_col = codes.shape[1]
    gi = np.zeros(d_col, dtype=np.int64) if group_size == -1 else np.arange(d_col) // group_size
    s32 = np.asarray(scales, np.float32)[:, gi]
    k32 = (codes.astype(np.int64) - np.asarray(zeros, np.int64)[:, gi]).astype(np.float32)
    return (s32 * k32).astype(np.float16)


def run_quantized_layer(X, packed, scales, zeros, d_in: int, bits: int, group_size: int, relu: bool = False):
    """The quantized layer run on tokens X [n, d_in] (xuzou.cn reading card,
    section 计算设置: the quantized block produces the next block's
    inputs): Y = act(X What^T) with What the fp16 model weight of
    ``model_weight_f16`` decoded from the packed words, the product exact
    (float64), act = ReLU if ``relu``, and Y rounded to fp16."""
    Wh = model_weight_f16(unpack(packed, d_in, bits), scales, zeros, group_size).astype(F64)
    Y = np.asarray(X, dtype=F64) @ Wh.T
    if relu:
        Y = np.maximum(Y, 0.0)
    return Y.astype(np.float16)


def quantize_mlp_block(X0, W_up, W_down, bits: int, group_size: int, block: int = 128, damp: float = 0.01,
                       decide=F64):
    """One MLP block quantized layer by layer (xuzou.cn reading card,
    section 计算设置): H_up from the block input X0 [tokens, d_model];
    quantize W_up [d_ff, d_model]; run the quantized up layer,
    X1 = fp16(relu(X0 What_up^T)) with What_up the fp16 model weight and the
    product exact; H_down from X1; quantize W_down [d_model, d_ff]; the block
    output X2 = fp16(X1 What_down^T) is the next block's input.
    Returns dict(up, down (quantize_layer dicts plus H, U, lam), X1, X2).
    """
    X0 = np.asarray(X0)
    out = {}
    H_up = hessian(X0)
    U_up, lam_up = prepare_hinv(H_up, damp)
    up = quantize_layer(W_up, U_up, bits, group_size, block, decide)
    up.update(H=H_up, U=U_up, lam=lam_up)
    Wh_up = model_weight_f16(up["codes"], up["scales"], up["zeros"], group_size)
    X1 = np.maximum(X0.astype(F64) @ Wh_up.astype(F64).T, 0.0).astype(np.float16)
    H_down = hessian(X1)
    U_down, lam_down = prepare_hinv(H_down, damp)
    down = quantize_layer(W_down, U_down, bits, group_size, block, decide)
    down.update(H=H_down, U=U_down, lam=lam_down)
    Wh_down = model_weight_f16(down["codes"], down["scales"], down["zeros"], group_size)
    X2 = (X1.astype(F64) @ Wh_down.astype(F64).T).astype(np.float16)
    out.update(up=up, down=down, X1=X1, X2=X2)
    return out


def layer_loss_direct(X: np.ndarray, W: np.ndarray, Wq: np.ndarray, lam: float = 0.0) -> float:
    """||X (W - Wq)^T||_F^2 + (lambda/2) ||W - Wq||_F^2.

    aiqz.cc, section 逐层量化: the layer objective is the squared Frobenius
    norm of the output difference. With H_d = 2 X^T X + lambda I the sum of
    the sweep's per-column losses equals half the H_d-weighted error
    quadratic, which is this quantity.
    """
    D = np.asarray(W, F64) - np.asarray(Wq, F64)
    Y = np.asarray(X, F64) @ D.T
    return float(np.sum(Y * Y) + 0.5 * lam * np.sum(D * D))


# --------------------------------------------------------------------------
# Packing
# --------------------------------------------------------------------------
def words_per_row(d_col: int, bits: int) -> int:
    return -(-d_col * bits // 32)


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """b-bit codes -> uint32 words, per row an LSB-first bitstream.

    mcipr.com "一文读懂GPTQ", section 三: low-bit codes are stored in 32-bit
    integer arrays. Bit i of a row's stream is bit (i mod b) of code i // b;
    word k holds stream bits [32k, 32k + 32).
    """
    codes = np.asarray(codes, dtype=np.uint64)
    d_row, d_col = codes.shape
    nw = words_per_row(d_col, bits)
    bitpos = np.arange(bits, dtype=np.uint64)
    stream = ((codes[:, :, None] >> bitpos) & np.uint64(1)).reshape(d_row, d_col * bits)
    padded = np.zeros((d_row, nw * 32), dtype=np.uint64)
    padded[:, : d_col * bits] = stream
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    words = (padded.reshape(d_row, nw, 32) * weights).sum(axis=2)
    return words.astype(np.uint32)


def unpack(words: np.ndarray, d_col: int, bits: int) -> np.ndarray:
    """Inverse of ``pack``."""
    words = np.asarray(words, dtype=np.uint64)
    d_row, nw = words.shape
    stream = ((words[:, :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).reshape(d_row, nw * 32)
    stream = stream[:, : d_col * bits].reshape(d_row, d_col, bits)
    vals = (stream << np.arange(bits, dtype=np.uint64)).sum(axis=2)
    return vals.astype(np.uint8)


# --------------------------------------------------------------------------
# Use of the packed layer: quantized matrix x full-precision vector
# --------------------------------------------------------------------------
def dequant_matvec(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, d_col: int, bits: int,
                   group_size: int, x: np.ndarray) -> np.ndarray:
    """Y = X What^T with What decoded from the packed words.

    xuzou.cn reading card, section 方法适配 (last paragraph) and section 瓶颈:
    inference multiplies the quantized matrix by full-precision activation
    vectors, dequantizing the weights on the fly, so that batch-1 generation
    reads the low-bit words instead of fp16 weights. What = s (code - z) per
    group (astro-blog survey, section 1.2).

    ``packed`` [d_row, words_per_row], ``scales``/``zeros`` [d_row, n_groups],
    ``x`` [batch, d_col] (any float dtype, upcast exactly). Returns
    [batch, d_row] in float64.
    """
    codes = unpack(packed, d_col, bits)
    What = dequantize(codes, scales, zeros, group_size)
    return np.asarray(x, dtype=F64) @ What.T
