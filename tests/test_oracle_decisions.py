"""Pins of the oracle's decision modes (runs on the CPU).

The GPU takes every rounding decision in float32; the oracle can take the
same decisions in float32 (``decide=np.float32``) on its own float64 values,
and the parity tests follow a row that crossed a near-tie by re-running the
oracle with that decision taken the other way (``flips``). Both devices are
pinned here against things other than the oracle itself:

* exact rational arithmetic (Python fractions, with a round-to-nearest-even
  to float32 written out below) for hand cases where the float32 and float64
  decisions differ;
* the float64 decisions on random layers: the two modes agree except where
  the float64 decision lay within 1e-6 grid steps of a rounding boundary;
* a direct re-solve of the free columns after every rounding (no Cholesky
  rows) with the same decision forced the other way, and the loss identity,
  which holds for any sequence of decisions the OBS update follows.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle.gptq_oracle as O
from tests.test_oracle_pins import rng, sweep_case


def rn32(q) -> Fraction:
    """The float32 nearest to the positive rational q, ties to even,
    computed exactly: q = m 2^(e-23) with 2^23 <= m < 2^24 before rounding."""
    q = Fraction(q)
    assert q > 0
    e = 0
    while q >= 2 ** (e + 1):
        e += 1
    while q < 2**e:
        e -= 1
    m = q / Fraction(2) ** (e - 23)
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return Fraction(n) * Fraction(2) ** (e - 23)


def test_rn32_agrees_with_float32_conversion():
    # the exact rounding above against the hardware conversion of float64 values
    for v in rng(3).uniform(1e-3, 1e3, 2000):
        assert rn32(Fraction(float(v))) == Fraction(float(np.float32(v)))
    assert rn32(Fraction(3, 2)) == Fraction(3, 2)
    assert rn32(1 + Fraction(1, 2**24)) == 1  # halfway, even mantissa below
    assert rn32(1 + Fraction(3, 2**24)) == 1 + Fraction(2, 2**23)  # halfway, even mantissa above


def test_float32_code_decision_hand_case():
    # w / s lies 3.7e-8 below 1.5: float64 rounds it to 1. Its nearest float32
    # is 1.5 itself (within half an ulp, 2^-24), an exact tie that rounds to
    # the even integer 2.
    s = float.fromhex("0x1.99999ep-4")
    w = float.fromhex("0x1.333336p-3")
    q = Fraction(w) / Fraction(s)
    assert float(np.float32(s)) == s and float(np.float32(w)) == w  # both exact in float32
    assert Fraction(3, 2) - Fraction(1, 2**24) < q < Fraction(3, 2) - Fraction(1, 2**50)
    assert rn32(q) == Fraction(3, 2)
    sv, zv, wv = np.array([s]), np.zeros(1), np.array([w])
    c64, m64 = O.quantize_codes(wv, sv, zv, 4, decide=np.float64, with_margin=True)
    c32, m32 = O.quantize_codes(wv, sv, zv, 4, decide=np.float32, with_margin=True)
    assert c64.tolist() == [1.0] and c32.tolist() == [2.0]
    assert m64[0] == pytest.approx(float(Fraction(3, 2) - q), rel=1e-6)  # distance to the boundary 1.5
    assert m32[0] == 0.0


def test_float32_zero_decision_hand_case():
    # 2 bits (maxq = 3), range [xmin, 1]: -xmin / s = 3 (-xmin) / (1 - xmin)
    # lies 1.3e-7 below 1.5, so float64 takes z = 1. In float32 the range
    # 1 - xmin, the scale (range / 3) and the quotient are each rounded; the
    # quotient lands on 1.5, which rounds to the even z = 2.
    xmin = -float.fromhex("0x1.fffffap-1")
    xmax = 1.0
    t_exact = -Fraction(xmin) * 3 / (Fraction(xmax) - Fraction(xmin))
    assert Fraction(3, 2) - t_exact > Fraction(1, 2**50)
    s32 = rn32(rn32(Fraction(xmax) - Fraction(xmin)) / 3)
    assert rn32(-Fraction(xmin) / s32) == Fraction(3, 2)
    x = np.array([[xmin, 0.25, xmax]])
    s64, z64, m64 = O.group_params(x, 2, decide=np.float64, with_margin=True)
    s32v, z32, m32 = O.group_params(x, 2, decide=np.float32, with_margin=True)
    assert z64.tolist() == [1.0] and z32.tolist() == [2.0]
    assert Fraction(float(s32v[0])) == s32
    assert Fraction(float(s64[0])) == Fraction(float((xmax - xmin) / 3))
    assert m64[0] < 1e-6 and m32[0] == 0.0


@pytest.mark.parametrize("bits,group,seed", [(4, 16, 0), (3, -1, 1), (8, 32, 2), (2, 64, 3), (4, 128, 4)])
def test_float32_decisions_equal_float64_except_at_near_ties(bits, group, seed):
    """Every row decided in float32 equals the float64 row up to its first
    differing decision, and that decision lay within 1e-6 grid steps of a
    rounding boundary in float64 (float32 quotients of the same values move
    by about 1e-7 of a step)."""
    X, W, H, U, lam = sweep_case(200, 256, 600, 50 + seed)
    W = W.astype(np.float32).astype(np.float64) * 30  # several grid steps apart
    a = O.quantize_layer(W, U, bits, group, block=32, decide=np.float64)
    b = O.quantize_layer(W, U, bits, group, block=32, decide=np.float32)
    g = 256 if group == -1 else group
    diverged = 0
    for r in range(W.shape[0]):
        cm = np.flatnonzero(a["codes"][r] != b["codes"][r])
        zm = np.flatnonzero(a["zeros"][r] != b["zeros"][r])
        firsts = [(int(cm[0]), "code")] if cm.size else []
        firsts += [(int(zm[0]) * g, "zero")] if zm.size else []
        if not firsts:
            assert np.allclose(a["scales"][r], b["scales"][r], rtol=2e-7, atol=0)
            continue
        diverged += 1
        col, kind = min(firsts, key=lambda t: (t[0], t[1] == "code"))
        if kind == "zero":
            assert a["zero_margin"][r, col // g] < 1e-6
        else:
            assert a["code_margin"][r, col] < 1e-6
        assert np.array_equal(a["codes"][r, :col], b["codes"][r, :col])
    assert diverged <= 2  # 51200 decisions, each within 1e-6 of a tie with probability ~2e-6


def brute_force_with_flip(w, Hd, bits, group, flip):
    """One row, re-solving the free columns directly after every rounding
    (v_R = w_R - H_RR^-1 H_RF (v_F - w_F)); the decision named by ``flip``
    ("code", column) or ("zero", group) takes the integer on the other side
    of its nearest rounding boundary. Decisions in float64, written without
    the oracle's quantizer functions."""
    d = w.shape[0]
    maxq = (1 << bits) - 1
    v = w.copy()
    codes, wq = np.zeros(d, int), np.zeros(d)

    def other(t):
        n = np.rint(t)
        return n + 1.0 if t > n else n - 1.0

    s = z = None
    for q in range(d):
        if q == 0 or (group != -1 and q % group == 0):
            seg = v if group == -1 else v[q : q + group]
            lo, hi = min(seg.min(), 0.0), max(seg.max(), 0.0)
            s = (hi - lo) / maxq
            t = -lo / s
            k = 0 if group == -1 else q // group
            z = other(t) if flip == ("zero", k) else np.rint(t)
        t = v[q] / s
        n = other(t) if flip == ("code", q) else np.rint(t)
        c = min(max(n + z, 0), maxq)
        codes[q], wq[q] = c, s * (c - z)
        F, R = np.arange(q + 1), np.arange(q + 1, d)
        v[F] = wq[F]
        if R.size:
            v[R] = w[R] - np.linalg.solve(Hd[np.ix_(R, R)], Hd[np.ix_(R, F)] @ (v[F] - w[F]))
    return codes, wq


@pytest.mark.parametrize("bits,group,flip", [
    (3, -1, ("code", 0)), (3, -1, ("code", 2)), (2, 3, ("zero", 1)), (4, 2, ("code", 3)),
    (3, 3, ("zero", 0)), (2, -1, ("zero", 0)),
])
def test_flip_continuation_matches_brute_force(bits, group, flip):
    X, W, H, U, lam = sweep_case(3, 6, 20, 70 + bits)
    W = W * 40
    Hd = H + lam * np.eye(6)
    for r in range(3):
        codes, wq = brute_force_with_flip(W[r].copy(), Hd, bits, group, flip)
        for B in (1, 2, 3, 6):
            if group != -1 and B % group and group % B:
                continue  # blocks and groups must nest
            out = O.quantize_layer(W[r : r + 1], U, bits, group, block=B, flips=[(0,) + flip])
            assert np.array_equal(out["codes"][0], codes), (r, B)
            assert np.allclose(out["Wq"][0], wq, atol=1e-12)


@pytest.mark.parametrize("bits,group", [(3, -1), (4, 8), (2, 16)])
def test_flipped_trajectories_keep_the_loss_identity(bits, group):
    """The loss identity holds for any decisions the OBS updates follow, so
    it holds for flipped continuations too; a continuation that forgot to
    carry the flipped value into the error would break it."""
    X, W, H, U, lam = sweep_case(6, 48, 300, 81)
    W = W * 20
    ng = 1 if group == -1 else 48 // group
    r_ = rng(bits)
    flips = [(r, "code", int(r_.integers(0, 48))) for r in range(6)]
    flips += [(r, "zero", int(r_.integers(0, ng))) for r in range(0, 6, 2)]
    base = O.quantize_layer(W, U, bits, group, block=16)
    out = O.quantize_layer(W, U, bits, group, block=16, flips=flips)
    assert not np.array_equal(out["codes"], base["codes"])
    D = W - out["Wq"]
    Hd = H + lam * np.eye(48)
    assert np.allclose(out["row_loss"], 0.5 * np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-10)
    assert out["loss"] == pytest.approx(O.layer_loss_direct(X, W, out["Wq"], lam), rel=1e-10)
    # on the grid of the (flipped) group parameters
    gi = np.zeros(48, int) if group == -1 else np.arange(48) // group
    t = out["Wq"] / out["scales"][:, gi] + out["zeros"][:, gi]
    assert np.allclose(t, out["codes"], atol=1e-9)


def test_flip_changes_only_its_row_and_reports_pre_flip_margins():
    _, W, _, U, _ = sweep_case(5, 40, 200, 90)
    W = W * 20
    base = O.quantize_layer(W, U, 3, 8, block=8)
    col = 17
    out = O.quantize_layer(W, U, 3, 8, block=8, flips=[(2, "code", col)])
    keep = [0, 1, 3, 4]
    assert np.array_equal(out["codes"][keep], base["codes"][keep])
    assert np.array_equal(out["row_loss"][keep], base["row_loss"][keep])
    assert np.array_equal(out["codes"][2, :col], base["codes"][2, :col])
    assert abs(int(out["codes"][2, col]) - int(base["codes"][2, col])) == 1
    assert out["code_margin"][2, col] == base["code_margin"][2, col]
    # the flipped code is the integer on the other side of w / s
    s = base["scales"][2, col // 8]
    t = out["code_margin"][2, col]
    assert 0.0 <= t <= 0.5 and s > 0


def test_flip_argument_errors():
    _, W, _, U, _ = sweep_case(2, 16, 60, 91)
    with pytest.raises(ValueError):
        O.quantize_layer(W, U, 4, -1, flips=[(0, "zero", 0)], symmetric=True)
    with pytest.raises(ValueError):
        O.quantize_layer(W, U, 4, -1, flips=[(2, "code", 0)])
    with pytest.raises(ValueError):
        O.quantize_layer(W, U, 4, 8, flips=[(0, "zero", 2)])
    with pytest.raises(ValueError):
        O.quantize_layer(W, U, 4, 8, flips=[(0, "scale", 0)])
