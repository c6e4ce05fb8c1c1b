"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: brute
force on tiny inputs, closed forms, invariants of the method, or an
independently written special case. Together they are chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand) fails at least one of them; the mutation tests at the
end plant such slips and check that the brute-force pin catches them.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle.gptq_oracle as O


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- Hessian
def test_hessian_brute_force_loops():
    X = rng(1).standard_normal((7, 5))
    H = O.hessian(X)
    for i in range(5):
        for j in range(5):
            s = 0.0
            for t in range(7):
                s += X[t, i] * X[t, j]
            assert abs(H[i, j] - 2.0 * s) < 1e-12


def test_hessian_hand_example():
    # tokens (1, 2) and (3, 4): sum of outer products [[10, 14], [14, 20]], times 2.
    H = O.hessian(np.array([[1.0, 2.0], [3.0, 4.0]]))
    assert np.array_equal(H, np.array([[20.0, 28.0], [28.0, 40.0]]))


def test_hessian_chunked_equals_whole():
    X = rng(2).standard_normal((300, 9))
    whole = O.hessian(X)
    parts = O.hessian([X[:100], X[100:101], X[101:]])
    assert np.allclose(whole, parts, rtol=1e-13, atol=1e-12)
    assert np.array_equal(O.hessian([], d=3), np.zeros((3, 3)))


# ------------------------------------------------------- inverse factor
def test_prepare_hinv_hand_2x2():
    # H = [[4, 2], [2, 2]], no damping: H^-1 = [[1/2, -1/2], [-1/2, 1]],
    # whose upper Cholesky factor is [[1/sqrt2, -1/sqrt2], [0, 1/sqrt2]].
    U, lam = O.prepare_hinv(np.array([[4.0, 2.0], [2.0, 2.0]]), 0.0)
    r = 1 / np.sqrt(2.0)
    assert lam == 0.0
    assert np.allclose(U, [[r, -r], [0.0, r]], atol=1e-15)


def test_prepare_hinv_diagonal_closed_form():
    h = np.array([1.0, 4.0, 9.0, 16.0])
    U, lam = O.prepare_hinv(np.diag(h), 0.1)
    assert lam == pytest.approx(0.1 * h.mean())
    assert np.allclose(U, np.diag(1.0 / np.sqrt(h + lam)), rtol=1e-14)


@pytest.mark.parametrize("d", [1, 2, 5, 33])
def test_prepare_hinv_factorizes_inverse(d):
    X = rng(d).standard_normal((4 * d + 3, d))
    H = O.hessian(X)
    U, lam = O.prepare_hinv(H, 0.01)
    Hd = H + lam * np.eye(d)
    assert np.array_equal(U, np.triu(U))
    assert np.all(np.diag(U) > 0)
    assert np.allclose(Hd @ (U.T @ U), np.eye(d), atol=1e-9)
    # Second derivation: the reversed ("UL") Cholesky of H_d, inverted.
    J = np.eye(d)[::-1]
    V = J @ np.linalg.cholesky(J @ Hd @ J) @ J
    assert np.allclose(U, np.linalg.inv(V), rtol=1e-9, atol=1e-12)


def test_prepare_hinv_rejects_indefinite():
    H = np.array([[1.0, 0.0], [0.0, -5.0]])
    with pytest.raises(O.NotPositiveDefinite):
        O.prepare_hinv(H, 0.01)
    with pytest.raises(O.NotPositiveDefinite):
        O.prepare_hinv(np.zeros((3, 3)), 0.01)  # lambda = 0


# ------------------------------------------------------------ sweep pins
def sweep_case(d_row, d_col, n_tok, seed, damp=0.01):
    r = rng(seed)
    X = r.standard_normal((n_tok, d_col))
    W = 0.02 * r.standard_normal((d_row, d_col))
    H = O.hessian(X)
    U, lam = O.prepare_hinv(H, damp)
    return X, W, H, U, lam


def test_hand_two_column_example():
    # W = [0.9, -0.25], H_d = [[4, 2], [2, 2]] (damp 0), 2 bits, one group.
    #   range [-0.25, 0.9]: s = 1.15/3, z = rint(0.25/s) = rint(0.652) = 1
    #   col 0: rint(0.9/s) = rint(2.348) = 2, code 3, what = 2s = 2.3/3,
    #          err = 0.9 - 2.3/3 = 2/15, e*U01 = -err, so w1 = -0.25 + 2/15 = -7/60
    #   col 1: rint((-7/60)/s) = rint(-0.304) = 0, code 1, what = 0, err = -7/60
    #   loss = (err0^2 + err1^2) / (2 * 1/2) = 4/225 + 49/3600 = 113/3600
    U, _ = O.prepare_hinv(np.array([[4.0, 2.0], [2.0, 2.0]]), 0.0)
    out = O.quantize_layer(np.array([[0.9, -0.25]]), U, bits=2, group_size=-1, block=128)
    assert out["codes"].tolist() == [[3, 1]]
    assert out["scales"][0, 0] == pytest.approx(1.15 / 3, rel=1e-15)
    assert out["zeros"][0, 0] == 1
    assert out["Wq"][0].tolist() == pytest.approx([2.3 / 3, 0.0], abs=1e-15)
    assert out["loss"] == pytest.approx(float(Fraction(113, 3600)), rel=1e-13)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("group", [-1, 8, 16])
def test_identity_hessian_reduces_to_rtn(bits, group):
    W = 0.02 * rng(bits + group).standard_normal((7, 48))
    lam_frac = 0.01
    U, lam = O.prepare_hinv(np.eye(48), lam_frac)
    out = O.quantize_layer(W, U, bits, group, block=16)
    codes, scales, zeros = O.rtn(W, bits, group)
    assert np.array_equal(out["codes"], codes)
    assert np.array_equal(out["scales"], scales)
    assert np.array_equal(out["zeros"], zeros)
    what = O.dequantize(codes, scales, zeros, group)
    assert out["loss"] == pytest.approx(0.5 * (1 + lam) * np.sum((W - what) ** 2), rel=1e-12)


def _symmetric_grid_rounding(w, bits):
    # The symmetric quantizer as defined in the astro-blog survey, section 1.2
    # (zero point 0, signed codes on [-2^(b-1), 2^(b-1) - 1]), with the scale
    # that maps the largest magnitude to the largest positive code:
    # s = max|w| / (2^(b-1) - 1); code = clamp(rint(w / s)); value s * code.
    top = 2 ** (bits - 1) - 1
    s = np.abs(w).max() / top
    code = np.clip(np.rint(w / s), -top - 1, top)
    return s * code


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("group", [-1, 16])
def test_symmetric_identity_hessian_is_plain_rounding(bits, group):
    W = 0.02 * rng(40 + bits).standard_normal((6, 32))
    U, _ = O.prepare_hinv(np.eye(32), 0.0)  # U = I: nothing is compensated
    out = O.quantize_layer(W, U, bits, group, block=8, symmetric=True)
    g = 32 if group == -1 else group
    ref = np.hstack([np.vstack([_symmetric_grid_rounding(r, bits) for r in W[:, k : k + g]]) for k in range(0, 32, g)])
    assert np.array_equal(out["Wq"], ref)
    assert np.all(out["zeros"] == 2 ** (bits - 1))


def test_symmetric_hand_example():
    # 3 bits: qmax = 3, s = 0.6 / 3 = 0.2, zero code 4. U = I.
    #   0.6 / 0.2 = 3 -> code 7; -0.25 / 0.2 = -1.25 -> -1 -> code 3;
    #   0.13 / 0.2 = 0.65 -> 1 -> code 5; 0 -> code 4
    U, _ = O.prepare_hinv(np.eye(4), 0.0)
    out = O.quantize_layer(np.array([[0.6, -0.25, 0.13, 0.0]]), U, 3, -1, block=128, symmetric=True)
    assert out["codes"].tolist() == [[7, 3, 5, 4]]
    assert out["scales"][0, 0] == pytest.approx(0.2, rel=1e-15) and out["zeros"][0, 0] == 4


@pytest.mark.parametrize("bits,group", [(4, -1), (3, 16), (2, 32)])
def test_symmetric_blocked_equals_unblocked_and_on_grid(bits, group):
    _, W, _, U, _ = sweep_case(5, 64, 400, 21)
    ref = O.quantize_layer(W, U, bits, group, block=1, symmetric=True)
    for B in (8, 32, 64):
        out = O.quantize_layer(W, U, bits, group, block=B, symmetric=True)
        assert np.array_equal(out["codes"], ref["codes"])
        assert np.allclose(out["Wq"], ref["Wq"], rtol=0, atol=1e-12)
    g = 64 if group == -1 else group
    sc = np.repeat(ref["scales"], g, axis=1)[:, :64]
    t = ref["Wq"] / sc + 2 ** (bits - 1)
    assert np.allclose(t, np.rint(t), atol=1e-9) and t.min() >= -1e-9 and t.max() <= 2**bits - 1 + 1e-9


def test_symmetric_gptq_beats_symmetric_rtn():
    X, W, H, U, lam = sweep_case(12, 48, 300, 5)
    out = O.quantize_layer(W, U, 3, -1, symmetric=True)
    codes, scales, zeros = O.rtn(W, 3, -1, symmetric=True)
    rtn_loss = O.layer_loss_direct(X, W, O.dequantize(codes, scales, zeros, -1), lam)
    assert out["loss"] < rtn_loss


def test_dequant_matvec_hand_example():
    # 2 rows, 3 columns, 4-bit, one group per row:
    #   row 0: s = 0.5, z = 8, codes [9, 7, 8] -> What [0.5, -0.5, 0]
    #   row 1: s = 2,   z = 1, codes [3, 1, 0] -> What [4, 0, -2]
    #   x = [[1, 2, 3], [0, 0, 1]] -> Y = [[-0.5, -2], [0, -2]]
    codes = np.array([[9, 7, 8], [3, 1, 0]])
    packed = O.pack(codes, 4)
    scales = np.array([[0.5], [2.0]])
    zeros = np.array([[8.0], [1.0]])
    y = O.dequant_matvec(packed, scales, zeros, 3, 4, -1, np.array([[1.0, 2.0, 3.0], [0.0, 0.0, 1.0]]))
    assert y.tolist() == [[-0.5, -2.0], [0.0, -2.0]]


@pytest.mark.parametrize("bits,group", [(3, 16), (4, 32), (2, -1), (8, 16)])
def test_dequant_matvec_unit_vectors_read_the_dequantized_columns(bits, group):
    # e_c picks column c of What = s (code - z); checked against the sweep's
    # own dequantized weights (Wq), which the on-grid pin ties to the codes.
    _, W, _, U, _ = sweep_case(3, 48, 200, 31)
    out = O.quantize_layer(W, U, bits, group, block=16)
    y = O.dequant_matvec(out["packed"], out["scales"], out["zeros"], 48, bits, group, np.eye(48))
    assert np.allclose(y.T, out["Wq"], rtol=0, atol=1e-15)


def test_decision_margins():
    # w/s = 2.5 (exact tie), 3.0, 2.4, -0.75 -> distance to the nearest
    # rounding boundary 0, 0.5, 0.1, 0.25 grid steps
    s = np.full(4, 0.125)
    c, m = O.quantize_codes(np.array([2.5, 3.0, 2.4, -0.75]) * 0.125, s, np.zeros(4), 4, with_margin=True)
    assert c.tolist() == [2, 3, 2, 0]
    assert m == pytest.approx([0.0, 0.5, 0.1, 0.25], abs=1e-12)
    # range [-0.3, 0.9] at 2 bits: s = 0.4, -xmin/s = 0.75 -> z = 1, margin 0.25
    s, z, zm = O.group_params(np.array([[-0.3, 0.9]]), 2, with_margin=True)
    assert s[0] == pytest.approx(0.4, rel=1e-15) and z[0] == 1 and zm[0] == pytest.approx(0.25, abs=1e-12)
    # with H = I nothing is compensated: each code's margin is that of the
    # weight itself on the round-to-nearest grid
    W = 0.02 * rng(5).standard_normal((5, 32))
    U, _ = O.prepare_hinv(np.eye(32), 0.0)
    out = O.quantize_layer(W, U, 3, 16, block=8)
    sc = np.repeat(out["scales"], 16, axis=1)
    t = W / sc
    assert out["code_margin"] == pytest.approx(0.5 - np.abs(t - np.rint(t)), abs=1e-12)
    assert out["zero_margin"].shape == (5, 2)
    assert np.all((out["code_margin"] >= 0) & (out["code_margin"] <= 0.5))


@pytest.mark.parametrize("bits,group,blocks", [(4, -1, [1, 2, 3, 5, 16, 128, 64]), (3, 8, [1, 2, 4, 8, 16, 32, 64]), (2, 32, [1, 4, 8, 32, 64])])
def test_blocked_equals_unblocked(bits, group, blocks):
    _, W, _, U, _ = sweep_case(6, 64, 400, 11)
    ref = O.quantize_layer(W, U, bits, group, block=1)
    for B in blocks:
        out = O.quantize_layer(W, U, bits, group, block=B)
        assert np.array_equal(out["codes"], ref["codes"]), B
        assert np.allclose(out["Wq"], ref["Wq"], rtol=1e-12, atol=1e-15), B
        assert out["loss"] == pytest.approx(ref["loss"], rel=1e-12)


@pytest.mark.parametrize("damp", [0.0, 0.01, 0.3])
@pytest.mark.parametrize("group", [-1, 4])
def test_loss_identity(damp, group):
    X, W, H, U, lam = sweep_case(5, 16, 200, 3, damp)
    out = O.quantize_layer(W, U, 3, group, block=8)
    direct = O.layer_loss_direct(X, W, out["Wq"], lam)
    assert out["loss"] == pytest.approx(direct, rel=1e-10)
    # per row: half the H_d-weighted quadratic of the weight error
    D = W - out["Wq"]
    Hd = H + lam * np.eye(16)
    assert np.allclose(out["row_loss"], 0.5 * np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-10)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_on_grid(bits):
    _, W, _, U, _ = sweep_case(9, 40, 300, 5)
    for group in (-1, 8):
        out = O.quantize_layer(W, U, bits, group, block=8)
        gi = np.zeros(40, int) if group == -1 else np.arange(40) // group
        t = out["Wq"] / out["scales"][:, gi] + out["zeros"][:, gi]
        assert np.allclose(t, np.rint(t), atol=1e-9)
        assert t.min() > -1e-9 and t.max() < (1 << bits) - 1 + 1e-9
        assert np.array_equal(np.rint(t).astype(np.uint8), out["codes"])
        assert np.all((out["zeros"] >= 0) & (out["zeros"] <= (1 << bits) - 1))


def brute_force(W, Hd, bits, group):
    """Re-solve the free columns directly after every rounding.

    After columns 0..q are fixed at their dequantized values, the remaining
    weights v_R minimise (v - w)^T H_d (v - w); the minimiser is
    v_R = w_R - H_RR^{-1} H_RF (v_F - w_F). Column q+1 is then rounded from
    that v. No Cholesky rows are used.
    """
    d_row, d = W.shape
    codes = np.zeros((d_row, d), np.uint8)
    Wq = np.zeros((d_row, d))
    for r in range(d_row):
        w = W[r].astype(float)
        v = w.copy()
        if group == -1:
            s, z = O.group_params(w[None, :], bits)
        for q in range(d):
            if group != -1 and q % group == 0:
                s, z = O.group_params(v[None, q : q + group], bits)
            c = O.quantize_codes(v[q : q + 1], s, z, bits)
            codes[r, q] = c[0]
            Wq[r, q] = (s * (c - z))[0]
            F = np.arange(q + 1)
            R = np.arange(q + 1, d)
            v[F] = Wq[r, F]
            if len(R):
                v[R] = w[R] - np.linalg.solve(Hd[np.ix_(R, R)], Hd[np.ix_(R, F)] @ (v[F] - w[F]))
    return codes, Wq


@pytest.mark.parametrize("bits,group,seed", list(itertools.product([2, 3, 4], [-1, 2], [0, 1, 2])))
def test_brute_force_4x4(bits, group, seed):
    X, W, H, U, lam = sweep_case(4, 4, 9, 100 + seed)
    W = W * 50  # spread the weights over several grid steps
    Hd = H + lam * np.eye(4)
    codes, Wq = brute_force(W, Hd, bits, group)
    for B in (1, 2, 4):
        out = O.quantize_layer(W, U, bits, group, block=B)
        assert np.array_equal(out["codes"], codes)
        assert np.allclose(out["Wq"], Wq, atol=1e-12)


def test_row_independence():
    _, W, _, U, _ = sweep_case(12, 32, 200, 8)
    full = O.quantize_layer(W, U, 4, 8, block=16)
    rows = np.array([0, 3, 4, 11])
    sub = O.quantize_layer(W[rows], U, 4, 8, block=16)
    assert np.array_equal(sub["codes"], full["codes"][rows])
    assert np.allclose(sub["row_loss"], full["row_loss"][rows], rtol=1e-13)
    assert np.array_equal(sub["scales"], full["scales"][rows])


def test_hessian_scale_invariance():
    _, W, H, _, _ = sweep_case(6, 24, 150, 9)
    U1, _ = O.prepare_hinv(H, 0.01)
    U2, _ = O.prepare_hinv(7.3 * H, 0.01)
    a = O.quantize_layer(W, U1, 3, 8, block=8)
    b = O.quantize_layer(W, U2, 3, 8, block=8)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.allclose(a["scales"], b["scales"], rtol=1e-12)
    assert b["loss"] == pytest.approx(7.3 * a["loss"], rel=1e-10)


def test_gptq_beats_rtn_on_correlated_inputs():
    # Not a theorem, but the pages' central claim (xuzou.cn, section 证据).
    r = rng(21)
    base = r.standard_normal((2000, 8))
    X = base @ r.standard_normal((8, 32)) + 0.1 * r.standard_normal((2000, 32))
    W = 0.02 * r.standard_normal((16, 32))
    H = O.hessian(X)
    U, lam = O.prepare_hinv(H, 0.01)
    out = O.quantize_layer(W, U, 3, -1, block=8)
    codes, scales, zeros = O.rtn(W, 3, -1)
    rtn_loss = O.layer_loss_direct(X, W, O.dequantize(codes, scales, zeros, -1), lam)
    assert out["loss"] < rtn_loss


def test_rejects_bad_arguments():
    U = np.eye(8)
    W = np.zeros((2, 8))
    with pytest.raises(ValueError):
        O.quantize_layer(W, U, 5, -1)
    with pytest.raises(ValueError):
        O.quantize_layer(W, U, 4, 3, block=8)  # neither divides the other
    with pytest.raises(ValueError):
        O.quantize_layer(W, np.eye(7), 4, -1)


def test_all_zero_row_and_degenerate_group():
    W = np.zeros((2, 8))
    W[1, 4:] = 0.5
    out = O.quantize_layer(W, np.eye(8), 4, 4, block=4)
    # all-zero group -> range [-1, 1]: s = 2/15, z = rint(7.5) = 8 (ties to even)
    assert out["scales"][0, 0] == pytest.approx(2 / 15)
    assert out["zeros"][0, 0] == 8
    assert np.all(out["Wq"][0] == 0)
    # positive-only group -> range [0, 0.5], z = 0, every 0.5 maps to code 15
    assert out["zeros"][1, 1] == 0 and np.all(out["codes"][1, 4:] == 15)


# ------------------------------------------------------------------ pack
def bigint_words(row, bits):
    """Independent packing: the row as one big integer, cut into 32-bit words."""
    v = 0
    for j, c in enumerate(row):
        v |= int(c) << (bits * j)
    nw = -(-len(row) * bits // 32)
    return [(v >> (32 * k)) & 0xFFFFFFFF for k in range(nw)]


def test_pack_hand_example_3bit():
    codes = np.array([[j % 8 for j in range(16)]], dtype=np.uint8)
    w = O.pack(codes, 3)
    # word 0: codes 0..9 at 3-bit steps, then the low 2 bits of code 10 (=2) at bit 30
    w0 = sum((j % 8) << (3 * j) for j in range(10)) | ((10 % 8) & 3) << 30
    # word 1: the high bit of code 10, then codes 11..15 from bit 1
    w1 = ((10 % 8) >> 2) | sum(((j % 8) << (3 * j - 32)) for j in range(11, 16))
    assert w.shape == (1, 2)
    assert int(w[0, 0]) == w0 and int(w[0, 1]) == w1


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d_col", [1, 7, 10, 11, 32, 33, 128, 200])
def test_pack_matches_bigint_and_roundtrips(bits, d_col):
    codes = rng(bits * d_col).integers(0, 1 << bits, size=(3, d_col)).astype(np.uint8)
    w = O.pack(codes, bits)
    assert w.shape == (3, O.words_per_row(d_col, bits))
    for r in range(3):
        assert [int(x) for x in w[r]] == bigint_words(codes[r], bits)
    assert np.array_equal(O.unpack(w, d_col, bits), codes)


# ------------------------------------------------------ mutation checks
def test_brute_force_catches_planted_mistakes():
    """Plant plausible mistakes in the oracle's inputs and check the pin fails."""
    X, W, H, U, lam = sweep_case(4, 4, 9, 7)
    W = W * 50
    Hd = H + lam * np.eye(4)
    codes, Wq = brute_force(W, Hd, 3, -1)
    Hinv = np.linalg.inv(Hd)
    mutants = {
        # the pages' demo loop: raw rows of the full inverse, no Cholesky rows
        "raw_inverse_rows": np.triu(Hinv / np.sqrt(np.diag(Hinv))[:, None]),
        "sign_flipped": 2 * np.diag(np.diag(U)) - U,
        "transposed": np.triu(U.T) + np.tril(np.zeros_like(U)),
        "dropped_diagonal_scale": np.triu(U, 1) + np.eye(4),
    }
    for name, Ubad in mutants.items():
        out = O.quantize_layer(W, Ubad, 3, -1, block=2)
        same = np.array_equal(out["codes"], codes) and np.allclose(out["Wq"], Wq, atol=1e-12)
        loss_ok = abs(out["loss"] - O.layer_loss_direct(X, W, out["Wq"], lam)) < 1e-10 * max(1.0, out["loss"])
        assert not (same and loss_ok), name


def test_run_quantized_layer_hand_example():
    # 2-bit codes [[1, 2], [3, 0]], one group per row, s = [0.5, 0.25], z = [1, 2]:
    # What = [[0, 0.5], [0.25, -0.5]]. X = [[2, 4], [1, -1]]:
    # X What^T = [[2, -1.5], [-0.5, 0.75]]; with ReLU [[2, 0], [0, 0.75]].
    packed = O.pack(np.array([[1, 2], [3, 0]]), 2)
    scales = np.array([[0.5], [0.25]], np.float32)
    zeros = np.array([[1], [2]])
    X = np.array([[2, 4], [1, -1]], np.float16)
    y = O.run_quantized_layer(X, packed, scales, zeros, 2, 2, -1)
    assert y.dtype == np.float16 and y.tolist() == [[2.0, -1.5], [-0.5, 0.75]]
    assert O.run_quantized_layer(X, packed, scales, zeros, 2, 2, -1, relu=True).tolist() == [[2.0, 0.0], [0.0, 0.75]]
    # the sum is rounded to fp16 once: 1 + 2^-11 + 2^-11 is exactly 1 + 2^-10
    packed = O.pack(np.array([[1, 1, 1]]), 2)
    X = np.array([[1.0, 2.0**-11, 2.0**-11]], np.float16)
    y = O.run_quantized_layer(X, packed, np.ones((1, 1), np.float32), np.zeros((1, 1)), 3, 2, -1)
    assert float(y[0, 0]) == 1.0 + 2.0**-10
