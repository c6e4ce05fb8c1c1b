"""Pins of the oracle's column-order variants (act-order and the greedy OBQ
order) and of its calibration pipeline (layers sharing an input, an MLP
block quantized layer by layer). No GPU.

Each pin checks the oracle against something other than itself: a hand
example, a pairwise restatement of the order, an invariance, the loss
identity in the original coordinates, a re-derivation of every greedy step
with directly inverted sub-Hessians, propagated activations re-derived entry
by entry, and planted mistakes (a wrong permutation composition,
full-precision propagation) that the pins must catch.
"""

import numpy as np
import pytest

import oracle.gptq_oracle as O


def _xh(seed, n, d, outliers=True):
    r = np.random.default_rng(seed)
    X = r.standard_normal((n, d))
    if outliers:  # a few loud channels, so the order matters
        X[:, r.choice(d, max(1, d // 5), replace=False)] *= 8.0
    return X, 2.0 * X.T @ X


def test_act_order_perm_hand_example():
    h = np.array([1.0, 3.0, 3.0, np.nan, 0.0, 2.0, -0.0, np.nan])
    assert O.act_order_perm(np.diag(h)).tolist() == [1, 2, 5, 0, 4, 6, 3, 7]


def test_act_order_perm_pairwise_order_with_ties():
    r = np.random.default_rng(3)
    h = r.integers(0, 6, size=200).astype(float)
    h[r.choice(200, 7, replace=False)] = np.nan
    p = O.act_order_perm(np.diag(h))
    assert sorted(p.tolist()) == list(range(200))
    for a in range(199):
        i, j = p[a], p[a + 1]
        hi, hj = h[i], h[j]
        if np.isnan(hi):
            assert np.isnan(hj) and i < j
        elif not np.isnan(hj):
            assert hi > hj or (hi == hj and i < j)


def test_inverse_perm():
    p = np.array([3, 0, 2, 1])
    inv = O.inverse_perm(p)
    assert inv.tolist() == [1, 3, 2, 0]
    assert np.array_equal(p[inv], np.arange(4)) and np.array_equal(inv[p], np.arange(4))


def test_act_order_with_descending_diag_is_the_natural_order():
    X, H = _xh(1, 64, 12, outliers=False)
    order = np.argsort(-np.diag(H), kind="stable")
    X, H = X[:, order], H[np.ix_(order, order)]  # diag now descending
    W = np.random.default_rng(2).standard_normal((5, 12))
    r = O.quantize_layer_act_order(W, H, 3, 4, block=4, damp=0.01)
    assert r["perm"].tolist() == list(range(12))
    U, _ = O.prepare_hinv(H, 0.01)
    ref = O.quantize_layer(W, U, 3, 4, block=4)
    assert np.array_equal(r["codes"], ref["codes"]) and np.array_equal(r["Wq_orig"], ref["Wq"])


@pytest.mark.parametrize("group", [-1, 4, 8])
def test_act_order_equivariance_under_input_permutation(group):
    X, H = _xh(4, 80, 16)
    W = np.random.default_rng(5).standard_normal((6, 16))
    P = np.random.default_rng(6).permutation(16)
    a = O.quantize_layer_act_order(W, H, 4, group, block=8)
    b = O.quantize_layer_act_order(W[:, P], H[np.ix_(P, P)], 4, group, block=8)
    assert np.array_equal(b["Wq_orig"], a["Wq_orig"][:, P])
    assert b["loss"] == a["loss"]


@pytest.mark.parametrize("bits,group", [(2, -1), (3, 4), (4, 8)])
def test_act_order_loss_identity_in_original_coordinates(bits, group):
    X, H = _xh(7, 96, 16)
    W = np.random.default_rng(8).standard_normal((5, 16))
    r = O.quantize_layer_act_order(W, H, bits, group, block=8, damp=0.05)
    direct = O.layer_loss_direct(X, W, r["Wq_orig"], r["lam"])
    assert r["loss"] == pytest.approx(direct, rel=1e-9)
    per_row = [O.layer_loss_direct(X, W[i : i + 1], r["Wq_orig"][i : i + 1], r["lam"]) for i in range(5)]
    assert np.allclose(r["row_loss"], per_row, rtol=1e-9)


def test_act_order_loss_identity_catches_a_wrong_composition():
    # Mutation: columns of W taken by the inverse permutation while the
    # Hessian is permuted by p. The identity must fail.
    X, H = _xh(9, 96, 16)
    W = np.random.default_rng(10).standard_normal((5, 16))
    p = O.act_order_perm(H)
    inv = O.inverse_perm(p)
    assert not np.array_equal(p, inv)
    U, lam = O.prepare_hinv(H[np.ix_(p, p)], 0.05)
    bad = O.quantize_layer(W[:, inv], U, 3, 4, block=8)
    wq_orig = bad["Wq"][:, O.inverse_perm(inv)]
    assert abs(bad["loss"] - O.layer_loss_direct(X, W, wq_orig, lam)) > 1e-6 * bad["loss"]


def test_act_order_groups_follow_the_permuted_order():
    X, H = _xh(11, 96, 16)
    W = np.random.default_rng(12).standard_normal((4, 16))
    r = O.quantize_layer_act_order(W, H, 3, 4, block=8)
    inv = O.inverse_perm(r["perm"])
    codes_orig = r["codes"][:, inv]
    g = r["g_idx"]
    assert np.array_equal(g, inv // 4)
    recon = r["scales"][:, g] * (codes_orig - r["zeros"][:, g])
    assert np.array_equal(recon, r["Wq_orig"])
    # every permuted group of 4 columns shares one grid, on which it lies
    for k in range(4):
        t = r["Wq"][:, 4 * k : 4 * k + 4] / r["scales"][:, k : k + 1] + r["zeros"][:, k : k + 1]
        assert np.allclose(t, np.rint(t), atol=1e-9)


def test_obq_in_natural_order_equals_the_fixed_order_sweep():
    X, H = _xh(13, 80, 10)
    W = np.random.default_rng(14).standard_normal((6, 10))
    U, _ = O.prepare_hinv(H, 0.01)
    ref = O.quantize_layer(W, U, 3, -1, block=128)
    ob = O.obq_greedy(W, H, 3, damp=0.01, order=np.arange(10))
    assert np.array_equal(ob["codes"], ref["codes"])
    assert np.allclose(ob["Wq"], ref["Wq"], rtol=0, atol=1e-12)
    assert ob["loss"] == pytest.approx(ref["loss"], rel=1e-9)


def test_obq_greedy_steps_against_directly_inverted_sub_hessians():
    X, H = _xh(15, 60, 7)
    W = np.random.default_rng(16).standard_normal((4, 7))
    damp, bits = 0.02, 3
    ob = O.obq_greedy(W, H, bits, damp=damp)
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(7)
    maxq = (1 << bits) - 1
    for r in range(4):
        w = W[r].copy()
        lo, hi = min(w.min(), 0.0), max(w.max(), 0.0)
        s = (hi - lo) / maxq
        z = np.rint(-lo / s)
        quant = lambda v: s * (np.clip(np.rint(v / s) + z, 0, maxq) - z)
        free = list(range(7))
        loss = 0.0
        for step in range(7):
            Hi = np.linalg.inv(Hd[np.ix_(free, free)])
            cost = [(w[f] - quant(w[f])) ** 2 / Hi[k, k] for k, f in enumerate(free)]
            k = int(np.argmin(cost))
            q = free[k]
            assert ob["order"][r, step] == q
            err = w[q] - quant(w[q])
            loss += err * err / (2 * Hi[k, k])
            w[free] -= err / Hi[k, k] * Hi[:, k]
            w[q] = quant(w[q])
            free.remove(q)
        assert np.allclose(ob["Wq"][r], w, atol=1e-12)
        assert ob["row_loss"][r] == pytest.approx(loss, rel=1e-9)


def test_obq_greedy_with_diagonal_hessian_is_round_to_nearest():
    W = np.random.default_rng(17).standard_normal((5, 9))
    H = np.diag(np.random.default_rng(18).uniform(1.0, 3.0, 9))
    ob = O.obq_greedy(W, H, 4, damp=0.0)
    codes, _, _ = O.rtn(W, 4, -1)
    assert np.array_equal(ob["codes"], codes)


# ----------------------------------------------------------------------------
# Calibration pipeline: layers sharing an input, and a block layer by layer
# ----------------------------------------------------------------------------
def test_shared_input_is_the_chunked_hessian_and_per_layer_sweeps():
    X, _ = _xh(19, 120, 12)
    Ws = [np.random.default_rng(20 + i).standard_normal((3 + i, 12)) for i in range(3)]
    r = O.quantize_shared_input([X[:50], X[50:90], X[90:]], Ws, 3, 4, block=4, damp=0.02)
    assert np.allclose(r["H"], 2.0 * X.T @ X, rtol=1e-12, atol=1e-12)
    for W, layer in zip(Ws, r["layers"]):
        one = O.quantize_layer(W, r["U"], 3, 4, block=4)
        assert np.array_equal(layer["codes"], one["codes"]) and layer["loss"] == one["loss"]
        # each layer's loss is its own output error on the shared input
        assert layer["loss"] == pytest.approx(O.layer_loss_direct(X, W, layer["Wq"], r["lam"]), rel=1e-9)


def test_model_weight_f16_rounds_the_float32_product():
    codes = np.array([[0, 7, 3]])
    s = np.array([[0.1]], np.float32)
    z = np.array([[2]])
    got = O.model_weight_f16(codes, s, z, -1)
    want = np.array([np.float16(np.float32(0.1) * np.float32(k)) for k in (-2, 5, 1)])
    assert got.dtype == np.float16 and np.array_equal(got[0], want)


def _mlp(seed, n=160, d_model=16, d_ff=24):
    r = np.random.default_rng(seed)
    X0 = r.standard_normal((n, d_model)).astype(np.float16)
    W_up = (0.3 * r.standard_normal((d_ff, d_model))).astype(np.float16)
    W_down = (0.3 * r.standard_normal((d_model, d_ff))).astype(np.float16)
    return X0, W_up, W_down


def test_mlp_block_propagates_through_the_quantized_up_layer():
    X0, W_up, W_down = _mlp(21)
    b = O.quantize_mlp_block(X0, W_up, W_down, 4, 8, block=8, damp=0.02)
    up, down = b["up"], b["down"]
    # X1 entries re-derived one by one: relu of the dot product with the fp16 model weight
    s32 = up["scales"].astype(np.float32)
    for i, j in [(0, 0), (5, 3), (159, 23), (77, 11)]:
        w = [np.float16(s32[j, c // 8] * np.float32(int(up["codes"][j, c]) - int(up["zeros"][j, c // 8])))
             for c in range(16)]
        dot = sum(float(X0[i, c]) * float(w[c]) for c in range(16))
        assert b["X1"][i, j] == np.float16(max(dot, 0.0))
    # each layer's loss is its output error on the input it was calibrated with
    assert up["loss"] == pytest.approx(O.layer_loss_direct(X0, W_up, up["Wq"], up["lam"]), rel=1e-9)
    assert down["loss"] == pytest.approx(O.layer_loss_direct(b["X1"], W_down, down["Wq"], down["lam"]), rel=1e-9)
    # the block output is the quantized down layer applied to X1
    Wd = O.model_weight_f16(down["codes"], down["scales"], down["zeros"], 8).astype(np.float64)
    assert np.array_equal(b["X2"], (b["X1"].astype(np.float64) @ Wd.T).astype(np.float16))


def test_mlp_block_down_hessian_is_not_from_full_precision_activations():
    # Mutation: activations propagated through the unquantized up layer. The
    # down layer's loss identity then fails, so the pin sees which input the
    # down layer was calibrated with.
    X0, W_up, W_down = _mlp(22)
    b = O.quantize_mlp_block(X0, W_up, W_down, 3, 8, block=8, damp=0.02)
    X1_fp = np.maximum(X0.astype(np.float64) @ W_up.astype(np.float64).T, 0.0).astype(np.float16)
    assert not np.array_equal(X1_fp, b["X1"])
    down = b["down"]
    direct_fp = O.layer_loss_direct(X1_fp, W_down, down["Wq"], down["lam"])
    assert abs(direct_fp - down["loss"]) > 1e-6 * down["loss"]
