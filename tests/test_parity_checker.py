"""The parity checker of tests/parity.py, exercised on the CPU.

The tested side here is made by the oracle itself: once from weights moved
by about 1e-7 relative (the size of float32 rounding), which must pass with
its near-tie flips followed, and once with planted mistakes, which must fail.
"""

import numpy as np
import pytest

import oracle.gptq_oracle as O
from tests.parity import ParityError, LayerOutputs, check_quant, rerun_for
from tests.test_oracle_pins import sweep_case


def as_outputs(out):
    return LayerOutputs(codes=out["codes"].copy(), scales=out["scales"].copy(), zeros=out["zeros"].astype(np.int32),
                  packed=out["packed"].copy(), row_loss=out["row_loss"].copy())


def layer(bits, group, seed=5, d_row=120, d_col=256):
    X, W, H, U, lam = sweep_case(d_row, d_col, 700, seed)
    return W * 30, U


@pytest.mark.parametrize("bits,group", [(4, 32), (3, -1), (8, 16), (2, 128)])
def test_noisy_rows_pass_through_their_near_tie_flips(bits, group):
    W, U = layer(bits, group)
    ref = O.quantize_layer(W, U, bits, group, 128, decide=np.float32)
    noisy = W * (1 + 2e-7 * np.random.default_rng(bits).standard_normal(W.shape))
    out = O.quantize_layer(noisy, U, bits, group, 128)
    s = check_quant(as_outputs(out), ref, bits, rerun_for(W, U, bits, group), max_flip_rows=0.5, log=None)
    assert s["match_followed"] == 1.0
    if bits == 8:
        assert s["flipped_rows"] > 0  # 255 levels: some decision always lands near a tie


def test_flipped_row_needs_the_near_tie():
    W, U = layer(4, 32)
    ref = O.quantize_layer(W, U, 4, 32, 128, decide=np.float32)
    # a row's nearest decision to a tie, and one far from any tie
    r = int(np.argmax(ref["code_margin"].min(axis=1) < 1e-3))
    near = int(np.argmin(ref["code_margin"][r]))
    far = int(np.argmax(ref["code_margin"][r]))
    assert ref["code_margin"][r, near] < 1e-3 < ref["code_margin"][r, far]
    ok = O.quantize_layer(W, U, 4, 32, 128, decide=np.float32, flips=[(r, "code", near)])
    check_quant(as_outputs(ok), ref, 4, rerun_for(W, U, 4, 32), log=None)
    bad = O.quantize_layer(W, U, 4, 32, 128, decide=np.float32, flips=[(r, "code", far)])
    with pytest.raises(ParityError, match="not a near-tie"):
        check_quant(as_outputs(bad), ref, 4, rerun_for(W, U, 4, 32), log=None)


def test_planted_mistakes_fail():
    W, U = layer(3, 64)
    ref = O.quantize_layer(W, U, 3, 64, 128, decide=np.float32)
    rerun = rerun_for(W, U, 3, 64)
    base = as_outputs(ref)
    check_quant(base, ref, 3, rerun, log=None)
    far = np.unravel_index(np.argmax(ref["code_margin"] * (ref["codes"] < 6)), ref["codes"].shape)

    t = as_outputs(ref)
    t.codes[far] += 1
    t.packed = O.pack(t.codes, 3)
    with pytest.raises(ParityError):
        check_quant(t, ref, 3, rerun, log=None)

    t = as_outputs(ref)
    t.codes[far] = (t.codes[far] + 2) % 8
    t.packed = O.pack(t.codes, 3)
    with pytest.raises(ParityError):
        check_quant(t, ref, 3, rerun, log=None)

    t = as_outputs(ref)
    t.scales[3, 1] *= 1.01
    with pytest.raises(ParityError, match="scale"):
        check_quant(t, ref, 3, rerun, log=None)

    t = as_outputs(ref)
    t.zeros[4, 2] += 1
    with pytest.raises(ParityError):
        check_quant(t, ref, 3, rerun, log=None)

    t = as_outputs(ref)
    t.row_loss[5] *= 1.05
    with pytest.raises(ParityError, match="loss"):
        check_quant(t, ref, 3, rerun, log=None)

    t = as_outputs(ref)
    t.packed[0, 0] ^= 1
    with pytest.raises(ParityError, match="packed"):
        check_quant(t, ref, 3, rerun, log=None)


def test_flipped_row_count_is_bounded():
    W, U = layer(4, 32)
    ref = O.quantize_layer(W, U, 4, 32, 128, decide=np.float32)
    rows = np.flatnonzero(ref["code_margin"].min(axis=1) < 1e-3)[:6]
    assert rows.size == 6
    flips = [(int(r), "code", int(np.argmin(ref["code_margin"][r]))) for r in rows]
    out = O.quantize_layer(W, U, 4, 32, 128, decide=np.float32, flips=flips)
    check_quant(as_outputs(out), ref, 4, rerun_for(W, U, 4, 32), max_flip_rows=0.05, log=None)
    with pytest.raises(ParityError, match="rows took"):
        check_quant(as_outputs(out), ref, 4, rerun_for(W, U, 4, 32), max_flip_rows=0.02, log=None)
