"""Parity of the calibration pipeline (layers sharing an input, an MLP block
quantized layer by layer) and of the dequantization, with the oracle (needs
an MI355X).

* gptq_dequantize: bit-exact against the float32 product rounded to the
  output type.
* Shared input: one Hessian over the chunks, one factor, each layer swept
  with it; each layer against the oracle as the plain sweep is compared, and
  the per-layer sweeps bit-exact against one stacked sweep of all rows
  (rows are independent given the factor).
* MLP block, end to end: the up layer against the oracle through near-tie
  continuations (tests/parity.py), which gives the oracle rows the GPU rows
  matched. The oracle runs its own quantized up layer from those rows on X0
  (X1'), and the GPU's X1 must lie within the fp32-summation bound of X1'
  element by element, allowing every fp16 weight one step of its own where
  the GPU's fp32 scale rounded differently. The oracle then quantizes the
  down layer from X1' alone, and the GPU's down layer (its own X1, H, U)
  passes the same continuation check against it; the block outputs X2 agree
  to fp16 rounding.
"""

import numpy as np
import pytest
import torch

import oracle.gptq_oracle as O
import post_weight_quantization_17_amd.pipeline as P
from tests.parity import rerun_for
from tests.test_gpu_parity import DEV, check_quant, gpu_tensor, rel_fro, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d_row,d_col,bits,group,dtype", [
    (1, 1, 4, -1, torch.float16),
    (7, 33, 3, 16, torch.float32),
    (5, 31, 2, 8, torch.float16),
    (64, 256, 4, 128, torch.float16),
    (100, 1000, 3, 40, torch.float32),
    (33, 4096, 8, 128, torch.float16),
])
def test_dequantize_parity(gpu, d_row, d_col, bits, group, dtype):
    r = np.random.default_rng(d_row + d_col)
    codes = r.integers(0, 2**bits, size=(d_row, d_col))
    ng = 1 if group == -1 else -(-d_col // group)
    scales = r.uniform(-0.05, 0.05, size=(d_row, ng)).astype(np.float32)
    zeros = r.integers(0, 2**bits, size=(d_row, ng)).astype(np.int32)
    packed = O.pack(codes, bits)
    out = gpu.gptq_dequantize(gpu_tensor(packed.view(np.int32)), gpu_tensor(scales), gpu_tensor(zeros), d_col, bits,
                              group, dtype)
    torch.cuda.synchronize()
    gi = np.zeros(d_col, np.int64) if group == -1 else np.arange(d_col) // group
    ref32 = scales[:, gi] * (codes - zeros[:, gi]).astype(np.float32)
    ref = ref32.astype(np.float16) if dtype == torch.float16 else ref32
    assert np.array_equal(out.cpu().numpy().view(np.uint8), ref.view(np.uint8))
    if dtype == torch.float16:
        assert np.array_equal(out.cpu().numpy(), O.model_weight_f16(codes, scales, zeros, group))


def test_dequantize_strided_output_and_bad_arguments(gpu):
    r = np.random.default_rng(3)
    codes = r.integers(0, 16, size=(9, 70))
    scales = r.uniform(0.01, 0.02, size=(9, 1)).astype(np.float32)
    zeros = r.integers(0, 16, size=(9, 1)).astype(np.int32)
    buf = torch.full((9, 80), -7.0, dtype=torch.float32, device=DEV)
    gpu.gptq_dequantize(gpu_tensor(O.pack(codes, 4).view(np.int32)), gpu_tensor(scales), gpu_tensor(zeros), 70, 4,
                        -1, out=buf[:, :70])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[:, :70], scales * (codes - zeros).astype(np.float32))
    assert np.all(got[:, 70:] == -7.0)  # untouched past d_col
    lib = gpu.load()
    p = buf.data_ptr()
    E = gpu.GPTQ_E_INVALID_ARG
    assert lib.gptq_dequantize(p, p, p, 4, 16, 5, -1, p, gpu.GPTQ_F32, 16, None) == E  # bits
    assert lib.gptq_dequantize(p, p, p, 4, 16, 4, 0, p, gpu.GPTQ_F32, 16, None) == E  # group
    assert lib.gptq_dequantize(p, p, p, 4, 16, 4, -1, p, 7, 16, None) == E  # dtype
    assert lib.gptq_dequantize(p, p, p, 4, 16, 4, -1, p, gpu.GPTQ_F32, 15, None) == E  # ld_out


def shared_inputs(seed, n, d, rows):
    r = np.random.default_rng(seed)
    X = r.standard_normal((n, d)).astype(np.float32)
    X[:, r.choice(d, max(1, d // 100), replace=False)] *= 20.0
    X *= r.lognormal(0.0, 0.5, size=(n, 1)).astype(np.float32)
    X = X.astype(np.float16)
    Ws = [(0.02 * r.standard_normal((k, d))).astype(np.float16) for k in rows]
    return X, Ws


@pytest.mark.parametrize("bits,group", [(4, 128), (3, -1)])
def test_shared_input_group(gpu, bits, group):
    """q/k/v: one Hessian over three calibration chunks, one factor, each
    layer swept with it."""
    d, rows = 640, (96, 96, 160)
    X, Ws = shared_inputs(11 + bits, 6000, d, rows)
    cuts = [0, 2000, 4100, 6000]
    chunks = [gpu_tensor(X[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    H, hv, layers = P.quantize_shared_input(chunks, [gpu_tensor(W) for W in Ws], bits, group)
    stacked = gpu.gptq_quantize_layer(torch.cat([gpu_tensor(W) for W in Ws]), hv.U, bits, group, 128)
    torch.cuda.synchronize()
    ref = O.quantize_shared_input([X[a:b] for a, b in zip(cuts[:-1], cuts[1:])], Ws, bits, group, damp=0.01,
                                  decide=np.float32)
    e = rel_fro(H.cpu().numpy(), ref["H"])
    say(f"shared input: H rel fro {e:.3g}")
    assert e < 1e-4
    r0 = 0
    for k, lay in enumerate(layers):
        r1 = r0 + rows[k]
        for name in ("codes", "scales", "zeros", "packed", "row_loss"):
            assert torch.equal(getattr(lay, name), getattr(stacked, name)[r0:r1]), (k, name)
        r0 = r1
    # against the oracle, from the oracle's own factor (the GPU factor differs by rounding only)
    for W in Ws:
        qk = gpu.gptq_quantize_layer(gpu_tensor(W), gpu_tensor(ref["U"].astype(np.float32)), bits, group, 128)
        torch.cuda.synchronize()
        U32 = ref["U"].astype(np.float32).astype(np.float64)
        check_quant(qk, O.quantize_layer(W, U32, bits, group, 128, decide=np.float32), bits,
                    rerun_for(W, U32, bits, group))


def within_fp16_bound(Y, A, Wh, relu, a_step):
    """Y (GPU, fp16) = act(A Wh^T) as the GPU computes it, against the exact
    product of the oracle's operands: fp32 summation moves each sum by at
    most (K + 2) 2^-24 sum |a w|; each fp16 weight may sit one fp16 step off
    (where the GPU's fp32 scale rounded to the other neighbour) and, with
    ``a_step``, each input too (the inputs are themselves such fp16
    outputs). Rounding and ReLU are monotone, so Y must lie between the fp16
    roundings of the two ends. Returns the share equal to the oracle's
    fp16 value."""
    A = A.astype(np.float64)
    K = A.shape[1]
    step = lambda v: np.abs(v) * 2.0**-10 + 2.0**-24  # one fp16 step (at least the subnormal step)
    exact = A @ Wh.T
    absA, absW = np.abs(A), np.abs(Wh)
    bound = (K + 2) * 2.0**-24 * (absA @ absW.T) + absA @ step(Wh).T
    if a_step:
        bound += step(A) @ (absW + step(Wh)).T
    lo, hi = exact - bound, exact + bound
    if relu:
        lo, hi, exact = np.maximum(lo, 0.0), np.maximum(hi, 0.0), np.maximum(exact, 0.0)
    lo16, hi16 = lo.astype(np.float16).astype(np.float64), hi.astype(np.float16).astype(np.float64)
    g = Y.astype(np.float64)
    bad = (g < lo16) | (g > hi16)
    assert not bad.any(), f"{int(bad.sum())} outputs outside the bound"
    return float(np.mean(g == exact.astype(np.float16).astype(np.float64)))


def test_mlp_block_pipeline(gpu):
    """Up layer, ReLU, down layer, quantized in order on the GPU and by the
    oracle, end to end (module docstring)."""
    n, d_model, d_ff, bits, group = 4096, 512, 1376, 4, 128
    r = np.random.default_rng(31)
    X0 = r.standard_normal((n, d_model)).astype(np.float32)
    X0[:, r.choice(d_model, 5, replace=False)] *= 10.0
    X0 = X0.astype(np.float16)
    W_up = (0.05 * r.standard_normal((d_ff, d_model))).astype(np.float16)
    W_down = (0.05 * r.standard_normal((d_model, d_ff))).astype(np.float16)
    b = P.quantize_mlp_block(gpu_tensor(X0), gpu_tensor(W_up), gpu_tensor(W_down), bits, group)
    torch.cuda.synchronize()
    assert int(b["hinv_up"].info.item()) == 0 and int(b["hinv_down"].info.item()) == 0
    # up layer: the oracle's chain from X0
    H_up = O.hessian(X0)
    assert rel_fro(b["H_up"].cpu().numpy(), H_up) < 1e-4
    U_up, _ = O.prepare_hinv(H_up, 0.01)
    ref_up = O.quantize_layer(W_up, U_up, bits, group, 128, decide=np.float32)
    s_up = check_quant(b["up"], ref_up, bits, rerun_for(W_up, U_up, bits, group), label="up layer")
    m = s_up["matched"]
    # X1: the oracle's quantized up layer from the matched oracle rows
    X1_ref = O.run_quantized_layer(X0, O.pack(m["codes"], bits), m["scales"], m["zeros"], d_model, bits, group,
                                   relu=True)
    Wh_up = O.model_weight_f16(m["codes"], m["scales"], m["zeros"], group).astype(np.float64)
    same = within_fp16_bound(b["X1"].cpu().numpy(), X0, Wh_up, True, False)
    say(f"mlp block: X1 within the bound; equal to the oracle's fp16 value {same:.6f}")
    assert same >= 0.9
    # down layer: the oracle's chain from X1' alone, the GPU's from its own X1
    H_dn = O.hessian(X1_ref)
    eh = rel_fro(b["H_down"].cpu().numpy(), H_dn)
    say(f"mlp block: H_down rel fro {eh:.3g}")
    assert eh < 1e-4
    U_dn, _ = O.prepare_hinv(H_dn, 0.01)
    ref_dn = O.quantize_layer(W_down, U_dn, bits, group, 128, decide=np.float32)
    s_dn = check_quant(b["down"], ref_dn, bits, rerun_for(W_down, U_dn, bits, group), label="down layer, end to end")
    md = s_dn["matched"]
    Wh_dn = O.model_weight_f16(md["codes"], md["scales"], md["zeros"], group).astype(np.float64)
    same2 = within_fp16_bound(b["X2"].cpu().numpy(), X1_ref, Wh_dn, False, True)
    X2_ref = O.run_quantized_layer(X1_ref, O.pack(md["codes"], bits), md["scales"], md["zeros"], d_ff, bits, group)
    ex2 = rel_fro(b["X2"].cpu().numpy(), X2_ref)
    say(f"mlp block: X2 within the bound, rel fro {ex2:.3g}, equal to the oracle's fp16 value {same2:.6f}")
    assert ex2 < 2.0**-10 and same2 >= 0.8
