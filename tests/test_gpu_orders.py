"""Parity of the column-order path (act-order permutation, gathers, and the
act-order layer) with the oracle (needs an MI355X).

The permutation and the gathers are integer and byte work: bit-exact. The
act-order layer is compared as the plain sweep is (codes equal but for
one-step flips at near-ties, scales, packing, loss). Inputs come from seeded
generators and the oracle only.
"""

import numpy as np
import pytest
import torch

import oracle.gptq_oracle as O
from tests.parity import rerun_for
from tests.test_gpu_parity import DEV, check_quant, gpu_tensor, say

pytestmark = pytest.mark.gpu


def diag_with_ties(d, seed):
    r = np.random.default_rng(seed)
    h = r.integers(0, 9, size=d).astype(np.float32)  # many ties
    m = r.random(d) < 0.3
    h[m] = r.standard_normal(int(m.sum())).astype(np.float32)  # distinct values, some negative
    h[r.random(d) < 0.05] = -0.0
    h[r.random(d) < 0.02] = np.nan
    return h


@pytest.mark.parametrize("d", [1, 2, 7, 255, 256, 257, 2048, 2049, 5000])
def test_act_order_perm_parity(gpu, d):
    h = diag_with_ties(d, d)
    r = np.random.default_rng(d + 1)
    ld = d + 3
    H = r.standard_normal((d, ld)).astype(np.float32)
    H[np.arange(d), np.arange(d)] = h
    Hd = gpu_tensor(H)[:, :d]  # row stride d + 3
    perm, inv = gpu.gptq_act_order_perm(Hd)
    torch.cuda.synchronize()
    ref = O.act_order_perm(H[:, :d].astype(np.float64))
    assert np.array_equal(perm.cpu().numpy(), ref)
    assert np.array_equal(inv.cpu().numpy(), O.inverse_perm(ref))


@pytest.mark.parametrize("dtype", [torch.uint8, torch.float16, torch.float32])
@pytest.mark.parametrize("use_rows,use_cols", [(True, True), (False, True), (True, False), (False, False)])
def test_gather_parity(gpu, dtype, use_rows, use_cols):
    r = np.random.default_rng(3)
    src_np = r.integers(0, 255, size=(37, 301)).astype(np.uint8) if dtype == torch.uint8 else \
        r.standard_normal((37, 301)).astype(np.float16 if dtype == torch.float16 else np.float32)
    buf = torch.zeros((37, 320), dtype=dtype, device=DEV)
    buf[:, :301] = gpu_tensor(src_np)
    src = buf[:, :301]  # row stride 320
    ri = r.integers(0, 37, size=50).astype(np.int32) if use_rows else None
    ci = r.permutation(301)[:200].astype(np.int32) if use_cols else None
    out, info = gpu.gptq_gather(src, None if ri is None else gpu_tensor(ri), None if ci is None else gpu_tensor(ci))
    torch.cuda.synchronize()
    ref = src_np[ri if ri is not None else np.arange(37)][:, ci if ci is not None else np.arange(301)]
    got = out.cpu().numpy()
    assert got.dtype == ref.dtype and np.array_equal(got.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))
    assert int(info.item()) == 0


@pytest.mark.parametrize("dtype,cols,ld", [
    (torch.float16, 777, 781),     # staged in LDS, rows not 16-byte aligned (element loads)
    (torch.uint8, 1000, 1003),     # the same for bytes
    (torch.float32, 20000, 20000), # 80 KB rows: gathered straight from global memory
    (torch.float16, 32768, 32768), # exactly 64 KB rows: the largest staged row
])
def test_gather_parity_row_layouts(gpu, dtype, cols, ld):
    r = np.random.default_rng(cols)
    rows = 9
    npdt = {torch.float16: np.float16, torch.float32: np.float32, torch.uint8: np.uint8}[dtype]
    src_np = (r.integers(0, 255, size=(rows, cols)) if dtype == torch.uint8 else r.standard_normal((rows, cols)))
    src_np = src_np.astype(npdt)
    buf = torch.zeros((rows, ld), dtype=dtype, device=DEV)
    buf[:, :cols] = gpu_tensor(src_np)
    src = buf[:, :cols]
    ri = r.permutation(rows).astype(np.int32)
    ci = r.integers(0, cols, size=cols + 5).astype(np.int32)
    out, info = gpu.gptq_gather(src, gpu_tensor(ri), gpu_tensor(ci))
    torch.cuda.synchronize()
    ref = np.ascontiguousarray(src_np[ri][:, ci])
    assert np.array_equal(out.cpu().numpy().view(np.uint8), ref.view(np.uint8))
    assert int(info.item()) == 0


def test_gather_reports_bad_indices(gpu):
    src = torch.arange(1, 1 + 6 * 10, dtype=torch.float32, device=DEV).reshape(6, 10)
    ri = torch.tensor([0, 5, 6, -1], dtype=torch.int32, device=DEV)
    ci = torch.tensor([9, 10, 0], dtype=torch.int32, device=DEV)
    out, info = gpu.gptq_gather(src, ri, ci)
    torch.cuda.synchronize()
    assert int(info.item()) == 1
    got = out.cpu().numpy()
    s = src.cpu().numpy()
    assert np.array_equal(got[:2], np.stack([s[0, [9, 0, 0]], s[5, [9, 0, 0]]]) * np.array([1, 0, 1]))
    assert np.all(got[2:] == 0)
    out, info = gpu.gptq_gather(src, ri[:2], ci[[0, 2]])
    torch.cuda.synchronize()
    assert int(info.item()) == 0


def test_order_abi_rejects_bad_arguments(gpu):
    lib = gpu.load()
    buf = torch.zeros(64, dtype=torch.int32, device=DEV)
    p = buf.data_ptr()
    E = gpu.GPTQ_E_INVALID_ARG
    assert lib.gptq_act_order_perm(p, 0, 1, p, p, None) == E
    assert lib.gptq_act_order_perm(p, 4, 3, p, p, None) == E
    assert lib.gptq_act_order_perm(p, 4, 4, p, None, None) == E
    assert lib.gptq_gather(p, 3, 2, 2, 2, None, 2, None, 2, p, 2, None, None) == E  # elem_bytes
    assert lib.gptq_gather(p, 4, 2, 4, 3, None, 2, None, 2, p, 2, None, None) == E  # ld_src < src_cols
    assert lib.gptq_gather(p, 4, 2, 2, 2, None, 2, None, 4, p, 3, None, None) == E  # ld_dst < cols
    assert lib.gptq_gather(None, 4, 2, 2, 2, None, 2, None, 2, p, 2, None, None) == E


def outlier_hessian(n, d, seed):
    r = np.random.default_rng(seed)
    X = r.standard_normal((n, d)).astype(np.float32)
    X[:, r.choice(d, max(1, d // 50), replace=False)] *= 20.0
    X *= r.lognormal(0.0, 0.5, size=(n, 1)).astype(np.float32)
    return O.hessian(X).astype(np.float32)  # the GPU's input; the oracle uses the same values


ACT_CASES = [
    (16, 128, 4, 128, np.float16),
    (33, 200, 3, 32, np.float16),
    (20, 300, 2, 64, np.float32),
    (64, 640, 3, -1, np.float16),
    (100, 1024, 4, 128, np.float16),
    (24, 512, 8, 16, np.float32),
]


@pytest.mark.parametrize("d_row,d_col,bits,group,wdt", ACT_CASES)
def test_act_order_layer_parity(gpu, d_row, d_col, bits, group, wdt):
    """perm -> H[p][:, p] and W[:, p] by gather -> factor -> sweep, against
    the oracle's act-order layer on the same fp32 Hessian."""
    say("act-order", d_row, d_col, bits, group, wdt.__name__)
    damp = 0.01
    H = outlier_hessian(4 * d_col + 64, d_col, d_col + bits)
    W = (0.02 * np.random.default_rng(d_row + d_col).standard_normal((d_row, d_col))).astype(wdt)
    Hg, Wg = gpu_tensor(H), gpu_tensor(W)
    perm, inv = gpu.gptq_act_order_perm(Hg)
    Hp, i1 = gpu.gptq_gather(Hg, perm, perm)
    hv = gpu.gptq_prepare_hinv(Hp, damp)
    Wp, i2 = gpu.gptq_gather(Wg, None, perm)
    q = gpu.gptq_quantize_layer(Wp, hv.U, bits, group, 128)
    codes_orig, i3 = gpu.gptq_gather(q.codes, None, inv)
    torch.cuda.synchronize()
    assert int(hv.info.item()) == 0 and int(i1.item()) == 0 and int(i2.item()) == 0 and int(i3.item()) == 0
    ref = O.quantize_layer_act_order(W, H.astype(np.float64), bits, group, 128, damp, decide=np.float32)
    assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    check_quant(q, ref, bits, rerun_for(W[:, ref["perm"]], ref["U"], bits, group))
    assert np.array_equal(codes_orig.cpu().numpy(), q.codes.cpu().numpy()[:, ref["perm"].argsort()])


def test_act_order_matvec_composition(gpu):
    """y = packed_p x[:, p]: the product of a layer stored in permuted order
    with activations gathered by the same permutation equals x What_orig^T."""
    d_row, d_col, bits, group = 300, 1024, 4, 128
    r = np.random.default_rng(21)
    codes = r.integers(0, 16, size=(d_row, d_col))
    packed = O.pack(codes, bits)
    scales = r.uniform(0.001, 0.02, size=(d_row, d_col // group)).astype(np.float32)
    zeros = r.integers(0, 16, size=(d_row, d_col // group)).astype(np.int32)
    p = r.permutation(d_col).astype(np.int32)
    x = r.standard_normal((2, d_col)).astype(np.float16)
    xg, info = gpu.gptq_gather(gpu_tensor(x), None, gpu_tensor(p))
    y = gpu.gptq_dequant_matvec(gpu_tensor(packed.view(np.int32)), gpu_tensor(scales), gpu_tensor(zeros), d_col,
                                bits, group, xg)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    What_p = O.dequantize(codes, scales.astype(np.float64), zeros.astype(np.float64), group)
    What_orig = np.empty_like(What_p)
    What_orig[:, p] = What_p
    ref = x.astype(np.float64) @ What_orig.T
    bound = 1e-5 * (np.abs(x.astype(np.float64)) @ np.abs(What_orig).T) + 1e-30
    assert np.all(np.abs(y.cpu().numpy() - ref) <= bound)
