"""The quantized layer run on token batches (gptq_dequant_gemm) against the
oracle's run_quantized_layer (needs an MI355X).

Both sides use the same fp16 weights s (code - z) (the fp32 product rounded
to fp16), products of fp16 values are exact, and the oracle sums in float64.
The kernel sums K = d_in products in fp32 in the MFMA's order, which moves
the sum by at most (K + 2) 2^-24 sum |x w| before the final rounding to
fp16; rounding is monotone, so every output must lie between the fp16
roundings of (exact - bound) and (exact + bound), ReLU applied to both. Most
outputs equal the oracle's fp16 value exactly (counted and bounded below).
"""

import numpy as np
import pytest
import torch

import oracle.gptq_oracle as O
from tests.test_gpu_parity import DEV, gpu_tensor, say

pytestmark = pytest.mark.gpu


def layer(d_out, d_in, bits, group, seed):
    r = np.random.default_rng(seed)
    ng = 1 if group == -1 else -(-d_in // group)
    codes = r.integers(0, 1 << bits, size=(d_out, d_in))
    scales = r.uniform(0.001, 0.03, size=(d_out, ng)).astype(np.float32)
    zeros = r.integers(0, 1 << bits, size=(d_out, ng)).astype(np.int32)
    return O.pack(codes, bits), scales, zeros


def tokens(n, d_in, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, d_in)).astype(np.float32)
    x[:, r.choice(d_in, max(1, d_in // 100), replace=False)] *= 20.0
    return x.astype(np.float16)


def check_gemm(y, X, packed, scales, zeros, d_in, bits, group, relu):
    Wh = O.model_weight_f16(O.unpack(packed, d_in, bits), scales, zeros, group).astype(np.float64)
    Xd = X.astype(np.float64)
    exact = Xd @ Wh.T
    bound = (d_in + 2) * 2.0**-24 * (np.abs(Xd) @ np.abs(Wh).T)
    lo, hi = exact - bound, exact + bound
    if relu:
        lo, hi = np.maximum(lo, 0.0), np.maximum(hi, 0.0)
    lo16, hi16 = lo.astype(np.float16).astype(np.float64), hi.astype(np.float16).astype(np.float64)
    g = y.astype(np.float64)
    ok = (g >= lo16) & (g <= hi16)
    assert ok.all(), f"{int((~ok).sum())} outputs outside the fp32-summation bound"
    ref = O.run_quantized_layer(X, packed, scales, zeros, d_in, bits, group, relu)
    same = float(np.mean(y.astype(np.float64) == ref.astype(np.float64)))
    say(f"  gemm: {y.size} outputs within the bound; equal to the oracle's fp16 value {same:.6f}")
    assert same >= 0.99
    return same


@pytest.mark.parametrize("n,d_out,d_in,bits,group,relu", [
    (1, 1, 64, 4, -1, False),
    (300, 200, 128, 4, 128, True),
    (1000, 130, 256, 3, -1, False),
    (77, 257, 192, 2, 64, True),
    (513, 384, 512, 8, 128, False),
    (4096, 1376, 512, 4, 128, True),
    (257, 129, 1408, 3, 128, True),
    (300, 70, 1376, 4, -1, False),  # d_in = 43 x 32: a last K tile of 32 columns
    (129, 33, 96, 2, -1, True),
])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "two_pass"])
def test_dequant_gemm_parity(gpu, n, d_out, d_in, bits, group, relu, fused):
    say("dequant gemm", n, d_out, d_in, bits, group, relu, "fused" if fused else "workspace")
    packed, scales, zeros = layer(d_out, d_in, bits, group, n + d_out)
    X = tokens(n, d_in, d_in + bits)
    y = gpu.gptq_dequant_gemm(gpu_tensor(packed.view(np.int32)), gpu_tensor(scales), gpu_tensor(zeros), d_in, bits,
                              group, gpu_tensor(X), relu=relu, fused=fused)
    torch.cuda.synchronize()
    check_gemm(y.cpu().numpy(), X, packed, scales, zeros, d_in, bits, group, relu)


@pytest.mark.parametrize("n,d_out,d_in,bits,group,relu", [
    (256, 256, 128, 4, 128, False),    # one tile, one block of 128 K
    (1000, 300, 512, 3, 128, True),    # ragged tokens and rows, four stages
    (2048, 768, 384, 2, -1, False),    # several tiles both ways, 12 stages
    (513, 520, 640, 8, 64, True),      # ragged, 8-bit, groups of 64
    (4096, 1024, 1024, 4, 128, True),  # token tiles a multiple of 8 (XCD order)
    (16384, 1100, 128, 4, 128, True),  # token tiles a multiple of 64: blocked XCD order, a last block of 1 weight tile
    (16384, 300, 256, 3, -1, False),   # blocked order with only a narrower block (2 weight tiles)
])
def test_dequant_gemm_two_pass_equals_fused(gpu, n, d_out, d_in, bits, group, relu):
    """The workspace form (weights dequantized once, K-major operands, the
    Hessian's pipeline) on shapes it takes, against the oracle's bound. It
    uses the same fp16 weights as the fused form; the fp32 sums run in a
    different order inside each 16-K MFMA step, so the two may differ by
    rounding: the fraction of equal outputs is reported. The workspace starts
    NaN-filled, so a read of anything the pre-passes did not write shows."""
    say("dequant gemm two-pass", n, d_out, d_in, bits, group, relu)
    packed, scales, zeros = layer(d_out, d_in, bits, group, 7 * n + d_out)
    X = tokens(n, d_in, d_in + 3 * bits)
    P, S, Z, XT = gpu_tensor(packed.view(np.int32)), gpu_tensor(scales), gpu_tensor(zeros), gpu_tensor(X)
    need = gpu.gptq_dequant_gemm_workspace_size(d_out, d_in, n)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN-filled fp16: nothing unwritten is read
    y2 = gpu.gptq_dequant_gemm(P, S, Z, d_in, bits, group, XT, relu=relu, ws=ws)
    y1 = gpu.gptq_dequant_gemm(P, S, Z, d_in, bits, group, XT, relu=relu, fused=True)
    torch.cuda.synchronize()
    a, b = y2.cpu().numpy(), y1.cpu().numpy()
    check_gemm(a, X, packed, scales, zeros, d_in, bits, group, relu)
    say(f"  two-pass equal to fused: {float(np.mean(a == b)):.6f}")
    lib = gpu.load()
    Y = torch.empty((n, d_out), dtype=torch.float16, device=DEV)
    assert lib.gptq_dequant_gemm(P.data_ptr(), S.data_ptr(), Z.data_ptr(), d_out, d_in, bits, group, XT.data_ptr(), n,
                                 d_in, Y.data_ptr(), d_out, int(relu), ws.data_ptr(), need - 1,
                                 None) == gpu.GPTQ_E_WORKSPACE


def test_dequant_gemm_strided_and_bad_arguments(gpu):
    """Strided X and Y rows (views), nothing written past d_out, no tokens,
    and the argument checks."""
    n, d_out, d_in, bits, group = 300, 96, 256, 4, 64
    packed, scales, zeros = layer(d_out, d_in, bits, group, 5)
    X = tokens(n, d_in, 6)
    Xbig = gpu_tensor(np.concatenate([X, np.ones((n, 64), np.float16)], axis=1))
    Ybig = torch.full((n, d_out + 40), -7.0, dtype=torch.float16, device=DEV)
    P, S, Z = gpu_tensor(packed.view(np.int32)), gpu_tensor(scales), gpu_tensor(zeros)
    gpu.gptq_dequant_gemm(P, S, Z, d_in, bits, group, Xbig[:, :d_in], Y=Ybig[:, :d_out])
    torch.cuda.synchronize()
    yb = Ybig.cpu().numpy()
    check_gemm(yb[:, :d_out], X, packed, scales, zeros, d_in, bits, group, False)
    assert np.all(yb[:, d_out:] == -7.0)
    e = gpu.gptq_dequant_gemm(P, S, Z, d_in, bits, group, Xbig[:0, :d_in])
    assert e.shape == (0, d_out)
    lib = gpu.load()
    p = Ybig.data_ptr()
    x = Xbig.data_ptr()
    assert lib.gptq_dequant_gemm(p, p, p, 8, 100, 4, -1, x, 4, 320, p, 8, 0, None, 0, None) == gpu.GPTQ_E_UNSUPPORTED  # d_in % 32
    assert lib.gptq_dequant_gemm(p, p, p, 8, 128, 4, 32, x, 4, 320, p, 8, 0, None, 0, None) == gpu.GPTQ_E_UNSUPPORTED  # group
    assert lib.gptq_dequant_gemm(p, p, p, 8, 128, 5, -1, x, 4, 320, p, 8, 0, None, 0, None) == gpu.GPTQ_E_INVALID_ARG  # bits
    assert lib.gptq_dequant_gemm(p, p, p, 8, 128, 4, -1, x, 4, 100, p, 8, 0, None, 0, None) == gpu.GPTQ_E_INVALID_ARG  # ldx
    assert lib.gptq_dequant_gemm(p, p, p, 8, 128, 4, -1, x, 4, 320, p, 8, 2, None, 0, None) == gpu.GPTQ_E_INVALID_ARG  # relu


@pytest.mark.parametrize("name,relu", [("mlp_up_11008x4096_4bit_g128", True), ("mlp_down_4096x11008_4bit_g128", False)])
def test_dequant_gemm_full_size_sampled(gpu, name, relu):
    """The quantized layer at the MLP block's full size (262144 tokens of the
    configuration's activations, its weight shape, 4-bit g128), both forms,
    in the launch configuration the benchmark's pipeline leg times. The
    oracle computes 64 seeded tokens x 256 seeded weight rows one by one, to
    the same fp32-summation bound and >= 99% equality as the small cases."""
    from workload import CONFIGS, activation_chunks
    cfg = CONFIGS[name]
    d_out, d_in, n, bits, group = cfg.d_row, cfg.d_col, cfg.n_tokens, cfg.bits, cfg.group_size
    say("dequant gemm full size", name, n, d_out, d_in, bits, group, relu)
    r = np.random.default_rng(1234)
    toks = np.sort(r.choice(n, 64, replace=False))
    rows = np.sort(r.choice(d_out, 256, replace=False))
    # a seeded packed layer (random words: every code value occurs), scales and zeros
    nw = d_in * bits // 32
    packed = r.integers(0, 2**32, size=(d_out, nw), dtype=np.uint64).astype(np.uint32)
    ng = -(-d_in // group)
    scales = r.uniform(0.001, 0.03, size=(d_out, ng)).astype(np.float32)
    zeros = r.integers(0, 1 << bits, size=(d_out, ng)).astype(np.int32)
    Xd = torch.empty((n, d_in), dtype=torch.float16, device=DEV)
    Xs = np.empty((64, d_in), dtype=np.float16)
    t = 0
    for ch in activation_chunks(cfg, threads=16):
        Xd[t:t + ch.shape[0]].copy_(torch.from_numpy(ch))
        sel = (toks >= t) & (toks < t + ch.shape[0])
        Xs[sel] = ch[toks[sel] - t]
        t += ch.shape[0]
    assert t == n
    P, S, Z = gpu_tensor(packed.view(np.int32)), gpu_tensor(scales), gpu_tensor(zeros)
    ti, ri = torch.from_numpy(toks).to(DEV), torch.from_numpy(rows).to(DEV)
    for fused in (False, True):
        y = gpu.gptq_dequant_gemm(P, S, Z, d_in, bits, group, Xd, relu=relu, fused=fused)
        ys = y.index_select(0, ti).index_select(1, ri).cpu().numpy()
        del y
        torch.cuda.synchronize()
        check_gemm(ys, Xs, packed[rows], scales[rows], zeros[rows], d_in, bits, group, relu)
