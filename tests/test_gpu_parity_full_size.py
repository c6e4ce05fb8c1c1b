"""Full-size parity for every layer configuration, in the launch configuration
the benchmark times (needs an MI355X).

* Hessian: the GPU computes H from the full activation matrix and the oracle
  computes the same H in float64, chunk by chunk; they are compared in full.
* Factor: both sides factor that oracle Hessian, rounded to fp32 as the
  library receives it, and are compared in full.
* Sweep: the GPU quantizes the whole weight matrix with the oracle's factor.
  The oracle sweeps a seeded sample of 256 rows; rows are independent given U.
  Each sampled row must equal the oracle's row or its continuation through
  near-tie decisions (tests/parity.py), once with the decisions taken in
  float32 (the kernel's precision) and once in float64.

No value from the HIP path is fed to the oracle.
"""

import numpy as np
import pytest
import torch

import oracle.gptq_oracle as O
from tests.parity import rerun_for
from tests.test_gpu_parity import DEV, check_quant, gpu_tensor, rel_fro, say
from workload import CONFIGS, activation_chunks, weights

pytestmark = pytest.mark.gpu

FULL_SIZE = [
    "attn_proj_4096x4096_4bit_g128",
    "mlp_up_11008x4096_4bit_g128",
    "attn_proj_4096x4096_3bit_g128",
    "attn_proj_4096x4096_3bit_rowwise",
    "mlp_down_4096x11008_4bit_g128",
    "opt175b_12288x12288_3bit_g128",
    "opt175b_49152x12288_3bit_g128",
]
N_SAMPLE_ROWS = 256

# Per activation recipe and damping: the oracle's H and U in fp32.
_cache = {}


def x_key(cfg):
    return (cfg.seed, cfg.n_tokens, cfg.d_col, cfg.x_dtype, cfg.outlier_frac, cfg.outlier_factor, cfg.token_scale)


def hessian_stage(gpu, cfg):
    """GPU H of the full X against the oracle's; returns the oracle's H."""
    Xd = torch.empty((cfg.n_tokens, cfg.d_col), dtype=getattr(torch, cfg.x_dtype), device=DEV)
    t = 0

    def uploaded_chunks():
        nonlocal t
        for ch in activation_chunks(cfg, threads=16):
            Xd[t : t + ch.shape[0]].copy_(torch.from_numpy(ch))
            t += ch.shape[0]
            yield ch

    H_ref = O.hessian(uploaded_chunks())
    assert t == cfg.n_tokens
    H = gpu.gptq_hessian_accumulate(Xd)
    torch.cuda.synchronize()
    del Xd
    Hc = H.cpu().numpy()
    del H
    torch.cuda.empty_cache()
    e = rel_fro(Hc, H_ref)
    say(f"{cfg.name}: H (d={cfg.d_col}, {cfg.n_tokens} tokens) rel fro {e:.3g}")
    assert e < 1e-4
    assert np.array_equal(Hc, Hc.T)  # both triangles written, identical
    return H_ref


def factor_stage(gpu, cfg, Hf):
    H32 = Hf.astype(np.float32)
    U_ref, lam = O.prepare_hinv(H32.astype(np.float64), cfg.damp)
    hv = gpu.gptq_prepare_hinv(gpu_tensor(H32), cfg.damp)
    torch.cuda.synchronize()
    assert int(hv.info.item()) == 0
    assert abs(float(hv.lam.item()) - lam) <= 1e-6 * lam
    U = hv.U.cpu().numpy()
    e = rel_fro(U, U_ref)
    say(f"{cfg.name}: U (d={cfg.d_col}) rel fro {e:.3g}")
    assert e < 1e-6
    assert np.all(np.tril(U, -1) == 0)
    return U_ref.astype(np.float32)


def prepared(gpu, cfg):
    """The oracle's factor in fp32 (after the Hessian and factor stages ran
    once for this activation recipe)."""
    return _prepared(gpu, cfg)[1]


def _prepared(gpu, cfg):
    key = x_key(cfg) + (cfg.damp,)
    if key not in _cache:
        Hf = hessian_stage(gpu, cfg)
        _cache[key] = (Hf.astype(np.float32), factor_stage(gpu, cfg, Hf))
    return _cache[key]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_layer(gpu, name):
    cfg = CONFIGS[name]
    say(f"full-size {name}: W {cfg.d_row}x{cfg.d_col}, X {cfg.n_tokens}x{cfg.d_col}, {cfg.bits}-bit g{cfg.group_size}")
    U32 = prepared(gpu, cfg)
    W = weights(cfg)
    q = gpu.gptq_quantize_layer(gpu_tensor(W), gpu_tensor(U32), cfg.bits, cfg.group_size, cfg.block)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7).choice(cfg.d_row, N_SAMPLE_ROWS, replace=False))
    rows[-1] = cfg.d_row - 1
    rows = np.unique(rows)
    U64 = U32.astype(np.float64)
    for decide in (np.float32, np.float64):
        # decisions in the kernel's precision, then in the oracle's own
        ref = O.quantize_layer(W[rows], U64, cfg.bits, cfg.group_size, cfg.block, decide=decide)
        check_quant(q, ref, cfg.bits, rerun_for(W[rows], U64, cfg.bits, cfg.group_size, cfg.block, decide=decide),
                    rows=rows, label=f"{name}, {decide.__name__} decisions")
    # outputs of every row are on the grid: zeros within range, scales positive
    zeros = q.zeros.cpu().numpy()
    assert zeros.min() >= 0 and zeros.max() <= (1 << cfg.bits) - 1
    assert bool(torch.all(q.scales > 0)) and bool(torch.isfinite(q.loss))


@pytest.mark.timeout(900)
def test_full_size_act_order_layer(gpu):
    """The 4096x4096 3-bit g128 layer in act-order, in the launch
    configuration the benchmark times: permutation (bit-exact), gathers,
    factor and sweep on the GPU; the oracle's act-order layer on 256 sampled
    rows from the same fp32 Hessian."""
    cfg = CONFIGS["attn_proj_4096x4096_3bit_g128"]
    say(f"full-size act-order {cfg.name}")
    H32, _ = _prepared(gpu, cfg)
    W = weights(cfg)
    Hg = gpu_tensor(H32)
    perm, inv = gpu.gptq_act_order_perm(Hg)
    Hp, i1 = gpu.gptq_gather(Hg, perm, perm)
    hv = gpu.gptq_prepare_hinv(Hp, cfg.damp)
    Wp, i2 = gpu.gptq_gather(gpu_tensor(W), None, perm)
    q = gpu.gptq_quantize_layer(Wp, hv.U, cfg.bits, cfg.group_size, cfg.block)
    torch.cuda.synchronize()
    assert int(hv.info.item()) == 0 and int(i1.item()) == 0 and int(i2.item()) == 0
    p = O.act_order_perm(H32.astype(np.float64))
    assert np.array_equal(perm.cpu().numpy(), p)
    U_ref, _ = O.prepare_hinv(H32.astype(np.float64)[np.ix_(p, p)], cfg.damp)
    e = rel_fro(hv.U.cpu().numpy(), U_ref)
    say(f"act-order U rel fro {e:.3g}")
    assert e < 1e-6
    rows = np.sort(np.random.default_rng(8).choice(cfg.d_row, N_SAMPLE_ROWS, replace=False))
    rows[-1] = cfg.d_row - 1
    rows = np.unique(rows)
    Wp_rows = W[rows][:, p]
    Up = U_ref.astype(np.float32).astype(np.float64)
    for decide in (np.float32, np.float64):
        ref = O.quantize_layer(Wp_rows, Up, cfg.bits, cfg.group_size, cfg.block, decide=decide)
        check_quant(q, ref, cfg.bits, rerun_for(Wp_rows, Up, cfg.bits, cfg.group_size, cfg.block, decide=decide),
                    rows=rows, label=f"act-order, {decide.__name__} decisions")
