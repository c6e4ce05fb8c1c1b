"""Parity of the HIP path with the float64 oracle (needs an MI355X).

Inputs always flow from the seeded generators or the oracle to the GPU; no
value produced by the HIP path is fed back into the oracle's arithmetic.
Tolerances: H within 1e-4 relative Frobenius error; every quantized row equal
to the oracle's row, or to the oracle's own continuation of that row through
decisions the oracle took within 1e-3 grid steps of a rounding boundary
(tests/parity.py), with codes and zeros exact, scales within 1e-3 relative
error and losses within 1%; packed words bit-exact for the same codes.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle.gptq_oracle as O
from tests import parity
from tests.parity import rerun_for
from workload import CONFIGS, activation_chunks, activations, weights
from workload.synth import small

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def rel_fro(a, b):
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def gpu_tensor(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def outputs(q, rows=None):
    """The GPU's quantize_layer outputs as numpy arrays (optionally a row subset)."""
    o = parity.LayerOutputs(codes=q.codes.cpu().numpy(), scales=q.scales.cpu().numpy(), zeros=q.zeros.cpu().numpy(),
                            packed=q.packed.cpu().numpy().view(np.uint32), row_loss=q.row_loss.cpu().numpy())
    if rows is not None:
        o = parity.LayerOutputs(*(getattr(o, f.name)[rows] for f in dataclasses.fields(o)))
    return o


def check_quant(q, ref, bits, rerun, rows=None, **kw):
    """The GPU rows against the oracle's (tests/parity.py): each row equal to
    the oracle's row, or to an oracle continuation through decisions the
    oracle took within 1e-3 grid steps of a tie; scales within 1e-3, zeros
    exact, losses within 1%, packing bit-exact."""
    return parity.check_quant(outputs(q, rows), ref, bits, rerun, log=say, **kw)


# ------------------------------------------------------------------ Hessian
def make_x(n, d, dtype, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, d)).astype(np.float32)
    if d >= 4:
        x[:, r.choice(d, max(1, d // 100), replace=False)] *= 20
    return x.astype(dtype)


@pytest.mark.parametrize(
    "n,d,dtype",
    [
        (1, 1, np.float16),
        (37, 3, np.float16),
        (1000, 100, np.float16),
        (5000, 300, np.float16),
        (2049, 513, np.float16),
        (33, 256, np.float16),
        (4096, 256, np.float32),
        (3001, 70, np.float32),
        (700, 130, np.float32),
    ],
)
def test_hessian_parity(gpu, n, d, dtype):
    say("hessian", n, d, dtype.__name__)
    X = make_x(n, d, dtype, n + d)
    H = gpu.gptq_hessian_accumulate(gpu_tensor(X))
    torch.cuda.synchronize()
    Hg = H.cpu().numpy()
    ref = O.hessian(X)
    assert rel_fro(Hg, ref) < 1e-4
    assert np.array_equal(Hg, Hg.T)


def test_hessian_accumulate_strided_and_empty(gpu):
    X = make_x(3000, 200, np.float16, 5)
    big = gpu_tensor(np.concatenate([X, np.ones((3000, 56), np.float16)], axis=1))
    view = big[:, :200]  # row stride 256 elements
    H = gpu.gptq_hessian_accumulate(view[:1000])
    gpu.gptq_hessian_accumulate(view[1000:], H=H, accumulate=True)
    gpu.gptq_hessian_accumulate(view[:0], H=H, accumulate=True)  # no tokens: unchanged
    torch.cuda.synchronize()
    assert rel_fro(H.cpu().numpy(), O.hessian(X)) < 1e-4
    Z = gpu.gptq_hessian_accumulate(view[:0])
    torch.cuda.synchronize()
    assert np.all(Z.cpu().numpy() == 0)


# ---------------------------------------------------- inverse-Hessian factor
@pytest.mark.parametrize("d", [1, 2, 63, 64, 65, 130, 256, 700, 1500])
def test_prepare_hinv_parity(gpu, d):
    say("hinv", d)
    X = make_x(3 * d + 50, d, np.float32, d)
    Href = O.hessian(X).astype(np.float32).astype(np.float64)  # the GPU's input, exactly
    hv = gpu.gptq_prepare_hinv(gpu_tensor(Href.astype(np.float32)), 0.01)
    torch.cuda.synchronize()
    assert int(hv.info.item()) == 0
    U, lam = O.prepare_hinv(Href, 0.01)
    Ug = hv.U.cpu().numpy()
    assert np.array_equal(Ug, np.triu(Ug))
    assert rel_fro(Ug, U) < 1e-6
    assert abs(float(hv.lam.item()) - lam) <= 1e-6 * lam


def test_prepare_hinv_rank_deficient_needs_damping(gpu):
    X = make_x(128, 256, np.float32, 1)  # fewer tokens than channels: singular H
    Href = O.hessian(X).astype(np.float32).astype(np.float64)
    hv = gpu.gptq_prepare_hinv(gpu_tensor(Href.astype(np.float32)), 0.01)
    torch.cuda.synchronize()
    assert int(hv.info.item()) == 0
    U, _ = O.prepare_hinv(Href, 0.01)
    assert rel_fro(hv.U.cpu().numpy(), U) < 1e-5


@pytest.mark.parametrize("d", [3, 100])
def test_prepare_hinv_reports_indefinite(gpu, d):
    H = -np.eye(d, dtype=np.float32)
    hv = gpu.gptq_prepare_hinv(gpu_tensor(H), 0.01)
    torch.cuda.synchronize()
    assert int(hv.info.item()) > 0
    Z = np.zeros((d, d), np.float32)  # lambda = 0: not positive definite
    hv = gpu.gptq_prepare_hinv(gpu_tensor(Z), 0.01)
    torch.cuda.synchronize()
    assert 1 <= int(hv.info.item()) <= d


@pytest.mark.parametrize("bad", [[10], [70], [130], [200], [280], [70, 200], [200, 70]])
def test_prepare_hinv_reports_the_first_breakdown(gpu, bad):
    """info = 1 + the H column of the first pivot that is not positive, in
    the factorization's order (H's columns from the last): a breakdown in
    either block of a super-panel, in a later one, and in the last, single
    block (d = 300 = 128 + 128 + 44 columns)."""
    d = 300
    h = np.ones(d, np.float32)
    for a in bad:  # a: position in the factorization's order
        h[d - 1 - a] = -1.0  # -1 + lambda < 0 with lambda = 0.01 * mean(diag H) < 0.01
    hv = gpu.gptq_prepare_hinv(gpu_tensor(np.diag(h)), 0.01)
    torch.cuda.synchronize()
    assert int(hv.info.item()) == 1 + (d - 1 - min(bad))


def test_prepare_hinv_nan_diagonal_fails_at_the_first_pivot(gpu):
    d = 300
    h = np.ones(d, np.float32)
    h[100] = np.nan  # lambda is NaN, so every damped pivot is
    hv = gpu.gptq_prepare_hinv(gpu_tensor(np.diag(h)), 0.01)
    torch.cuda.synchronize()
    assert int(hv.info.item()) == d


@pytest.mark.parametrize("d", [300, 700])
def test_prepare_hinv_under_graph_capture(gpu, d):
    """The factor's two streams captured into one HIP graph: every replay, with
    eager work and eager factor calls between replays, gives the eager U, lambda
    and info to the bit."""
    say("hinv graph", d)
    X = make_x(3 * d + 50, d, np.float32, d + 7)
    H = gpu_tensor(O.hessian(X).astype(np.float32))
    ws = torch.empty(gpu.gptq_prepare_hinv_workspace_size(d), dtype=torch.uint8, device=DEV)
    ref = gpu.gptq_prepare_hinv(H, 0.01, ws=ws)  # also creates the auxiliary stream before capture
    torch.cuda.synchronize()
    assert int(ref.info.item()) == 0
    out = gpu.Hinv(torch.empty_like(ref.U), torch.empty_like(ref.lam), torch.empty_like(ref.info))
    wsg = torch.empty_like(ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu.gptq_prepare_hinv(H, 0.01, ws=wsg, out=out)
    torch.cuda.synchronize()
    for _ in range(3):
        out.U.fill_(float("nan"))
        out.info.fill_(-1)
        wsg.fill_(255)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.U.view(torch.int32), ref.U.view(torch.int32))
        assert torch.equal(out.lam, ref.lam) and int(out.info.item()) == 0
        again = gpu.gptq_prepare_hinv(H, 0.01, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(again.U.view(torch.int32), ref.U.view(torch.int32))
    U, _ = O.prepare_hinv(O.hessian(X).astype(np.float32).astype(np.float64), 0.01)
    assert rel_fro(out.U.cpu().numpy(), U) < 1e-6


def test_layer_path_under_graph_capture(gpu):
    """Hessian, factor and sweep (with packing and loss) captured into one HIP
    graph: three replays, with eager layer calls between them, give the eager
    outputs to the bit."""
    cfg = small(CONFIGS["attn_proj_4096x4096_4bit_g128"], d_row=96, d_col=640, n_tokens=9000)
    say("layer graph", cfg.name, cfg.d_row, cfg.d_col, cfg.n_tokens)
    Xd = torch.from_numpy(activations(cfg, threads=1)).to(DEV)
    Wd = torch.from_numpy(weights(cfg)).to(DEV)

    def layer(H=None, hws=None, fws=None, hv=None, qws=None, q=None):
        H = gpu.gptq_hessian_accumulate(Xd, H=H, ws=hws)
        hv = gpu.gptq_prepare_hinv(H, cfg.damp, ws=fws, out=hv)
        return H, hv, gpu.gptq_quantize_layer(Wd, hv.U, cfg.bits, cfg.group_size, cfg.block, ws=qws, out=q)

    He, hve, qe = layer()
    torch.cuda.synchronize()
    like = lambda t: None if t is None else torch.empty_like(t)
    H = torch.empty_like(He)
    hws = torch.empty(gpu.gptq_hessian_workspace_size(cfg.n_tokens, cfg.d_col, Xd.dtype), dtype=torch.uint8, device=DEV)
    fws = torch.empty(gpu.gptq_prepare_hinv_workspace_size(cfg.d_col), dtype=torch.uint8, device=DEV)
    qws = torch.empty(
        gpu.gptq_quantize_layer_workspace_size(cfg.d_row, cfg.d_col, cfg.bits, cfg.group_size, cfg.block),
        dtype=torch.uint8, device=DEV)
    hv = gpu.Hinv(like(hve.U), like(hve.lam), like(hve.info))
    q = gpu.Quantized(*(like(getattr(qe, f.name)) for f in dataclasses.fields(gpu.Quantized)))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(H, hws, fws, hv, qws, q)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in (H, hv.U, q.scales, q.loss):
            t.fill_(float("nan"))
        for t in (hws, fws, qws, q.codes, q.packed, q.zeros):
            t.fill_(255 if t.dtype == torch.uint8 else -1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(H.view(torch.int32), He.view(torch.int32))
        assert torch.equal(hv.U.view(torch.int32), hve.U.view(torch.int32)) and int(hv.info.item()) == 0
        for f in dataclasses.fields(gpu.Quantized):
            a, b = getattr(q, f.name), getattr(qe, f.name)
            if b is not None:
                assert torch.equal(a.reshape(-1).view(torch.uint8), b.reshape(-1).view(torch.uint8)), f.name
        layer()
        torch.cuda.synchronize()


@pytest.mark.parametrize("d", [65, 300, 700])
def test_stages_ignore_workspace_contents(gpu, d):
    """Each stage gives the same result to the bit from a workspace of zero
    bytes and from one of 0xff bytes (NaN in every float slot): no kernel
    reads a workspace entry before a kernel of the same call wrote it."""
    X = make_x(3 * d + 50, d, np.float16, d + 7)
    Xg = gpu_tensor(X)
    W = gpu_tensor((0.02 * np.random.default_rng(d).standard_normal((48, d))).astype(np.float16))
    outs = []
    for fill in (0, 255):
        wsh = torch.full((gpu.gptq_hessian_workspace_size(Xg.shape[0], d, torch.float16),), fill, dtype=torch.uint8,
                         device=DEV)
        H = gpu.gptq_hessian_accumulate(Xg, ws=wsh)
        wsu = torch.full((gpu.gptq_prepare_hinv_workspace_size(d),), fill, dtype=torch.uint8, device=DEV)
        hv = gpu.gptq_prepare_hinv(H, 0.01, ws=wsu)
        wsq = torch.full((gpu.gptq_quantize_layer_workspace_size(48, d, 4, 32, 128),), fill, dtype=torch.uint8,
                         device=DEV)
        q = gpu.gptq_quantize_layer(W, hv.U, 4, 32, 128, ws=wsq)
        torch.cuda.synchronize()
        assert int(hv.info.item()) == 0
        outs.append([H.cpu(), hv.U.cpu(), q.codes.cpu(), q.scales.cpu(), q.row_loss.cpu()])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    U_ref, _ = O.prepare_hinv(O.hessian(X), 0.01)
    assert rel_fro(outs[1][1].numpy(), U_ref) < 1e-5


# ------------------------------------------------------------------- sweep
def oracle_u(d, seed, n=None):
    X = make_x(n or (4 * d + 64), d, np.float32, seed)
    U, _ = O.prepare_hinv(O.hessian(X), 0.01)
    return U.astype(np.float32)  # the GPU's input; the oracle uses the same values


SWEEP_CASES = [
    (1, 1, 4, -1, np.float32),
    (5, 7, 3, -1, np.float32),
    (16, 128, 4, 128, np.float16),
    (17, 129, 4, 16, np.float32),
    (33, 200, 3, 32, np.float16),
    (64, 256, 4, 128, np.float16),
    (20, 300, 2, 64, np.float32),
    (48, 384, 8, 128, np.float16),
    (40, 512, 3, 256, np.float16),
    (31, 260, 4, 256, np.float32),
    (64, 640, 3, -1, np.float16),
    (100, 1024, 4, 128, np.float16),
]


@pytest.mark.parametrize("d_row,d_col,bits,group,wdt", SWEEP_CASES)
def test_quantize_layer_parity(gpu, d_row, d_col, bits, group, wdt):
    say("sweep", d_row, d_col, bits, group, wdt.__name__)
    U = oracle_u(d_col, d_col + bits)
    W = (0.02 * np.random.default_rng(d_row + d_col).standard_normal((d_row, d_col))).astype(wdt)
    q = gpu.gptq_quantize_layer(gpu_tensor(W), gpu_tensor(U), bits, group, 128)
    torch.cuda.synchronize()
    ref = O.quantize_layer(W, U, bits, group, 128, decide=np.float32)
    check_quant(q, ref, bits, rerun_for(W, U, bits, group))
    assert float(q.loss.item()) == pytest.approx(float(np.sum(q.row_loss.cpu().numpy().astype(np.float64))), rel=1e-6)


LAZY_SHAPES = [
    (40, 1300, 4, -1, np.float32),  # ragged: 10 full blocks and a 20-column tail
    (64, 2048, 3, 128, np.float16),  # whole tiles
    (33, 1100, 4, 16, np.float16),
]


@pytest.mark.parametrize("d_row,d_col,bits,group,wdt", LAZY_SHAPES)
def test_lazy_batch_widths(gpu, d_row, d_col, bits, group, wdt):
    """Lazy batches are exact (the deferred update applies the same rank-1
    updates later), so every width gives the same layer: on the GPU each
    element sees the same fp32 operations in the same order for every width
    (widths above the block defer in two levels, widths that divide it nest
    inside it), so all widths agree to the bit with B = 128; each also passes
    the oracle's own sweep at that width."""
    say("lazy widths", d_row, d_col, bits, group, wdt.__name__)
    U = oracle_u(d_col, d_col + 3 * bits)
    W = (0.02 * np.random.default_rng(d_row * d_col).standard_normal((d_row, d_col))).astype(wdt)
    Wd, Ud = gpu_tensor(W), gpu_tensor(U)
    base = gpu.gptq_quantize_layer(Wd, Ud, bits, group, 128)
    widths = [1, 2, 16, 64, 256, 512, 1024]
    outs = {}
    for B in widths:
        if group != -1 and B % group and group % B:
            continue  # blocks and groups must nest
        outs[B] = gpu.gptq_quantize_layer(Wd, Ud, bits, group, B)
    torch.cuda.synchronize()
    for B, q in outs.items():
        for name in ("codes", "scales", "zeros", "packed", "row_loss", "loss"):
            assert torch.equal(getattr(q, name).reshape(-1).view(torch.uint8),
                               getattr(base, name).reshape(-1).view(torch.uint8)), (B, name)
    for B in (1, 256, 1024):
        if B in outs:
            ref = O.quantize_layer(W, U, bits, group, B, decide=np.float32)
            check_quant(outs[B], ref, bits, rerun_for(W, U, bits, group, B), label=f"block {B}")


@pytest.mark.parametrize("bits,group", [(4, -1), (3, 128), (2, 32), (8, 16)])
def test_identity_hessian_is_rtn_bit_exact(gpu, bits, group):
    d_col = 384
    W = (0.02 * np.random.default_rng(bits).standard_normal((40, d_col))).astype(np.float32)
    U = (np.eye(d_col) / np.sqrt(1.01)).astype(np.float32)
    q = gpu.gptq_quantize_layer(gpu_tensor(W), gpu_tensor(U), bits, group, 128)
    torch.cuda.synchronize()
    ref = O.quantize_layer(W, U, bits, group, 128, decide=np.float32)
    assert np.array_equal(q.codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(q.zeros.cpu().numpy(), ref["zeros"].astype(np.int32))
    assert np.allclose(q.scales.cpu().numpy(), ref["scales"], rtol=1e-7)


def _random_layers(n=24, seed=20261203):
    """Seeded random layers: shape, width, group (whole row, or a multiple of
    16 that divides or is divided by the 128-column block), grid, and the
    dtypes of the weights and activations; tokens from half to three times
    the width (the Hessian is rank-deficient below the width)."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d_row, d_col = int(r.integers(1, 300)), int(r.integers(1, 700))
        bits = int(r.choice([2, 3, 4, 8]))
        group = int(r.choice([-1, 16, 32, 64, 128, 256, 384, 512]))
        sym = bool(r.integers(0, 2))
        wdt = np.float16 if r.integers(0, 2) else np.float32
        xdt = np.float16 if r.integers(0, 2) else np.float32
        n_tok = int(r.integers(max(1, d_col // 2), 3 * d_col + 2))
        out.append((d_row, d_col, bits, group, sym, wdt, xdt, n_tok))
    return out


RANDOM_LAYERS = _random_layers()


@pytest.mark.parametrize("case", range(len(RANDOM_LAYERS)))
def test_layer_path_random_shapes(gpu, case):
    """Hessian and factor from seeded activations against the oracle's own
    chain, then the sweep on the oracle's factor against the oracle's sweep
    (same near-tie criteria as the fixed cases)."""
    d_row, d_col, bits, group, sym, wdt, xdt, n_tok = RANDOM_LAYERS[case]
    say("random layer", case, d_row, d_col, bits, group, "sym" if sym else "asym", wdt.__name__, xdt.__name__, n_tok)
    X = make_x(n_tok, d_col, xdt, 1000 + case)
    W = (0.02 * np.random.default_rng(2000 + case).standard_normal((d_row, d_col))).astype(wdt)
    H = gpu.gptq_hessian_accumulate(gpu_tensor(X))
    hv = gpu.gptq_prepare_hinv(H, 0.01)
    torch.cuda.synchronize()
    Href = O.hessian(X)
    assert rel_fro(H.cpu().numpy(), Href) < 1e-4
    Uref, lam = O.prepare_hinv(Href, 0.01)
    assert int(hv.info.item()) == 0
    # fp32 H, fp64 factor: U's error is H's rounding times the damped conditioning
    assert rel_fro(hv.U.cpu().numpy(), Uref) < 5e-3
    assert abs(float(hv.lam.item()) - lam) <= 1e-4 * lam
    U32 = Uref.astype(np.float32)
    q = gpu.gptq_quantize_layer(gpu_tensor(W), gpu_tensor(U32), bits, group, 128, symmetric=sym)
    torch.cuda.synchronize()
    ref = O.quantize_layer(W, U32, bits, group, 128, decide=np.float32, symmetric=sym)
    check_quant(q, ref, bits, rerun_for(W, U32, bits, group, symmetric=sym), max_flip_rows=0.05)


SYM_CASES = [
    (16, 128, 4, 128, np.float16),
    (33, 200, 3, 32, np.float16),
    (20, 300, 2, 64, np.float32),
    (64, 256, 3, 128, np.float16),
    (64, 640, 8, -1, np.float16),
]


@pytest.mark.parametrize("d_row,d_col,bits,group,wdt", SYM_CASES)
def test_quantize_layer_parity_symmetric(gpu, d_row, d_col, bits, group, wdt):
    say("sweep symmetric", d_row, d_col, bits, group, wdt.__name__)
    U = oracle_u(d_col, d_col + 2 * bits)
    W = (0.02 * np.random.default_rng(3 * d_row + d_col).standard_normal((d_row, d_col))).astype(wdt)
    q = gpu.gptq_quantize_layer(gpu_tensor(W), gpu_tensor(U), bits, group, 128, symmetric=True)
    torch.cuda.synchronize()
    ref = O.quantize_layer(W, U, bits, group, 128, decide=np.float32, symmetric=True)
    check_quant(q, ref, bits, rerun_for(W, U, bits, group, symmetric=True))
    assert np.all(q.zeros.cpu().numpy() == 2 ** (bits - 1))


@pytest.mark.parametrize("bits,group", [(4, -1), (3, 128), (2, 32), (8, 16)])
def test_identity_hessian_symmetric_is_rtn_bit_exact(gpu, bits, group):
    d_col = 384
    W = (0.02 * np.random.default_rng(10 + bits).standard_normal((40, d_col))).astype(np.float32)
    U = (np.eye(d_col) / np.sqrt(1.01)).astype(np.float32)
    q = gpu.gptq_quantize_layer(gpu_tensor(W), gpu_tensor(U), bits, group, 128, symmetric=True)
    torch.cuda.synchronize()
    ref = O.quantize_layer(W, U, bits, group, 128, decide=np.float32, symmetric=True)
    assert np.array_equal(q.codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(q.zeros.cpu().numpy(), ref["zeros"].astype(np.int32))
    assert np.allclose(q.scales.cpu().numpy(), ref["scales"], rtol=1e-7)


@pytest.mark.parametrize("d_row,d_col,bits,group,wdt", [
    (80, 384, 4, 128, np.float16),  # 8 waves, one partial super-block
    (64, 2048, 3, 128, np.float16),  # 8 waves, four 512-column super-blocks
    (4112, 1280, 4, 256, np.float32),  # 4-wave whole-tile form (groups wider than a block)
    (31, 260, 4, 256, np.float32),  # the checked form
    (16384, 12288, 3, 128, np.float16),  # 32 rows per workgroup, super-blocks
])
def test_quantize_is_deterministic(gpu, d_row, d_col, bits, group, wdt):
    """Three calls, each with a fresh workspace (whose memory may still hold
    an earlier call's working copy), give the same bits. U is any
    upper-triangular factor with a positive diagonal."""
    say("determinism", d_row, d_col, bits, group, wdt.__name__)
    r = np.random.default_rng(d_row + d_col)
    U = np.triu(r.standard_normal((d_col, d_col), dtype=np.float32)) * np.float32(0.3 / np.sqrt(d_col))
    U[np.diag_indices(d_col)] = 1.0
    Ud = gpu_tensor(U)
    Wd = gpu_tensor((0.02 * r.standard_normal((d_row, d_col), dtype=np.float32)).astype(wdt))
    del U
    qs = [gpu.gptq_quantize_layer(Wd, Ud, bits, group, 128) for _ in range(3)]
    torch.cuda.synchronize()
    for q in qs[1:]:
        for name in ("codes", "scales", "zeros", "packed", "row_loss", "loss"):
            assert torch.equal(getattr(q, name), getattr(qs[0], name)), name


# -------------------------------------------------------------------- pack
@pytest.mark.parametrize("wdt,bits,group", [(np.float16, 3, 128), (np.float32, 4, -1), (np.float16, 4, 256),
                                            (np.float16, 3, 512), (np.float16, 4, 384)])
def test_tall_layer_row_groups_are_bit_identical(gpu, wdt, bits, group):
    """Tile-aligned layers with at least 16384 rows (a multiple of 32) and
    12288 columns take 32 rows per workgroup and 512-column super-blocks
    (groups of at most 128 columns), others 16 rows and no super-blocks. A
    row element's fp32 MFMA sequence is the same either way, so the
    16384-row layer and the same layer one 16-row group shorter agree bit
    for bit on the rows both have;
    the tall one also matches the oracle on sampled rows. Groups wider than
    a block (256, 384, 512) read columns past the block for their
    statistics. U is any upper-triangular factor with a positive diagonal
    (both sides take it as given)."""
    d_row, d_col = 16384, 12288
    r = np.random.default_rng(98)
    U = (np.triu(r.standard_normal((d_col, d_col), dtype=np.float32)) * 1e-3 + np.eye(d_col, dtype=np.float32))
    W = (0.02 * r.standard_normal((d_row, d_col), dtype=np.float32)).astype(wdt)
    Ud, Wd = gpu_tensor(U), gpu_tensor(W)
    qa = gpu.gptq_quantize_layer(Wd, Ud, bits, group, 128)
    qb = gpu.gptq_quantize_layer(Wd[: d_row - 16].contiguous(), Ud, bits, group, 128)
    torch.cuda.synchronize()
    for name in ("codes", "scales", "zeros", "packed", "row_loss"):
        assert torch.equal(getattr(qa, name)[: d_row - 16], getattr(qb, name)), name
    rows = np.unique(np.append(r.choice(d_row, 24, replace=False), [0, 31, d_row - 1]))
    ref = O.quantize_layer(W[rows], U.astype(np.float64), bits, group, 128, decide=np.float32)
    check_quant(qa, ref, bits, rerun_for(W[rows], U, bits, group), rows=rows)


@pytest.mark.parametrize("wdt,bits,group", [(np.float16, 4, 128), (np.float32, 3, -1)])
def test_update_forms_are_bit_identical(gpu, wdt, bits, group):
    """Tile-aligned layers (here 4096 rows) run 8 waves per 16-row workgroup,
    the extra 4 only in the deferred update, and defer the update of columns
    past a 512-column super-block to its end; one more row makes the layer
    ragged, and it runs the checked 4-wave form, which updates after every
    block. A row element's fp32 MFMA sequence is the same in both, so the
    shared rows agree bit for bit."""
    d_col = 1280  # two 512-column super-blocks and a half one
    U = oracle_u(d_col, 96)
    W = (0.02 * np.random.default_rng(95).standard_normal((4097, d_col))).astype(wdt)
    Ud, Wd = gpu_tensor(U), gpu_tensor(W)
    qa = gpu.gptq_quantize_layer(Wd[:4096].contiguous(), Ud, bits, group, 128)
    qb = gpu.gptq_quantize_layer(Wd, Ud, bits, group, 128)
    torch.cuda.synchronize()
    for name in ("codes", "scales", "zeros", "packed", "row_loss"):
        assert torch.equal(getattr(qa, name), getattr(qb, name)[:4096]), name
    rows = np.unique(np.append(np.random.default_rng(94).choice(4096, 48, replace=False), [0, 4095]))
    check_quant(qa, O.quantize_layer(W[rows], U.astype(np.float64), bits, group, 128, decide=np.float32), bits,
                rerun_for(W[rows], U, bits, group), rows=rows)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d_row,d_col", [(1, 1), (3, 10), (7, 11), (5, 128), (9, 1000)])
def test_pack_parity(gpu, bits, d_row, d_col):
    codes = np.random.default_rng(bits * d_col).integers(0, 1 << bits, size=(d_row, d_col)).astype(np.uint8)
    p = gpu.gptq_pack_codes(gpu_tensor(codes), bits)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy().view(np.uint32), O.pack(codes, bits))


# ------------------------------------------------------- ABI error paths
def test_abi_rejects_bad_arguments(gpu):
    U = torch.zeros((64, 64), dtype=torch.float32, device=DEV)
    W = torch.zeros((4, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(gpu.GptqError) as e:
        gpu.gptq_quantize_layer(W, U, 5, -1)
    assert e.value.status == gpu.GPTQ_E_INVALID_ARG
    with pytest.raises(gpu.GptqError) as e:
        gpu.gptq_quantize_layer(W, U, 4, 48)  # neither divides the other
    assert e.value.status == gpu.GPTQ_E_INVALID_ARG
    with pytest.raises(gpu.GptqError) as e:
        gpu.gptq_quantize_layer(W, U, 4, -1, block=96)  # neither a power of two below 128 nor a multiple of 128
    assert e.value.status == gpu.GPTQ_E_UNSUPPORTED
    with pytest.raises(gpu.GptqError) as e:
        gpu.gptq_prepare_hinv(U, damp=-1.0)
    assert e.value.status == gpu.GPTQ_E_INVALID_ARG
    lib = gpu.load()
    X = torch.zeros((8, 16), dtype=torch.float16, device=DEV)
    H = torch.zeros((16, 16), dtype=torch.float32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    st = lib.gptq_hessian_accumulate(X.data_ptr(), 0, 8, 16, 16, H.data_ptr(), 0, ws.data_ptr(), 16, None)
    assert st == gpu.GPTQ_E_WORKSPACE
    st = lib.gptq_hessian_accumulate(X.data_ptr(), 0, 8, 16, 8, H.data_ptr(), 0, ws.data_ptr(), 16, None)
    assert st == gpu.GPTQ_E_INVALID_ARG
    # symmetric must be 0 or 1 (checked before any launch or output access)
    st = lib.gptq_quantize_layer(W.data_ptr(), 0, 4, 64, U.data_ptr(), 4, -1, 128, 2, H.data_ptr(), H.data_ptr(),
                                 H.data_ptr(), H.data_ptr(), H.data_ptr(), None, ws.data_ptr(), 16, None)
    assert st == gpu.GPTQ_E_INVALID_ARG


# -------------------------------------------------------- whole layer path
def run_chain(gpu, cfg, X, W):
    H = gpu.gptq_hessian_accumulate(gpu_tensor(X) if isinstance(X, np.ndarray) else X)
    hv = gpu.gptq_prepare_hinv(H, cfg.damp)
    q = gpu.gptq_quantize_layer(gpu_tensor(W), hv.U, cfg.bits, cfg.group_size, cfg.block)
    torch.cuda.synchronize()
    return H, hv, q


def test_chain_tiny_fp32_layer(gpu):
    """The 256x256 fp32 layer with 4096 tokens, rowwise 4-bit: full chain."""
    cfg = CONFIGS["tiny_256x256_fp32_4bit_rowwise"]
    X, W = activations(cfg, threads=1), weights(cfg)
    H, hv, q = run_chain(gpu, cfg, X, W)
    Href = O.hessian(X)
    assert rel_fro(H.cpu().numpy(), Href) < 1e-4
    U, lam = O.prepare_hinv(Href, cfg.damp)
    assert int(hv.info.item()) == 0
    assert rel_fro(hv.U.cpu().numpy(), U) < 1e-3
    ref = O.quantize_layer(W, U, cfg.bits, cfg.group_size, cfg.block, decide=np.float32)
    check_quant(q, ref, cfg.bits, rerun_for(W, U, cfg.bits, cfg.group_size, cfg.block))


@pytest.mark.parametrize("name", ["attn_proj_4096x4096_3bit_g128", "attn_proj_4096x4096_3bit_rowwise", "mlp_down_4096x11008_4bit_g128"])
def test_chain_reduced_layers(gpu, name):
    """Each layer config at reduced size (same distributions), full chain."""
    cfg = small(CONFIGS[name], d_row=96, d_col=640 if "11008" not in name else 1152, n_tokens=9000)
    say("chain", cfg.name, cfg.d_row, cfg.d_col, cfg.n_tokens)
    X, W = activations(cfg, threads=4), weights(cfg)
    H, hv, q = run_chain(gpu, cfg, X, W)
    Href = O.hessian(X)
    assert rel_fro(H.cpu().numpy(), Href) < 1e-4
    U, _ = O.prepare_hinv(Href, cfg.damp)
    ref = O.quantize_layer(W, U, cfg.bits, cfg.group_size, cfg.block, decide=np.float32)
    check_quant(q, ref, cfg.bits, rerun_for(W, U, cfg.bits, cfg.group_size, cfg.block))


@pytest.mark.timeout(900)
def test_chain_full_size_attention_layer(gpu):
    """4096x4096 fp16 layer, 262144 fp16 tokens, 4-bit g128, in the launch
    configuration the benchmark times. H is compared in full; the sweep on a
    seeded subset of 256 rows (rows are independent given U)."""
    cfg = CONFIGS["attn_proj_4096x4096_4bit_g128"]
    say("full-size", cfg.name)
    Xd = torch.empty((cfg.n_tokens, cfg.d_col), dtype=torch.float16, device=DEV)
    t = 0

    def uploaded_chunks():
        nonlocal t
        for ch in activation_chunks(cfg, threads=8):
            Xd[t : t + ch.shape[0]] = torch.from_numpy(ch).to(DEV)
            t += ch.shape[0]
            yield ch

    Href = O.hessian(uploaded_chunks())
    assert t == cfg.n_tokens
    W = weights(cfg)
    H, hv, q = run_chain(gpu, cfg, Xd, W)
    e = rel_fro(H.cpu().numpy(), Href)
    say("H rel fro", e)
    assert e < 1e-4
    U, _ = O.prepare_hinv(Href, cfg.damp)
    eu = rel_fro(hv.U.cpu().numpy(), U)
    say("U rel fro", eu)
    assert int(hv.info.item()) == 0 and eu < 1e-5
    rows = np.sort(np.random.default_rng(0).choice(cfg.d_row, 256, replace=False))
    ref = O.quantize_layer(W[rows], U, cfg.bits, cfg.group_size, cfg.block, decide=np.float32)
    check_quant(q, ref, cfg.bits, rerun_for(W[rows], U, cfg.bits, cfg.group_size, cfg.block), rows=rows)
