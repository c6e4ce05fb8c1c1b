"""Parity of the packed-layer matrix-vector product with the oracle (needs an
MI355X).

Inputs are seeded: random codes packed by the oracle, random scales and
zeros, fp16 activations. The oracle computes in float64 from the same
values. Tolerance: fp32 accumulation over d_col terms, so every output is
within 1e-5 of the sum of |What[r][c] x[c]| over its row (about 2^-24 per
term, with a wide margin), plus bit-identical repeats.
"""

import numpy as np
import pytest
import torch

import oracle.gptq_oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def make_inputs(d_row, d_col, bits, group, batch, seed):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 2**bits, size=(d_row, d_col), dtype=np.int64)
    ng = 1 if group == -1 else -(-d_col // group)
    scales = r.uniform(0.001, 0.02, size=(d_row, ng)).astype(np.float32)
    zeros = r.integers(0, 2**bits, size=(d_row, ng)).astype(np.int32)
    x = r.standard_normal((batch, d_col)).astype(np.float16)
    return O.pack(codes, bits), scales, zeros, x


def run(gpu, d_row, d_col, bits, group, batch, seed, ldx=None, off=1):
    packed, scales, zeros, x = make_inputs(d_row, d_col, bits, group, batch, seed)
    ref = O.dequant_matvec(packed, scales.astype(np.float64), zeros.astype(np.float64), d_col, bits, group, x)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    pk = g(packed.view(np.int32))
    if ldx is None:
        xd = g(x)
    else:  # rows of x ldx apart (view into a wider buffer, offset by `off` elements)
        buf = torch.zeros((batch, ldx), dtype=torch.float16, device=DEV)
        buf[:, off : off + d_col] = g(x)
        xd = buf[:, off : off + d_col]
    y = gpu.gptq_dequant_matvec(pk, g(scales), g(zeros), d_col, bits, group, xd)
    y2 = gpu.gptq_dequant_matvec(pk, g(scales), g(zeros), d_col, bits, group, xd)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)  # deterministic
    codes = O.unpack(packed, d_col, bits)
    What = O.dequantize(codes, scales.astype(np.float64), zeros.astype(np.float64), group)
    bound = 1e-5 * (np.abs(x.astype(np.float64)) @ np.abs(What).T) + 1e-30
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
    return y


@pytest.mark.parametrize(
    "d_row,d_col,bits,group,batch",
    [
        (1, 1, 4, -1, 1),
        (7, 33, 3, 16, 1),
        (5, 31, 2, 8, 2),
        (64, 256, 4, 128, 1),
        (100, 1000, 2, 40, 1),
        (33, 4096, 3, 128, 3),
        (16, 128, 8, 32, 9),
        (129, 2048, 4, -1, 4),
        (4096, 4096, 4, 128, 1),
        (12288, 4096, 3, 128, 1),
        # groups of 32-column multiples with aligned activations: the
        # code-pair kernel, with a partial last unit, no full unit at all,
        # and each rows-per-wave choice (1, 2 and 4 rows)
        (70, 1000, 3, -1, 2),
        (3, 24, 4, -1, 1),
        (40, 1024, 8, 32, 2),
        (300, 2048, 2, 64, 1),
        (5000, 776, 8, -1, 1),
        (9000, 296, 4, -1, 3),
        (8193, 4128, 3, 32, 2),
        # more row blocks than resident waves: several row blocks per wave
        (20000, 512, 4, 128, 1),
        (40000, 264, 2, -1, 2),
        # the MFMA form (128-column super-units, groups of 128-multiples, more
        # than two vectors or tall layers): a ragged last group of 256, rows
        # not a multiple of 64, exactly 16 and 17 vectors (two passes), an
        # LDS chunk boundary (9 super-units), every code width
        (100, 640, 2, 256, 5),
        (70, 1024, 8, -1, 16),
        (50, 512, 3, 128, 17),
        (9000, 1152, 4, 128, 1),
        (8192, 1024, 2, 128, 1),
        (300, 2048, 8, 128, 3),
    ],
)
def test_dequant_matvec_parity(gpu, d_row, d_col, bits, group, batch):
    run(gpu, d_row, d_col, bits, group, batch, seed=d_row + 7 * d_col + bits)


def test_dequant_matvec_strided_unaligned_activations(gpu):
    run(gpu, 40, 300, 3, 16, 3, seed=5, ldx=302, off=1)


def test_dequant_matvec_strided_aligned_activations(gpu):
    # 16-byte aligned rows ldx apart: the code-pair kernel with ldx != d_col
    run(gpu, 64, 1000, 3, -1, 3, seed=6, ldx=1040, off=8)
    run(gpu, 64, 1024, 4, 128, 2, seed=7, ldx=1032, off=8)
    run(gpu, 64, 1024, 3, 128, 5, seed=8, ldx=1040, off=8)  # the MFMA form


def test_dequant_matvec_rejects_bad_arguments(gpu):
    lib = gpu.load()
    buf = torch.zeros(64, dtype=torch.int32, device=DEV)
    p = buf.data_ptr()
    assert lib.gptq_dequant_matvec(p, p, p, 4, 16, 5, -1, p, 1, 16, p, None) == gpu.GPTQ_E_INVALID_ARG  # bits
    assert lib.gptq_dequant_matvec(p, p, p, 4, 16, 4, 12, p, 1, 16, p, None) == gpu.GPTQ_E_INVALID_ARG  # group
    assert lib.gptq_dequant_matvec(p, p, p, 4, 16, 4, -1, p, 1, 8, p, None) == gpu.GPTQ_E_INVALID_ARG  # ldx
    assert lib.gptq_dequant_matvec(p, p, p, 4, 16, 4, -1, p, 0, 16, p, None) == gpu.GPTQ_E_INVALID_ARG  # batch


@pytest.mark.parametrize("d_row,d_col,bits,group", [(49152, 12288, 3, 128), (11008, 4096, 4, 128)])
def test_dequant_matvec_full_size_sampled_rows(gpu, d_row, d_col, bits, group):
    """Full-size layers, in the launch configuration the benchmark times:
    random words (every bit pattern is a valid code stream), the oracle on a
    seeded sample of rows."""
    r = np.random.default_rng(d_row + bits)
    nw = -(-d_col * bits // 32)
    packed = r.integers(0, 2**32, size=(d_row, nw), dtype=np.uint64).astype(np.uint32)
    ng = d_col // group
    scales = r.uniform(0.001, 0.02, size=(d_row, ng)).astype(np.float32)
    zeros = r.integers(0, 2**bits, size=(d_row, ng)).astype(np.int32)
    x = r.standard_normal((1, d_col)).astype(np.float16)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    y = gpu.gptq_dequant_matvec(g(packed.view(np.int32)), g(scales), g(zeros), d_col, bits, group, g(x))
    torch.cuda.synchronize()
    rows = np.unique(np.append(r.choice(d_row, 384, replace=False), [0, d_row - 1]))
    sc, zr = scales[rows].astype(np.float64), zeros[rows].astype(np.float64)
    ref = O.dequant_matvec(packed[rows], sc, zr, d_col, bits, group, x)
    What = O.dequantize(O.unpack(packed[rows], d_col, bits), sc, zr, group)
    bound = 1e-5 * (np.abs(x.astype(np.float64)) @ np.abs(What).T) + 1e-30
    err = np.abs(y.cpu().numpy()[:, rows].astype(np.float64) - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
