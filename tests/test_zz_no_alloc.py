"""The allocation-free sweep entry point against the workspace one (needs an
MI355X).

gptq_quantize_layer_noalloc runs the same kernels as gptq_quantize_layer
with the library's static scratch in place of the caller's workspace, so its
outputs must equal the workspace entry point's to the bit. Two calls in a
row, the second with a smaller, ragged layer, show that nothing the first
call left in the scratch leaks into the second. Calls go through the C ABI.
"""

import ctypes

import numpy as np
import pytest
import torch

from tests.test_gpu_parity import DEV, gpu_tensor, say

pytestmark = pytest.mark.gpu

FIELDS = ("codes", "scales", "zeros", "packed", "row_loss", "loss")


def _outputs(g, d_row, d_col, bits, group):
    return g._quantized_like(d_row, d_col, bits, group, True, DEV)


def _call_noalloc(g, W, U, bits, group, out):
    lib = g.load()
    d_row, d_col = W.shape
    return lib.gptq_quantize_layer_noalloc(
        W.data_ptr(), g._dtype_code(W), d_row, d_col, U.data_ptr(), bits, group, 128, 0, out.codes.data_ptr(),
        out.scales.data_ptr(), out.zeros.data_ptr(), out.packed.data_ptr(), out.loss.data_ptr(),
        out.row_loss.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _upper_factor(d, seed):
    r = np.random.default_rng(seed)
    U = np.triu(r.standard_normal((d, d), dtype=np.float32)) * np.float32(2e-3) + np.eye(d, dtype=np.float32)
    return gpu_tensor(U)


def _same(a, b):
    for f in FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        assert torch.equal(x.reshape(-1).view(torch.uint8), y.reshape(-1).view(torch.uint8)), f


def test_noalloc_matches_workspace_entry_point(gpu):
    """4096 x 4096 fp16 (the largest layer the scratch holds: 2^24 weights),
    then 300 x 700 fp32 with ragged blocks; each against gptq_quantize_layer
    bit for bit, with the outputs filled with garbage beforehand."""
    cases = [(4096, 4096, 4, 128, np.float16, 11), (300, 700, 3, 64, np.float32, 12)]
    for d_row, d_col, bits, group, wdt, seed in cases:
        say("noalloc", d_row, d_col, bits, group, wdt.__name__)
        assert d_row * d_col <= gpu.GPTQ_NOALLOC_MAX_WEIGHTS
        W = gpu_tensor((0.02 * np.random.default_rng(seed).standard_normal((d_row, d_col))).astype(wdt))
        U = _upper_factor(d_col, seed + 100)
        ref = gpu.gptq_quantize_layer(W, U, bits, group, 128)
        out = _outputs(gpu, d_row, d_col, bits, group)
        for t in (out.scales, out.row_loss, out.loss):
            t.fill_(float("nan"))
        for t in (out.codes, out.zeros, out.packed):
            t.fill_(-1 if t.dtype != torch.uint8 else 255)
        st = _call_noalloc(gpu, W, U, bits, group, out)
        assert st == gpu.GPTQ_OK, gpu.status_string(st)
        torch.cuda.synchronize()
        _same(out, ref)
        # the Python binding calls the same entry point
        again = gpu.gptq_quantize_layer_noalloc(W, U, bits, group)
        torch.cuda.synchronize()
        _same(again, ref)


def test_noalloc_rejects_layers_beyond_its_scratch(gpu):
    """Sizes past the static scratch come back as GPTQ_E_TOO_LARGE before
    anything is enqueued (the outputs stay untouched)."""
    lib = gpu.load()
    W = torch.zeros((8, 16), dtype=torch.float16, device=DEV)
    U = torch.eye(16, dtype=torch.float32, device=DEV)
    out = _outputs(gpu, 8, 16, 4, -1)
    out.codes.fill_(7)
    p = out.codes.data_ptr()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    too_wide = 1 + gpu.GPTQ_NOALLOC_MAX_WEIGHTS // 4096
    for d_row, d_col in [(4096, too_wide), (gpu.GPTQ_NOALLOC_MAX_ROWS + 16, 16)]:
        st = lib.gptq_quantize_layer_noalloc(W.data_ptr(), 0, d_row, d_col, U.data_ptr(), 4, -1, 128, 0, p, p, p, p,
                                             p, None, s)
        assert st == gpu.GPTQ_E_TOO_LARGE, st
    assert gpu.status_string(gpu.GPTQ_E_TOO_LARGE).startswith("layer larger")
    # argument errors come first, as for gptq_quantize_layer
    st = lib.gptq_quantize_layer_noalloc(W.data_ptr(), 0, 8, 16, U.data_ptr(), 5, -1, 128, 0, p, p, p, p, p, None, s)
    assert st == gpu.GPTQ_E_INVALID_ARG
    torch.cuda.synchronize()
    assert bool(torch.all(out.codes == 7))
