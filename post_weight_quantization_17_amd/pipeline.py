"""Calibration pipeline over the library's entry points.

xuzou.cn reading card of the GPTQ paper, section 计算设置: the model is
quantized one block at a time; calibration data run through a block give
each layer's Hessian, the layers are quantized, and the quantized block is
run to produce the next block's inputs. Two pieces of that:

* ``quantize_shared_input``: layers that read the same input (the q/k/v
  projections) share one Hessian, accumulated over the calibration chunks
  (``accumulate``), and one factor; each layer is then swept with it, so
  each layer's loss is the library's own fp64 sum.
* ``quantize_mlp_block``: up layer, ReLU, down layer, quantized in order,
  the down layer calibrated on the output of the quantized up layer.

Every step runs in the library's kernels, the quantized layers included
(``gptq_dequant_gemm``: tokens x packed weights on the fp16 MFMA with the
ReLU in its epilogue; with its workspace, the weights are dequantized once
and both operands are taken K-major). torch only provides device memory,
workspaces and streams.
"""

from __future__ import annotations

from typing import Iterable, List, Sequence

import torch

from . import (
    Quantized,
    gptq_dequant_gemm,
    gptq_hessian_accumulate,
    gptq_prepare_hinv,
    gptq_quantize_layer,
)


def quantize_shared_input(chunks: Iterable[torch.Tensor], Ws: Sequence[torch.Tensor], bits: int, group_size: int,
                          block: int = 128, damp: float = 0.01, symmetric: bool = False):
    """One Hessian over all calibration chunks ([tokens_i, d] each), one
    factor, and each layer in ``Ws`` ([rows_k, d] each) swept with it.
    Returns (H, hinv, list of Quantized, one per layer)."""
    H = None
    for i, X in enumerate(chunks):
        H = gptq_hessian_accumulate(X, H=H, accumulate=i > 0)
    if H is None:
        raise ValueError("no calibration chunks")
    hv = gptq_prepare_hinv(H, damp)
    layers: List[Quantized] = [gptq_quantize_layer(Wk, hv.U, bits, group_size, block, symmetric=symmetric)
                               for Wk in Ws]
    return H, hv, layers


def quantize_mlp_block(X0: torch.Tensor, W_up: torch.Tensor, W_down: torch.Tensor, bits: int, group_size: int,
                       block: int = 128, damp: float = 0.01):
    """Quantize an MLP block layer by layer: H_up from X0 [tokens, d_model]
    (fp16), quantize W_up [d_ff, d_model]; X1 = relu(X0 What_up^T) (fp16)
    from the quantized up layer; H_down from X1, quantize W_down
    [d_model, d_ff]; X2 = X1 What_down^T (fp16) is the block output.
    Returns a dict with the Hessians, factors, quantized layers, X1 and X2."""
    d_model = X0.shape[1]
    d_ff = W_up.shape[0]
    H_up = gptq_hessian_accumulate(X0)
    hv_up = gptq_prepare_hinv(H_up, damp)
    q_up = gptq_quantize_layer(W_up, hv_up.U, bits, group_size, block)
    X1 = gptq_dequant_gemm(q_up.packed, q_up.scales, q_up.zeros, d_model, bits, group_size, X0, relu=True)
    H_down = gptq_hessian_accumulate(X1)
    hv_down = gptq_prepare_hinv(H_down, damp)
    q_down = gptq_quantize_layer(W_down, hv_down.U, bits, group_size, block)
    X2 = gptq_dequant_gemm(q_down.packed, q_down.scales, q_down.zeros, d_ff, bits, group_size, X1)
    return dict(H_up=H_up, hinv_up=hv_up, up=q_up, X1=X1, H_down=H_down, hinv_down=hv_down, down=q_down, X2=X2)
