"""Calibration pipeline over the library's entry points.

xuzou.cn reading card of the GPTQ paper, section 计算设置: the model is
quantized one block at a time; calibration data run through a block give
each layer's Hessian, the layers are quantized, and the quantized block is
run to produce the next block's inputs. Two pieces of that:

* ``quantize_shared_input``: layers that read the same input (the q/k/v
  projections) share one Hessian, accumulated over the calibration chunks
  (``accumulate``), and one factor; their rows are swept together in one
  call, since rows are independent given the factor.
* ``quantize_mlp_block``: up layer, ReLU, down layer, quantized in order,
  the down layer calibrated on the output of the quantized up layer.

Every step of the method runs in the library's kernels. Running the
quantized layers on the calibration tokens (a [tokens x d_in] x [d_in x d_out]
product, with the weights dequantized to fp16 by ``gptq_dequantize``) is a
plain dense GEMM and uses torch's library GEMM; the block's ReLU is torch's.
"""

from __future__ import annotations

from typing import Iterable, List, Sequence

import torch

from . import (
    Quantized,
    gptq_dequantize,
    gptq_hessian_accumulate,
    gptq_prepare_hinv,
    gptq_quantize_layer,
)


def quantize_shared_input(chunks: Iterable[torch.Tensor], Ws: Sequence[torch.Tensor], bits: int, group_size: int,
                          block: int = 128, damp: float = 0.01, symmetric: bool = False):
    """One Hessian over all calibration chunks ([tokens_i, d] each), one
    factor, and the rows of all layers in ``Ws`` ([rows_k, d] each, one
    dtype) swept in one call. Returns (H, hinv, stacked Quantized, per-layer
    list of Quantized views)."""
    H = None
    for i, X in enumerate(chunks):
        H = gptq_hessian_accumulate(X, H=H, accumulate=i > 0)
    if H is None:
        raise ValueError("no calibration chunks")
    hv = gptq_prepare_hinv(H, damp)
    W = torch.cat(list(Ws), dim=0)
    q = gptq_quantize_layer(W, hv.U, bits, group_size, block, symmetric=symmetric)
    layers: List[Quantized] = []
    r0 = 0
    for Wk in Ws:
        r1 = r0 + Wk.shape[0]
        rl = q.row_loss[r0:r1]
        layers.append(Quantized(q.codes[r0:r1], q.scales[r0:r1], q.zeros[r0:r1], q.packed[r0:r1],
                                rl.double().sum(), rl))
        r0 = r1
    return H, hv, q, layers


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
    Wh_up = gptq_dequantize(q_up.packed, q_up.scales, q_up.zeros, d_model, bits, group_size, torch.float16)
    X1 = torch.matmul(X0, Wh_up.t())
    X1.relu_()
    H_down = gptq_hessian_accumulate(X1)
    hv_down = gptq_prepare_hinv(H_down, damp)
    q_down = gptq_quantize_layer(W_down, hv_down.U, bits, group_size, block)
    Wh_down = gptq_dequantize(q_down.packed, q_down.scales, q_down.zeros, d_ff, bits, group_size, torch.float16)
    X2 = torch.matmul(X1, Wh_down.t())
    return dict(H_up=H_up, hinv_up=hv_up, up=q_up, X1=X1, H_down=H_down, hinv_down=hv_down, down=q_down, X2=X2)
