"""Float64 CPU oracle for the GPTQ layer path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it, and it shares no code
with the HIP library.
"""

from .gptq_oracle import (  # noqa: F401
    damped,
    dequantize,
    group_params,
    hessian,
    layer_loss_direct,
    pack,
    prepare_hinv,
    quantize_layer,
    rtn,
    unpack,
)
