"""Writes oracle_snapshot.json: the oracle's outputs on a tiny seeded layer.

The pages print no numeric worked example for this method (the aiqz.cc demo
prints its two MSEs only when run), so no fixture here holds the pages'
values. This snapshot is written by the oracle alone (``oracle/`` and the
seeded ``workload`` generator, nothing from the HIP library) and guards the
oracle's arithmetic against unnoticed changes: a change that alters it must
regenerate the file and say which passage of the pages justifies it.

Run:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle.gptq_oracle as O  # noqa: E402
from workload import CONFIGS, activations, weights  # noqa: E402
from workload.synth import small  # noqa: E402


def snapshot_config():
    return small(CONFIGS["attn_proj_4096x4096_3bit_g128"], d_row=6, d_col=48, n_tokens=300, group_size=16, block=16)


def compute():
    cfg = snapshot_config()
    X = activations(cfg, threads=1)
    W = weights(cfg)
    H = O.hessian(X)
    U, lam = O.prepare_hinv(H, cfg.damp)
    out = O.quantize_layer(W, U, cfg.bits, cfg.group_size, cfg.block)
    return dict(
        config=cfg.__dict__,
        lambda_=lam,
        H_diag=np.diag(H).tolist(),
        U_diag=np.diag(U).tolist(),
        codes=out["codes"].tolist(),
        scales=out["scales"].tolist(),
        zeros=out["zeros"].tolist(),
        packed=[[int(v) for v in r] for r in out["packed"]],
        loss=out["loss"],
    )


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_snapshot.json"), "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", os.path.join(HERE, "oracle_snapshot.json"))
