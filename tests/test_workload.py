"""Host-side checks of the seeded synthetic input generator."""

import numpy as np

from workload import CONFIGS, activation_chunks, n_outliers, outlier_channels, weights
from workload.synth import CHUNK, small


def test_configs_shapes_and_outlier_counts():
    c = CONFIGS
    assert n_outliers(c["tiny_256x256_fp32_4bit_rowwise"]) == 3
    assert n_outliers(c["attn_proj_4096x4096_4bit_g128"]) == 20
    assert n_outliers(c["mlp_down_4096x11008_4bit_g128"]) == 55
    assert n_outliers(c["opt175b_12288x12288_3bit_g128"]) == 12
    assert c["attn_proj_4096x4096_4bit_g128"].n_tokens == 262144
    assert c["opt175b_49152x12288_3bit_g128"].d_row == 49152


def test_generator_is_deterministic_and_chunk_addressable():
    cfg = small(CONFIGS["attn_proj_4096x4096_4bit_g128"], d_col=64, d_row=8, n_tokens=2 * CHUNK + 5)
    a = np.concatenate(list(activation_chunks(cfg, threads=1)))
    b = np.concatenate(list(activation_chunks(cfg, threads=4)))
    assert a.dtype == np.float16 and a.shape == (cfg.n_tokens, 64)
    assert np.array_equal(a, b)
    w1, w2 = weights(cfg), weights(cfg)
    assert w1.dtype == np.float16 and np.array_equal(w1, w2)
    assert np.array_equal(weights(cfg, rows=np.array([1, 5])), w1[[1, 5]])
    # outlier channels carry the factor: their mean square is far larger
    ms = np.mean(a.astype(np.float64) ** 2, axis=0)
    oc = outlier_channels(cfg)
    assert len(oc) == 0 or ms[oc].min() > 50 * np.median(ms)
