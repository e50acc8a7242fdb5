"""The seeded generator is deterministic and has the stated structure."""

import numpy as np
import torch

from post_weight_quantization_18_amd import synthetic as S


def test_generator_is_deterministic_and_seeded_per_layer():
    cfg = S.scaled(S.CONFIGS["toy768"], m=64, d=128, n_tokens=2048)
    w1, x1 = S.make_layer(cfg)
    w2, x2 = S.make_layer(cfg)
    assert torch.equal(w1, w2) and torch.equal(x1, x2)
    other = S.scaled(S.CONFIGS["opt175b-k"], m=64, d=128, n_tokens=2048)
    assert not torch.equal(S.make_weights(other), S.make_weights(S.scaled(S.CONFIGS["opt175b-q"], m=64, d=128,
                                                                          n_tokens=2048)))


def test_generator_shapes_dtypes_and_structure():
    cfg = S.CONFIGS["toy768"]
    w, x = S.make_layer(cfg)
    assert w.shape == (768, 768) and w.dtype == torch.float32
    assert x.shape == (4096, 768) and x.dtype == torch.float16
    wn = w.double().numpy()
    col_std = wn.std(axis=0)
    assert np.sum(col_std > 0.1) == 8                    # eight x10 outlier input columns
    assert 0.015 < np.median(col_std) < 0.025
    xv = x.double().numpy().var(axis=0)
    assert np.sum(xv > 50) == 6                          # six x20 activation channels
    ev = np.linalg.eigvalsh(np.cov(x.double().numpy().T))
    assert ev[-1] / ev[len(ev) // 2] > 20                # strongly correlated, decaying spectrum


def test_config_table_matches_the_workloads():
    c = S.CONFIGS
    assert (c["opt2.7b-fc1"].m, c["opt2.7b-fc1"].d, c["opt2.7b-fc1"].n_tokens) == (10240, 2560, 262144)
    assert (c["opt175b-fc2"].m, c["opt175b-fc2"].d) == (12288, 49152)
    assert c["opt13b-attn"].group == 128 and c["opt13b-attn"].bits == 3
    assert c["opt175b-fc1-ternary"].grid == "ternary"
    assert len(S.OPT175B_BLOCK) == 6
