"""Seeded inputs and FLOP/parameter accounting (CPU)."""
import json
import math
import os

import numpy as np

from dense_decoder_only_amd import accounting as acc
from synthetic import CONFIGS, bf16_bits_to_f32, make_tokens, to_bf16_bits, zipf_ids


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _scale():
    with open(os.path.join(GOLDEN, "d20_scale.json")) as f:
        return json.load(f)


def test_param_counts():
    d20 = CONFIGS["d20"]
    assert acc.total_params(d20) == 502_005_760
    # with full K/V heads the d20 count is the page's approximate d20 size
    full = acc.total_params(d20, kv_heads=d20.n_head)
    assert full == 560_988_160
    assert abs(full - _scale()["d20_params_approx"]) / _scale()["d20_params_approx"] < 0.005
    assert acc.total_params(CONFIGS["tiny"]) == 491_520
    assert acc.total_params(CONFIGS["d26"]) == 949_092_352


def test_flops_convention_matches_pages():
    d20 = CONFIGS["d20"]
    assert acc.matmul_params(d20) == 418_119_680
    assert acc.flops_per_token(d20) == 6 * 418_119_680 + 6 * 20 * 10 * 128 * 2048
    # the page's token budget is 20 tokens per parameter, and 6 N D over it is
    # its approximate total compute
    g = _scale()
    assert abs(g["d20_tokens"] - g["tokens_per_param"] * g["d20_params_approx"]) < 1e6
    full = acc.total_params(d20, kv_heads=d20.n_head)
    assert abs(6 * full * g["d20_tokens"] - g["d20_total_flops_approx"]) / g["d20_total_flops_approx"] < 0.07


def test_zipf_marginals():
    rng = np.random.default_rng(0)
    V = 65536
    ids = zipf_ids(rng, V, 400_000, 1.1)
    assert ids.min() >= 0 and ids.max() < V
    w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    p0 = 1.0 / w.sum()
    assert abs(np.mean(ids == 0) - p0) < 5 * math.sqrt(p0 * (1 - p0) / ids.size)
    assert abs(np.mean(ids == 1) - p0 * 2 ** -1.1) < 0.003


def test_tokens_seeded_and_shaped():
    cfg = CONFIGS["small"]
    a = make_tokens(cfg)
    b = make_tokens(cfg)
    assert a.shape == (cfg.batch, cfg.seq_len + 1) and a.dtype == np.int32
    np.testing.assert_array_equal(a, b)


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38, np.inf], np.float32)
    bits = to_bf16_bits(x)
    back = bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: 1 + 2^-6 is even.
    np.testing.assert_array_equal(back[:5], np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5], np.float32))
    assert np.isinf(back[6])
    # against torch's own fp32 -> bf16 conversion (also round to nearest even)
    import torch
    r = np.random.default_rng(3).standard_normal(10000).astype(np.float32)
    t = torch.tensor(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(to_bf16_bits(r), t)
