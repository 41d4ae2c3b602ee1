"""Pins of the inference oracle (oracle/decode.py) and their sensitivity.

decode_attention is held against torch's CPU float64 scaled_dot_product_attention
(an independent textbook routine), against the last row of the causal
attention oracle (itself pinned), and against two exact special cases.
prefix_logits is held against the loss path (its rows give the forward's
cross entropy), and against causality: the row of position t from the prefix
0..t equals the row t of the whole sequence, which is what makes a key/value
cache exact.
"""
import inspect
import math
import textwrap

import numpy as np
import pytest
import torch

import oracle
from oracle import decode as od
from oracle import model as om
from synthetic import CONFIGS, make_inputs


def _rand(*shape, seed=0):
    return np.random.default_rng(seed + sum(shape)).standard_normal(shape)


def test_decode_attention_matches_library_sdpa():
    H, n, hd = 5, 37, 16
    q, k, v = _rand(H, hd), _rand(n, hd, seed=1), _rand(n, hd, seed=2)
    scale = 1 / math.sqrt(hd)
    tq = torch.from_numpy(q)[None, :, None, :]                       # [1, H, 1, hd]
    tk = torch.from_numpy(k)[None, None].expand(1, H, n, hd).contiguous()
    tv = torch.from_numpy(v)[None, None].expand(1, H, n, hd).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, :, 0].numpy()
    np.testing.assert_allclose(od.decode_attention(q, k, v, scale), ref, rtol=1e-12, atol=1e-14)


def test_decode_attention_is_last_row_of_causal_attention():
    T, H, hd = 19, 3, 8
    q, k, v = _rand(T, H, hd), _rand(T, 1, hd, seed=3), _rand(T, 1, hd, seed=4)
    o, _ = om.attention(q, k, v, 0.3)
    for t in (0, 7, T - 1):
        got = od.decode_attention(q[t], k[: t + 1, 0], v[: t + 1, 0], 0.3)
        np.testing.assert_allclose(got, o[t], rtol=1e-13, atol=1e-15)


def test_decode_attention_special_cases():
    H, hd = 4, 8
    q, v1 = _rand(H, hd), _rand(1, hd, seed=5)
    # one cached position: every head returns that value exactly
    np.testing.assert_array_equal(od.decode_attention(q, _rand(1, hd, seed=6), v1, 0.5), np.repeat(v1, H, 0))
    # identical keys: uniform weights, the mean of the values
    n = 9
    k = np.repeat(_rand(1, hd, seed=7), n, 0)
    v = _rand(n, hd, seed=8)
    np.testing.assert_allclose(od.decode_attention(q, k, v, 0.5), np.repeat(v.mean(0, keepdims=True), H, 0),
                               rtol=1e-13)


def test_decode_attention_permutation_invariant():
    H, n, hd = 3, 12, 8
    q, k, v = _rand(H, hd), _rand(n, hd, seed=9), _rand(n, hd, seed=10)
    perm = np.random.default_rng(0).permutation(n)
    np.testing.assert_allclose(od.decode_attention(q, k[perm], v[perm], 0.4), od.decode_attention(q, k, v, 0.4),
                               rtol=1e-13)


def _tiny():
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, 1)
    return cfg, inp, oracle.to_f64_params(inp["weights"])


def test_prefix_logits_give_the_forward_loss():
    cfg, inp, p = _tiny()
    ids, y = inp["ids"][0], inp["targets"][0]
    zc = od.prefix_logits(cfg, p, ids)
    assert zc.shape == (cfg.seq_len, cfg.vocab) and np.all(np.abs(zc) < cfg.softcap)
    lt, _ = om.sequence_forward(cfg, p, ids, y, keep_cache=False)
    lse = np.log(np.exp(zc - zc.max(1, keepdims=True)).sum(1)) + zc.max(1)
    np.testing.assert_allclose(lse - zc[np.arange(len(y)), y], lt, rtol=1e-13)


def test_prefix_logits_rows_are_causal():
    cfg, inp, p = _tiny()
    ids = inp["ids"][0]
    full = od.prefix_logits(cfg, p, ids)
    for t in (0, 5, 31, cfg.seq_len - 2):
        part = od.prefix_logits(cfg, p, ids[: t + 1])
        np.testing.assert_allclose(part[-1], full[t], rtol=1e-12, atol=1e-13)


MUTATIONS = [
    ("decode_attention", "s = (q @ k.T) * scale", "s = q @ k.T"),
    ("decode_attention", "p = e / e.sum(axis=1, keepdims=True)", "p = e / e.sum(axis=0, keepdims=True)"),
    ("decode_attention", "return p @ v", "return p @ k"),
    ("decode_attention", "p = e / e.sum(axis=1, keepdims=True)", "p = e"),
    ("prefix_logits", 'return cache["zc"]', 'return cache["zc"] / cfg.softcap'),
]
PINS = [test_decode_attention_matches_library_sdpa, test_decode_attention_is_last_row_of_causal_attention,
        test_decode_attention_special_cases, test_decode_attention_permutation_invariant,
        test_prefix_logits_give_the_forward_loss, test_prefix_logits_rows_are_causal]


@pytest.mark.parametrize("fn,old,new", MUTATIONS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTATIONS)])
def test_some_pin_catches_mutation(monkeypatch, fn, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(od, fn)))
    assert src.count(old) == 1, (fn, old)
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant {fn}>", "exec"), od.__dict__, ns)
    monkeypatch.setattr(od, fn, ns[fn])
    caught = False
    for t in PINS:
        try:
            t()
        except Exception:
            caught = True
            break
    assert caught, f"no pin detects {fn}: {old!r} -> {new!r}"
