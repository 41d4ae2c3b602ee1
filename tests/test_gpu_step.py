"""Whole-step parity: nc_step_fwd_bwd against the fp64 oracle.

Tolerances (the readings of the target): fp32 configuration: loss rel 1e-4,
every gradient max-rel 1e-3.  bf16 configurations: loss rel 2e-3, every
gradient cosine >= 0.999 and max-rel <= 3e-2, where
max-rel = ||g - g*||_inf / ||g*||_inf per parameter tensor.

At the full d12/d20/d26 sizes the oracle cannot run the whole batch in a
test, so the step runs at the full batch (the benchmark's launch
configuration) and sampled sequences' per-token losses are compared with the
oracle's forward of those sequences; gradients are compared on a one-sequence
batch of the same model."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import cosine, dev_to_f64, max_rel, run_step
from synthetic import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _check_grads(cfg, got, ref, bf16):
    for k, g in got.items():
        g = dev_to_f64(g)
        assert np.all(np.isfinite(g)), k
        mr = max_rel(g, ref[k])
        if bf16:
            cs = cosine(g, ref[k])
            assert cs >= 0.999 and mr <= 3e-2, (k, cs, mr)
        else:
            assert mr <= 1e-3, (k, mr)


def _check_embed_rows(ids, dE):
    absent = np.setdiff1d(np.arange(dE.shape[0]), ids)
    assert np.all(dev_to_f64(dE)[absent] == 0.0), "embedding rows of absent ids must be exactly zero"


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_step_full_parity(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    out = run_step(cfg, inp)
    assert out["status"] == 0
    p = oracle.to_f64_params(inp["weights"])
    ref = oracle.step(cfg, p, inp["ids"], inp["targets"], inp["token_bytes"])
    bf16 = cfg.dtype == "bf16"
    tol_loss = 2e-3 if bf16 else 1e-4
    assert float(out["loss"]) == pytest.approx(ref["loss"], rel=tol_loss)
    assert float(out["bpb"]) == pytest.approx(ref["bpb"], rel=tol_loss)
    lt = dev_to_f64(out["loss_tok"])
    assert max_rel(lt, ref["loss_tok"]) < (2e-2 if bf16 else 1e-4)
    _check_grads(cfg, out["grads"], ref["grads"], bf16)
    _check_embed_rows(inp["ids"], out["grads"]["embed"])


def test_step_deterministic_accumulating_and_causal():
    cfg = CONFIGS["small"]
    inp = make_inputs(cfg)
    a = run_step(cfg, inp)
    b = run_step(cfg, inp)
    assert torch.equal(a["loss"], b["loss"]) and torch.equal(a["loss_tok"], b["loss_tok"])
    for k in a["grads"]:
        assert torch.equal(a["grads"][k], b["grads"][k]), k
    # accumulate = 1 adds the step's gradient to what is there
    acc = {k: v.clone() for k, v in a["grads"].items()}
    c = run_step(cfg, inp, accumulate=1, grads=acc)
    for k in acc:
        # (base + p1) + p2 vs base + (p1 + p2): equal up to fp32 rounding
        torch.testing.assert_close(c["grads"][k], 2 * a["grads"][k], rtol=1e-5, atol=1e-12)
    # future tokens do not change earlier per-token losses, bit for bit
    S = inp["S"].copy()
    t0 = 200
    r = np.random.default_rng(3000 + cfg.index)
    S[0, t0 + 2:] = r.integers(0, cfg.vocab, S.shape[1] - t0 - 2)
    d = run_step(cfg, inp, ids=np.ascontiguousarray(S[:, :-1]), targets=np.ascontiguousarray(S[:, 1:]))
    assert torch.equal(d["loss_tok"][0, : t0 + 1], a["loss_tok"][0, : t0 + 1])
    assert not torch.equal(d["loss_tok"][0, t0 + 1:], a["loss_tok"][0, t0 + 1:])
    assert torch.equal(d["loss_tok"][1:], a["loss_tok"][1:])


@pytest.mark.parametrize("name", ["d12", "d20", "d26"])
def test_step_full_size_sampled_losses(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    out = run_step(cfg, inp)
    assert out["status"] == 0
    lt = dev_to_f64(out["loss_tok"])
    assert np.all(np.isfinite(lt))
    # the reported mean and bits-per-byte agree with the per-token losses
    assert float(out["loss"]) == pytest.approx(lt.mean(), rel=1e-5)
    assert float(out["bpb"]) == pytest.approx(lt.sum() / (math.log(2) * 4.8 * lt.size), rel=1e-5)
    _check_embed_rows(inp["ids"], out["grads"]["embed"])
    for k, g in out["grads"].items():
        assert torch.isfinite(g).all(), k
    p = oracle.to_f64_params(inp["weights"])
    b = cfg.batch - 1  # a sampled sequence
    ref, _ = oracle.sequence_forward(cfg, p, inp["ids"][b], inp["targets"][b], keep_cache=False)
    assert lt[b].mean() == pytest.approx(ref.mean(), rel=2e-3)
    assert max_rel(lt[b], ref) < 2e-2


@pytest.mark.parametrize("name", ["d12"])
def test_step_full_size_gradients_one_sequence(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    out = run_step(cfg, inp, batch=1)
    p = oracle.to_f64_params(inp["weights"])
    ref = oracle.step(cfg, p, inp["ids"][:1], inp["targets"][:1], inp["token_bytes"])
    assert float(out["loss"]) == pytest.approx(ref["loss"], rel=2e-3)
    _check_grads(cfg, out["grads"], ref["grads"], True)
