"""Pins for the fp64 oracle: checks against what the definition and the
mathematics fix, none of which re-types the oracle's own formulas.

Kinds of pin used here: closed forms, invariants, special cases that reduce
to a textbook or library routine (torch's CPU scaled-dot-product attention and
autograd in float64, scipy's logsumexp), brute force on tiny inputs, and
central finite differences of the whole model.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import model as om
from synthetic import CONFIGS, make_inputs

RNG = np.random.default_rng(12345)


def _rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- RMSNorm --

def test_rmsnorm_unit_rms():
    x = _rand(7, 33) * 3.0
    eps = 1e-6
    y, r = om.rms_norm(x, eps)
    ms = np.mean(x * x, axis=-1)
    got = np.sqrt(np.mean(y * y, axis=-1))
    np.testing.assert_allclose(got, np.sqrt(ms / (ms + eps)), rtol=1e-14)
    np.testing.assert_allclose(r[:, 0], 1.0 / np.sqrt(ms + eps), rtol=1e-14)


def test_rmsnorm_scale_invariance_and_bwd_orthogonality():
    # y(a x) = y(x) at eps = 0, hence the input gradient is orthogonal to x.
    x = _rand(5, 16)
    y1, _ = om.rms_norm(x, 0.0)
    y2, _ = om.rms_norm(3.7 * x, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-14, atol=1e-15)
    y, r = om.rms_norm(x, 0.0)
    g = _rand(5, 16)
    dx = om.rms_norm_bwd(g, y, r)
    np.testing.assert_allclose(np.sum(dx * x, axis=-1), 0.0, atol=1e-13)


def test_rmsnorm_bwd_finite_difference():
    x = _rand(3, 12)
    g = _rand(3, 12)
    eps = 1e-6
    y, r = om.rms_norm(x, eps)
    dx = om.rms_norm_bwd(g, y, r)
    h = 1e-6
    fd = np.zeros_like(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            fd[i, j] = (np.sum(g * om.rms_norm(xp, eps)[0]) - np.sum(g * om.rms_norm(xm, eps)[0])) / (2 * h)
    np.testing.assert_allclose(dx, fd, rtol=1e-7, atol=1e-9)


# ------------------------------------------------------------------- RoPE --

def test_rope_identity_at_position_zero_and_pair_norms():
    T, hd = 9, 16
    th = om.rope_angles(T, hd, 10000.0)
    x = _rand(T, 3, hd)
    y = om.rope(x, th)
    np.testing.assert_array_equal(y[0], x[0])
    n_in = x[..., : hd // 2] ** 2 + x[..., hd // 2:] ** 2
    n_out = y[..., : hd // 2] ** 2 + y[..., hd // 2:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13)


def test_rope_frequency_closed_form():
    # hd = 4, base = 100: pair i rotates at 100**(-2i/4): i = 0 -> 1 rad per
    # position, i = 1 -> 0.1 rad per position.  Unit vector e_1 (the first
    # element of pair 1) at position 3 goes to (cos 0.3, sin 0.3) in
    # components (1, 3).
    th = om.rope_angles(4, 4, 100.0)
    np.testing.assert_allclose(th[3], [3.0, 0.3], rtol=1e-15)
    x = np.zeros((4, 4)); x[3, 1] = 1.0
    y = om.rope(x, th)
    np.testing.assert_allclose(y[3], [0.0, math.cos(0.3), 0.0, math.sin(0.3)], atol=1e-15)
    x = np.zeros((4, 4)); x[2, 0] = 1.0
    y = om.rope(x, th)
    np.testing.assert_allclose(y[2], [math.cos(2.0), 0.0, math.sin(2.0), 0.0], atol=1e-15)


def test_rope_relative_position():
    # <rope(q, t+s), rope(k, u+s)> = <rope(q, t), rope(k, u)>
    hd, T = 32, 40
    th = om.rope_angles(T, hd, 10000.0)
    q, k = _rand(hd), _rand(hd)
    Q = np.tile(q, (T, 1)); K = np.tile(k, (T, 1))
    rq, rk = om.rope(Q, th), om.rope(K, th)
    base = rq[5] @ rk[2]
    for s in (1, 7, 30):
        np.testing.assert_allclose(rq[5 + s] @ rk[2 + s], base, rtol=1e-12)


def test_rope_bwd_is_inverse():
    T, hd = 11, 8
    th = om.rope_angles(T, hd, 10000.0)
    x = _rand(T, 2, hd)
    np.testing.assert_allclose(om.rope_bwd(om.rope(x, th), th), x, rtol=1e-13, atol=1e-14)


def test_qknorm_commutes_with_rope():
    T, hd = 13, 16
    th = om.rope_angles(T, hd, 10000.0)
    x = _rand(T, 4, hd)
    a = om.rms_norm(om.rope(x, th), 1e-6)[0]
    b = om.rope(om.rms_norm(x, 1e-6)[0], th)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


# -------------------------------------------------------------- attention --

def _sdpa_reference(q, k, v, scale):
    """torch CPU float64 scaled-dot-product attention, K/V repeated per head."""
    T, Hq, hd = q.shape
    Hkv = k.shape[1]
    rep = Hq // Hkv
    qt = torch.tensor(q).permute(1, 0, 2)
    kt = torch.tensor(np.repeat(k, rep, axis=1)).permute(1, 0, 2)
    vt = torch.tensor(np.repeat(v, rep, axis=1)).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_attention_matches_library_sdpa_mqa():
    T, H, hd = 24, 3, 16
    q, k, v = _rand(T, H, hd), _rand(T, 1, hd), _rand(T, 1, hd)
    o, P = om.attention(q, k, v, 1 / math.sqrt(hd))
    np.testing.assert_allclose(o, _sdpa_reference(q, k, v, 1 / math.sqrt(hd)), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=1e-14)
    assert np.all(np.triu(P, 1) == 0.0)
    # row 0 attends only to itself
    np.testing.assert_array_equal(o[0], np.repeat(v[0], H, axis=0))


def test_mqa_equals_mha_with_replicated_kv():
    T, H, hd = 10, 4, 8
    q, k, v = _rand(T, H, hd), _rand(T, 1, hd), _rand(T, 1, hd)
    o1, _ = om.attention(q, k, v, 0.3)
    o2, _ = om.attention(q, np.repeat(k, H, axis=1), np.repeat(v, H, axis=1), 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)
    do = _rand(T, H, hd)
    _, P1 = om.attention(q, k, v, 0.3)
    dq1, dk1, dv1 = om.attention_bwd(do, q, k, v, P1, 0.3)
    kr, vr = np.repeat(k, H, axis=1), np.repeat(v, H, axis=1)
    _, P2 = om.attention(q, kr, vr, 0.3)
    dq2, dk2, dv2 = om.attention_bwd(do, q, kr, vr, P2, 0.3)
    np.testing.assert_allclose(dq1, dq2, rtol=1e-13)
    np.testing.assert_allclose(dk1[:, 0], dk2.sum(1), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv1[:, 0], dv2.sum(1), rtol=1e-12, atol=1e-13)


def test_attention_bwd_matches_library_autograd():
    T, H, hd = 17, 2, 8
    scale = 1 / math.sqrt(hd)
    q, k, v, do = _rand(T, H, hd), _rand(T, 1, hd), _rand(T, 1, hd), _rand(T, H, hd)
    _, P = om.attention(q, k, v, scale)
    dq, dk, dv = om.attention_bwd(do, q, k, v, P, scale)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2), kt.expand(T, H, hd).permute(1, 0, 2),
        vt.expand(T, H, hd).permute(1, 0, 2), is_causal=True, scale=scale)
    (o.permute(1, 0, 2) * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


# ------------------------------------------------------ softcap and CE --

def test_softcap_bounds_and_small_signal():
    c = 15.0
    z = np.array([-1e6, -300.0, -40.0, 0.0, 1e-3, 40.0, 300.0, 1e6])
    zc = om.softcap(z, c)
    assert np.all(np.abs(zc) <= c)
    assert np.all(np.abs(zc[2:-2]) < c)
    # tanh series: c tanh(z/c) = z - z^3 / (3 c^2) + O(z^5)
    zs = np.array([1e-3, -2e-3, 0.05])
    np.testing.assert_allclose(om.softcap(zs, c), zs - zs ** 3 / (3 * c * c), rtol=1e-9)


def test_cross_entropy_against_logsumexp():
    z = _rand(6, 50) * 4
    y = RNG.integers(0, 50, 6)
    loss, lse = om.cross_entropy(z, y)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=1e-14)
    np.testing.assert_allclose(loss, -scipy.special.log_softmax(z, axis=1)[np.arange(6), y], rtol=1e-13)


def test_embed_bwd_brute_force_and_conservation():
    V, d, n = 11, 5, 40
    ids = RNG.integers(0, V, n)
    de = _rand(n, d)
    dE = om.embed_bwd(ids, de, V)
    ref = np.zeros((V, d))
    for t in range(n):
        for j in range(d):
            ref[ids[t], j] += de[t, j]
    np.testing.assert_allclose(dE, ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dE.sum(0), de.sum(0), rtol=1e-12)
    absent = np.setdiff1d(np.arange(V), ids)
    assert np.all(dE[absent] == 0.0)


# -------------------------------------------------- composed-model pins --

def _tiny(batch=2):
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, batch)
    return cfg, inp, oracle.to_f64_params(inp["weights"])


def test_zero_unembedding_gives_log_vocab():
    cfg, inp, p = _tiny()
    p["unembed"][:] = 0.0
    r = oracle.step(cfg, p, inp["ids"], inp["targets"], inp["token_bytes"])
    assert r["loss"] == pytest.approx(math.log(cfg.vocab), rel=1e-15)
    # with U = 0 every other gradient vanishes and dU[v] = (1/M) sum_t (1/V - [y_t = v]) h_t
    for k in ("embed", "w_qkv", "w_o", "w_fc", "w_proj"):
        assert np.all(r["grads"][k] == 0.0)
    M = inp["ids"].size
    hs = []
    for b in range(inp["ids"].shape[0]):
        _, cache = oracle.sequence_forward(cfg, p, inp["ids"][b], inp["targets"][b])
        hs.append(cache["h"])
    h = np.concatenate(hs)
    y = inp["targets"].reshape(-1)
    onehot = np.zeros((M, cfg.vocab)); onehot[np.arange(M), y] = 1
    dU = (1.0 / cfg.vocab - onehot).T @ h / M
    np.testing.assert_allclose(r["grads"]["unembed"], dU, rtol=1e-10, atol=1e-15)


def test_bits_per_byte_closed_form():
    cfg, inp, p = _tiny()
    r = oracle.step(cfg, p, inp["ids"], inp["targets"], inp["token_bytes"], want_grads=False)
    # the per-id byte table is float32, so each entry is float32(4.8)
    assert r["bpb"] == pytest.approx(r["loss"] / (float(np.float32(4.8)) * math.log(2)), rel=1e-13)
    # 1 / (4.8 ln 2) = 0.3005617..., stated to six digits
    assert r["bpb"] == pytest.approx(0.300561 * r["loss"], rel=5e-6)


def _head_only_loss(cfg, p, ids, y):
    """Closed form when every block adds nothing: loss of softcap(rms(rms(E[ids])) U^T)."""
    e = p["embed"][ids]
    x0 = e / np.sqrt(np.mean(e * e, -1, keepdims=True) + cfg.eps)
    h = x0 / np.sqrt(np.mean(x0 * x0, -1, keepdims=True) + cfg.eps)
    z = cfg.softcap * np.tanh((h @ p["unembed"].T) / cfg.softcap)
    return scipy.special.logsumexp(z, axis=1) - z[np.arange(len(y)), y], h


def test_blocks_off_reduces_to_head():
    cfg, inp, p = _tiny(1)
    p["w_o"][:] = 0.0
    p["w_proj"][:] = 0.0
    lt, _ = oracle.sequence_forward(cfg, p, inp["ids"][0], inp["targets"][0], keep_cache=False)
    ref, _ = _head_only_loss(cfg, p, inp["ids"][0], inp["targets"][0])
    np.testing.assert_allclose(lt, ref, rtol=1e-12)


def test_uniform_attention_special_case():
    # W_q = W_k = 0 -> q, k are 0 after RoPE and QK norm -> every query
    # averages the values of its prefix: o_t = mean_{u<=t} v_u for each head.
    # One layer, MLP off (W_fc = 0): x1 = x0 + concat_h(o) Wo^T.
    cfg, inp, p = _tiny(1)
    from dataclasses import replace
    cfg1 = replace(cfg, n_layer=1)
    H, hd, d = cfg.n_head, cfg.head_dim, cfg.d_model
    p1 = {k: (v[:1] if v.ndim == 3 else v) for k, v in p.items()}
    p1["w_qkv"] = p1["w_qkv"].copy(); p1["w_qkv"][0, : (H + 1) * hd] = 0.0
    p1["w_fc"] = np.zeros_like(p1["w_fc"])
    ids, y = inp["ids"][0], inp["targets"][0]
    lt, _ = oracle.sequence_forward(cfg1, p1, ids, y, keep_cache=False)
    e = p1["embed"][ids]
    x0 = e / np.sqrt(np.mean(e * e, -1, keepdims=True) + cfg.eps)
    a = x0 / np.sqrt(np.mean(x0 * x0, -1, keepdims=True) + cfg.eps)
    v = a @ p1["w_qkv"][0, (H + 1) * hd:].T                     # [T, hd]
    cm = np.cumsum(v, axis=0) / np.arange(1, len(ids) + 1)[:, None]
    x1 = x0 + np.tile(cm, (1, H)) @ p1["w_o"][0].T
    h = x1 / np.sqrt(np.mean(x1 * x1, -1, keepdims=True) + cfg.eps)
    z = cfg.softcap * np.tanh((h @ p1["unembed"].T) / cfg.softcap)
    ref = scipy.special.logsumexp(z, axis=1) - z[np.arange(len(y)), y]
    np.testing.assert_allclose(lt, ref, rtol=1e-11)


def test_relu2_mlp_special_case():
    # Attention off (Wo = 0).  W_fc = [I; -I; 0; 0], W_proj = [I, I, 0, 0]
    # give relu(m)^2 + relu(-m)^2 = m^2 elementwise: x1 = x0 + rms(x0)^2.
    cfg, inp, p = _tiny(1)
    from dataclasses import replace
    cfg1 = replace(cfg, n_layer=1)
    d, F = cfg.d_model, cfg.d_ff
    p1 = {k: (v[:1].copy() if v.ndim == 3 else v) for k, v in p.items()}
    p1["w_o"][:] = 0.0
    wfc = np.zeros((1, F, d)); wfc[0, :d] = np.eye(d); wfc[0, d: 2 * d] = -np.eye(d)
    wpr = np.zeros((1, d, F)); wpr[0, :, :d] = np.eye(d); wpr[0, :, d: 2 * d] = np.eye(d)
    p1["w_fc"], p1["w_proj"] = wfc, wpr
    ids, y = inp["ids"][0], inp["targets"][0]
    lt, _ = oracle.sequence_forward(cfg1, p1, ids, y, keep_cache=False)
    e = p1["embed"][ids]
    x0 = e / np.sqrt(np.mean(e * e, -1, keepdims=True) + cfg.eps)
    m = x0 / np.sqrt(np.mean(x0 * x0, -1, keepdims=True) + cfg.eps)
    x1 = x0 + m * m
    h = x1 / np.sqrt(np.mean(x1 * x1, -1, keepdims=True) + cfg.eps)
    z = cfg.softcap * np.tanh((h @ p1["unembed"].T) / cfg.softcap)
    ref = scipy.special.logsumexp(z, axis=1) - z[np.arange(len(y)), y]
    np.testing.assert_allclose(lt, ref, rtol=1e-11)


def test_causality_future_tokens_do_not_change_past_losses():
    cfg, inp, p = _tiny(1)
    S = inp["S"].copy()
    t0 = 30
    lt1, _ = oracle.sequence_forward(cfg, p, S[0, :-1], S[0, 1:], keep_cache=False)
    rng = np.random.default_rng(3000 + cfg.index)
    S[0, t0 + 2:] = rng.integers(0, cfg.vocab, S.shape[1] - t0 - 2)
    lt2, _ = oracle.sequence_forward(cfg, p, S[0, :-1], S[0, 1:], keep_cache=False)
    np.testing.assert_allclose(lt2[: t0 + 1], lt1[: t0 + 1], rtol=1e-15, atol=0)
    assert not np.allclose(lt2[t0 + 1:], lt1[t0 + 1:])


@pytest.mark.slow
def test_whole_model_gradient_finite_differences():
    """Central differences of the mean loss on the tiny config, h = 1e-5."""
    cfg, inp, p = _tiny()
    ids, tg = inp["ids"], inp["targets"]
    r = oracle.step(cfg, p, ids, tg)
    rng = np.random.default_rng(7)
    hstep = 1e-5

    def loss_of(pp):
        return oracle.step(cfg, pp, ids, tg, want_grads=False)["loss"]

    present = np.unique(ids)
    for name, g in r["grads"].items():
        flat_g = g.reshape(-1)
        if name == "embed":
            rows = rng.choice(present, 20)
            cols = rng.integers(0, cfg.d_model, 20)
            coords = rows * cfg.d_model + cols
        else:
            coords = rng.choice(flat_g.size, 20, replace=False)
        scale = np.abs(flat_g).max()
        for ci in coords:
            pp = {k: v.copy() for k, v in p.items()}
            pp[name].reshape(-1)[ci] += hstep
            lp = loss_of(pp)
            pp[name].reshape(-1)[ci] -= 2 * hstep
            lm = loss_of(pp)
            fd = (lp - lm) / (2 * hstep)
            assert abs(fd - flat_g[ci]) <= 1e-6 * scale + 1e-6 * abs(flat_g[ci]), (name, ci, fd, flat_g[ci])
