"""fp64 oracle: the plain definition of the nanochat-style dense decoder step.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
HIP path.

Sources (page title, section):
  [NEWS]  "Karpathy再放大招：8000行代碼復現ChatGPT全棧，最低成本僅100美元，4小時跑完"
          (shdongyou.cn), section 技術細節與問答 — the architecture list: dense
          Transformer, rotary embeddings and no positional embedding, QK norm,
          untied embedding and unembedding, a norm right after the token
          embedding, relu-squared MLP, RMSNorm without learnable parameters,
          linear layers without biases, multi-query attention, logit softcap.
  [NANO]  "Karpathy 的 nano 諧系：nanoGPT、llm.c 到 nanochat" (quidproquo.cc),
          section nanochat — pretraining loss is reported in bits per byte;
          the tokenizer averages about 4.8 characters per token.

Readings where the pages are silent (the GPU path takes the same ones):
  R1  eps = 1e-6 inside the square root, the same for every norm.
  R2  norms: after the embedding, before attention and before the MLP in each
      layer, and a final one before the unembedding ("like Llama").
  R3  pre-norm residual x <- x + f(rms(x)), no scaling.
  R4  RoPE pairs (i, i + hd/2), rotation by +theta,
      theta(t, i) = t * base**(-2 i / hd), base 10000, positions 0..T-1 per row.
  R5  RoPE first, then the per-head RMS norm (they commute exactly).
  R6  attention scale 1/sqrt(hd).
  R7  softcap z' = c tanh(z / c), c = 15.
  R8  relu^2(u) = max(u, 0)^2, derivative 2 max(u, 0).
  R9  natural-log cross entropy, mean over all B*T tokens.
  R10 bits per byte = sum(loss) / (ln 2 * sum(bytes[target])).
  R15 one sequence per row, plain causal mask.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# Building blocks
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Parameter-free RMSNorm over the last axis [NEWS: RMSNorm has no gain].

    y = x / sqrt(mean(x^2) + eps).  Returns (y, r) with r = 1/sqrt(ms + eps)
    (shape x.shape[:-1] + (1,)).
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r, r


def rms_norm_bwd(g: np.ndarray, y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Gradient through y = x * r(x): dx = r * (g - y * mean(g * y)).

    Derivation: dy_i/dx_j = r (delta_ij - y_i y_j / n) with n the last-axis
    length, so dx_j = r (g_j - y_j * sum_i(g_i y_i) / n).
    """
    return r * (g - y * np.mean(g * y, axis=-1, keepdims=True))


def rope_angles(T: int, hd: int, base: float) -> np.ndarray:
    """theta[t, i] = t * base**(-2 i / hd), t < T, i < hd/2 [NEWS: RoPE; R4]."""
    t = np.arange(T, dtype=F64)[:, None]
    i = np.arange(hd // 2, dtype=F64)[None, :]
    return t * base ** (-2.0 * i / hd)


def rope(x: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Rotate pairs (x_i, x_{i+hd/2}) by +theta.

    x: [T, ..., hd]; theta: [T, hd/2] (broadcast over the middle axes).
    """
    half = x.shape[-1] // 2
    th = theta.reshape(theta.shape[:1] + (1,) * (x.ndim - 2) + theta.shape[1:])
    c, s = np.cos(th), np.sin(th)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_bwd(g: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Adjoint of ``rope``: the rotation is orthogonal, so rotate by -theta."""
    return rope(g, -theta)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Causal softmax attention, one sequence [NEWS: multi-query attention].

    q: [T, Hq, hd]; k, v: [T, Hkv, hd] with Hq a multiple of Hkv; query head h
    reads K/V head h // (Hq / Hkv).  With Hkv = 1 this is multi-query
    attention.  Returns (o [T, Hq, hd], P [Hq, T, T]) where
    P[h, t, u] = softmax_u(q[t,h] . k[u] * scale) over u <= t, 0 for u > t.
    """
    T, Hq, hd = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    mask = np.tril(np.ones((T, T), dtype=bool))
    o = np.empty_like(q)
    P = np.empty((Hq, T, T), dtype=q.dtype)
    for h in range(Hq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        P[h] = p
        o[:, h, :] = p @ v[:, g, :]
    return o, P


def attention_bwd(do: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                  P: np.ndarray, scale: float):
    """Gradients of ``attention`` w.r.t. q, k, v.

    Per query head h (K/V head g): dV_g += P^T dO, dP = dO V^T,
    dS = P * (dP - rowsum(dP * P)), dQ = scale dS K, dK_g += scale dS^T Q.
    Shared K/V heads sum their contributions over the query heads they serve.
    """
    T, Hq, hd = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        g = h // group
        p = P[h]
        dv[:, g, :] += p.T @ do[:, h, :]
        dp = do[:, h, :] @ v[:, g, :].T
        ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
        dq[:, h, :] = scale * (ds @ k[:, g, :])
        dk[:, g, :] += scale * (ds.T @ q[:, h, :])
    return dq, dk, dv


def relu2(u: np.ndarray) -> np.ndarray:
    """relu(u)^2 [NEWS: relu-squared MLP activation]."""
    return np.maximum(u, 0.0) ** 2


def softcap(z: np.ndarray, c: float) -> np.ndarray:
    """Logit softcap z' = c tanh(z / c) [NEWS: logit softcap; R7]."""
    return c * np.tanh(z / c)


def cross_entropy(zc: np.ndarray, y: np.ndarray):
    """Per-row natural-log cross entropy of logits zc [T, V] against y [T].

    Returns (loss_t [T], lse [T]) with lse = log sum_v exp(zc[t, v]).
    """
    m = zc.max(axis=1, keepdims=True)
    lse = (m + np.log(np.sum(np.exp(zc - m), axis=1, keepdims=True)))[:, 0]
    return lse - zc[np.arange(zc.shape[0]), y], lse


def relu2_bwd(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Gradient through relu(u)^2: g * 2 max(u, 0) (zero at u = 0)."""
    return g * 2.0 * np.maximum(u, 0.0)


def softcap_xent_bwd(zc: np.ndarray, lse: np.ndarray, y: np.ndarray, c: float, dloss: float) -> np.ndarray:
    """Gradient of dloss * sum_t loss_t w.r.t. the raw logits z (zc = softcap(z)).

    d loss_t / d zc_tv = softmax(zc_t)_v - [v = y_t]; d zc / d z = 1 - tanh^2 = 1 - (zc/c)^2.
    """
    T = zc.shape[0]
    dzc = np.exp(zc - lse[:, None])
    dzc[np.arange(T), y] -= 1.0
    dzc *= dloss
    return dzc * (1.0 - (zc / c) ** 2)


def embed_bwd(ids: np.ndarray, de: np.ndarray, V: int) -> np.ndarray:
    """Scatter-add of embedding-row gradients: dE[v] = sum_{t: ids[t]=v} de[t]."""
    dE = np.zeros((V, de.shape[-1]), dtype=de.dtype)
    np.add.at(dE, ids.reshape(-1), de.reshape(-1, de.shape[-1]))
    return dE


# ----------------------------------------------------------------------------
# One sequence, forward and backward
# ----------------------------------------------------------------------------

def to_f64_params(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=F64) for k, v in weights.items()}


def sequence_forward(cfg, p: Dict[str, np.ndarray], ids: np.ndarray, y: np.ndarray,
                     keep_cache: bool = True):
    """Forward of one sequence (ids, y: [T]).  Returns (loss_t [T], cache).

    The composition follows [NEWS]: token embedding, norm, L pre-norm blocks of
    (QKV projection, RoPE, QK norm, causal MQA, output projection) and
    (relu^2 MLP), a final norm, untied unembedding, softcap, cross entropy.
    """
    T = ids.shape[0]
    L, d, H, hd = cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim
    Hkv = cfg.n_kv_head
    eps, c = cfg.eps, cfg.softcap
    scale = 1.0 / math.sqrt(hd)
    theta = rope_angles(T, hd, cfg.rope_base)

    e = p["embed"][ids]                       # token embedding gather
    x0, r0 = rms_norm(e, eps)                 # norm after the embedding
    x = x0
    layers = []
    for l in range(L):
        a, ra = rms_norm(x, eps)
        qkv = a @ p["w_qkv"][l].T             # bias-free projection
        q = qkv[:, : H * hd].reshape(T, H, hd)
        k = qkv[:, H * hd: (H + Hkv) * hd].reshape(T, Hkv, hd)
        v = qkv[:, (H + Hkv) * hd:].reshape(T, Hkv, hd)
        qn, rq = rms_norm(rope(q, theta), eps)   # RoPE, then QK norm (R5)
        kn, rk = rms_norm(rope(k, theta), eps)
        o, _ = attention(qn, kn, v, scale)
        of = o.reshape(T, H * hd)
        x = x + of @ p["w_o"][l].T
        m, rm = rms_norm(x, eps)
        u = m @ p["w_fc"][l].T
        a2 = relu2(u)
        x = x + a2 @ p["w_proj"][l].T
        if keep_cache:
            layers.append(dict(a=a, ra=ra, qn=qn, rq=rq, kn=kn, rk=rk, v=v, of=of,
                               m=m, rm=rm, u=u, a2=a2))
    h, rf = rms_norm(x, eps)
    z = h @ p["unembed"].T
    zc = softcap(z, c)
    loss_t, lse = cross_entropy(zc, y)
    cache = None
    if keep_cache:
        cache = dict(ids=ids, y=y, x0=x0, r0=r0, layers=layers, h=h, rf=rf, zc=zc,
                     lse=lse, theta=theta)
    return loss_t, cache


def sequence_backward(cfg, p: Dict[str, np.ndarray], cache, dloss: float,
                      grads: Dict[str, np.ndarray]) -> None:
    """Accumulate into ``grads`` the gradient of dloss * sum_t loss_t.

    For the mean loss over M tokens the caller passes dloss = 1/M.
    """
    L, d, H, hd = cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim
    Hkv = cfg.n_kv_head
    c = cfg.softcap
    scale = 1.0 / math.sqrt(hd)
    theta = cache["theta"]
    y, zc, lse, h = cache["y"], cache["zc"], cache["lse"], cache["h"]
    T = y.shape[0]

    # cross entropy and softcap
    dz = softcap_xent_bwd(zc, lse, y, c, dloss)
    grads["unembed"] += dz.T @ h
    dh = dz @ p["unembed"]
    dx = rms_norm_bwd(dh, h, cache["rf"])

    for l in reversed(range(L)):
        C = cache["layers"][l]
        # MLP block: x_out = x_mid + relu(m W1^T)^2 W2^T
        grads["w_proj"][l] += dx.T @ C["a2"]
        da2 = dx @ p["w_proj"][l]
        du = relu2_bwd(da2, C["u"])
        grads["w_fc"][l] += du.T @ C["m"]
        dm = du @ p["w_fc"][l]
        dx = dx + rms_norm_bwd(dm, C["m"], C["rm"])
        # attention block: x_mid = x_in + attn(...) Wo^T
        grads["w_o"][l] += dx.T @ C["of"]
        do = (dx @ p["w_o"][l]).reshape(T, H, hd)
        _, P = attention(C["qn"], C["kn"], C["v"], scale)   # recompute P
        dqn, dkn, dv = attention_bwd(do, C["qn"], C["kn"], C["v"], P, scale)
        dq = rope_bwd(rms_norm_bwd(dqn, C["qn"], C["rq"]), theta)
        dk = rope_bwd(rms_norm_bwd(dkn, C["kn"], C["rk"]), theta)
        dqkv = np.concatenate([dq.reshape(T, H * hd), dk.reshape(T, Hkv * hd),
                               dv.reshape(T, Hkv * hd)], axis=1)
        grads["w_qkv"][l] += dqkv.T @ C["a"]
        da = dqkv @ p["w_qkv"][l]
        dx = dx + rms_norm_bwd(da, C["a"], C["ra"])

    de = rms_norm_bwd(dx, cache["x0"], cache["r0"])
    grads["embed"] += embed_bwd(cache["ids"], de, p["embed"].shape[0])


def step(cfg, p: Dict[str, np.ndarray], ids: np.ndarray, targets: np.ndarray,
         token_bytes: np.ndarray | None = None, want_grads: bool = True,
         seq_indices=None):
    """Full training step: mean loss, bits per byte, parameter gradients.

    ids, targets: [B, T].  Sequences interact only through the mean, so they
    are processed one at a time and the gradient of each is added with weight
    1/M, M = B*T [R9].  ``seq_indices`` restricts the work to some sequences
    (the returned loss is then the mean over those, with M their token count).

    Returns dict(loss, bpb, loss_tok [B', T], grads or None).
    """
    B, T = ids.shape
    seqs = list(range(B)) if seq_indices is None else list(seq_indices)
    M = len(seqs) * T
    if token_bytes is None:
        token_bytes = np.full(cfg.vocab, cfg.bytes_per_token)
    tb = np.asarray(token_bytes, dtype=F64)
    grads = None
    if want_grads:
        grads = {k: np.zeros_like(v, dtype=F64) for k, v in p.items()}
    losses = []
    for b in seqs:
        loss_t, cache = sequence_forward(cfg, p, ids[b], targets[b], keep_cache=want_grads)
        losses.append(loss_t)
        if want_grads:
            sequence_backward(cfg, p, cache, 1.0 / M, grads)
        del cache
    loss_tok = np.stack(losses)
    total = float(loss_tok.sum())
    nbytes = float(tb[targets[seqs]].sum())
    return dict(loss=total / M, bpb=total / (math.log(2.0) * nbytes),
                loss_tok=loss_tok, grads=grads)
