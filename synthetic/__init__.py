"""Seeded synthetic inputs for the dense-decoder training step.

This module is shared by the fp64 oracle (``oracle/``) and the HIP path
(``dense_decoder_only_amd``).  It holds shapes, seeds and random draws only:
none of the model's arithmetic lives here.

Workload recipe (the pages train on FineWeb-EDU token shards, which are not
available; these draws stand in for them):

* token ids: i.i.d. finite Zipf(s=1.1) over the vocabulary, P(id = r-1) is
  proportional to r**-1.1 for r = 1..V, drawn by inverse CDF from fp64
  uniforms of ``numpy.random.default_rng(1000 + cfg.index)``; an array of
  shape [B, T+1] whose first T columns are the inputs and whose last T columns
  are the targets (targets are the inputs shifted by one position);
* weights: ``default_rng(2000 + cfg.index)``, drawn in the order
  E, then per layer Wq, Wk, Wv, Wo, W1, W2, then U, each a float32
  standard normal times 1/sqrt(fan_in) with fan_in = the stored matrix's
  second axis ([out, in] -> in; E and U are [V, d] -> d);
* bf16 configurations consume the round-to-nearest-even bf16 copy of those
  fp32 masters (the oracle reads the same rounded values in fp64);
* bytes per token: a per-id table, constant 4.8 (the tokenizer's average
  compression on its training corpus, nano-series page, section nanochat).

Model shapes follow the nanochat depth ladder: width 64 per layer of depth,
head_dim 128 (64 in the tiny configuration), one shared K/V head, MLP width
4x, vocabulary 65,536, sequence length 2048.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np

__all__ = [
    "ModelConfig",
    "CONFIGS",
    "get_config",
    "zipf_ids",
    "make_tokens",
    "make_weights",
    "to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "PARAM_NAMES",
]


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    index: int
    n_layer: int
    d_model: int
    n_head: int
    head_dim: int
    d_ff: int
    vocab: int
    seq_len: int
    batch: int
    dtype: str  # "f32" or "bf16"
    n_kv_head: int = 1
    softcap: float = 15.0
    rope_base: float = 10000.0
    eps: float = 1e-6
    zipf_s: float = 1.1
    bytes_per_token: float = 4.8

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    @property
    def qkv_dim(self) -> int:
        return (self.n_head + 2 * self.n_kv_head) * self.head_dim

    def with_batch(self, batch: int) -> "ModelConfig":
        return dataclasses.replace(self, batch=batch)


CONFIGS: Dict[str, ModelConfig] = {
    "tiny": ModelConfig("tiny", 0, n_layer=2, d_model=128, n_head=2, head_dim=64, d_ff=512,
                        vocab=512, seq_len=64, batch=2, dtype="f32"),
    "small": ModelConfig("small", 1, n_layer=4, d_model=256, n_head=2, head_dim=128, d_ff=1024,
                         vocab=8192, seq_len=512, batch=8, dtype="bf16"),
    "d12": ModelConfig("d12", 2, n_layer=12, d_model=768, n_head=6, head_dim=128, d_ff=3072,
                       vocab=65536, seq_len=2048, batch=16, dtype="bf16"),
    "d20": ModelConfig("d20", 3, n_layer=20, d_model=1280, n_head=10, head_dim=128, d_ff=5120,
                       vocab=65536, seq_len=2048, batch=32, dtype="bf16"),
    "d26": ModelConfig("d26", 4, n_layer=26, d_model=1664, n_head=13, head_dim=128, d_ff=6656,
                       vocab=65536, seq_len=2048, batch=32, dtype="bf16"),
}

# Parameter tensors, in the layout both sides consume.  Per-layer matrices are
# stacked on a leading layer axis; every matrix is stored [out, in].
PARAM_NAMES = ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")


def get_config(name: str) -> ModelConfig:
    return CONFIGS[name]


def zipf_ids(rng: np.random.Generator, vocab: int, shape, s: float = 1.1) -> np.ndarray:
    """Finite Zipf(s) ids in [0, vocab) by inverse CDF over fp64 uniforms."""
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    w = ranks ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(size=shape, dtype=np.float64)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def make_tokens(cfg: ModelConfig, batch: int | None = None, seed: int | None = None) -> np.ndarray:
    """Token stream S [B, T+1] (int32); inputs S[:, :T], targets S[:, 1:]."""
    b = cfg.batch if batch is None else batch
    rng = np.random.default_rng(1000 + cfg.index if seed is None else seed)
    return zipf_ids(rng, cfg.vocab, (b, cfg.seq_len + 1), cfg.zipf_s)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_weights(cfg: ModelConfig, seed: int | None = None) -> Dict[str, np.ndarray]:
    """fp32 master weights, stacked per layer, in the draw order of the recipe."""
    rng = np.random.default_rng(2000 + cfg.index if seed is None else seed)
    L, d, H, hd, F, V = cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.d_ff, cfg.vocab
    kv = cfg.n_kv_head

    def draw(out_dim, in_dim):
        w = rng.standard_normal((out_dim, in_dim), dtype=np.float32)
        w *= np.float32(1.0 / np.sqrt(in_dim))
        return w

    embed = draw(V, d)
    w_qkv = np.empty((L, cfg.qkv_dim, d), np.float32)
    w_o = np.empty((L, d, H * hd), np.float32)
    w_fc = np.empty((L, F, d), np.float32)
    w_proj = np.empty((L, d, F), np.float32)
    for l in range(L):
        w_qkv[l, : H * hd] = draw(H * hd, d)
        w_qkv[l, H * hd: (H + kv) * hd] = draw(kv * hd, d)
        w_qkv[l, (H + kv) * hd:] = draw(kv * hd, d)
        w_o[l] = draw(d, H * hd)
        w_fc[l] = draw(F, d)
        w_proj[l] = draw(d, F)
    unembed = draw(V, d)
    return {"embed": embed, "w_qkv": w_qkv, "w_o": w_o, "w_fc": w_fc,
            "w_proj": w_proj, "unembed": unembed}


def make_inputs(cfg: ModelConfig, batch: int | None = None):
    """Everything one step consumes.

    Returns a dict with
      ``S`` int32 [B, T+1], ``ids`` int32 [B, T], ``targets`` int32 [B, T],
      ``token_bytes`` float32 [V] (constant 4.8),
      ``master`` fp32 weights, and ``weights``: the values the step consumes
      (fp32 masters for f32 configs, bf16-rounded values held in fp32 for
      bf16 configs) plus ``weights_bf16`` (uint16 bit patterns, bf16 only).
    """
    S = make_tokens(cfg, batch)
    master = make_weights(cfg)
    out = {
        "S": S,
        "ids": np.ascontiguousarray(S[:, :-1]),
        "targets": np.ascontiguousarray(S[:, 1:]),
        "token_bytes": np.full(cfg.vocab, cfg.bytes_per_token, np.float32),
        "master": master,
    }
    if cfg.dtype == "bf16":
        bits = {k: to_bf16_bits(v) for k, v in master.items()}
        out["weights_bf16"] = bits
        out["weights"] = {k: bf16_bits_to_f32(v) for k, v in bits.items()}
    else:
        out["weights"] = master
    return out
