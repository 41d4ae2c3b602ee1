"""Inference with a key/value cache on the GPU, against the fp64 oracle.

* Small-M GEMMs (the decode projections; M <= 128 rows take their own
  kernel inside nc_gemm_bf16) against a float64 library matmul of the same
  bf16 inputs, every epilogue they serve.
* nc_mqa_decode_attn against oracle.decode_attention, ragged lengths across
  the 64-position chunks, an empty sequence, and NaN in every cache slot past
  a sequence's length (a read there would poison the output); at the d20
  decode shape (32 sequences, 10 heads, 2048 positions) as well.
* nc_prefill + nc_decode_step against oracle.prefix_logits: the small
  configuration with a short prompt, then decode steps at per-sequence
  positions (one sequence rewrites a position, as a sampler that backs off
  would); and the d20 configuration (32 x 2040 prompt, max_len 2048) on a
  sampled sequence.

Tolerances (bf16 model, the gradient reading of the training tests): every
logits row within max-rel 3e-2 of the oracle and cosine >= 0.999; attention
outputs within bf16 rounding (2^-8 relative) plus fp32 accumulation.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, PARAM_NAMES, bf16_tensor_from_bits, dev_to_f64
from synthetic import CONFIGS, make_inputs, make_tokens

pytestmark = pytest.mark.gpu


def _nc():
    from dense_decoder_only_amd import nc
    nc.load()
    return nc


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def _within(got, ref, bound, what):
    bad = ~(np.abs(got - ref) <= bound)  # NaN counts as outside
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside; first at {i}: got {got[i]} ref {ref[i]}; "
                             f"rows {np.unique(np.argwhere(bad)[:, 0])[:16]}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (7, 96, 320), (32, 1536, 1280), (33, 64, 5120), (128, 256, 1280),
                                   (100, 8192, 256), (32, 1280, 5120), (5, 65536, 1280), (3, 16, 128)])
def test_small_m_gemm_matches_library_matmul(M, N, K):
    n = _nc()
    r = np.random.default_rng(M * 7 + N + K)
    A = _bf16(r.standard_normal((M, K)))
    W = _bf16(r.standard_normal((N, K)) / math.sqrt(K))
    ref = dev_to_f64(A) @ dev_to_f64(W).T
    scale = np.abs(ref).max()
    # fp32 store
    C = torch.empty(M, N, device=DEV)
    n.nc_gemm_bf16(0, 1, M, N, K, A, K, W, K, C, N)
    torch.cuda.synchronize()
    assert np.abs(dev_to_f64(C) - ref).max() <= 2e-5 * scale
    # fp32 accumulate (the residual add of the decode projections)
    base = torch.randn(M, N, device=DEV)
    C2 = base.clone()
    n.nc_gemm_bf16(0, 1, M, N, K, A, K, W, K, C2, N, beta=1.0)
    torch.cuda.synchronize()
    assert np.abs(dev_to_f64(C2) - (dev_to_f64(base) + ref)).max() <= 2e-5 * scale + 1e-6
    # bf16 store and relu^2 (bf16)
    Cb = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    n.nc_gemm_bf16(0, 1, M, N, K, A, K, W, K, Cb, N)
    torch.cuda.synchronize()
    _within(dev_to_f64(Cb), ref, 2 ** -8 * np.abs(ref) + 2e-5 * scale, "bf16 store")
    n.nc_gemm_bf16(0, 1, M, N, K, A, K, W, K, Cb, N, epilogue=n.NC_EPI_RELU2_SQ)
    torch.cuda.synchronize()
    r2 = np.maximum(ref, 0.0) ** 2
    _within(dev_to_f64(Cb), r2, 2 ** -8 * r2 + 4e-5 * scale * scale, "relu2")


def _decode_attn_case(B, H, max_len, lens, seed):
    n = _nc()
    r = np.random.default_rng(seed)
    hd = 128
    q = _unit_rms(r.standard_normal((B, H, hd)))
    k = _unit_rms(r.standard_normal((B, max_len, hd)))
    v = r.standard_normal((B, max_len, hd))
    q_d, k_d, v_d = _bf16(q), _bf16(k), _bf16(v)
    for b, L in enumerate(lens):  # poison everything past the length
        k_d[b, L:] = float("nan")
        v_d[b, L:] = float("nan")
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = torch.empty(B, H, hd, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(n.nc_mqa_decode_workspace_bytes(B, H, max_len), dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(hd)
    n.nc_mqa_decode_attn(q_d, k_d, v_d, lens_d, B, H, hd, max_len, scale, o, ws)
    torch.cuda.synchronize()
    got = dev_to_f64(o)
    qr, kr, vr = dev_to_f64(q_d), dev_to_f64(k_d), dev_to_f64(v_d)
    assert np.all(np.isfinite(got))
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(got[b] == 0.0)
            continue
        ref = oracle.decode_attention(qr[b], kr[b, :L], vr[b, :L], scale)
        err = np.abs(got[b] - ref)
        assert np.all(err <= 2 ** -8 * np.abs(ref) + 2e-3 * np.abs(ref).max()), (b, L, err.max())


def _unit_rms(x):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def test_decode_attention_ragged_and_empty():
    _decode_attn_case(7, 10, 300, [1, 63, 64, 65, 300, 0, 129], seed=1)
    _decode_attn_case(3, 2, 64, [64, 1, 37], seed=2)
    _decode_attn_case(2, 16, 130, [130, 127], seed=3)
    _decode_attn_case(3, 32, 200, [200, 65, 2], seed=6)


def test_decode_attention_d20_shape():
    r = np.random.default_rng(4)
    lens = [int(x) for x in r.integers(1, 2049, 32)]
    lens[0], lens[1] = 2048, 1
    _decode_attn_case(32, 10, 2048, lens, seed=5)


def _device_params(inp):
    return {k: bf16_tensor_from_bits(inp["weights_bf16"][k]) for k in PARAM_NAMES}


def _check_logits(got, ref, what):
    for b in range(ref.shape[0]):
        g, z = got[b], ref[b]
        mr = np.abs(g - z).max() / np.abs(z).max()
        cos = float(g @ z / (np.linalg.norm(g) * np.linalg.norm(z)))
        assert mr <= 3e-2 and cos >= 0.999, (what, b, mr, cos)


def test_prefill_then_decode_small():
    n = _nc()
    T0, B, max_len = 40, 3, 48
    cfg = dataclasses.replace(CONFIGS["small"], seq_len=T0, batch=B)
    inp = make_inputs(CONFIGS["small"])
    params = _device_params(inp)
    p64 = oracle.to_f64_params(inp["weights"])
    prompts = make_tokens(cfg, seed=11)[:, :T0]
    extra = make_tokens(cfg, seed=12)[:, :4]
    ccfg = n.make_config(cfg)
    kv = torch.empty(n.nc_kv_cache_bytes(ccfg, max_len), dtype=torch.uint8, device=DEV)
    ws = torch.empty(n.nc_infer_workspace_bytes(ccfg, max_len), dtype=torch.uint8, device=DEV)
    logits = torch.empty(B, cfg.vocab, device=DEV)
    n.nc_prefill(ccfg, params, torch.from_numpy(prompts).to(DEV), kv, max_len, logits, ws)
    torch.cuda.synchronize()
    assert n.nc_sync_status(ws) == n.NC_OK
    ref = np.stack([oracle.prefix_logits(cfg, p64, prompts[b])[-1] for b in range(B)])
    _check_logits(dev_to_f64(logits), ref, "prefill")
    # decode: sequence 1 writes position T0 twice (a rewrite), then T0 + 1 twice
    cache_tokens = [list(prompts[b]) for b in range(B)]
    for j in range(4):
        pos = [T0 + j if b != 1 else T0 + j // 2 for b in range(B)]
        ids = [int(extra[b, j]) for b in range(B)]
        n.nc_decode_step(ccfg, params, torch.tensor(ids, dtype=torch.int32, device=DEV),
                         torch.tensor(pos, dtype=torch.int32, device=DEV), kv, max_len, logits, ws)
        torch.cuda.synchronize()
        assert n.nc_sync_status(ws) == n.NC_OK
        rows = []
        for b in range(B):
            del cache_tokens[b][pos[b]:]
            cache_tokens[b].append(ids[b])
            rows.append(oracle.prefix_logits(cfg, p64, np.array(cache_tokens[b], dtype=np.int32))[-1])
        _check_logits(dev_to_f64(logits), np.stack(rows), f"decode step {j}")


def test_decode_steps_replay_from_a_graph():
    """Three decode steps captured once into a HIP graph (the library records
    kernels only, no memset nodes) replay to the eager logits bit for bit,
    with eager prefills and synchronizations between the replays."""
    n = _nc()
    T0, B, max_len, steps = 24, 2, 32, 3
    cfg = dataclasses.replace(CONFIGS["small"], seq_len=T0, batch=B)
    inp = make_inputs(CONFIGS["small"])
    params = _device_params(inp)
    prompts = torch.from_numpy(make_tokens(cfg, seed=21)[:, :T0]).to(DEV)
    extra = make_tokens(cfg, seed=22)[:, :steps]
    ccfg = n.make_config(cfg)
    kv = torch.empty(n.nc_kv_cache_bytes(ccfg, max_len), dtype=torch.uint8, device=DEV)
    ws = torch.empty(n.nc_infer_workspace_bytes(ccfg, max_len), dtype=torch.uint8, device=DEV)
    logits = torch.empty(B, cfg.vocab, device=DEV)
    pos = [torch.full((B,), T0 + j, dtype=torch.int32, device=DEV) for j in range(steps)]
    ids = [torch.from_numpy(np.ascontiguousarray(extra[:, j])).to(DEV) for j in range(steps)]
    out = torch.empty(steps, B, cfg.vocab, device=DEV)

    def decode():  # library launches only: each step writes its own logits rows
        st = torch.cuda.current_stream()
        for j in range(steps):
            n.nc_decode_step(ccfg, params, ids[j], pos[j], kv, max_len, out[j], ws, stream=st)

    n.nc_prefill(ccfg, params, prompts, kv, max_len, logits, ws)
    decode()
    torch.cuda.synchronize()
    assert n.nc_sync_status(ws) == n.NC_OK
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        decode()
    torch.cuda.synchronize()
    for r in range(3):
        n.nc_prefill(ccfg, params, prompts, kv, max_len, logits, ws)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert n.nc_sync_status(ws) == n.NC_OK
        assert torch.equal(out, ref), f"replay {r} differs from the eager steps"


def test_decode_flags_bad_position_and_id():
    n = _nc()
    cfg = dataclasses.replace(CONFIGS["small"], seq_len=8, batch=2)
    inp = make_inputs(CONFIGS["small"])
    params = _device_params(inp)
    ccfg = n.make_config(cfg)
    kv = torch.zeros(n.nc_kv_cache_bytes(ccfg, 16), dtype=torch.uint8, device=DEV)
    ws = torch.empty(n.nc_infer_workspace_bytes(ccfg, 16), dtype=torch.uint8, device=DEV)
    logits = torch.empty(2, cfg.vocab, device=DEV)
    ids = torch.tensor([1, 2], dtype=torch.int32, device=DEV)
    n.nc_decode_step(ccfg, params, ids, torch.tensor([3, 16], dtype=torch.int32, device=DEV), kv, 16, logits, ws)
    assert n.nc_sync_status(ws) == n.NC_ERR_DEVICE_FLAG
    bad = torch.tensor([1, cfg.vocab], dtype=torch.int32, device=DEV)
    n.nc_decode_step(ccfg, params, bad, torch.tensor([3, 4], dtype=torch.int32, device=DEV), kv, 16, logits, ws)
    assert n.nc_sync_status(ws) == n.NC_ERR_DEVICE_FLAG
    n.nc_decode_step(ccfg, params, ids, torch.tensor([3, 4], dtype=torch.int32, device=DEV), kv, 16, logits, ws)
    assert n.nc_sync_status(ws) == n.NC_OK
    with pytest.raises(n.NcError):  # unsupported: fp32 configuration
        n.nc_prefill(n.make_config(CONFIGS["tiny"]), params, ids, kv, 64, logits, ws)


def test_prefill_then_decode_d20_sampled():
    """The d20 decode workload (32 sequences, a 2040-token prompt, max_len
    2048): prefill, then one decode step, checked on one sequence against the
    oracle's forward over 2041 tokens."""
    n = _nc()
    T0, max_len, b = 2040, 2048, 5
    base = CONFIGS["d20"]
    cfg = dataclasses.replace(base, seq_len=T0)
    inp = make_inputs(base)
    params = _device_params(inp)
    prompts = np.ascontiguousarray(inp["ids"][:, :T0])
    nxt = np.ascontiguousarray(inp["ids"][:, T0])
    ccfg = n.make_config(cfg)
    kv = torch.empty(n.nc_kv_cache_bytes(ccfg, max_len), dtype=torch.uint8, device=DEV)
    ws = torch.empty(n.nc_infer_workspace_bytes(ccfg, max_len), dtype=torch.uint8, device=DEV)
    lp = torch.empty(cfg.batch, cfg.vocab, device=DEV)
    ld = torch.empty(cfg.batch, cfg.vocab, device=DEV)
    n.nc_prefill(ccfg, params, torch.from_numpy(prompts).to(DEV), kv, max_len, lp, ws)
    n.nc_decode_step(ccfg, params, torch.from_numpy(nxt).to(DEV),
                     torch.full((cfg.batch,), T0, dtype=torch.int32, device=DEV), kv, max_len, ld, ws)
    torch.cuda.synchronize()
    assert n.nc_sync_status(ws) == n.NC_OK
    assert np.all(np.isfinite(dev_to_f64(lp))) and np.all(np.isfinite(dev_to_f64(ld)))
    del params, kv
    p64 = oracle.to_f64_params(inp["weights"])
    z = oracle.prefix_logits(cfg, p64, np.concatenate([prompts[b], nxt[b:b + 1]]))
    _check_logits(dev_to_f64(lp[b:b + 1]), z[T0 - 1:T0], "d20 prefill")
    _check_logits(dev_to_f64(ld[b:b + 1]), z[T0:T0 + 1], "d20 decode")
