"""Parity at the launch configuration the d12/d20/d26 training step runs.

The per-kernel tests elsewhere stop at sizes the oracle finishes in seconds.
Several code paths only run at the full shapes:
  - attention's dK/dV keeps whole query ranges once the B x T/128 key blocks
    alone fill the GPU (32 x 2048 tokens);
  - the weight-gradient products reduce K = B T = 65,536 over 5, 8 or 10
    deterministic k-splits, the 8-split form giving each XCD whole splits;
  - the cross entropy stores one [M, V] buffer of 2^32 entries and its
    gradient products contract over all of it.
The tests here run those launches and compare with the fp64 oracle (or, for
the plain contractions, a float64 matmul of the same rounded operands).

Whole steps: the oracle cannot run 32 sequences of the full model in a test,
but sequences interact only through the mean loss.  A batch made of two
distinct sequences, each repeated B/2 times (in a seeded random order), has
exactly the mean-loss gradient of the two-sequence batch, which the oracle
computes.  Tolerances are the bf16 readings of the target: loss rel 2e-3,
every gradient cosine >= 0.999 and max-rel <= 3e-2 with
max-rel = ||g - g*||_inf / ||g*||_inf per parameter tensor.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_close, cosine, dev_to_f64, max_rel, run_step
from synthetic import CONFIGS, bf16_bits_to_f32, make_inputs, to_bf16_bits, zipf_ids

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def nc():
    from dense_decoder_only_amd import nc as _nc
    _nc.load()
    return _nc


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def bf16_pair(x32):
    """fp32 array -> (device bf16 tensor, the same rounded values as fp32 on the host)."""
    bits = to_bf16_bits(x32)
    dev = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return dev, bf16_bits_to_f32(bits)


def unit_rms(x):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


# ------------------------------------------------------------- attention --

@pytest.mark.parametrize("H", [10, 13])
def test_attention_full_size(H):
    """(B, T) = (32, 2048) with H = 10 (d20) and 13 (d26) query heads: the
    dK/dV kernel takes whole query ranges here.  Distinct random sequences;
    o, lse, dq, dk and dv of three sequences compared element by element."""
    n = nc()
    B, T, hd = 32, 2048, 128
    M, Q = B * T, (H + 2) * hd
    r = np.random.default_rng(5000 + H)
    qkv32 = np.empty((M, Q), np.float32)
    qkv32[:, : (H + 1) * hd] = unit_rms(r.standard_normal((M, H + 1, hd), dtype=np.float32)).reshape(M, -1)
    qkv32[:, (H + 1) * hd:] = r.standard_normal((M, hd), dtype=np.float32)
    qkv, qkv_h = bf16_pair(qkv32)
    dout, do_h = bf16_pair(r.standard_normal((M, H * hd), dtype=np.float32))
    scale = 1 / math.sqrt(hd)
    o = torch.empty(M, H * hd, dtype=BF16, device=DEV)
    lse = torch.empty(M * H, dtype=F32, device=DEV)
    n.nc_mqa_attn_fwd(qkv, B, T, H, hd, scale, o, lse)
    # the backward consumes the forward's own o (D = rowsum(dO o) is part of it)
    dq = torch.full((M, Q), float("nan"), dtype=F32, device=DEV)
    ws = torch.empty(n.nc_mqa_attn_bwd_workspace_bytes(B, T, H), dtype=torch.uint8, device=DEV)
    n.nc_mqa_attn_bwd(qkv, o, dout, lse, B, T, H, hd, scale, dq, ws)
    torch.cuda.synchronize()
    og = dev_to_f64(o).reshape(B, T, H, hd)
    lg = dev_to_f64(lse).reshape(B, T, H)
    dqg = dev_to_f64(dq).reshape(B, T, H + 2, hd)
    assert np.all(np.isfinite(dqg)), "every dq/dk/dv element must be written"
    q4 = qkv_h.reshape(B, T, H + 2, hd)
    do4 = do_h.reshape(B, T, H, hd)
    for b in (0, 17, 31):
        q = q4[b, :, :H].astype(np.float64)
        k = q4[b, :, H:H + 1].astype(np.float64)
        v = q4[b, :, H + 1:].astype(np.float64)
        ref_o, P = oracle.attention(q, k, v, scale)
        # lse from the oracle's probabilities: log of the normaliser at row t,
        # recovered as s_tt - log P_tt on the diagonal (P_tt > 0)
        s_diag = np.einsum("thd,td->ht", q, k[:, 0]) * scale
        ref_lse = (s_diag - np.log(np.einsum("htt->ht", P))).T
        assert_close(og[b], ref_o, 2 ** -8, 1e-3, f"attn o (b={b})")
        assert_close(lg[b], ref_lse, 1e-5, 1e-6, f"attn lse (b={b})")
        dq_r, dk_r, dv_r = oracle.attention_bwd(do4[b].astype(np.float64), q, k, v, P, scale)
        for name, got, ref in (("dq", dqg[b, :, :H], dq_r), ("dk", dqg[b, :, H], dk_r[:, 0]),
                               ("dv", dqg[b, :, H + 1], dv_r[:, 0])):
            note(f"attn H={H} b={b} {name}: max_rel {max_rel(got, ref):.3e} cos {cosine(got, ref):.7f}")
            assert_close(got, ref, 2e-2, 5e-3, f"attn {name} (b={b})")
            assert cosine(got, ref) > 0.9999, (name, b, cosine(got, ref))


# ----------------------------------------------- weight-gradient products --

@pytest.mark.parametrize("M,N", [(5120, 1280), (1280, 5120), (1536, 1280), (1280, 1280)])
def test_weight_gradient_gemm_full_k(M, N):
    """dW = dY^T X at d20 with K = B T = 65,536 (dW_fc, dW_proj, dW_qkv,
    dW_o), with the workspace the step gives it, so the split count is the
    step's; sampled output rows (every row tile's edges) against a float64
    matmul, with and without accumulation."""
    n = nc()
    K = 65536
    r = np.random.default_rng(6000 + M + N)
    A, A_h = bf16_pair(r.standard_normal((K, M), dtype=np.float32))
    Bm, B_h = bf16_pair(r.standard_normal((K, N), dtype=np.float32))
    wsb = n.nc_gemm_workspace_bytes(M, N, K)
    assert wsb > 0, "these shapes take the split-K path"
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    C = torch.full((M, N), float("nan"), dtype=F32, device=DEV)
    n.nc_gemm_bf16(1, 0, M, N, K, A, M, Bm, N, C, N, ws=ws)
    C0_h = r.standard_normal((M, N)).astype(np.float32)
    C1 = torch.from_numpy(C0_h).to(DEV)
    n.nc_gemm_bf16(1, 0, M, N, K, A, M, Bm, N, C1, N, beta=1.0, ws=ws)
    C2 = torch.empty((M, N), dtype=F32, device=DEV)
    n.nc_gemm_bf16(1, 0, M, N, K, A, M, Bm, N, C2, N, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(C, C2), "split-K must be deterministic"
    edges = sorted({e for t in range(0, M, 256) for e in (t, t + 1, t + 127, t + 255) if e < M})
    rows = np.array(sorted(set(edges) | set(r.choice(M, 16, replace=False).tolist())))
    ref = A_h[:, rows].astype(np.float64).T @ B_h.astype(np.float64)
    got = C.cpu().numpy()[rows].astype(np.float64)
    note(f"wgrad {M}x{N}x{K}: max_rel {max_rel(got, ref):.3e}")
    assert_close(got, ref, 1e-4, 2e-5, f"dW {M}x{N}")
    got1 = C1.cpu().numpy()[rows].astype(np.float64)
    assert_close(got1, C0_h[rows].astype(np.float64) + ref, 1e-4, 2e-5, f"dW {M}x{N} accumulate")


# ---------------------------------------------------- cross entropy, dU --

def test_softcap_xent_two_chunks_dU_elementwise():
    """Two vocabulary chunks (M V > 2^32), dU compared element by element over
    the whole vocabulary.  One row in 16 of h is non-zero (random rows); the
    others are exactly zero, so they add exactly nothing to dU = dz^T h and
    the oracle needs the log-sum-exp of the non-zero rows only.  A read of a
    wrong h row or a wrong dz row lands on a zero row and shows."""
    n = nc()
    M, d, V, c = 65536, 64, 65536 + 256, 15.0
    r = np.random.default_rng(78)
    nz = np.sort(r.choice(M, M // 16, replace=False))
    h32 = np.zeros((M, d), np.float32)
    h32[nz] = unit_rms(r.standard_normal((nz.size, d), dtype=np.float32))
    h, h_h = bf16_pair(h32)
    U, U_h = bf16_pair((r.standard_normal((V, d), dtype=np.float32) / np.float32(math.sqrt(d))))
    y_np = zipf_ids(r, V, M)
    y_np[nz[:64]] = V - 1 - np.arange(64)  # targets in the second chunk
    y = torch.from_numpy(y_np).to(DEV)
    ws = torch.empty(n.nc_softcap_xent_workspace_bytes(M, d, V), dtype=torch.uint8, device=DEV)
    lse = torch.empty(M, dtype=F32, device=DEV)
    ltok = torch.empty(M, dtype=F32, device=DEV)
    loss = torch.empty(1, dtype=F32, device=DEV)
    bpb = torch.empty(1, dtype=F32, device=DEV)
    n.nc_softcap_xent_fwd(h, U, y, None, c, lse, ltok, loss, bpb, ws)
    dh = torch.empty(M, d, dtype=F32, device=DEV)
    dU = torch.full((V, d), float("nan"), dtype=F32, device=DEV)
    n.nc_softcap_xent_bwd(h, U, y, lse, c, 1.0 / M, dh, 0, dU, 0, ws)
    assert n.nc_sync_status(ws) == n.NC_OK
    h64, U64 = h_h[nz].astype(np.float64), U_h.astype(np.float64)
    zc = oracle.softcap(h64 @ U64.T, c)
    lt_ref, lse_ref = oracle.cross_entropy(zc, y_np[nz])
    assert_close(lse.cpu().numpy()[nz], lse_ref, 2e-6, 0, "xent lse (non-zero rows)")
    assert_close(ltok.cpu().numpy()[nz], lt_ref, 1e-5, 1e-5, "xent loss_tok (non-zero rows)")
    dz = oracle.softcap_xent_bwd(zc, lse_ref, y_np[nz], c, 1.0 / M)
    del zc
    got_dU = dU.cpu().numpy().astype(np.float64)
    ref_dU = dz.T @ h64
    note(f"xent dU: max_rel {max_rel(got_dU, ref_dU):.3e} cos {cosine(got_dU, ref_dU):.7f}")
    assert_close(got_dU, ref_dU, 1e-2, 5e-3, "xent dU (every element)")
    got_dh = dh.cpu().numpy()[nz].astype(np.float64)
    assert_close(got_dh, dz @ U64, 1e-2, 5e-3, "xent dh (non-zero rows)")
    # the zero rows' dh is dz U with dz = (1/V - onehot) / M exactly (z = 0):
    zr = np.setdiff1d(np.arange(M), nz)[:32]
    dz0 = np.full((zr.size, V), 1.0 / V)
    dz0[np.arange(zr.size), y_np[zr]] -= 1.0
    assert_close(dh.cpu().numpy()[zr].astype(np.float64), (dz0 / M) @ U64, 1e-2, 5e-3, "xent dh (zero rows)")


def test_softcap_xent_flags_out_of_range_targets():
    """A target outside [0, V) raises the flag in the workspace; that row has
    z' at the target = 0 and counts no bytes; no other row changes."""
    n = nc()
    c = 15.0
    for M, d, V in ((264, 128, 1024), (264, 200, 1024)):  # fused epilogue, chunked path
        r = np.random.default_rng(M + d)
        h, h_h = bf16_pair(unit_rms(r.standard_normal((M, d), dtype=np.float32)))
        U, U_h = bf16_pair(r.standard_normal((V, d), dtype=np.float32) / np.float32(math.sqrt(d)))
        y_np = zipf_ids(r, V, M)
        bad = np.array([3, 9, 200])
        y_np[bad] = [V, -1, 1 << 30]
        y = torch.from_numpy(y_np).to(DEV)
        tb_np = np.full(V, 4.8, np.float32)
        tb_np[::5] = 3.0
        tb = torch.from_numpy(tb_np).to(DEV)
        ws = torch.empty(n.nc_softcap_xent_workspace_bytes(M, d, V), dtype=torch.uint8, device=DEV)
        ws.fill_(0xFF)  # stale contents
        lse = torch.empty(M, dtype=F32, device=DEV)
        ltok = torch.empty(M, dtype=F32, device=DEV)
        loss = torch.empty(1, dtype=F32, device=DEV)
        bpb = torch.empty(1, dtype=F32, device=DEV)
        n.nc_softcap_xent_fwd(h, U, y, tb, c, lse, ltok, loss, bpb, ws)
        assert n.nc_sync_status(ws) == n.NC_ERR_DEVICE_FLAG
        zc = oracle.softcap(h_h.astype(np.float64) @ U_h.astype(np.float64).T, c)
        good = np.setdiff1d(np.arange(M), bad)
        lt_ref, lse_ref = oracle.cross_entropy(zc[good], y_np[good])
        lt = ltok.cpu().numpy().astype(np.float64)
        assert_close(lse.cpu().numpy()[good], lse_ref, 2e-6, 0, "lse of valid rows")
        assert_close(lt[good], lt_ref, 1e-5, 1e-5, "loss_tok of valid rows")
        assert_close(lt[bad], lse.cpu().numpy()[bad].astype(np.float64), 0, 0, "flagged rows: loss = lse")
        nbytes = tb_np[y_np[good]].astype(np.float64).sum()
        assert float(bpb) == pytest.approx(lt.sum() / (math.log(2) * nbytes), rel=1e-5)
        # valid targets again: the flag starts clear on every call
        y.copy_(torch.from_numpy(np.where(y_np < 0, 0, np.minimum(y_np, V - 1)).astype(np.int32)))
        n.nc_softcap_xent_fwd(h, U, y, tb, c, lse, ltok, loss, bpb, ws)
        assert n.nc_sync_status(ws) == n.NC_OK


def test_step_flags_out_of_range_target():
    cfg = CONFIGS["small"]
    inp = make_inputs(cfg, batch=2)
    tg = inp["targets"][:2].copy()
    tg[1, 7] = cfg.vocab
    out = run_step(cfg, inp, batch=2, targets=tg)
    from dense_decoder_only_amd import nc as _nc
    assert out["status"] == _nc.NC_ERR_DEVICE_FLAG
    assert torch.isfinite(out["loss"]).all()
    ok = run_step(cfg, inp, batch=2)
    assert ok["status"] == _nc.NC_OK


# ------------------------------------------------------------ whole step --

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["d12", "d20", "d26"])
def test_step_full_batch_gradients(name):
    """nc_step_fwd_bwd at the full batch of the configuration (the launches
    the benchmark times), every parameter gradient against the oracle.  The
    batch repeats two distinct sequences B/2 times each in a seeded random
    order; its mean-loss gradient equals the oracle's over those two."""
    cfg = CONFIGS[name]
    B = cfg.batch
    inp = make_inputs(cfg)
    order = np.random.default_rng(4000 + cfg.index).permutation(np.repeat([0, 1], B // 2))
    S2 = inp["S"][:2]
    S = S2[order]
    ids, tg = np.ascontiguousarray(S[:, :-1]), np.ascontiguousarray(S[:, 1:])
    out = run_step(cfg, inp, ids=ids, targets=tg)
    assert out["status"] == 0
    torch.cuda.synchronize()
    note(f"{name}: GPU step done, running the oracle on 2 sequences")
    p = oracle.to_f64_params(inp["weights"])
    ref = oracle.step(cfg, p, np.ascontiguousarray(S2[:, :-1]), np.ascontiguousarray(S2[:, 1:]),
                      inp["token_bytes"])
    del p
    note(f"{name}: loss {float(out['loss']):.7f} oracle {ref['loss']:.7f}")
    assert float(out["loss"]) == pytest.approx(ref["loss"], rel=2e-3)
    assert float(out["bpb"]) == pytest.approx(ref["bpb"], rel=2e-3)
    lt = dev_to_f64(out["loss_tok"])
    for b in range(B):
        assert max_rel(lt[b], ref["loss_tok"][order[b]]) < 2e-2, b
    for k, g in out["grads"].items():
        g64 = dev_to_f64(g)
        assert np.all(np.isfinite(g64)), k
        cs, mr = cosine(g64, ref["grads"][k]), max_rel(g64, ref["grads"][k])
        note(f"{name} grad {k}: cos {cs:.6f} max_rel {mr:.3e}")
        assert cs >= 0.999 and mr <= 3e-2, (k, cs, mr)
    absent = np.setdiff1d(np.arange(cfg.vocab), ids)
    assert np.all(dev_to_f64(out["grads"]["embed"])[absent] == 0.0)
