"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing device results with fp64 oracle results."""
import numpy as np
import torch

DEV = "cuda"


def bf16_tensor_from_bits(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def to_dev(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp32/fp64 array -> device tensor; bf16 via round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).to(DEV)


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rounded(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """The fp64 values of x after rounding to `dtype` (what the device consumes)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype).double().numpy()


def max_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_inf / ||ref||_inf."""
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def cosine(got: np.ndarray, ref: np.ndarray) -> float:
    a, b = got.reshape(-1), ref.reshape(-1)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def assert_close(got, ref, rtol, atol_frac, what=""):
    """|got - ref| <= rtol |ref| + atol_frac * max|ref| elementwise."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref)
    bound = rtol * np.abs(ref) + atol_frac * scale
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} outside tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} (max_rel {max_rel(got, ref):.3e})")


PARAM_NAMES = ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")


def run_step(cfg, inp, batch=None, accumulate=0, grads=None, ids=None, targets=None):
    """Run nc_step_fwd_bwd on the seeded inputs; returns device tensors."""
    from dense_decoder_only_amd import nc
    import dataclasses
    B = cfg.batch if batch is None else batch
    c = dataclasses.replace(cfg, batch=B)
    wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if cfg.dtype == "bf16":
        params = {k: bf16_tensor_from_bits(inp["weights_bf16"][k]) for k in PARAM_NAMES}
    else:
        params = {k: to_dev(inp["weights"][k], torch.float32) for k in PARAM_NAMES}
    if grads is None:
        grads = {k: torch.full(params[k].shape, float("nan"), dtype=torch.float32, device=DEV) for k in PARAM_NAMES}
    ids_np = inp["ids"][:B] if ids is None else ids
    tg_np = inp["targets"][:B] if targets is None else targets
    idt = torch.from_numpy(np.ascontiguousarray(ids_np)).to(DEV)
    tgt = torch.from_numpy(np.ascontiguousarray(tg_np)).to(DEV)
    tb = torch.from_numpy(inp["token_bytes"]).to(DEV)
    ccfg = nc.make_config(c)
    ws = torch.empty(nc.nc_step_workspace_bytes(ccfg), dtype=torch.uint8, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    bpb = torch.empty(1, dtype=torch.float32, device=DEV)
    ltok = torch.empty(B, cfg.seq_len, dtype=torch.float32, device=DEV)
    nc.nc_step_fwd_bwd(ccfg, params, grads, accumulate, idt, tgt, tb, ws, loss, bpb, ltok)
    status = nc.nc_sync_status(ws)
    del ws
    return dict(loss=loss, bpb=bpb, loss_tok=ltok, grads=grads, status=status, params=params, wdt=wdt)
