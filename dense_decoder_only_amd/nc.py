"""ctypes binding of libnc (include/nc.h).

Argument marshalling only: every function here has the name of the C entry
point it calls, takes torch tensors where the C function takes device
pointers, passes ``torch.cuda.current_stream()`` as the stream, and raises
``NcError`` when the call returns an error.  All computation happens in the
HIP kernels of libnc.so; there is no fallback of any kind.  If the library
has not been built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnc.so")

NC_OK, NC_ERR_INVALID_ARG, NC_ERR_UNSUPPORTED, NC_ERR_WORKSPACE, NC_ERR_HIP, NC_ERR_DEVICE_FLAG = range(6)
NC_F32, NC_BF16 = 0, 1
NC_EPI_STORE, NC_EPI_RELU2, NC_EPI_RELU2_BWD, NC_EPI_RELU2_SQ, NC_EPI_RELU2_BWD_SQ = 0, 1, 2, 3, 4
(NC_PROBE_OFF, NC_PROBE_GEMM_WGRAD, NC_PROBE_GEMM_NT, NC_PROBE_ATTN_FWD, NC_PROBE_ATTN_DQ,
 NC_PROBE_ATTN_DKV, NC_PROBE_GEMM_SKINNY, NC_PROBE_DECODE_ATTN, NC_PROBE_GEMM) = range(9)

c_int, c_i64, c_f, c_sz, c_p = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class NcError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libnc error {code}: {msg}")
        self.code = code


class nc_config(ctypes.Structure):
    _fields_ = [("n_layer", c_int), ("d_model", c_int), ("n_head", c_int), ("head_dim", c_int),
                ("n_kv_head", c_int), ("d_ff", c_int), ("vocab", c_int), ("seq_len", c_int), ("batch", c_int),
                ("softcap", c_f), ("rope_base", c_f), ("eps", c_f), ("dtype", c_int)]


class nc_params(ctypes.Structure):
    _fields_ = [(n, c_p) for n in ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")]


class nc_grads(ctypes.Structure):
    _fields_ = [(n, c_p) for n in ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")] + [("accumulate", c_int)]


# name -> (restype, argtypes)
_SIGS = {
    "nc_last_error": (ctypes.c_char_p, []),
    "nc_version": (ctypes.c_char_p, []),
    "nc_debug_mode": (ctypes.c_int, []),
    "nc_sync_status": (c_int, [c_p, c_p]),
    "nc_adamw_step": (c_int, [c_p, c_p, c_p, c_p, c_p, c_i64, c_int, c_f, c_f, c_f, c_f, c_f, c_f, c_p]),
    "nc_probe_start": (c_int, [c_int, c_int]),
    "nc_probe_stop": (c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64),
                              ctypes.POINTER(ctypes.c_double)]),
    "nc_step_workspace_bytes": (c_sz, [ctypes.POINTER(nc_config)]),
    "nc_step_fwd_bwd": (c_int, [ctypes.POINTER(nc_config), ctypes.POINTER(nc_params), ctypes.POINTER(nc_grads),
                                c_p, c_p, c_p, c_p, c_sz, c_p, c_p, c_p, c_p]),
    "nc_embed_fwd": (c_int, [c_p, c_i64, c_p, c_int, c_i64, c_int, c_p, c_p, c_p, c_f, c_p, c_p]),
    "nc_embed_bwd_workspace_bytes": (c_sz, [c_i64, c_i64, c_int]),
    "nc_embed_bwd": (c_int, [c_p, c_i64, c_p, c_int, c_p, c_i64, c_int, c_p, c_sz, c_p]),
    "nc_rmsnorm_fwd": (c_int, [c_p, c_int, c_i64, c_int, c_f, c_p, c_int, c_p, c_p]),
    "nc_rmsnorm_bwd": (c_int, [c_p, c_int, c_p, c_int, c_p, c_i64, c_int, c_p, c_int, c_p, c_p]),
    "nc_rope_table": (c_int, [c_p, c_int, c_int, c_f, c_p]),
    "nc_rope_qknorm_fwd": (c_int, [c_p, c_int, c_int, c_int, c_int, c_int, c_p, c_f, c_p, c_p, c_p]),
    "nc_rope_qknorm_bwd": (c_int, [c_p, c_p, c_p, c_p, c_p, c_int, c_int, c_int, c_int, c_int, c_p, c_p]),
    "nc_mqa_attn_fwd": (c_int, [c_p, c_int, c_int, c_int, c_int, c_int, c_f, c_p, c_p, c_p]),
    "nc_mqa_attn_bwd_workspace_bytes": (c_sz, [c_int, c_int, c_int]),
    "nc_mqa_attn_bwd": (c_int, [c_p, c_p, c_p, c_p, c_int, c_int, c_int, c_int, c_int, c_f, c_p, c_p, c_sz, c_p]),
    "nc_gemm_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "nc_gemm_bf16": (c_int, [c_int, c_int, c_i64, c_i64, c_i64, c_p, c_i64, c_p, c_i64, c_p, c_int, c_i64, c_f,
                             c_int, c_p, c_p, c_int, c_p, c_sz, c_p]),
    "nc_relu2_mlp": (c_int, [c_p, c_p, c_p, c_int, c_i64, c_int, c_int, c_p, c_p, c_p, c_p]),
    "nc_relu2_mlp_bwd": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_int, c_i64, c_int, c_int, c_p, c_p, c_p, c_int,
                                 c_p, c_p, c_sz, c_p]),
    "nc_kv_cache_bytes": (c_sz, [ctypes.POINTER(nc_config), c_int]),
    "nc_infer_workspace_bytes": (c_sz, [ctypes.POINTER(nc_config), c_int]),
    "nc_prefill": (c_int, [ctypes.POINTER(nc_config), ctypes.POINTER(nc_params), c_p, c_p, c_int, c_p, c_p, c_sz,
                           c_p]),
    "nc_decode_step": (c_int, [ctypes.POINTER(nc_config), ctypes.POINTER(nc_params), c_p, c_p, c_p, c_int, c_p, c_p,
                               c_sz, c_p]),
    "nc_mqa_decode_workspace_bytes": (c_sz, [c_int, c_int, c_int]),
    "nc_mqa_decode_attn": (c_int, [c_p, c_p, c_p, c_p, c_int, c_int, c_int, c_int, c_f, c_p, c_p, c_sz, c_p]),
    "nc_mqa_decode_attn_noalloc": (c_int, [c_p, c_p, c_p, c_p, c_int, c_int, c_int, c_int, c_f, c_p, c_p]),
    "nc_softcap_xent_workspace_bytes": (c_sz, [c_i64, c_int, c_int]),
    "nc_softcap_xent_fwd": (c_int, [c_p, c_p, c_int, c_p, c_p, c_i64, c_int, c_int, c_f, c_p, c_p, c_p, c_p, c_p,
                                    c_sz, c_p]),
    "nc_softcap_xent_bwd": (c_int, [c_p, c_p, c_int, c_p, c_p, c_i64, c_int, c_int, c_f, c_f, c_p, c_int, c_p,
                                    c_int, c_p, c_sz, c_p]),
}

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnc.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first with `python -m dense_decoder_only_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def exported_names():
    return list(_SIGS)


def _check(rc: int) -> None:
    if rc != NC_OK:
        raise NcError(rc, load().nc_last_error().decode())


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return NC_F32
    if dt == torch.bfloat16:
        return NC_BF16
    raise ValueError(f"unsupported dtype {dt}")


def make_config(cfg) -> nc_config:
    """nc_config from a synthetic.ModelConfig-like object."""
    return nc_config(cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                     cfg.seq_len, cfg.batch, cfg.softcap, cfg.rope_base, cfg.eps,
                     NC_BF16 if cfg.dtype == "bf16" else NC_F32)


# --------------------------------------------------------------------------- calls

def nc_version() -> str:
    return load().nc_version().decode()


def nc_debug_mode() -> bool:
    return bool(load().nc_debug_mode())


def nc_last_error() -> str:
    return load().nc_last_error().decode()


def nc_sync_status(flag, stream=None) -> int:
    """Returns the status code (NC_OK or NC_ERR_DEVICE_FLAG) instead of raising on the flag."""
    return load().nc_sync_status(_p(flag), _stream(stream))


def nc_adamw_step(master, m, v, grad, weights_lp, t, lr, beta1, beta2, eps, weight_decay, grad_scale=1.0,
                  stream=None) -> None:
    _check(load().nc_adamw_step(_p(master), _p(m), _p(v), _p(grad), _p(weights_lp), master.numel(), int(t),
                                lr, beta1, beta2, eps, weight_decay, grad_scale, _stream(stream)))


def nc_probe_start(family: int, max_launches: int) -> None:
    _check(load().nc_probe_start(int(family), int(max_launches)))


def nc_probe_stop() -> tuple:
    """Returns (total_ms, launches, flops) of the bracketed launches."""
    ms, n, fl = ctypes.c_double(), c_i64(), ctypes.c_double()
    _check(load().nc_probe_stop(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl)))
    return ms.value, n.value, fl.value


def nc_step_workspace_bytes(cfg: nc_config) -> int:
    return load().nc_step_workspace_bytes(ctypes.byref(cfg))


def nc_step_fwd_bwd(cfg: nc_config, params: dict, grads: dict, accumulate: int, ids, targets, token_bytes, ws,
                    loss, bpb, loss_tok=None, stream=None) -> None:
    names = ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")
    p = nc_params(*[_p(params[n]) for n in names])
    g = nc_grads(*[_p(grads[n]) for n in names], int(accumulate))
    _check(load().nc_step_fwd_bwd(ctypes.byref(cfg), ctypes.byref(p), ctypes.byref(g), _p(ids), _p(targets),
                                  _p(token_bytes), _p(ws), ws.numel() * ws.element_size(), _p(loss), _p(bpb),
                                  _p(loss_tok), _stream(stream)))


def nc_embed_fwd(ids, table, rows_out=None, x_out=None, rstd=None, eps=1e-6, flag=None, stream=None) -> None:
    V, d = table.shape
    _check(load().nc_embed_fwd(_p(ids), ids.numel(), _p(table), dtype_code(table.dtype), V, d, _p(rows_out),
                               _p(x_out), _p(rstd), eps, _p(flag), _stream(stream)))


def nc_embed_bwd_workspace_bytes(n: int, V: int, d: int) -> int:
    return load().nc_embed_bwd_workspace_bytes(n, V, d)


def nc_embed_bwd(ids, de, dtable, accumulate, ws, stream=None) -> None:
    V, d = dtable.shape
    _check(load().nc_embed_bwd(_p(ids), ids.numel(), _p(de), d, _p(dtable), V, int(accumulate), _p(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))


def nc_rmsnorm_fwd(x, y, rstd=None, eps=1e-6, stream=None) -> None:
    d = x.shape[-1]
    _check(load().nc_rmsnorm_fwd(_p(x), dtype_code(x.dtype), x.numel() // d, d, eps, _p(y), dtype_code(y.dtype),
                                 _p(rstd), _stream(stream)))


def nc_rmsnorm_bwd(dy, y, rstd, dx, accumulate=0, dx_bf16=None, stream=None) -> None:
    d = dy.shape[-1]
    _check(load().nc_rmsnorm_bwd(_p(dy), dtype_code(dy.dtype), _p(y), dtype_code(y.dtype), _p(rstd),
                                 dy.numel() // d, d, _p(dx), int(accumulate), _p(dx_bf16), _stream(stream)))


def nc_rope_table(table, T: int, hd: int, base: float, stream=None) -> None:
    _check(load().nc_rope_table(_p(table), T, hd, base, _stream(stream)))


def nc_rope_qknorm_fwd(qkv, B, T, H, hd, table, eps, rstd_q, rstd_k, stream=None) -> None:
    _check(load().nc_rope_qknorm_fwd(_p(qkv), dtype_code(qkv.dtype), B, T, H, hd, _p(table), eps, _p(rstd_q),
                                     _p(rstd_k), _stream(stream)))


def nc_rope_qknorm_bwd(dqkv_hat, qkv_hat, rstd_q, rstd_k, table, B, T, H, hd, dqkv, stream=None) -> None:
    _check(load().nc_rope_qknorm_bwd(_p(dqkv_hat), _p(qkv_hat), _p(rstd_q), _p(rstd_k), _p(table),
                                     dtype_code(qkv_hat.dtype), B, T, H, hd, _p(dqkv), _stream(stream)))


def nc_mqa_attn_fwd(qkv, B, T, H, hd, scale, o, lse, stream=None) -> None:
    _check(load().nc_mqa_attn_fwd(_p(qkv), dtype_code(qkv.dtype), B, T, H, hd, scale, _p(o), _p(lse),
                                  _stream(stream)))


def nc_mqa_attn_bwd_workspace_bytes(B, T, H) -> int:
    return load().nc_mqa_attn_bwd_workspace_bytes(B, T, H)


def nc_mqa_attn_bwd(qkv, o, dout, lse, B, T, H, hd, scale, dqkv_hat, ws, stream=None) -> None:
    _check(load().nc_mqa_attn_bwd(_p(qkv), _p(o), _p(dout), _p(lse), dtype_code(qkv.dtype), B, T, H, hd, scale,
                                  _p(dqkv_hat), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def nc_gemm_workspace_bytes(M, N, K) -> int:
    return load().nc_gemm_workspace_bytes(M, N, K)


def nc_gemm_bf16(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, beta=0.0, epilogue=NC_EPI_STORE, aux=None,
                 aux_out=None, ws=None, stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().nc_gemm_bf16(transA, transB, M, N, K, _p(A), lda, _p(B), ldb, _p(C), dtype_code(C.dtype), ldc,
                               beta, epilogue, _p(aux), _p(aux_out), dtype_code(A.dtype), _p(ws), ws_bytes,
                               _stream(stream)))


def nc_relu2_mlp(m, w_fc, w_proj, x, u_out, a2_out, stream=None) -> None:
    M, d = m.shape
    F = w_fc.shape[0]
    _check(load().nc_relu2_mlp(_p(m), _p(w_fc), _p(w_proj), dtype_code(m.dtype), M, d, F, _p(x), _p(u_out),
                               _p(a2_out), _stream(stream)))


def nc_relu2_mlp_bwd(g_lp, m, u, a2, w_fc, w_proj, dm, dw_fc, dw_proj, accumulate, du_buf, ws=None,
                     stream=None) -> None:
    M, d = m.shape
    F = w_fc.shape[0]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().nc_relu2_mlp_bwd(_p(g_lp), _p(m), _p(u), _p(a2), _p(w_fc), _p(w_proj), dtype_code(m.dtype), M, d,
                                   F, _p(dm), _p(dw_fc), _p(dw_proj), int(accumulate), _p(du_buf), _p(ws), ws_bytes,
                                   _stream(stream)))


def nc_softcap_xent_workspace_bytes(M, d, V) -> int:
    return load().nc_softcap_xent_workspace_bytes(M, d, V)


def nc_softcap_xent_fwd(h, U, tgt, token_bytes, softcap, lse, loss_tok, loss, bpb, ws, stream=None) -> None:
    M, d = h.shape
    V = U.shape[0]
    _check(load().nc_softcap_xent_fwd(_p(h), _p(U), dtype_code(h.dtype), _p(tgt), _p(token_bytes), M, d, V, softcap,
                                      _p(lse), _p(loss_tok), _p(loss), _p(bpb), _p(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def nc_softcap_xent_bwd(h, U, tgt, lse, softcap, dloss, dh, dh_accumulate, dU, dU_accumulate, ws,
                        stream=None) -> None:
    M, d = h.shape
    V = U.shape[0]
    _check(load().nc_softcap_xent_bwd(_p(h), _p(U), dtype_code(h.dtype), _p(tgt), _p(lse), M, d, V, softcap, dloss,
                                      _p(dh), int(dh_accumulate), _p(dU), int(dU_accumulate), _p(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))


_PARAM_NAMES = ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")


def nc_kv_cache_bytes(cfg: nc_config, max_len: int) -> int:
    return load().nc_kv_cache_bytes(ctypes.byref(cfg), max_len)


def nc_infer_workspace_bytes(cfg: nc_config, max_len: int) -> int:
    return load().nc_infer_workspace_bytes(ctypes.byref(cfg), max_len)


def nc_prefill(cfg: nc_config, params: dict, ids, kv_cache, max_len: int, logits, ws, stream=None) -> None:
    p = nc_params(*[_p(params[n]) for n in _PARAM_NAMES])
    _check(load().nc_prefill(ctypes.byref(cfg), ctypes.byref(p), _p(ids), _p(kv_cache), max_len, _p(logits), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)))


def nc_decode_step(cfg: nc_config, params: dict, ids, pos, kv_cache, max_len: int, logits, ws, stream=None) -> None:
    p = nc_params(*[_p(params[n]) for n in _PARAM_NAMES])
    _check(load().nc_decode_step(ctypes.byref(cfg), ctypes.byref(p), _p(ids), _p(pos), _p(kv_cache), max_len,
                                 _p(logits), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def nc_mqa_decode_workspace_bytes(B: int, H: int, max_len: int) -> int:
    return load().nc_mqa_decode_workspace_bytes(B, H, max_len)


def nc_mqa_decode_attn(q, k_cache, v_cache, lens, B, H, hd, max_len, scale, o, ws, stream=None) -> None:
    _check(load().nc_mqa_decode_attn(_p(q), _p(k_cache), _p(v_cache), _p(lens), B, H, hd, max_len, scale, _p(o),
                                     _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def nc_mqa_decode_attn_noalloc(q, k_cache, v_cache, lens, B, H, hd, max_len, scale, o, stream=None) -> None:
    _check(load().nc_mqa_decode_attn_noalloc(_p(q), _p(k_cache), _p(v_cache), _p(lens), B, H, hd, max_len, scale,
                                             _p(o), _stream(stream)))
