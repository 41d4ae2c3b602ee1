"""C ABI checks that need no GPU: the library loads, exports every entry point
include/nc.h declares, the binding covers exactly those, and host-side
validation rejects bad arguments before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nc.h")
LIB = os.path.join(ROOT, "dense_decoder_only_amd", "libnc.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libnc.so not built")


def declared_names():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_names()
    for n in ("nc_embed_fwd", "nc_embed_bwd", "nc_rmsnorm_fwd", "nc_rmsnorm_bwd", "nc_rope_qknorm_fwd",
              "nc_rope_qknorm_bwd", "nc_mqa_attn_fwd", "nc_mqa_attn_bwd", "nc_relu2_mlp", "nc_gemm_bf16",
              "nc_softcap_xent_fwd", "nc_softcap_xent_bwd", "nc_step_fwd_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_names() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_the_header():
    from dense_decoder_only_amd import nc
    assert sorted(nc.exported_names()) == declared_names()


def test_version_and_host_validation():
    from dense_decoder_only_amd import nc
    lib = nc.load()
    assert b"gfx950" in lib.nc_version()
    # null operands: rejected on the host, nothing enqueued
    rc = lib.nc_gemm_bf16(0, 1, 256, 256, 256, None, 256, None, 256, None, nc.NC_F32, 256, 0.0,
                          nc.NC_EPI_STORE, None, None, nc.NC_BF16, None, 0, None)
    assert rc == nc.NC_ERR_INVALID_ARG
    assert "null" in nc.nc_last_error()
    # unsupported head_dim
    rc = lib.nc_mqa_attn_fwd(ctypes.c_void_p(16), nc.NC_BF16, 1, 64, 2, 96, 0.1, ctypes.c_void_p(16),
                             ctypes.c_void_p(16), None)
    assert rc == nc.NC_ERR_UNSUPPORTED
    # bad beta
    rc = lib.nc_gemm_bf16(0, 1, 8, 8, 8, ctypes.c_void_p(16), 8, ctypes.c_void_p(16), 8, ctypes.c_void_p(16),
                          nc.NC_F32, 8, 0.5, nc.NC_EPI_STORE, None, None, nc.NC_BF16, None, 0, None)
    assert rc == nc.NC_ERR_INVALID_ARG


def test_step_workspace_query_and_config_validation():
    from dense_decoder_only_amd import nc
    from synthetic import CONFIGS
    sizes = {}
    for name, cfg in CONFIGS.items():
        c = nc.make_config(cfg)
        sizes[name] = nc.nc_step_workspace_bytes(c)
        assert sizes[name] > 0
    assert sizes["d20"] > sizes["d12"] > sizes["small"] > sizes["tiny"]
    assert sizes["d26"] < 200 * 2 ** 30  # fits one MI355X with the weights
    bad = nc.make_config(CONFIGS["tiny"])
    bad.n_kv_head = 2
    assert nc.nc_step_workspace_bytes(bad) == 0
    lib = nc.load()
    p, g = nc.nc_params(), nc.nc_grads()
    rc = lib.nc_step_fwd_bwd(ctypes.byref(bad), ctypes.byref(p), ctypes.byref(g), None, None, None, None, 0, None,
                             None, None, None)
    assert rc == nc.NC_ERR_INVALID_ARG
    ok = nc.make_config(CONFIGS["tiny"])
    rc = lib.nc_step_fwd_bwd(ctypes.byref(ok), ctypes.byref(p), ctypes.byref(g), None, None, None, None, 0, None,
                             None, None, None)
    assert rc == nc.NC_ERR_INVALID_ARG


def test_kernel_timer_rejects_unknown_families():
    from dense_decoder_only_amd import nc
    lib = nc.load()
    for fam in (-1, nc.NC_PROBE_GEMM + 1):
        assert lib.nc_probe_start(fam, 4) == nc.NC_ERR_INVALID_ARG
        assert "unknown family" in nc.nc_last_error()
    assert lib.nc_probe_start(nc.NC_PROBE_GEMM, -1) == nc.NC_ERR_INVALID_ARG


def test_adamw_host_validation():
    from dense_decoder_only_amd import nc
    lib = nc.load()
    rc = lib.nc_adamw_step(None, None, None, None, None, 16, 1, 1e-3, 0.9, 0.95, 1e-8, 0.0, 1.0, None)
    assert rc == nc.NC_ERR_INVALID_ARG and "null" in nc.nc_last_error()


def test_inference_size_queries_and_validation():
    import dataclasses
    from dense_decoder_only_amd import nc
    from synthetic import CONFIGS
    lib = nc.load()
    small = nc.make_config(dataclasses.replace(CONFIGS["small"], seq_len=16, batch=2))
    assert nc.nc_kv_cache_bytes(small, 32) == 4 * 2 * 2 * 32 * 128 * 2  # L x (K, V) x B x max_len x 128 x bf16
    assert nc.nc_infer_workspace_bytes(small, 32) > 0
    # unsupported or inconsistent configurations report 0 bytes
    assert nc.nc_kv_cache_bytes(nc.make_config(CONFIGS["tiny"]), 128) == 0      # fp32, head_dim 64
    assert nc.nc_kv_cache_bytes(small, 8) == 0                                   # max_len < prompt length
    big_b = nc.make_config(dataclasses.replace(CONFIGS["small"], batch=129))
    assert nc.nc_infer_workspace_bytes(big_b, 1024) == 0                         # more than 128 sequences
    # errors are returned on the host, before anything is enqueued
    p = nc.nc_params(*[None] * 6)
    rc = lib.nc_prefill(ctypes.byref(small), ctypes.byref(p), None, None, 32, None, None, 0, None)
    assert rc == nc.NC_ERR_INVALID_ARG and "null parameter" in nc.nc_last_error()
    tiny = nc.make_config(CONFIGS["tiny"])
    rc = lib.nc_decode_step(ctypes.byref(tiny), ctypes.byref(p), None, None, None, 128, None, None, 0, None)
    assert rc == nc.NC_ERR_UNSUPPORTED
    assert nc.nc_mqa_decode_workspace_bytes(0, 10, 64) == 0
    fake = ctypes.c_void_p(1 << 20)
    rc = lib.nc_mqa_decode_attn(fake, fake, fake, fake, 2, 10, 64, 64, 0.1, fake, fake, 1 << 20, None)
    assert rc == nc.NC_ERR_UNSUPPORTED and "head_dim" in nc.nc_last_error()
    rc = lib.nc_mqa_decode_attn(fake, fake, fake, fake, 2, 40, 128, 64, 0.1, fake, fake, 1 << 20, None)
    assert rc == nc.NC_ERR_UNSUPPORTED
    rc = lib.nc_mqa_decode_attn(fake, fake, fake, fake, 2, 10, 128, 64, 0.1, fake, fake, 16, None)
    assert rc == nc.NC_ERR_WORKSPACE


def _debug_mode_in_child(env_value):
    """nc_debug_mode() and a host-rejected call in a fresh process (the switch is read once per process)."""
    import subprocess
    import sys
    code = ("import ctypes, sys; sys.path.insert(0, %r); from dense_decoder_only_amd import nc; lib = nc.load(); "
            "rc = lib.nc_gemm_bf16(0, 1, 256, 256, 256, None, 256, None, 256, None, nc.NC_F32, 256, 0.0, "
            "nc.NC_EPI_STORE, None, None, nc.NC_BF16, None, 0, None); "
            "print(lib.nc_debug_mode(), rc == nc.NC_ERR_INVALID_ARG)" % ROOT)
    env = dict(os.environ)
    env.pop("NC_DEBUG", None)
    if env_value is not None:
        env["NC_DEBUG"] = env_value
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    return out.stdout.split()


def test_debug_mode_follows_the_environment():
    assert _debug_mode_in_child(None) == ["0", "True"]
    assert _debug_mode_in_child("0") == ["0", "True"]
    # on: argument errors are still reported as such (nothing was enqueued to check)
    assert _debug_mode_in_child("1") == ["1", "True"]


def test_noalloc_decode_attention_host_validation():
    from dense_decoder_only_amd import nc
    lib = nc.load()
    fake = ctypes.c_void_p(256)
    # 128 sequences x 32 heads x 4096 positions need more partials than the fixed scratch holds
    assert nc.nc_mqa_decode_workspace_bytes(128, 32, 4096) > 16 << 20
    rc = lib.nc_mqa_decode_attn_noalloc(fake, fake, fake, fake, 128, 32, 128, 4096, 0.1, fake, None)
    assert rc == nc.NC_ERR_WORKSPACE and "scratch" in nc.nc_last_error()
    # unsupported shape: rejected before any scratch is touched
    rc = lib.nc_mqa_decode_attn_noalloc(fake, fake, fake, fake, 0, 32, 128, 4096, 0.1, fake, None)
    assert rc != nc.NC_OK
