"""nc_mqa_decode_attn_noalloc: decode attention whose chunk partials live in
the library's own device scratch array instead of a caller workspace.

It runs the same kernels as nc_mqa_decode_attn, so on the same inputs its
output must equal that entry point's bit for bit; two calls in a row, the
second smaller than the first, check that nothing of the first call's
scratch contents reaches the second.  Cache rows past each sequence's length
hold NaN, so a read there would show.  The first call is also checked
against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, dev_to_f64

pytestmark = pytest.mark.gpu


def _nc():
    from dense_decoder_only_amd import nc
    nc.load()
    return nc


def _unit_rms(x):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def _case(n, seed, B, H, max_len, lens):
    r = np.random.default_rng(seed)
    hd = 128
    q = torch.from_numpy(_unit_rms(r.standard_normal((B, H, hd))).astype(np.float32)).to(torch.bfloat16).to(DEV)
    k = torch.from_numpy(_unit_rms(r.standard_normal((B, max_len, hd))).astype(np.float32)).to(torch.bfloat16).to(DEV)
    v = torch.from_numpy(r.standard_normal((B, max_len, hd)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    for b, L in enumerate(lens):
        k[b, L:] = float("nan")
        v[b, L:] = float("nan")
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(hd)
    o_ws = torch.empty(B, H, hd, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(n.nc_mqa_decode_workspace_bytes(B, H, max_len), dtype=torch.uint8, device=DEV)
    n.nc_mqa_decode_attn(q, k, v, lens_d, B, H, hd, max_len, scale, o_ws, ws)
    o = torch.full((B, H, hd), float("nan"), dtype=torch.bfloat16, device=DEV)
    n.nc_mqa_decode_attn_noalloc(q, k, v, lens_d, B, H, hd, max_len, scale, o)
    torch.cuda.synchronize()
    return o, o_ws, (q, k, v, scale)


def test_noalloc_decode_attention_matches_workspace_call():
    n = _nc()
    # first call: the d20 decode shape (32 sequences, 10 heads, 2048 positions)
    r = np.random.default_rng(11)
    lens = [int(x) for x in r.integers(1, 2049, 32)]
    lens[0], lens[1], lens[2] = 2048, 1, 0
    o1, ref1, (q, k, v, scale) = _case(n, 12, 32, 10, 2048, lens)
    assert torch.equal(o1, ref1)
    got, qr, kr, vr = dev_to_f64(o1), dev_to_f64(q), dev_to_f64(k), dev_to_f64(v)
    assert np.all(got[2] == 0.0)
    for b in (0, 1, 17):
        ref = oracle.decode_attention(qr[b], kr[b, :lens[b]], vr[b, :lens[b]], scale)
        assert np.all(np.abs(got[b] - ref) <= 2 ** -8 * np.abs(ref) + 2e-3 * np.abs(ref).max()), b
    # second call, smaller: fewer sequences, heads and positions
    o2, ref2, _ = _case(n, 13, 3, 4, 200, [200, 65, 0])
    assert torch.equal(o2, ref2)
    assert torch.all(o2[2] == 0)


def test_noalloc_decode_attention_rejects_shapes_beyond_its_scratch():
    n = _nc()
    lib = n.load()
    fake = torch.empty(16, dtype=torch.uint8, device=DEV)
    # 128 sequences x 32 heads x 4096 positions need 68 MB of partials
    assert n.nc_mqa_decode_workspace_bytes(128, 32, 4096) > 16 << 20
    rc = lib.nc_mqa_decode_attn_noalloc(fake.data_ptr(), fake.data_ptr(), fake.data_ptr(), fake.data_ptr(),
                                        128, 32, 128, 4096, 0.1, fake.data_ptr(), None)
    assert rc == n.NC_ERR_WORKSPACE and "scratch" in n.nc_last_error()
