"""Benchmark: training tokens/s of one forward+backward step of the dense
decoder (libnc.nc_step_fwd_bwd) on one MI355X, on synthetic inputs.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d20]

Prints ONE JSON line on stdout.  A step is the whole hot path (embedding,
every layer forward and backward, softcap cross entropy, all parameter
gradients) over one batch; inputs and weights are resident in HBM before the
timed region.  Besides the throughput it reports
  * roofline: the dominant kernel's achieved TFLOP/s against the bf16 matrix
    peak, timed live with HIP events on the stream it runs on, over separate
    steps after the timed region (the headline steps run without the events);
  * cpu_baseline: the fp64 oracle timed on this host's cores on a bounded
    sample of the same workload;
  * optimizer: the AdamW update over every parameter (HBM roofline) and the
    whole training iteration;
  * decode: prefill and one-token decode steps of the same model with a
    key/value cache (HBM rooflines of the decode attention and the small-M
    GEMMs).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/sec (fwd+bwd) at d20 seq 2048 on 1 MI355X; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_device_inputs(cfg, torch, nc):
    from synthetic import make_inputs
    inp = make_inputs(cfg)
    dev = "cuda"
    names = ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")
    if cfg.dtype == "bf16":
        params = {k: torch.from_numpy(inp["weights_bf16"][k].view(np.int16)).view(torch.bfloat16).to(dev) for k in names}
    else:
        params = {k: torch.from_numpy(inp["weights"][k]).to(dev) for k in names}
    grads = {k: torch.zeros(params[k].shape, dtype=torch.float32, device=dev) for k in names}
    ids = torch.from_numpy(inp["ids"]).to(dev)
    tgt = torch.from_numpy(inp["targets"]).to(dev)
    tb = torch.from_numpy(inp["token_bytes"]).to(dev)
    ccfg = nc.make_config(cfg)
    ws = torch.empty(nc.nc_step_workspace_bytes(ccfg), dtype=torch.uint8, device=dev)
    return inp, ccfg, params, grads, ids, tgt, tb, ws


FAMILIES = {
    # name: (probe family, kernel symbol in the profiles, what it computes,
    #        committed counter summary giving its HBM bytes per launch)
    "gemm": ("NC_PROBE_GEMM", "gemm_pipe_kernel<E, TN>",
             "every GEMM of the step: projections, relu^2 MLP, logits, activation and weight gradients",
             "gemm_pipe_kernel_d20_traffic.md"),
    "wgrad": ("NC_PROBE_GEMM_WGRAD", "gemm_pipe_kernel<E, true>",
              "weight-gradient GEMMs dW = dY^T X (K = tokens, split-K partial products)", None),
    "nt": ("NC_PROBE_GEMM_NT", "gemm_pipe_kernel<E, false>",
           "K-contiguous GEMMs (forward projections and activation gradients)", None),
    "attn_fwd": ("NC_PROBE_ATTN_FWD", "attn_fwd_kernel", "causal MQA attention forward", None),
    "attn_dq": ("NC_PROBE_ATTN_DQ", "attn_dq_kernel", "attention backward, dQ", None),
    "attn_dkv": ("NC_PROBE_ATTN_DKV", "attn_dkv_kernel", "attention backward, dK and dV", None),
}
DOMINANT = "gemm"    # largest share of kernel time in the committed kernel-trace summary


def stored_traffic(summary):
    """HBM bytes per launch from a committed counter summary under profiles/,
    or None if there is none or the kernel's source has changed since the
    counters were taken."""
    import hashlib
    if summary is None:
        return None
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    src = fields.get("source")
    if not src or "traffic_bytes_per_launch" not in fields:
        return None
    digest = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    if digest != fields.get("source_sha256"):
        return None
    return float(fields["traffic_bytes_per_launch"])


def roofline(name, ms, launches, flops, workload):
    fam = FAMILIES[name]
    achieved = flops / (ms / 1e3) / 1e12
    return {
        "kernel": f"{fam[1]}: {fam[2]}",
        "avg_launch_us": 1e3 * ms / max(launches, 1),
        "launches": launches,
        "flops_per_launch": flops / max(launches, 1),
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        # the stored counter figures are per launch of the d20 step
        "traffic": stored_traffic(fam[3]) if workload == "d20" else None,
    }


def host_cpu_and_blas():
    """(CPU model name, numpy's BLAS library and version, BLAS threads)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '?')}"
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:
        pass
    return model, blas, int(threads)


def cpu_baseline(cfg, inp, budget_tokens=None):
    """The fp64 oracle, untouched, on a bounded sample: forward+backward of the
    first `n` tokens of sequence 0 with the full model."""
    import oracle
    cpu, blas, cores = host_cpu_and_blas()
    n = budget_tokens or cfg.seq_len
    p = oracle.to_f64_params(inp["weights"])
    ids = inp["ids"][:1, :n]
    tg = inp["targets"][:1, :n]
    t0 = time.perf_counter()
    oracle.step(cfg, p, ids, tg, inp["token_bytes"])
    dt = time.perf_counter() - t0
    return {
        "value": round(n / dt, 3),
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, forward+backward of the first {n} tokens of one sequence, "
                  f"full {cfg.name} model ({cfg.n_layer} layers, vocab {cfg.vocab}); {dt:.1f} s "
                  f"on {cpu}, BLAS {blas} with {cores} threads",
        "cpu": cpu,
        "blas": blas,
    }


ADAMW_BYTES_PER_PARAM = 30   # read p, m, v, g (fp32); write p, m, v (fp32) and the bf16 copy


def optimizer_leg(cfg, inp, torch, nc, params, grads, step, s, reps=5):
    """Times nc_adamw_step over every parameter tensor (HBM-bound: 30 B per
    parameter in a bf16 configuration, 28 B in fp32), then whole training
    iterations (forward + backward + AdamW with the bf16 refresh).  Runs after
    the timed region of the headline metric and leaves it untouched."""
    names = ("embed", "w_qkv", "w_o", "w_fc", "w_proj", "unembed")
    bf16 = cfg.dtype == "bf16"
    master = {k: torch.from_numpy(inp["master"][k]).to("cuda") for k in names}
    m = {k: torch.zeros_like(master[k]) for k in names}
    v = {k: torch.zeros_like(master[k]) for k in names}
    n = sum(master[k].numel() for k in names)
    hp = dict(beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)

    def adamw(t):
        for k in names:
            nc.nc_adamw_step(master[k], m[k], v[k], grads[k], params[k] if bf16 else None, t, 1e-4,
                             stream=s, **hp)

    adamw(1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for t in range(2, 2 + reps):
        adamw(t)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    bpp = ADAMW_BYTES_PER_PARAM if bf16 else ADAMW_BYTES_PER_PARAM - 2
    gbs = n * bpp / (ms * 1e-3) / 1e9
    e0.record(s)
    for t in range(2 + reps, 2 + 2 * reps):
        step()
        adamw(t)
    e1.record(s)
    torch.cuda.synchronize()
    it_ms = e0.elapsed_time(e1) / reps
    for k in names:
        del master[k], m[k], v[k]
    log(f"[bench] adamw over {n} parameters: {ms:.3f} ms, {gbs:.0f} GB/s; "
        f"training iteration {it_ms:.2f} ms ({cfg.tokens / (it_ms * 1e-3):.0f} tok/s)")
    return {"kernel": "adamw_kernel", "params": n, "bytes_per_param": bpp, "ms": round(ms, 4),
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "launches": 6,
            "iteration_ms": round(it_ms, 3), "iteration_tokens_per_s": round(cfg.tokens / (it_ms * 1e-3), 1)}


def decode_leg(cfg, torch, nc, params, s, steps=64, max_len=2048):
    """Inference on the same model: prefill of B prompts of max_len - steps
    tokens, then `steps` decode steps (one token per sequence, positions
    max_len - steps .. max_len - 1).  HBM-bound: a step reads every projection
    weight and U once (small-M GEMMs) and each sequence's cached keys and
    values once per layer (decode attention).  Timed with HIP events on the
    launch stream; the per-kernel times come from the library's kernel timer
    in two extra passes (one family each), the bytes are counted here from
    the known positions."""
    import dataclasses
    from synthetic import make_tokens
    T0 = max_len - steps
    icfg = dataclasses.replace(cfg, seq_len=T0)
    ccfg = nc.make_config(icfg)
    B, L, d, H, F, V = cfg.batch, cfg.n_layer, cfg.d_model, cfg.n_head, cfg.d_ff, cfg.vocab
    kv = torch.empty(nc.nc_kv_cache_bytes(ccfg, max_len), dtype=torch.uint8, device="cuda")
    ws = torch.empty(nc.nc_infer_workspace_bytes(ccfg, max_len), dtype=torch.uint8, device="cuda")
    logits = torch.empty(B, V, device="cuda")
    toks = torch.from_numpy(make_tokens(cfg, seed=4242)).to("cuda")  # [B, 2049], Zipf(1.1)
    prompts = toks[:, :T0].contiguous()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def prefill():
        nc.nc_prefill(ccfg, params, prompts, kv, max_len, logits, ws, stream=s)

    prefill()
    torch.cuda.synchronize()
    e0.record(s)
    prefill()
    e1.record(s)
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    pos = [torch.full((B,), T0 + j, dtype=torch.int32, device="cuda") for j in range(steps)]
    ids = [toks[:, T0 + j].contiguous() for j in range(steps)]

    def run(family=None):
        if family is not None:  # room for every launch of the decode steps (5 per layer at most)
            nc.nc_probe_start(getattr(nc, family), (5 * L + 8) * steps)
        e0.record(s)
        for j in range(steps):
            nc.nc_decode_step(ccfg, params, ids[j], pos[j], kv, max_len, logits, ws, stream=s)
        e1.record(s)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        return ms, (nc.nc_probe_stop() if family is not None else None)

    run()
    ms, _ = run()
    if nc.nc_sync_status(ws) != nc.NC_OK:
        raise RuntimeError("device flag raised during decoding")
    _, (att_ms, att_n, _) = run("NC_PROBE_DECODE_ATTN")
    _, (gem_ms, gem_n, gem_bytes) = run("NC_PROBE_GEMM_SKINNY")
    # algorithmic bytes
    Q, HD = (H + 2) * 128, H * 128
    w_bytes = 2 * (L * (Q * d + d * HD + F * d + d * F) + V * d)
    mean_len = T0 + (steps + 1) / 2.0                    # positions T0 .. T0 + steps - 1, lengths pos + 1
    kv_bytes_launch = B * mean_len * 128 * 2 * 2 + 2 * B * H * 128 * 2
    act_bytes = 2 * L * B * (Q + HD + F + d) * 2 + B * V * 4
    step_bytes = w_bytes + L * kv_bytes_launch + act_bytes
    att_us = 1e3 * att_ms / att_n
    att_gbs = kv_bytes_launch / (att_us * 1e-6) / 1e9
    gem_gbs = gem_bytes / (gem_ms * 1e-3) / 1e9
    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode {cfg.name}: {ms:.3f} ms/step ({B / (ms * 1e-3):.0f} tok/s), {step_gbs:.0f} GB/s over "
        f"{step_bytes / 1e9:.3f} GB; attention {att_us:.1f} us/launch {att_gbs:.0f} GB/s; small-M GEMMs "
        f"{gem_gbs:.0f} GB/s; prefill {prefill_ms:.1f} ms")
    return {
        "workload": f"{cfg.name} decode: {B} sequences, one token each at positions {T0}..{max_len - 1} "
                    f"(cache max_len {max_len}), after a {T0}-token prefill",
        "tokens_per_s": round(B / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
        "step_bytes": int(step_bytes), "step_achieved_GBs": round(step_gbs, 1),
        "step_frac": round(step_gbs / PEAK_HBM_GBS, 4),
        "attention": {"kernel": "decode_attn_split_kernel + decode_attn_combine_kernel", "bound": "hbm",
                      "achieved": round(att_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(att_gbs / PEAK_HBM_GBS, 4), "avg_launch_us": round(att_us, 2),
                      "bytes_per_launch": int(kv_bytes_launch)},
        "gemm": {"kernel": "gemm_skinny_kernel", "bound": "hbm", "achieved": round(gem_gbs, 1),
                 "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gem_gbs / PEAK_HBM_GBS, 4),
                 "launches_per_step": gem_n // steps, "avg_launch_us": round(1e3 * gem_ms / gem_n, 2)},
        "prefill_tokens_per_s": round(B * T0 / (prefill_ms * 1e-3), 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d20", choices=["tiny", "small", "d12", "d20", "d26"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=None)
    ap.add_argument("--roofline-kernel", default=DOMINANT, choices=sorted(FAMILIES))
    ap.add_argument("--roofline-steps", type=int, default=5,
                    help="steps run after the timed region with the kernel timer armed (0: none)")
    ap.add_argument("--no-decode", action="store_true", help="skip the prefill / decode timings")
    ap.add_argument("--no-optimizer", action="store_true", help="skip the AdamW and full-iteration timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with one 1 GiB device-to-device copy (counter calibration runs)")
    a = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", a.gpus))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from synthetic import CONFIGS
    from dense_decoder_only_amd import accounting, nc
    nc.load()
    cfg = CONFIGS[a.config]
    log(f"[bench] config {cfg.name}: building inputs")
    inp, ccfg, params, grads, ids, tgt, tb, ws = build_device_inputs(cfg, torch, nc)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    bpb = torch.empty(1, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()

    def step():
        nc.nc_step_fwd_bwd(ccfg, params, grads, 0, ids, tgt, tb, ws, loss, bpb, None, stream=s)

    for i in range(a.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{a.warmup} loss {float(loss):.4f}")
    if nc.nc_sync_status(ws) != nc.NC_OK:
        raise RuntimeError("device flag raised during warmup")
    torch.cuda.synchronize()
    # headline: the timed steps run with the kernel timer disarmed
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(a.steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = e0.elapsed_time(e1) / 1e3
    # roofline of the dominant kernel: separate steps with the kernel timer armed
    fam = FAMILIES[a.roofline_kernel]
    rsteps = max(a.roofline_steps, 1)
    nc.nc_probe_start(getattr(nc, fam[0]), 512 * rsteps)
    for _ in range(rsteps):
        step()
    torch.cuda.synchronize()
    roof = roofline(a.roofline_kernel, *nc.nc_probe_stop(), cfg.name)
    roof["steps"] = rsteps
    elapsed = max(wall, gpu_s)
    tokens = cfg.tokens * a.steps
    value = tokens / elapsed
    flops = accounting.flops_per_step(cfg) * a.steps
    tflops = flops / elapsed / 1e12
    log(f"[bench] {a.steps} steps in {elapsed:.3f} s: {value:.0f} tok/s, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.2f}% of bf16 peak), loss {float(loss):.4f} bpb {float(bpb):.4f}")

    log(f"[bench] {roof['kernel']}: {roof['launches']} launches, {roof['avg_launch_us']:.1f} us/launch, "
        f"{roof['achieved']} TFLOP/s")
    opt = None if a.no_optimizer else optimizer_leg(cfg, inp, torch, nc, params, grads, step, s)
    dec = None
    if not a.no_decode and cfg.dtype == "bf16" and cfg.head_dim == 128:
        dec = decode_leg(cfg, torch, nc, params, s)
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB device to device (calibration)")
    base = None
    if not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        base = cpu_baseline(cfg, inp, a.cpu_tokens)
        log(f"[bench] cpu baseline {base['value']} tok/s on {base['cores']} threads")
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(1e3 * elapsed / a.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Zipf(1.1) token ids, random-init weights)",
        "config": {
            "workload": f"{cfg.name}: depth {cfg.n_layer}, d_model {cfg.d_model}, {cfg.n_head} heads x "
                        f"{cfg.head_dim}, 1 KV head, MLP {cfg.d_ff}, vocab {cfg.vocab}, seq {cfg.seq_len}, "
                        f"batch {cfg.batch} ({cfg.tokens} tokens/step), fwd+bwd",
            "global_batch": cfg.batch,
            "seq_len": cfg.seq_len,
            "parallelism": "single GPU",
        },
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "roofline_kernel": {k: roof[k] for k in ("kernel", "launches", "avg_launch_us", "flops_per_launch",
                                                  "steps")},
        "cpu_baseline": base,
        "optimizer": opt,
        "decode": dec,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
