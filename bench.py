"""Benchmark of the Wan2.1 DiT hot path on one MI355X.

Workload: the 1.3B-shaped DiT block at 480P (latent 21x60x104, L = 32760
tokens, dim 1536, 12 heads of 128, FFN 8960, 512 text tokens), bf16 operands
with fp32 accumulation, seeded synthetic weights N(0, 0.02) and activations
N(0, 1).  One timed "step" is one pass of the hot path over that input: the
shared timestep MLP (wan_tmlp_fwd) followed by one full block
(wan_dit_block_fwd: LayerNorm+modulate, QKV GEMMs, flash self-attention,
out-projection with gated residual, cross-attention, FFN with gated residual).
Inputs are resident in HBM before timing starts; the block updates the
residual stream in place, so successive timed steps chain blocks.

Prints one JSON line (tokens/s of the block, attention roofline, CPU oracle
baseline on a bounded sample).  ``--gpus`` above 1 is refused: the library
runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_SCLK_MHZ = 2400.0        # the shader clock the published peaks are quoted at

# HBM bytes per self-attention launch of this workload, from two rocprofv3
# --pmc passes over `bench.py --traffic-pass` (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch), each scaled by what the counter reads for a plain 512 MiB
# copy (fetch x2.00, write x1.00); see profiles/k_attn_bf16_wan1.3b_block_480p.md.
# Valid only for the kernel sources they were taken on: reported as null
# once k_attn.hip, common.hpp or attn.hpp change.
ATTN_TRAFFIC = {
    "sources_sha256": "97fe764837f7bdc2d94a0e36b80849e69831605cb63adc228379ddbb1d900a47",
    "fetch_kib": 453210, "write_kib": 120571, "fetch_scale": 2.00, "write_scale": 1.00,
}


def attn_sources_sha256() -> str:
    import hashlib
    csrc = os.path.join(ROOT, "video_diffusion_transformer_block_amd", "csrc")
    h = hashlib.sha256()
    for f in ("k_attn.hip", "common.hpp", "attn.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def attn_traffic_bytes():
    """Calibrated HBM bytes of one self-attention launch of the 1.3B 480P
    workload (the counters were taken on that shape only), or None."""
    t = ATTN_TRAFFIC
    if attn_sources_sha256() != t["sources_sha256"]:
        return None
    return int(round(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])))


class ClockSampler:
    """Samples the GPU shader clock while a timed region runs: a host thread
    reads the driver's current-level line (the one marked '*') of
    /sys/class/drm/card*/device/pp_dpm_sclk every `period` seconds.  Used as a
    context manager; `mhz()` is the mean over the samples, or None when the
    file is not there."""

    def __init__(self, period: float = 0.002):
        import glob
        import threading
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = cards[0] if len(cards) == 1 else None
        self.period, self.samples = period, []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if self.path else None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self._thread:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()
        return False

    def mhz(self):
        return sum(self.samples) / len(self.samples) if self.samples else None


def clock_fields(clock, achieved_tf):
    """The sampled shader clock and the MFMA peak at that clock.  The driver's
    level is only a sample of the running clock: a rate above the peak at the
    sampled clock shows that the samples missed it (seen under a profiler),
    and then no fraction is given."""
    mhz = clock.mhz()
    out = {"sclk_mhz": None if mhz is None else round(mhz, 1), "sclk_samples": len(clock.samples),
           "peak_at_sclk": None, "frac_at_sclk": None}
    if mhz is not None:
        peak = PEAK_BF16_TFLOPS * mhz / PEAK_SCLK_MHZ
        out["peak_at_sclk"] = round(peak, 1)
        if achieved_tf <= peak:
            out["frac_at_sclk"] = round(achieved_tf / peak, 4)
        else:
            out["sclk_note"] = "the sampled level is below the clock the measured rate needs"
    return out


def block_flops(B, L, d, H, F, Lc, Li=0):
    hd = d // H
    M = B * L
    gemm = 2 * M * d * (3 * d) + 2 * M * d * d + 2 * M * d * d + 2 * B * Lc * d * 2 * d \
        + 2 * M * d * d + 2 * 2 * M * F * d
    if Li:
        gemm += 2 * B * Li * d * 2 * d
    sa = 4 * B * H * L * L * hd
    ca = 4 * B * H * L * (Lc + Li) * hd
    return gemm, sa, ca


def cpu_baseline(work, inp, tw, bw, budget_s: float = 25.0):
    """The CPU oracle, as it stands, on a bounded sample of the same block:
    oracle.block(..., rows=r) for two sample sizes r1 < r2 (every sampled run
    still projects K/V for all L tokens); the full block's time is
    extrapolated linearly in r to r = L and turned into tokens/s."""
    import numpy as np
    import oracle.wan_oracle as O
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(i.get("num_threads", 1) for i in info)
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        pass
    m = work.model
    L = work.L
    m_vec = O.tmlp(inp["t"], tw["w1"], tw["b1"], tw["w2"], tw["b2"])
    rng = np.random.default_rng(0)
    times = {}
    for r in (2048, 8192):
        rows = np.sort(rng.choice(L, size=r, replace=False))
        t0 = time.perf_counter()
        O.block(inp["x"], m_vec, bw, inp["ctx"], m.heads, m.eps, rows=rows)
        times[r] = time.perf_counter() - t0
    (r1, t1), (r2, t2) = sorted(times.items())
    per_row = max((t2 - t1) / (r2 - r1), 1e-9)
    fixed = max(t1 - per_row * r1, 0.0)
    full = fixed + per_row * L
    return {"value": work.batch * L / full, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "blas_threads": int(threads), "blas": blas, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"oracle.block on {r1} and {r2} sampled query rows of the same input "
                      f"(K/V for all {L} tokens each time; {t1:.1f}s and {t2:.1f}s); full-block time "
                      f"{full:.1f}s extrapolated linearly in the row count"}


def cpu_model() -> str:
    """The host CPU's model name (what lscpu prints as 'Model name')."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def block_gemm_leg(W, B, L, d, F, stream, reps=10):
    """The block's Linear layers on its own kernels (wan_linear_fwd), HIP events
    on the launch stream: Q||K (bf16 out), V^T (the swapped-operand GEMM),
    the d x d out-projection (float32 out, as the residual epilogue), the
    cross-attention query, FFN up (GELU) and FFN down (float32 out)."""
    import torch
    M = B * L
    shapes = [("qk", M, 2 * d, d, 0), ("vt", d, L, d, 0), ("oproj", M, d, d, 1), ("ca_q", M, d, d, 0),
              ("ffn_up", M, F, d, 2), ("ffn_down", M, d, F, 1)]
    g = torch.Generator(device="cpu").manual_seed(11)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res, tot_ms, tot_fl = {}, 0.0, 0.0
    for name, m, n, k, mode in shapes:
        x = torch.randn((m, k), generator=g).to(torch.bfloat16).cuda()
        w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16).cuda()
        b = (torch.randn(n, generator=g) * 0.02).to(torch.bfloat16).cuda()
        y = torch.empty((m, n), dtype=torch.float32 if mode == 1 else torch.bfloat16, device="cuda")
        run = lambda: W.linear_fwd(x, w, b, y, m, n, k, mode, stream)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fl = 2.0 * m * n * k
        mult = 2 if name in ("oproj", "ca_q") else 1      # the block runs two of the d x d shapes each
        tot_ms += ms * mult
        tot_fl += fl * mult
        res[name] = {"M": m, "N": n, "K": k, "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                     "frac": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    return {"kernel": "k_gemm_bf16", "shapes": res, "sum_ms": round(tot_ms, 4),
            "tflops": round(tot_fl / tot_ms / 1e9, 1), "frac": round(tot_fl / tot_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "note": "sum over the block's GEMMs (the d x d projection shape counted for the SA and CA "
                    "out-projections and for the CA query and Q-side shapes it stands for)"}


def ln_leg(W, B, L, d, stream, reps=20):
    """LayerNorm + modulate of the residual stream (wan_ln_modulate_fwd): 4 B
    read + 2 B written per element, against HBM's 8 TB/s."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(13)
    x = torch.randn((B, L, d), generator=g).cuda()
    mod = (torch.randn((B, 6 * d), generator=g) * 0.3).cuda()
    h = torch.empty((B * L, d), dtype=torch.bfloat16, device="cuda")
    run = lambda: W.ln_modulate_fwd(x, B, L, d, mod, 0, 1e-6, h, stream)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    by = 6.0 * B * L * d
    return {"kernel": "k_ln_mod_reg", "ms": round(ms, 4), "bytes": int(by), "gbs": round(by / ms / 1e6, 1),
            "peak_gbs": PEAK_HBM_GBS, "frac": round(by / ms / 1e6 / PEAK_HBM_GBS, 4)}


def step_leg(W, work, steps=2, warmup=1):
    """The full denoising step of a step workload (the 1.3B guidance pair: 30
    blocks, B = 2, L = 32760): wan_dit_step_fwd, weights drawn on the device
    (N(0, 0.02), bf16), HIP events on the launch stream."""
    import torch

    import synth
    m = work.model
    B, L = work.batch, work.L
    cfg = W.make_cfg(dim=m.dim, heads=m.heads, ffn=m.ffn, n_blocks=m.n_blocks, in_ch=m.in_ch,
                     out_ch=m.out_ch, freq_dim=m.freq_dim, text_len=m.text_len, eps=m.eps, dtype=m.dtype)
    mw = synth.device_model_weights(work)
    mws, keep = W.model_weights(mw, [W.block_weights(b) for b in mw["blocks"]])
    inp = synth.workload_inputs(work)
    lat = torch.from_numpy(inp["latent"]).cuda()
    t = torch.from_numpy(inp["t"]).cuda()
    ctx = torch.from_numpy(inp["ctx"]).to(torch.bfloat16).cuda()
    out = torch.empty((B, 16, work.lat_f, work.lat_h, work.lat_w), dtype=torch.float32, device="cuda")
    ws = torch.empty(W.workspace_bytes(cfg, B, work.lat_f, work.lat_h, work.lat_w), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: W.dit_step_fwd(cfg, lat, t, ctx, None, mws, out, ws, stream)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite step output")
    gemm_f, sa_f, ca_f = block_flops(B, L, m.dim, m.heads, m.ffn, m.text_len)
    fl = m.n_blocks * (gemm_f + sa_f + ca_f)
    return {"workload": work.name, "blocks": m.n_blocks, "batch": B, "tokens": L, "steps": steps,
            "ms_per_step": round(ms, 3), "latent_tokens_per_s": round(B * L / (ms * 1e-3), 1),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def traffic_pass(W, B, L, d, H, dev):
    """Kernels for the HBM-traffic counters: the self-attention launch of the
    workload and, as the calibration reference, a plain copy of 512 MiB
    (reads 512 MiB, writes 512 MiB)."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(7)
    qk = (torch.randn((B * L, 2 * d), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    Lp = (L + 63) // 64 * 64
    vt = torch.randn((d, B * Lp), generator=g).to(torch.bfloat16).to(dev)
    o = torch.empty((B * L, d), dtype=torch.bfloat16, device=dev)
    src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        W.attention_fwd(qk, 2 * d, qk[:, d:], 2 * d, vt, B * Lp, Lp, o, d, B, H, L, L, q_scaled=True)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_pass": "done", "copy_bytes": 512 << 20}), flush=True)


def sampler_bench(n_steps: int, warmup: int):
    """Sampler steps of the 1.3B guidance pair at 480P (30 blocks, B = 2:
    conditional and unconditional contexts, one latent): wan_sample_fwd with
    the cross-attention K/V cache against the plain path (wan_dit_step_fwd,
    which projects the text K/V in every block, + wan_euler_fwd)."""
    import torch

    import synth
    import video_diffusion_transformer_block_amd as W
    work = synth.WORKLOADS["wan1.3b-step-480p-cfg2"]
    m = work.model
    B, L = work.batch, work.L
    cfg = W.make_cfg(dim=m.dim, heads=m.heads, ffn=m.ffn, n_blocks=m.n_blocks, in_ch=m.in_ch,
                     out_ch=m.out_ch, freq_dim=m.freq_dim, text_len=m.text_len, eps=m.eps,
                     dtype=m.dtype)
    mw = synth.device_model_weights(work)
    mws, keep = W.model_weights(mw, [W.block_weights(b) for b in mw["blocks"]])
    inp = synth.workload_inputs(work)
    lat0 = torch.from_numpy(inp["latent"][:1].repeat(B, 0)).cuda()
    ctx = torch.from_numpy(inp["ctx"]).to(torch.bfloat16).cuda()
    ws = torch.empty(W.sample_workspace_bytes(cfg, B, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    cache = torch.empty(W.kv_cache_bytes(cfg, B), dtype=torch.uint8, device="cuda")
    vel = torch.empty((B, 16) + tuple(lat0.shape[2:]), dtype=torch.float32, device="cuda")
    tb = torch.zeros(B, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        torch.cuda.synchronize()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    fill_ms = [timed(lambda: W.kv_cache_fwd(cfg, B, ctx, None, mws, cache, ws, stream))
               for _ in range(3)][-1]
    lat = lat0.clone()
    W.sample_fwd(cfg, lat, warmup, cache, mws, ws, True, 5.0, stream)
    lat = lat0.clone()
    cached_ms = timed(lambda: W.sample_fwd(cfg, lat, n_steps, cache, mws, ws, True, 5.0, stream))

    def plain():
        for k in range(n_steps):
            tb.fill_(1000.0 * k / n_steps)
            W.dit_step_fwd(cfg, lat, tb, ctx, None, mws, vel, ws, stream)
            W.euler_fwd(lat, vel, 1.0 / n_steps, True, 5.0, stream)

    lat = lat0.clone()
    plain_ms = timed(plain)
    if not bool(torch.isfinite(lat).all()):
        raise RuntimeError("non-finite sample")
    # the same cached sampler with every block in FP8 (weights quantised once, outside the timing)
    qbuf = torch.empty(W.model_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
    quant_ms = timed(lambda: W.quantize_model_fp8(cfg, mws, qbuf, stream))
    ws8 = torch.empty(W.fp8_workspace_bytes(cfg, B, work.lat_f, work.lat_h, work.lat_w, True),
                      dtype=torch.uint8, device="cuda")
    lat = lat0.clone()
    W.sample_fp8_fwd(cfg, lat, warmup, cache, mws, qbuf, ws8, True, 5.0, stream)
    lat = lat0.clone()
    fp8_ms = timed(lambda: W.sample_fp8_fwd(cfg, lat, n_steps, cache, mws, qbuf, ws8, True, 5.0, stream))
    if not bool(torch.isfinite(lat).all()):
        raise RuntimeError("non-finite FP8 sample")
    # ... and with every block's self-attention in 8 bits as well (cfg attn8)
    cfg8 = W.make_cfg(dim=m.dim, heads=m.heads, ffn=m.ffn, n_blocks=m.n_blocks, in_ch=m.in_ch,
                      out_ch=m.out_ch, freq_dim=m.freq_dim, text_len=m.text_len, eps=m.eps,
                      dtype=m.dtype, attn8=True)
    del ws8
    ws8 = torch.empty(W.fp8_workspace_bytes(cfg8, B, work.lat_f, work.lat_h, work.lat_w, True),
                      dtype=torch.uint8, device="cuda")
    lat = lat0.clone()
    W.sample_fp8_fwd(cfg8, lat, warmup, cache, mws, qbuf, ws8, True, 5.0, stream)
    lat = lat0.clone()
    a8_ms = timed(lambda: W.sample_fp8_fwd(cfg8, lat, n_steps, cache, mws, qbuf, ws8, True, 5.0, stream))
    if not bool(torch.isfinite(lat).all()):
        raise RuntimeError("non-finite FP8 + 8-bit attention sample")
    per_c, per_p, per_8, per_a8 = cached_ms / n_steps, plain_ms / n_steps, fp8_ms / n_steps, a8_ms / n_steps
    print(json.dumps({
        "sampler": "wan1.3b-480p guidance pair (30 blocks, B=2, L=32760, 512 text tokens)",
        "steps": n_steps, "guidance": 5.0,
        "ms_per_step_cached": round(per_c, 3), "ms_per_step_plain": round(per_p, 3),
        "kv_cache_fill_ms": round(fill_ms, 3),
        "saving_per_step_ms": round(per_p - per_c, 3),
        "latent_tokens_per_s_cached": round(B * L / (per_c * 1e-3), 1),
        "ms_per_step_cached_fp8_blocks": round(per_8, 3), "fp8_speedup": round(per_c / per_8, 4),
        "fp8_weight_quantisation_ms": round(quant_ms, 3),
        "ms_per_step_cached_fp8_attn8": round(per_a8, 3), "fp8_attn8_speedup": round(per_c / per_a8, 4),
        "dtype": "bf16 (and fp8 e4m3 block Linear layers; and 8-bit self-attention)",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) latent and text)",
    }), flush=True)


def gemm_bench(reps: int):
    """The block's Linear layers of the 1.3B model at 480P (M = 32760 tokens) in
    bf16 (wan_linear_fwd) and FP8 (wan_linear_fp8_fwd on operands quantised
    beforehand; the per-token quantisation of the activations is timed on its
    own).  Seeded N(0, 1) activations, N(0, 0.02) weights."""
    import torch

    import video_diffusion_transformer_block_amd as W
    M = 32760
    shapes = [("qk", 3072, 1536, 0), ("oproj", 1536, 1536, 1), ("ffn_up", 8960, 1536, 2),
              ("ffn_down", 1536, 8960, 1)]
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    g = torch.Generator(device="cpu").manual_seed(11)
    res = {}
    for name, N, K, mode in shapes:
        x = torch.randn((M, K), generator=g).to(torch.bfloat16).cuda()
        w = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16).cuda()
        b = (torch.randn(N, generator=g) * 0.02).to(torch.bfloat16).cuda()
        y = torch.empty((M, N), dtype=torch.float32 if mode == 1 else torch.bfloat16, device="cuda")
        qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sx = torch.empty(M, dtype=torch.float32, device="cuda")
        qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sw = torch.empty(1, dtype=torch.float32, device="cuda")
        W.quantize_tensor_fp8(w, qw, sw, torch.empty(256, dtype=torch.uint8, device="cuda"), stream)
        W.quantize_rows_fp8(x, qx, sx, stream)
        fl = 2.0 * M * N * K
        ms_bf = timed(lambda: W.linear_fwd(x, w, b, y, M, N, K, mode, stream))
        ms_f8 = timed(lambda: W.linear_fp8_fwd(qx, sx, qw, sw, b, y, M, N, K, mode, stream))
        ms_q = timed(lambda: W.quantize_rows_fp8(x, qx, sx, stream))
        res[name] = {"M": M, "N": N, "K": K,
                     "bf16_ms": round(ms_bf, 4), "bf16_tflops": round(fl / ms_bf / 1e9, 1),
                     "fp8_ms": round(ms_f8, 4), "fp8_tflops": round(fl / ms_f8 / 1e9, 1),
                     "fp8_frac_of_fp8_peak": round(fl / ms_f8 / 1e9 / PEAK_FP8_TFLOPS, 4),
                     "quant_rows_ms": round(ms_q, 4),
                     "quant_rows_gbs": round(M * K * 3 / ms_q / 1e6, 1)}
    print(json.dumps({"gemm": "1.3B block Linear layers at 480P, bf16 vs FP8 (E4M3)",
                      "shapes": res, "peak_bf16_tflops": PEAK_BF16_TFLOPS,
                      "peak_fp8_tflops": PEAK_FP8_TFLOPS, "data": "synthetic"}), flush=True)


def fp8_block_bench(steps: int, warmup: int):
    """The 1.3B block at 480P (L = 32760) with bf16 Linear layers
    (wan_dit_block_fwd) and with E4M3 ones (wan_dit_block_fp8_fwd, weights
    quantised once beforehand, activation quantisation inside the timed
    region), same weights and inputs."""
    import numpy as np
    import torch

    import synth
    import video_diffusion_transformer_block_amd as W
    work = synth.WORKLOADS["wan1.3b-block-480p"]
    m = work.model
    B, L, d = work.batch, work.L, m.dim
    cfg = W.make_cfg(dim=d, heads=m.heads, ffn=m.ffn, n_blocks=1, text_len=m.text_len, eps=m.eps,
                     dtype="bf16")
    inp = synth.workload_inputs(work)
    bw = synth.block_weights(work, 0)

    def up(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
        return (t.to(torch.bfloat16) if dt == "bf16" else t).cuda()

    bwd = {k: up(v, "f32" if k == "mod_bias" else "bf16") for k, v in bw.items()}
    desc = W.block_weights(bwd)
    x0 = up(inp["x"], "f32")
    x = x0.clone()
    ctx = up(inp["ctx"], "bf16")
    mod = (torch.randn((B, 6 * d), generator=torch.Generator().manual_seed(5)) * 0.3).cuda()
    stream = torch.cuda.current_stream()
    qbuf = torch.empty(W.block_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
    W.quantize_block_fp8(cfg, desc, qbuf, stream)
    ws = torch.empty(W.block_fp8_workspace_bytes(cfg, B, work.lat_f, work.Hp, work.Wp),
                     dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        x.copy_(x0)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    geo = (B, work.lat_f, work.Hp, work.Wp)
    ms_bf = timed(lambda: W.dit_block_fwd(cfg, x, *geo, mod, desc, ctx, None, ws, stream))
    ms_f8 = timed(lambda: W.dit_block_fp8_fwd(cfg, x, *geo, mod, desc, qbuf, ctx, None, ws, stream))
    if not bool(torch.isfinite(x).all()):
        raise RuntimeError("non-finite FP8 block output")
    print(json.dumps({"fp8_block": f"{work.name}: bf16 vs FP8 (E4M3) Linear layers",
                      "tokens": B * L, "steps": steps, "warmup": warmup,
                      "bf16_ms": round(ms_bf, 4), "fp8_ms": round(ms_f8, 4),
                      "speedup": round(ms_bf / ms_f8, 4),
                      "fp8_tokens_per_s": round(B * L / (ms_f8 * 1e-3), 1), "data": "synthetic"}),
          flush=True)


def fp8_block_leg(W, cfg, work, bwd, mod, ctx, stream, steps, warmup, bf16_ms, tmlp,
                  label="fp8 e4m3 Linear layers, bf16 attention"):
    """Time the step with wan_dit_block_fp8_fwd in place of the bf16 block (the
    same t-MLP call first; weights quantised once beforehand; the per-token
    activation quantisation is inside the timed region), on its own copy of
    the residual stream.  With cfg.attn8 the self-attention runs in 8 bits
    (its Int8 / E4M3 quantisation inside the timed region too)."""
    import torch
    desc = W.block_weights(bwd)
    qbuf = torch.empty(W.block_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
    W.quantize_block_fp8(cfg, desc, qbuf, stream)
    ws = torch.empty(W.block_fp8_workspace_bytes(cfg, work.batch, work.lat_f, work.Hp, work.Wp),
                     dtype=torch.uint8, device="cuda")
    x = torch.randn((work.batch, work.L, cfg.dim), generator=torch.Generator().manual_seed(3)).cuda()
    geo = (work.batch, work.lat_f, work.Hp, work.Wp)
    def step8():
        tmlp()
        W.dit_block_fp8_fwd(cfg, x, *geo, mod, desc, qbuf, ctx, None, ws, stream)

    for _ in range(max(1, warmup)):
        step8()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step8()
    e1.record(stream)
    torch.cuda.synchronize()
    ms8 = e0.elapsed_time(e1) / steps
    if not bool(torch.isfinite(x).all()):
        raise RuntimeError("non-finite FP8 block output")
    return {"ms_per_step": round(ms8, 4), "tokens_per_s": round(work.batch * work.L / (ms8 * 1e-3), 1),
            "speedup_vs_bf16": round(bf16_ms / ms8, 4), "dtype": label}


def attn8_leg(W, B, L, d, H, qk, vt, Lp, stream, n_att, bf16_attn_ms, sa_f):
    """The 8-bit self-attention kernel on its own (Int8 / E4M3 copies of the
    same q, k, V^T made once), timed with HIP events on the launch stream,
    and the three quantisers it needs, timed separately."""
    import torch
    D, nkb = H * 128, Lp // 64
    q8 = torch.empty((B * L, D), dtype=torch.int8, device="cuda")
    qs = torch.empty((B * L, H), dtype=torch.float32, device="cuda")
    k8 = torch.empty((B * L, D), dtype=torch.int8, device="cuda")
    ks = torch.empty((B, H, nkb), dtype=torch.float32, device="cuda")
    v8 = torch.empty((D, B * Lp), dtype=torch.uint8, device="cuda")
    vs = torch.empty((B, D), dtype=torch.float32, device="cuda")
    o = torch.empty((B * L, d), dtype=torch.bfloat16, device="cuda")
    quant = lambda: W.attention_8bit_quantize(qk, 2 * d, qk[:, d:], 2 * d, vt, B * Lp, Lp, B, H, L, L, q8, qs,
                                              k8, ks, v8, vs, stream)
    run = lambda: W.attention_8bit_q_fwd(q8, qs, k8, ks, v8, vs, o, d, B, H, L, L, q_scaled=True,
                                         stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, f in (("quant", quant), ("attn", run)):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_att):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / n_att
    if not bool(torch.isfinite(o.float()).all()):
        raise RuntimeError("non-finite 8-bit attention output")
    tf = sa_f / (res["attn"] * 1e-3) / 1e12
    return {"kernel": "k_attn_i8f8", "launch_ms": round(res["attn"], 4), "tflops": round(tf, 1),
            "peak": PEAK_FP8_TFLOPS, "frac_of_8bit_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "quantise_ms": round(res["quant"], 4),
            "speedup_vs_bf16_attention": round(bf16_attn_ms / res["attn"], 4),
            "speedup_incl_quantise": round(bf16_attn_ms / (res["attn"] + res["quant"]), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", type=int, default=2,
                    help="block workload id (2: wan1.3b-block-480p, 4: wan14b-block-720p)")
    ap.add_argument("--sampler", type=int, default=0, metavar="STEPS",
                    help="time STEPS sampler steps of the 1.3B guidance pair with and without the "
                         "cross-attention K/V cache (prints its own JSON line) instead of the block")
    ap.add_argument("--gemm", action="store_true",
                    help="time the block's Linear layers in bf16 and FP8 (prints its own JSON line)")
    ap.add_argument("--fp8-block", action="store_true",
                    help="time the 1.3B block with bf16 and with FP8 Linear layers "
                         "(prints its own JSON line)")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="only run 3 self-attention launches and 3 plain 512-MiB device copies "
                         "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE and their calibration)")
    args = ap.parse_args()
    if args.traffic_pass:
        args.no_cpu_baseline = True
        args.warmup, args.steps = 1, 1
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    if args.sampler:
        sampler_bench(args.sampler, max(1, args.warmup))
        return
    if args.gemm:
        gemm_bench(10)
        return
    if args.fp8_block:
        fp8_block_bench(args.steps, max(1, args.warmup))
        return

    import numpy as np
    import torch

    import synth
    import video_diffusion_transformer_block_amd as W

    work = synth.by_id(args.config)
    assert work.kind == "block"
    m = work.model
    B, L, d, H, F = work.batch, work.L, m.dim, m.heads, m.ffn
    dev = "cuda"
    cfg = W.make_cfg(dim=d, heads=H, ffn=F, n_blocks=1, text_len=m.text_len, eps=m.eps,
                     dtype=m.dtype)

    inp = synth.workload_inputs(work)
    tw = synth.tmlp_weights(work)
    bw = synth.block_weights(work, 0)

    def up(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
        return (t.to(torch.bfloat16) if dt == "bf16" else t).to(dev)

    twd = {k: up(v, m.dtype) for k, v in tw.items()}
    bwd = {k: up(v, "f32" if k == "mod_bias" else m.dtype) for k, v in bw.items()}
    x = up(inp["x"], "f32")
    t = up(inp["t"], "f32")
    ctx = up(inp["ctx"], m.dtype)
    mod = torch.empty((B, 6 * d), dtype=torch.float32, device=dev)
    ws = torch.empty(W.workspace_bytes(cfg, B, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device=dev)
    tws = torch.empty(B * (d + m.freq_dim) * 4, dtype=torch.uint8, device=dev)
    tws_c, bws_c = W.tmlp_weights(twd), W.block_weights(bwd)
    stream = torch.cuda.current_stream()

    def step():
        W.tmlp_fwd(cfg, t, tws_c, mod, tws, stream)
        W.dit_block_fwd(cfg, x, B, work.lat_f, work.Hp, work.Wp, mod, bws_c, ctx, None, ws, stream)

    for _ in range(args.warmup):
        step()
    # events the library records around each timed step's self-attention launch
    # (wan_set_attention_events): the dominant kernel timed inside the timed region
    sa_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for a, b in sa_ev:      # a first record creates the underlying events
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clock:
        e0.record(stream)
        t_wall = time.perf_counter()
        for i in range(args.steps):
            W.set_attention_events(*sa_ev[i])
            step()
        e1.record(stream)
        W.set_attention_events(None, None)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    sa_ms = [a.elapsed_time(b) for a, b in sa_ev]
    attn_block_ms = sum(sa_ms) / len(sa_ms)
    if not all(math.isfinite(v) for v in x[0, :4, :4].flatten().tolist()):
        raise RuntimeError("non-finite block output")

    if args.traffic_pass:
        traffic_pass(W, B, L, d, H, dev)
        return
    # ---- the dominant kernel (self-attention), timed on its own stream with HIP events
    hd = d // H
    g = torch.Generator(device="cpu").manual_seed(7)
    qk = (torch.randn((B * L, 2 * d), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    Lp = (L + 63) // 64 * 64
    vt = torch.randn((d, B * Lp), generator=g).to(torch.bfloat16).to(dev)
    o = torch.empty((B * L, d), dtype=torch.bfloat16, device=dev)

    def attn():
        # queries pre-scaled by log2(e)/sqrt(hd), as the block's Q projection writes them
        W.attention_fwd(qk, 2 * d, qk[:, d:], 2 * d, vt, B * Lp, Lp, o, d, B, H, L, L, stream,
                        q_scaled=True)

    for _ in range(2):
        attn()
    n_att = max(3, args.steps // 2)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n_att):
        attn()
    e1.record(stream)
    torch.cuda.synchronize()
    attn_ms = e0.elapsed_time(e1) / n_att

    gemm_f, sa_f, ca_f = block_flops(B, L, d, H, F, m.text_len)
    attn_tf = sa_f / (attn_block_ms * 1e-3) / 1e12
    attn_solo_tf = sa_f / (attn_ms * 1e-3) / 1e12
    block_tf = (gemm_f + sa_f + ca_f) / (ms * 1e-3) / 1e12
    tokens_s = B * L / (ms * 1e-3)

    out = {
        "metric": "DiT block tokens/s + attn TFLOP/s (% bf16 MFMA peak), 1.3B @ 480P L=32760"
                  if args.config == 2 else f"DiT block tokens/s + attn TFLOP/s (% bf16 MFMA peak), {work.name}",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {"workload": work.name, "batch": B, "latent": [16, work.lat_f, work.lat_h, work.lat_w],
                   "tokens": L, "dim": d, "heads": H, "ffn": F, "text_tokens": m.text_len},
        "attn_tflops": round(attn_tf, 1),
        "attn_frac_of_peak": round(attn_tf / PEAK_BF16_TFLOPS, 4),
        "block_tflops": round(block_tf, 1),
        "block_frac_of_peak": round(block_tf / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "k_attn_bf16", "achieved": round(attn_tf, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4), "traffic": attn_traffic_bytes() if args.config == 2 else None,
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 counters, copy-calibrated)",
                     "algorithmic_bytes": 4 * B * L * d * 2,
                     "launch_ms": round(attn_block_ms, 4),
                     "launch_ms_where": "the timed steps' own self-attention launches (HIP events the "
                                        "library records around them on the launch stream)",
                     "launches": len(sa_ms),
                     "standalone_launch_ms": round(attn_ms, 4),
                     "standalone_tflops": round(attn_solo_tf, 1),
                     "flop_per_launch": sa_f,
                     # the same against the peak at the shader clock sampled during the timed steps
                     **clock_fields(clock, attn_tf)},
        "wall_s_timed": round(t_wall, 3),
    }
    if m.dtype == "bf16":   # the same block with its six Linear layers in FP8 (E4M3), same inputs
        tm = lambda: W.tmlp_fwd(cfg, t, tws_c, mod, tws, stream)
        out["fp8_block"] = fp8_block_leg(W, cfg, work, bwd, mod, ctx, stream, args.steps, args.warmup, ms, tm)
        # ... and with the 8-bit self-attention as well
        cfg8 = W.make_cfg(dim=d, heads=H, ffn=F, n_blocks=1, text_len=m.text_len, eps=m.eps, dtype=m.dtype,
                          attn8=True)
        out["fp8_attn8_block"] = fp8_block_leg(W, cfg8, work, bwd, mod, ctx, stream, args.steps, args.warmup,
                                               ms, tm, "fp8 e4m3 Linear layers, 8-bit self-attention "
                                                       "(Int8 QK^T, E4M3 PV)")
        out["attn8"] = attn8_leg(W, B, L, d, H, qk, vt, Lp, stream, n_att, attn_ms, sa_f)
    out["gemm"] = block_gemm_leg(W, B, L, d, F, stream)
    out["ln_modulate"] = ln_leg(W, B, L, d, stream)
    if args.config == 2:
        out["c3_step"] = step_leg(W, synth.WORKLOADS["wan1.3b-step-480p-cfg2"])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(work, inp, tw, bw)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
