#!/usr/bin/env python3
"""Throughput of one classifier-free-guided denoising step of the 48-block
Lens MM-DiT at 1024x1024 (64 x 64 = 4096 image tokens + 512 text tokens) on
one MI355X.

A step is the whole hot path: lens_dit_forward on a batch of 2 (cond and
uncond samples sharing x and t: timestep MLP, AdaLN of all blocks, img_in,
txt_norm + txt_in, 48 double-stream blocks, norm_out + proj_out) followed by
lens_flow_step_rescaled (Lens's norm-rescaled CFG at scale 5.0 + Euler
update + bf16 copy of x for the next forward).  Weights are random-init bf16 (N(0, 0.02)), inputs are seeded
synthetic tensors of the real shapes, and everything is resident in HBM
before the timed region starts.

Prints one JSON line.  `value` is achieved TFLOP/s over the whole step
(algorithmic FLOPs: 2 M N K per GEMM, 4 S_q S_kv d H for attention over
valid keys).  A second timed region records HIP events around every kernel
launch (the library's opt-in timer) for the per-family breakdown and the
roofline of the dominant kernel family.  `cpu_baseline` times the fp64
oracle on a bounded sample (one block at the same shape) on the host cores.
`fp8_variant` times the same step with the block projections as MX fp8
GEMMs (weights quantized on the device from the same bf16 weights) and
reports the cosine of its velocity against the bf16 step's on one input.
`turbo_1440` times a second workload: whole 4-step Turbo-style sampling
jobs at 1440x1440 (90 x 90 = 8100 image tokens + 512 text tokens, batch 1,
no CFG), with its own kernel breakdown and roofline.  `value` is always the
bf16 1024x1024 CFG step.
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

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published

S_IMG, S_TXT, GRID = 4096, 512, (64, 64)
CFG_SCALE = 5.0
LOOP_STEPS = 20
# Turbo-style sampling at 1440^2: 90 x 90 image tokens + 512 text tokens,
# batch 1, 4 Euler steps, no CFG (guidance 1.0)
TURBO_GRID, TURBO_TXT, TURBO_STEPS = (90, 90), 512, 4


def block_flops(d, S_img, S_txt, B, q_valid=None, kv_valid=None):
    """Algorithmic FLOPs of one block for B samples (AdaLN included)."""
    D, F, H = d.hidden, d.mlp, d.heads
    gemm = 0
    for S in (S_img, S_txt):
        gemm += 2 * B * S * D * (3 * D + D + 2 * F) + 2 * B * S * F * D
    adaln = 2 * 2 * B * D * 6 * D
    Sq = S_img + S_txt if q_valid is None else q_valid
    Skv = S_img + S_txt if kv_valid is None else kv_valid
    attn = 4 * B * Sq * Skv * d.head_dim * H
    return gemm, attn, adaln


def sclk_mhz():
    """Current shader clock from the amdgpu driver's pp_dpm_sclk (the line
    marked '*'), or None where the file is not readable."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            text = open(path).read()
        except OSError:
            continue
        for line in text.splitlines():
            if line.rstrip().endswith("*"):
                m = re.search(r"(\d+)\s*[Mm]hz", line)
                if m:
                    return int(m.group(1))
    return None


def step_flops(d, S_img, S_txt, B):
    g, a, m = block_flops(d, S_img, S_txt, B)
    D = d.hidden
    emb = 2 * B * (S_img * d.in_ch * D + S_txt * d.txt_layers * d.txt_feat * D + S_img * D * d.out_ch)
    tmlp = 2 * B * (d.t_freq * D + D * D + D * 2 * D)
    return {"gemm_blocks": d.n_blocks * g, "attention": d.n_blocks * a, "adaln": d.n_blocks * m,
            "gemm_embed": emb, "small": tmlp,
            "total": d.n_blocks * (g + a + m) + emb + tmlp}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_dit_step_1024_traffic.md")
GEMM_SRC = os.path.join(ROOT, "text_image_flow_amd", "csrc", "gemm.hip")


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when that summary is missing or was taken on
    a different GEMM source than the one built now."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in text.splitlines() if l.startswith(("traffic_bytes_per_launch:", "gemm_source_sha256:")))
    if not fields:
        return None
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    if fields.get("gemm_source_sha256", "").strip() != sha:
        return None
    return float(fields["traffic_bytes_per_launch"])


def family_roofline(L, ms, n, steps, fam_flops):
    """Per-family breakdown from the library's kernel timer and the
    roofline of the dominant MFMA family (gemm or attention)."""
    kernels = {}
    for i, name in enumerate(L.KERNEL_NAMES):
        if n[i] == 0:
            continue
        e = {"ms_per_step": round(ms[i] / steps, 4), "launches_per_step": n[i] // steps,
             "avg_launch_us": round(1e3 * ms[i] / n[i], 2)}
        if name in fam_flops:
            e["TFLOP/s"] = round(fam_flops[name] / (ms[i] / steps * 1e-3) / 1e12, 1)
        kernels[name] = e
    dom = max(("gemm", "attention"), key=lambda k: kernels.get(k, {}).get("ms_per_step", 0))
    i = L.KERNEL_NAMES.index(dom)
    per_launch_flops = fam_flops[dom] / (n[i] / steps)
    avg_s = ms[i] / n[i] * 1e-3
    ach = per_launch_flops / avg_s / 1e12
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flops_per_launch": per_launch_flops, "avg_launch_us": round(avg_s * 1e6, 2)}
    return kernels, roof


def turbo_sampling(d, cfg, dit, jobs, warmup, timer):
    """One 1440^2 Turbo-style sampling job per repetition: 4 x
    (lens_dit_forward at B = 1 + lens_flow_step without CFG) from the same
    seeded latent, uniform time grid; inputs resident before timing."""
    import torch
    import synth
    import text_image_flow_amd as T
    from text_image_flow_amd import _lib as L
    from text_image_flow_amd import device as dv
    gh, gw = TURBO_GRID
    S = gh * gw
    x0 = synth.latents(1, S, d)
    x_init = dv.upload(x0)
    x = x_init.clone()
    x_act = dv.upload(synth.bf16_round(x0), T.LENS_BF16)
    x_act_init = x_act.clone()
    feats = dv.upload(synth.text_features(1, TURBO_TXT, d, seed=synth.SEED_TEXT_COND), T.LENS_BF16)
    ip, tp = dv.upload(synth.image_positions(gh, gw)), dv.upload(synth.text_positions(TURBO_TXT))
    ts, dts = dv.time_grid(TURBO_STEPS)
    t_tab = dv.upload(ts[:, None].copy())
    v = torch.empty((1, S, d.out_ch), dtype=torch.float32, device="cuda")
    ws = dv.Workspace()
    ws.get(T.lens_dit_workspace_bytes(cfg, 1, S, TURBO_TXT))
    torch.cuda.synchronize()

    def job():
        x.copy_(x_init)
        x_act.copy_(x_act_init)
        for k in range(TURBO_STEPS):
            dv.dit_forward(cfg, dit, x_act, feats, t_tab[k], ip, tp, None, v, ws)
            dv.flow_step(x, v, None, float(dts[k]), 1.0, x_act, T.LENS_BF16)

    for _ in range(warmup):
        job()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(jobs):
        job()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_job = e0.elapsed_time(e1) / jobs
    assert torch.isfinite(x).all().item(), "non-finite Turbo output"
    fl = step_flops(d, S, TURBO_TXT, 1)
    out = {"workload": "Lens MM-DiT Turbo-style sampling, 1440x1440", "image_tokens": S, "text_tokens": TURBO_TXT,
           "batch": 1, "steps": TURBO_STEPS, "cfg": "none (guidance 1.0)", "jobs_timed": jobs,
           "ms_per_job": round(ms_job, 3), "ms_per_step": round(ms_job / TURBO_STEPS, 3),
           "TFLOP/s": round(fl["total"] * TURBO_STEPS / (ms_job * 1e-3) / 1e12, 2),
           "pct_of_bf16_peak": round(100 * fl["total"] * TURBO_STEPS / (ms_job * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "flops_per_step": fl["total"], "kernels": None, "roofline": None}
    if timer:
        L.check(T.lens_timer_start((1 << L.LENS_KERNEL_COUNT) - 1))
        torch.cuda.synchronize()
        job()
        torch.cuda.synchronize()
        st, ms, n = T.lens_timer_stop()
        L.check(st)
        fam = {"gemm": fl["gemm_blocks"] + fl["gemm_embed"], "attention": fl["attention"],
               "adaln": fl["adaln"] + fl["small"]}
        out["kernels"], out["roofline"] = family_roofline(L, ms, n, TURBO_STEPS, fam)
    return out


def cpu_baseline(d):
    """The oracle as it stands, on one block at 1024^2 (B = 1), fp64."""
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = synth.block_weights(0, dtype="bf16")
    hi, ht, temb = synth.block_inputs(1, S_IMG, S_TXT, dtype="bf16")
    ip, tp = synth.image_positions(*GRID), synth.text_positions(S_TXT)
    t0 = time.perf_counter()
    O.block_forward(w, hi, ht, temb, ip, tp, None)
    dt = time.perf_counter() - t0
    g, a, m = block_flops(d, S_IMG, S_TXT, 1)
    return {"value": round((g + a + m) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"oracle.block_forward: one block at 1024^2 (4096 image + 512 text tokens), B=1, fp64 numpy, "
                      f"{dt:.2f} s for {(g + a + m) / 1e9:.1f} GFLOP; host os.cpu_count()={os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timer", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the MX fp8 variant")
    ap.add_argument("--no-b1", action="store_true",
                    help="skip the B = 1 forward and the clock-sampling pass (profiles of the B = 2 step alone)")
    ap.add_argument("--no-turbo", action="store_true", help="skip the 1440^2 Turbo-style sampling workload")
    ap.add_argument("--copy-kernel-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path has no multi-GPU part (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_kernel_bytes:
        n = args.copy_kernel_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel_bytes": n * 4, "launches": 3}))
        return

    import synth
    import text_image_flow_amd as T
    from text_image_flow_amd import _lib as L
    from text_image_flow_amd import device as dv

    dv.require_gpu()
    torch.cuda.set_device(0)
    d = synth.LENS
    cfg = T.default_config(T.LENS_BF16)
    B = 2

    # ---- weights and inputs, resident in HBM before timing
    t_setup = time.perf_counter()
    top = synth.top_weights(d)
    blocks = [dv.DeviceBlock(w, T.LENS_BF16) for _, w in synth.all_block_weights(d, threads=16)]
    dit = dv.DeviceDit(top, blocks, T.LENS_BF16)
    x0 = synth.latents(1, S_IMG, d)
    x = dv.upload(x0)                                                   # f32 latent tokens [1, S, 128]
    x_act = dv.upload(np.concatenate([synth.bf16_round(x0)] * B), T.LENS_BF16)
    feats = dv.upload(np.concatenate([synth.text_features(1, S_TXT, d, seed=synth.SEED_TEXT_COND),
                                      synth.text_features(1, S_TXT, d, seed=synth.SEED_TEXT_UNCOND)]), T.LENS_BF16)
    ip, tp = dv.upload(synth.image_positions(*GRID)), dv.upload(synth.text_positions(S_TXT))
    ts, dts = dv.time_grid(LOOP_STEPS)
    t_tab = dv.upload(np.repeat(ts[:, None], B, axis=1))
    v = torch.empty((B, S_IMG, d.out_ch), dtype=torch.float32, device="cuda")
    ws = dv.Workspace()
    ws.get(T.lens_dit_workspace_bytes(cfg, B, S_IMG, S_TXT))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    k_state = [0]
    model = [cfg, dit]

    def step():
        k = k_state[0] % LOOP_STEPS
        k_state[0] += 1
        dv.dit_forward(model[0], model[1], x_act, feats, t_tab[k], ip, tp, None, v, ws)
        dv.flow_step_rescaled(x, v[:1], v[1:], float(dts[k]), CFG_SCALE, x_act[:1], T.LENS_BF16)
        x_act[1:].copy_(x_act[:1])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(v).all().item() and torch.isfinite(x).all().item(), "non-finite output"

    fl = step_flops(d, S_IMG, S_TXT, B)
    tflops = fl["total"] / (ms_step * 1e-3) / 1e12

    # ---- B = 1 forward (the cond half alone), same weights and shapes
    fl1 = step_flops(d, S_IMG, S_TXT, 1)["total"]
    b1, clock = None, None
    for _ in range(0 if args.no_b1 else args.warmup):
        dv.dit_forward(cfg, dit, x_act[:1], feats[:1], t_tab[0][:1], ip, tp, None, v[:1], ws)
    torch.cuda.synchronize()
    if not args.no_b1:
        e0.record(stream)
        for k in range(args.steps):
            dv.dit_forward(cfg, dit, x_act[:1], feats[:1], t_tab[k % LOOP_STEPS][:1], ip, tp, None, v[:1], ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_b1 = e0.elapsed_time(e1) / args.steps
        b1 = {"ms": round(ms_b1, 3), "TFLOP/s": round(fl1 / (ms_b1 * 1e-3) / 1e12, 2),
              "pct_of_bf16_peak": round(100 * fl1 / (ms_b1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2), "flops": fl1}

    # ---- shader clock while the same steps run (sampled in a separate,
    # untimed pass so the sampling thread cannot delay the timed launches)
    if not args.no_b1 and sclk_mhz() is not None:
        import threading
        samples, done = [], threading.Event()

        def sampler():
            while not done.is_set():
                c = sclk_mhz()
                if c is not None:
                    samples.append(c)
                time.sleep(0.02)

        th = threading.Thread(target=sampler, daemon=True)
        th.start()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        done.set()
        th.join()
        if samples:
            med = sorted(samples)[len(samples) // 2]
            clock = {"sclk_mhz_median": med, "sclk_mhz_min": min(samples), "sclk_mhz_max": max(samples),
                     "samples": len(samples), "source": "amdgpu pp_dpm_sclk current level, sampled every 20 ms "
                                                        "during an untimed pass of the same steps",
                     "pct_of_bf16_peak_at_measured_clock": round(100 * tflops / (PEAK_BF16_TFLOPS * med / 2400.0), 2)}

    # ---- second timed region: per-family kernel timing with HIP events
    kernels, roof = {}, None
    if not args.no_kernel_timer:
        L.check(T.lens_timer_start((1 << L.LENS_KERNEL_COUNT) - 1))
        torch.cuda.synchronize()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        st, ms, n = T.lens_timer_stop()
        L.check(st)
        fam_flops = {"gemm": fl["gemm_blocks"] + fl["gemm_embed"], "attention": fl["attention"],
                     "adaln": fl["adaln"] + fl["small"]}
        kernels, roof = family_roofline(L, ms, n, args.steps, fam_flops)
        roof["traffic"] = measured_traffic() if roof["kernel"] == "gemm" else None

    # ---- MX fp8 variant of the same step (not the headline value)
    fp8 = None
    if not args.no_fp8:
        cfg8 = T.default_config(T.LENS_BF16)
        cfg8.gemm_fp8 = 1
        dit8 = dv.DeviceDit(top, [dv.DeviceBlock.fp8_copy(b) for b in blocks], T.LENS_BF16)
        ws.get(T.lens_dit_workspace_bytes(cfg8, B, S_IMG, S_TXT))
        # velocity of both variants on the current input
        va = torch.empty_like(v)
        dv.dit_forward(cfg, dit, x_act, feats, t_tab[0], ip, tp, None, va, ws)
        dv.dit_forward(cfg8, dit8, x_act, feats, t_tab[0], ip, tp, None, v, ws)
        torch.cuda.synchronize()
        a, b8 = va.double().flatten(), v.double().flatten()
        cosv = float((a @ b8) / (a.norm() * b8.norm()))
        model[:] = [cfg8, dit8]
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms8 = e0.elapsed_time(e1) / args.steps
        fk = {}
        if not args.no_kernel_timer:
            L.check(T.lens_timer_start((1 << L.LENS_KERNEL_COUNT) - 1))
            for _ in range(args.steps):
                step()
            torch.cuda.synchronize()
            st8, ms_k, n_k = T.lens_timer_stop()
            L.check(st8)
            for i, name in enumerate(L.KERNEL_NAMES):
                if n_k[i]:
                    fk[name] = {"ms_per_step": round(ms_k[i] / args.steps, 4)}
        model[:] = [cfg, dit]
        fp8 = {"ms_per_step": round(ms8, 3), "TFLOP/s": round(fl["total"] / (ms8 * 1e-3) / 1e12, 2),
               "speedup_vs_bf16": round(ms_step / ms8, 3), "v_cosine_vs_bf16": round(cosv, 6),
               "format": "MX fp8: e4m3 elements, E8M0 scale per 32 along K, weights and activations of the "
                         "block projections (qkv, out, w1, w3, w2)", "kernels": fk}

    # ---- 1440^2 Turbo-style sampling (a second workload, not the headline value)
    turbo = None
    if not args.no_turbo:
        turbo = turbo_sampling(d, cfg, dit, max(1, min(args.steps, 3)), 1, not args.no_kernel_timer)

    cpu = None if args.no_cpu_baseline else cpu_baseline(d)

    out = {
        "metric": "ms & TFLOP/s per 48-block DiT step at 1024^2 (4096+512 tok), % bf16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Lens MM-DiT CFG denoising step, 1024x1024", "image_tokens": S_IMG,
                   "text_tokens": S_TXT, "batch": B, "cfg": "cond+uncond in one batch, norm-rescaled, scale 5.0",
                   "blocks": d.n_blocks, "hidden": d.hidden, "heads": d.heads, "mlp": d.mlp,
                   "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": fl["total"], "wall_s": round(wall, 3), "setup_s": round(setup_s, 1),
        "b1_forward": b1, "clock": clock,
        "kernels": kernels, "roofline": roof, "cpu_baseline": cpu, "fp8_variant": fp8, "turbo_1440": turbo,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
