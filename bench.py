"""Training-step benchmark: tokens/s and MFU of one GPT training step on one GPU.

    python bench.py [--steps K] [--warmup W] [--config gpt2_124m] [--no-cpu-baseline]

One step = forward + loss readback + backward + global grad norm + clip +
AdamW, through the C ABI, on seeded synthetic Zipf tokens already resident in
HBM and N(0, 0.02) weights.  W untimed warm-up steps, then exactly K timed
steps between device synchronisations.  MFU uses the per-token FLOP formula
of the nanochat page ("FLOPs-Berechnung im Detail") against the MI355X dense
bf16 MFMA peak.  A second, separately run pass brackets every kernel with HIP
events (gpt_profile_*) to give the dominant kernel's achieved rate against its
roofline; the CPU oracle is timed on a bounded sample of the same workload.
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
METRIC = "training tokens/sec on 1 GPU + MFU vs bf16 MFMA peak, GPT-2 124M shape"


# Call sites that launch exactly one kernel (see gpt_site in include/gpt.h):
# each maps to one kernel specialisation in rocprofv3 traces.  (lmhead_dx is
# split over K: a GEMM plus the fixed-order reduction; attn_bwd is two kernels;
# ln_bwd, cross_entropy, embed_bwd and grad_norm include their reductions.)
SINGLE_KERNEL_SITES = ["embed_fwd", "ln_fwd", "qkv_fwd", "attn_fwd", "proj_fwd", "fc_fwd",
                       "fcproj_fwd", "lmhead_fwd", "lmhead_dw", "fcproj_dx", "fc_dx",
                       "proj_dx", "qkv_dx", "adamw", "block_dw", "block_dw_reduce"]


def load_traffic(site):
    """HBM bytes per launch of `site` from the committed PMC summary, if it was
    taken on the current kernel sources (else None)."""
    from decoder_only_gpt_amd import profile_run
    path = os.path.join(ROOT, "profiles", f"traffic_{site}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != profile_run.kernel_source_sha():
        return None
    return round(t["hbm_bytes_per_launch"], 1)


def workload_name(cfg, name):
    return (f"{name}: decoder-only GPT training step, B={cfg['B']} T={cfg['T']} "
            f"V={cfg['vocab_size']}/{cfg['padded_vocab']} L={cfg['n_layer']} H={cfg['n_head']} "
            f"C={cfg['n_embd']} F={cfg['mlp_hidden']} {cfg['precision']}")


def cpu_baseline(cfg, min_seconds=10.0, max_steps=6):
    """Time the oracle's full step (fp32 NumPy) on one sequence of the same
    model, repeated on successive sequences until at least `min_seconds` of
    CPU work (at most `max_steps` steps) so the sample is not one short run."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from decoder_only_gpt_amd import synth
    cores = len(os.sched_getaffinity(0))  # the host cores this process may use
    p = synth.init_params(cfg, seed=0)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    steps = 0
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        while steps < max_steps and (steps == 0 or time.perf_counter() - t0 < min_seconds):
            idx, tgt = synth.tokens(cfg, B=1, T=cfg["T"], seed=1 + steps)
            r = oracle.step(cfg, p, m, v, idx, tgt, steps + 1, dtype=np.float32)
            p, m, v = r["p"], r["m"], r["v"]
            steps += 1
        dt = time.perf_counter() - t0
    return {"value": round(steps * cfg["T"] / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{steps} steps of one sequence each (B=1, T={cfg['T']}) of the same model, "
                      f"full step (forward, backward, norm, AdamW) in float32 NumPy; {dt:.1f} s"}


def muon_ns_flops(cfg, steps=5):
    """Matrix-product FLOPs of the Newton-Schulz iterations of one Muon step:
    per matrix [r, c] with s = min(r, c), l = max(r, c) and per iteration,
    the Gram product 2 s^2 l, A A 2 s^3 and the update product 2 s^2 l."""
    C, F = cfg["n_embd"], cfg["mlp_hidden"]
    total = 0
    for r, c in ((3 * C, C), (C, C), (F, C), (C, F)):
        s_, l_ = min(r, c), max(r, c)
        total += 4 * s_ * s_ * l_ + 2 * s_ ** 3
    return total * steps * cfg["n_layer"]


def time_muon(model, cfg, torch, gpt, reps=5):
    """The hybrid optimizer step (Muon on the block matrices, AdamW on the rest)
    in place of AdamW: HIP events on the stream it runs on, after one untimed
    call, on fixed synthetic gradients."""
    g = torch.randn(model.n_params, generator=torch.Generator().manual_seed(5)) * 1e-3
    g = g.cuda()
    ms = []
    for r in range(reps + 1):
        model.set_buffer(gpt.BUF_GRADS, g)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        model.muon_step(1000 + r, 1.0)
        e1.record()
        torch.cuda.synchronize()
        if r:
            ms.append(e0.elapsed_time(e1))
    t = sorted(ms)[len(ms) // 2]
    fl = muon_ns_flops(cfg)
    return {"ms": round(t, 3), "ns_flop": fl, "ns_tflops_over_step": round(fl / (t * 1e-3) / 1e12, 1)}


def decode_bytes(cfg, B, pos):
    """HBM bytes one decode step must read at context length pos: every
    weight matrix once (the tied lm_head is wte), the LayerNorm and bias
    vectors, the B embedding rows, and the cached keys and values of all
    layers (positions 0..pos-1), plus the new cache rows and the logits written."""
    C, F, L, H = cfg["n_embd"], cfg["mlp_hidden"], cfg["n_layer"], cfg["n_head"]
    act = 2 if cfg["precision"] == "bf16" else 4
    Vp = cfg["padded_vocab"]
    mats = L * (3 * C * C + C * C + 2 * F * C) + Vp * C
    vecs = L * (4 * C + (3 * C + C + F + C + 2 * C if cfg["bias"] else 0)) + 2 * C
    kv_read = 2 * L * B * pos * C * act
    writes = 2 * L * B * C * act + B * Vp * act
    return mats * act + vecs * 4 + 2 * B * C * 4 + kv_read + writes


def time_decode(model, cfg, torch, gpt, np, B=16, prefill=512, steps=64):
    """Decode throughput with the key/value cache: B sequences, a prompt of
    `prefill` tokens fed one position at a time (untimed), then `steps`
    timed decode steps (one token per sequence each), HIP events on the
    stream they run on."""
    g = gpt.Generator(model, B, prefill + steps)
    rng = np.random.default_rng(9)
    toks = torch.from_numpy(rng.integers(0, cfg["vocab_size"], (prefill + steps, B),
                                         dtype=np.int32)).cuda()
    for t in range(prefill):
        g.step(toks[t])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(prefill, prefill + steps):
        g.step(toks[t])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    byts = np.mean([decode_bytes(cfg, B, pos) for pos in range(prefill, prefill + steps)])
    return {"batch": B, "context": [prefill, prefill + steps], "ms_per_step": round(ms, 4),
            "tokens_per_s": round(B / (ms * 1e-3), 1),
            "hbm_bytes_per_step": int(byts), "achieved_gbs": round(byts / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gpt2_124m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=3)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from decoder_only_gpt_amd import gpt, presets, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = presets.preset(args.config)
    B, T = cfg["B"], cfg["T"]
    model = gpt.Model(cfg)
    model.set_params(synth.init_params(cfg, seed=0))
    idx, tgt = synth.tokens(cfg, seed=1)
    d_idx = torch.from_numpy(idx.reshape(-1)).cuda()
    d_tgt = torch.from_numpy(tgt.reshape(-1)).cuda()
    torch.cuda.synchronize()

    losses = []
    for _ in range(args.warmup):
        losses.append(model.train_step(d_idx, d_tgt)["loss"])
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for k in range(args.steps):
        losses.append(model.train_step(d_idx, d_tgt)["loss"])
        ev[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
    ms_per_step = wall * 1e3 / args.steps

    tokens = B * T
    value = tokens * args.steps / wall
    fpt = model.sizes.flops_per_token
    mfu = fpt * value / (PEAK_BF16_TFLOPS * 1e12)

    # Kernel timing pass (separate steps, same work): HIP events around every
    # launch, on the stream the kernels run on.
    model.profile_begin()
    for _ in range(args.profile_steps):
        model.train_step(d_idx, d_tgt)
    kstats, sstats = model.profile_end()
    per_kind = {}
    for k, s in kstats.items():
        if s["launches"]:
            per_kind[k] = {
                "ms_per_step": round(s["ms"] / args.profile_steps, 4),
                "launches_per_step": s["launches"] // args.profile_steps,
                "tflops": round(s["flops"] / (s["ms"] * 1e-3) / 1e12, 2) if s["flops"] else None,
                "gbs": round(s["bytes"] / (s["ms"] * 1e-3) / 1e9, 1) if s["bytes"] else None,
            }
    per_site = {k: {"ms_per_step": round(s["ms"] / args.profile_steps, 4),
                    "launches_per_step": s["launches"] // args.profile_steps}
                for k, s in sstats.items() if s["launches"]}
    # Dominant kernel: the call site with the most time per step among those that
    # launch a single kernel (rocprofv3's top kernel: the grouped weight gradients).
    single = [k for k in SINGLE_KERNEL_SITES if sstats[k]["launches"]]
    dom = max(single, key=lambda k: sstats[k]["ms"])
    ds = sstats[dom]
    avg_s = ds["ms"] * 1e-3 / ds["launches"]
    traffic = load_traffic(dom)
    if ds["flops"]:
        per_launch = ds["flops"] / ds["launches"]
        ach = per_launch / avg_s / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_per_launch": per_launch, "avg_launch_us": round(avg_s * 1e6, 2),
                "launches_per_step": ds["launches"] // args.profile_steps}
    else:
        per_launch = ds["bytes"] / ds["launches"]
        ach = per_launch / avg_s / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_per_launch": per_launch, "avg_launch_us": round(avg_s * 1e6, 2),
                "launches_per_step": ds["launches"] // args.profile_steps}

    muon = time_muon(model, cfg, torch, gpt)
    decode = time_decode(model, cfg, torch, gpt, np=np)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg["precision"] == "bf16" else "f32",
        "data": "synthetic (seeded Zipf token ids, N(0,0.02) weights)",
        "config": {"workload": workload_name(cfg, args.config), "global_batch": B, "seq_len": T,
                   "parallelism": "none (1 GPU)"},
        "mfu": round(mfu, 4), "flops_per_token": fpt, "peak_tflops": PEAK_BF16_TFLOPS,
        "step_ms_median": round(float(np.median(step_ms)), 3),
        "step_ms_min": round(float(np.min(step_ms)), 3),
        "loss_first": round(losses[0], 4), "loss_last": round(losses[-1], 4),
        "kernels": per_kind, "sites": per_site, "roofline": roof, "muon_step": muon,
        "decode": decode,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
