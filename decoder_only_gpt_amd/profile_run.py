"""Workloads for rocprofv3 runs and the summaries committed from them.

    python -m decoder_only_gpt_amd.profile_run step [--config gpt2_124m] [--steps 3]
        a few training steps (forward, loss, backward, norm, AdamW) of a preset
    python -m decoder_only_gpt_amd.profile_run muon [--config gpt2_124m] [--steps 3]
        a few hybrid Muon + AdamW optimizer steps on fixed synthetic gradients
    python -m decoder_only_gpt_amd.profile_run decode [--config gpt2_124m] [--batch 16]
        [--prefill 512] [--steps 64]
        key/value-cache decode steps after a prompt fed one position at a time
    python -m decoder_only_gpt_amd.profile_run copy [--mib 1024]
        one plain device-to-device copy of a known size (counter calibration)
    python -m decoder_only_gpt_amd.profile_run summarize-stats CSV OUT --command "..."
        rocprofv3 --stats kernel table -> short text summary
    python -m decoder_only_gpt_amd.profile_run summarize-mfma CSV OUT --command "..."
        rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE counter rows -> per-kernel
        fraction of SIMD cycles the matrix units were busy
    python -m decoder_only_gpt_amd.profile_run summarize-timeline CSV OUT --command "..."
        rocprofv3 --kernel-trace rows of concurrent steps -> per step: busy fraction,
        fraction with two or more kernels running, idle gaps (and where they fall)
    python -m decoder_only_gpt_amd.profile_run summarize-traffic --kernel SUBSTR
        --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --copy-mib N OUT --command "..."
        per-dispatch FETCH_SIZE / WRITE_SIZE of one kernel, scaled by the same counters
        on the copy of known size -> JSON used by bench.py
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def kernel_source_sha() -> str:
    """Hash of the HIP sources the measured kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def run_step(config: str, steps: int, concurrent: bool = False):
    """A few training steps.  Unless `concurrent`, inside a kernel-timing window,
    which keeps every kernel on one stream (as the benchmark's per-kernel pass
    does), so a trace times each kernel alone."""
    import torch
    from decoder_only_gpt_amd import gpt, presets, synth
    cfg = presets.preset(config)
    m = gpt.Model(cfg)
    m.set_params(synth.init_params(cfg, seed=0))
    idx, tgt = synth.tokens(cfg, seed=1)
    di = torch.from_numpy(idx.reshape(-1)).cuda()
    dt = torch.from_numpy(tgt.reshape(-1)).cuda()
    if not concurrent:
        m.profile_begin()
    for i in range(steps):
        r = m.train_step(di, dt)
        print(f"step {i} loss {r['loss']:.4f}", flush=True)
    if not concurrent:
        m.profile_end()
    torch.cuda.synchronize()


def run_muon(config: str, steps: int):
    """A few hybrid optimizer steps (Muon on the block matrices, AdamW on the rest)."""
    import torch
    from decoder_only_gpt_amd import gpt, presets, synth
    cfg = presets.preset(config)
    m = gpt.Model(cfg)
    m.set_params(synth.init_params(cfg, seed=0))
    g = torch.from_numpy(synth.normal(m.n_params, seed=5, scale=1e-3)).cuda()
    for i in range(steps):
        m.set_buffer(gpt.BUF_GRADS, g)
        m.muon_step(i + 1, 1.0)
        torch.cuda.synchronize()
        print(f"muon step {i}", flush=True)


def run_decode(config: str, batch: int, prefill: int, steps: int):
    import numpy as np
    import torch
    from decoder_only_gpt_amd import gpt, presets, synth
    cfg = presets.preset(config)
    m = gpt.Model(cfg, B=1, T=8)
    m.set_params(synth.init_params(cfg, seed=0))
    g = gpt.Generator(m, batch, prefill + steps)
    rng = np.random.default_rng(9)
    toks = torch.from_numpy(rng.integers(0, cfg["vocab_size"], (prefill + steps, batch),
                                         dtype=np.int32)).cuda()
    for t in range(prefill + steps):
        g.step(toks[t])
        if t % 128 == 0 or t == prefill + steps - 1:
            torch.cuda.synchronize()
            print(f"decode position {t}", flush=True)


def run_copy(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB", flush=True)


def summarize_stats(csv_path: str, out_path: str, command: str, top: int = 40):
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}",
             f"# kernel sources sha: {kernel_source_sha()}",
             f"# total kernel time {total / 1e6:.3f} ms over the profiled run", "",
             f"{'calls':>6} {'total_ms':>9} {'avg_us':>9} {'pct':>6}  kernel"]
    for r in rows[:top]:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"{int(r['Calls']):>6} {float(r['TotalDurationNs']) / 1e6:>9.3f} "
                     f"{float(r['AverageNs']) / 1e3:>9.2f} {float(r['Percentage']):>6.2f}  {name}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU.  rocprofv3 sums a counter over
# its hardware instances: GRBM_GUI_ACTIVE over the 8 XCDs (so the sum is 8x
# the elapsed GPU cycles) and SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs.
N_XCD, N_SIMD = 8, 1024


def summarize_mfma(csv_path: str, out_path: str, command: str, top: int = 40):
    """Per kernel: mean over dispatches of MFMA-busy cycles / (elapsed cycles x
    SIMDs), elapsed cycles = GRBM_GUI_ACTIVE / XCDs."""
    disp = {}
    for r in csv.DictReader(open(csv_path)):
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        d = disp.setdefault(key, {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if "Start_Timestamp" in r and "End_Timestamp" in r:
            d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    per = {}
    for (_, name), d in disp.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in d or not d.get("GRBM_GUI_ACTIVE"):
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / N_XCD
        frac = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        e = per.setdefault(name, {"n": 0, "frac": 0.0, "cyc": 0.0, "busy": 0.0})
        e["n"] += 1
        e["frac"] += frac
        e["cyc"] += cyc
        e["busy"] += d["SQ_VALU_MFMA_BUSY_CYCLES"]
    rows = sorted(per.items(), key=lambda kv: -kv[1]["cyc"])
    lines = ["# rocprofv3 MFMA utilisation per kernel",
             f"# command: {command}",
             f"# kernel sources sha: {kernel_source_sha()}",
             f"# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} XCDs x {N_SIMD} SIMDs),",
             "#   averaged over a kernel's dispatches (counters summed over their hardware instances);",
             "#   cyc = elapsed GPU cycles per dispatch (GRBM_GUI_ACTIVE / 8)", "",
             f"{'calls':>6} {'mfma_busy':>9} {'kcyc':>9}  kernel"]
    for name, e in rows[:top]:
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"{e['n']:>6} {e['frac'] / e['n']:>9.3f} {e['cyc'] / e['n'] / 1e3:>9.1f}  {name}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _short(name: str) -> str:
    for pre in ("void gpt::(anonymous namespace)::", "gpt::(anonymous namespace)::", "gpt::"):
        name = name.replace(pre, "")
    return name.split("(")[0][:44]


def summarize_timeline(csv_path: str, out_path: str, command: str, marker: str = "embed_fwd_kernel"):
    """Kernel trace of back-to-back training steps: a step runs from one
    embedding lookup to the next.  Per whole step: its length, the fraction
    of it with at least one kernel running (busy) and with two or more, and
    the idle gaps; for the median step, every gap with the kernels around it."""
    with open(csv_path) as f:
        rows = list(csv.DictReader(f))
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                for r in rows)
    starts = [b for b, e, n in ev if marker in n]
    steps = []
    for a, b in zip(starts[1:-1], starts[2:]):  # whole steps only (the first may be warm-up)
        ks = [(s, e, n) for s, e, n in ev if a <= s < b]
        busy, gaps, cur_s, cur_e, last = 0, [], None, None, None
        for s, e, n in ks:
            if cur_e is not None and s > cur_e:
                busy += cur_e - cur_s
                gaps.append(((cur_e - a) / 1e3, (s - cur_e) / 1e3, last, n))
                cur_s = None
            if cur_s is None:
                cur_s = s
            if cur_e is None or e > cur_e:
                cur_e, last = e, n
        busy += cur_e - cur_s
        pts = sorted([(s, 1) for s, e, n in ks] + [(min(e, b), -1) for s, e, n in ks])
        two, run, prev = 0, 0, a
        for t, d in pts:
            if run >= 2:
                two += t - prev
            run += d
            prev = t
        steps.append(dict(ms=(b - a) / 1e6, busy=busy / (b - a), two=two / (b - a), gaps=gaps))
    lines = ["# Kernel timeline of concurrent training steps", f"# command: {command}",
             f"# kernel sources sha: {kernel_source_sha()}",
             "# busy = fraction of the step with a kernel running; 2+ = with two or more", "",
             "  step      ms   busy     2+   idle_us  gaps"]
    for i, st in enumerate(steps):
        idle = sum(g for _, g, _, _ in st["gaps"])
        lines.append(f"  {i:4d} {st['ms']:7.3f}  {st['busy']:.3f}  {st['two']:.3f}  {idle:8.1f}"
                     f"  {len(st['gaps']):4d}")
    if steps:
        med = sorted(steps, key=lambda x: x["ms"])[len(steps) // 2]
        lines += ["", "gaps of the median step (offset in the step, idle time, kernels around it):"]
        for off, g, p_, n in med["gaps"]:
            lines.append(f"  {off:9.1f} us  {g:5.1f} us  {_short(p_):44s} -> {_short(n)}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:12 + len(steps)]))


def _per_dispatch(csv_path: str, counter: str, substr: str):
    vals = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and substr in r["Kernel_Name"]:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {substr!r} in {csv_path}")
    return sum(vals) / len(vals), len(vals)


def summarize_traffic(args):
    fetch, nf = _per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    write, nw = _per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    cf, _ = _per_dispatch(args.copy_fetch, "FETCH_SIZE", args.copy_kernel)
    cw, _ = _per_dispatch(args.copy_write, "WRITE_SIZE", args.copy_kernel)
    known_kib = args.copy_mib * 1024.0
    sf, sw = known_kib / cf, known_kib / cw
    out = {
        "kernel": args.kernel, "site": args.site, "command": args.command,
        "kernel_source_sha": kernel_source_sha(),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "dispatches": [nf, nw],
        "copy_mib": args.copy_mib, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "scale_fetch": sf, "scale_write": sw,
        "hbm_bytes_per_launch": (fetch * sf + write * sw) * 1024.0,
    }
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("step")
    p.add_argument("--config", default="gpt2_124m")
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--concurrent", action="store_true",
                   help="the streams of training (forward chains, weight gradients and "
                        "AdamW groups beside the main chain) instead of one timed stream")
    p = sub.add_parser("muon")
    p.add_argument("--config", default="gpt2_124m")
    p.add_argument("--steps", type=int, default=3)
    p = sub.add_parser("decode")
    p.add_argument("--config", default="gpt2_124m")
    p.add_argument("--batch", type=int, default=16)
    p.add_argument("--prefill", type=int, default=512)
    p.add_argument("--steps", type=int, default=64)
    p = sub.add_parser("copy")
    p.add_argument("--mib", type=int, default=1024)
    p = sub.add_parser("summarize-stats")
    p.add_argument("csv")
    p.add_argument("out")
    p.add_argument("--command", required=True)
    p = sub.add_parser("summarize-mfma")
    p.add_argument("csv")
    p.add_argument("out")
    p.add_argument("--command", required=True)
    p = sub.add_parser("summarize-timeline")
    p.add_argument("csv")
    p.add_argument("out")
    p.add_argument("--command", required=True)
    p = sub.add_parser("summarize-traffic")
    p.add_argument("out")
    p.add_argument("--kernel", required=True)
    p.add_argument("--site", required=True)
    p.add_argument("--copy-kernel", default="copy")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-fetch", required=True)
    p.add_argument("--copy-write", required=True)
    p.add_argument("--copy-mib", type=int, default=1024)
    p.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "step":
        sys.path.insert(0, ROOT)
        run_step(a.config, a.steps, a.concurrent)
    elif a.cmd == "muon":
        sys.path.insert(0, ROOT)
        run_muon(a.config, a.steps)
    elif a.cmd == "decode":
        sys.path.insert(0, ROOT)
        run_decode(a.config, a.batch, a.prefill, a.steps)
    elif a.cmd == "copy":
        run_copy(a.mib)
    elif a.cmd == "summarize-stats":
        summarize_stats(a.csv, a.out, a.command)
    elif a.cmd == "summarize-mfma":
        summarize_mfma(a.csv, a.out, a.command)
    elif a.cmd == "summarize-timeline":
        summarize_timeline(a.csv, a.out, a.command)
    else:
        summarize_traffic(a)


if __name__ == "__main__":
    main()
