"""The profile summaries (host-only parsing of rocprofv3 CSV output) on small
synthetic traces whose answers are known by construction."""

import csv

from decoder_only_gpt_amd import profile_run


def _write(path, rows, fields):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_timeline_busy_overlap_and_gaps(tmp_path):
    # Five 10 us steps, each: the embedding lookup [0, 1) us, a product [0.5, 3)
    # beside it, an idle microsecond, a LayerNorm [4, 9), then idle to the next step.
    rows = []
    for k in range(5):
        t = k * 10000
        rows += [
            dict(Start_Timestamp=t, End_Timestamp=t + 1000,
                 Kernel_Name="gpt::(anonymous namespace)::embed_fwd_kernel(int const*)"),
            dict(Start_Timestamp=t + 500, End_Timestamp=t + 3000,
                 Kernel_Name="void gpt::(anonymous namespace)::gemm_big8_kernel<0, 0, 6>(x)"),
            dict(Start_Timestamp=t + 4000, End_Timestamp=t + 9000,
                 Kernel_Name="void gpt::(anonymous namespace)::ln_fwd_kernel<2>(y)"),
        ]
    src, out = tmp_path / "trace.csv", tmp_path / "timeline.txt"
    _write(src, rows, ["Start_Timestamp", "End_Timestamp", "Kernel_Name"])
    profile_run.summarize_timeline(str(src), str(out), "synthetic")
    lines = out.read_text().splitlines()
    table = [l.split() for l in lines if l[:6].strip().isdigit()]
    assert len(table) == 3  # whole steps only: the first and the last are left out
    for step in table:
        ms, busy, two, idle = (float(x) for x in step[1:5])
        gaps = int(step[5])
        assert abs(ms - 0.010) < 1e-9
        assert abs(busy - 0.8) < 1e-9   # 3 us + 5 us of 10
        assert abs(two - 0.05) < 1e-9   # [0.5, 1) us
        assert abs(idle - 1.0) < 1e-9 and gaps == 1
    assert any("gemm_big8_kernel<0, 0, 6>" in l and "-> ln_fwd_kernel<2>" in l for l in lines)
