"""Host-side checks of bench.py: the multi-GPU refusal, the algorithmic byte count the roofline
is computed from (against the oracle's byte model), and the planner-made plans."""
import os
import subprocess
import sys

import numpy as np

import bench
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_follow_the_oracle_byte_model():
    """Per cell: every (token, head) of the history reads the source cell's bytes (the 4-bit
    low plane weighted by the cell's hot fraction), plus q (bf16), out (fp32) and one page-table
    entry per 32 tokens; exact tokens read 512 B."""
    plan = np.array([[4, 2], [0, 0], [4, 2]], np.uint8)
    B, N, H = 3, 256, 16
    hot = np.linspace(0.1, 0.6, plan.size)
    total, per_cell = bench.algorithmic_bytes(plan, hot, B, N, H=H)
    i = 0
    expect = []
    for t in range(3):
        for l in range(2):
            cell = plan[t:t + 1, l:l + 1] if plan[t, l] else np.array([[plan[2, l]]], np.uint8)
            ref = O.cache_bytes_ref(cell, num_kv_heads=H)
            src = int(plan[2, l]) if plan[t, l] == 0 else int(plan[t, l])
            per_tok = ref["read_hi_only"] + (hot[i] * (ref["read_all_hot"] - ref["read_hi_only"]) if src == 4 else 0)
            expect.append(B * N * per_tok + B * H * 128 * 6 + B * (N // 32) * 4)
            i += 1
    assert np.allclose(per_cell, expect, rtol=1e-12)
    assert np.isclose(total, sum(expect), rtol=1e-12)
    # a sink and a window: 32 + 256 exact tokens at 512 B per head instead of quantized history
    t2, _ = bench.algorithmic_bytes(plan, hot, B, N + 288, H=H, n_hist=N, n_exact=288)
    assert np.isclose(t2 - total, len(expect) * B * 288 * H * 512 + len(expect) * B * (288 // 32) * 4, rtol=1e-12)


def test_planner_plans_for_the_benchmark():
    for name in ["knapsack_r", "knapsack_m"]:
        plan = bench.knapsack_plan(name, 24, 4, 1, 32)
        assert plan.shape == (4, 24) and set(np.unique(plan)) <= {0, 2, 4}
        assert (plan[3] != 0).all()


def test_kernel_hash_ignores_comments_only():
    """The stored traffic counters stay valid across comment and whitespace edits, not code edits."""
    a = bench.source_digest(["int a; // x\n/* y\n z */ int b;\n"])
    assert a == bench.source_digest(["int a;\n  int b; // other words\n"])
    assert a != bench.source_digest(["int a; int c;"])
    assert len(bench.kernel_hash()) == 16


def test_cpu_baseline_all_cores_child(tmp_path):
    """The all-cores CPU baseline: the sample written to disk is read back by a child Python
    (importing no GPU library), which runs one oracle worker per available core and reports how
    many rows each decoded in how long."""
    from quantized_kv_decode_amd import synth
    B, N, H = 2, 64, 16
    k = synth.keys(B, N, H, 128, 5)[0].double().numpy()
    v = synth.values(B, N, H, 128, 5)[0].double().numpy()
    q = synth.queries(B, H, 128, 6).double().numpy()
    heads = [O.quantize_head(k[:, h], v[:, h], 4, 128) for h in range(H)]
    pool = O.pack_pool(4, 32, [heads], np.arange(N // 32)[None, :], N // 32)
    cells = [(4, pool)]
    rows = [(0, h, q[:, h].copy(), k[:0, h], v[:0, h], k[N:, h], v[N:, h]) for h in range(3)]
    cfg = dict(B=B, N=N, S=0, n_hist=N, split=0)
    t, d = bench._time_rows(cells, rows, cfg, 0.01, 0.05)
    assert d >= 1 and t > 0
    path = str(tmp_path / "sample.npz")
    bench._write_sample(path, cells, rows, cfg, 0.01, 0.2)
    pj = bench._run_pool(path, 0.2)
    assert pj["workers"] >= 1 and len(pj["runs"]) == pj["workers"]
    assert all(dd >= 1 and tt > 0 for tt, dd in pj["runs"])
