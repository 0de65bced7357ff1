"""Benchmark: one LoopKV decode step (every cell's fused decode-attention launch, in model order)
on one MI355X, on a synthetic Ouro-1.4B-shaped cache.

Default workload: 24 layers x 4 loops = 96 cells, 16 KV heads x 128, batch 64, context 8192,
seeded plan of 40% INT4 / 35% INT2 / 25% reuse-the-final-loop, tau = 0.01, one split per row.
A step is the 96 decode launches back to back on one stream; inputs are resident in HBM.

Prints one JSON line: value = microseconds per decode step (lower is better), plus the achieved
algorithmic HBM bandwidth of the decode kernel against MI355X's 8 TB/s (`roofline`) and the
fp64 CPU oracle timed on a bounded sample on this host (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
# Algorithmic bytes per (token, head) read by decode, 128-channel value groups.
INT4_BASE, INT4_LO, INT2_BYTES = 116.0, 32.0, 84.0

WORKLOADS = {
    # name: (layers, loops, batch, context, p_int4, p_reuse, split_tokens, heavy_tail)
    "ouro1.4b-96cells-b64-ctx8k": (24, 4, 64, 8192, 0.40, 0.25, 0, False),
    "ouro2.6b-192cells-b16-ctx32k": (48, 4, 16, 32768, 0.30, 0.25, 8192, True),
    "one-layer-4loops-b8-ctx4k": (1, 4, 8, 4096, None, None, 2048, False),
    "single-cell-b1-ctx256": (1, 1, 1, 256, "single", None, 64, False),
    # batch 1: 16 rows per cell, so the library splits each row (split_tokens = LOOPKV_SPLIT_AUTO)
    "ouro1.4b-96cells-b1-ctx8k": (24, 4, 1, 8192, 0.40, 0.25, "auto", False),
}
# The same caches in the paper's serving setting: a 32-token sink and a 256-token window stay
# exact bf16 (read as 512 bytes per (token, head)), the groups between them are quantized history.
NEAR = {"ouro1.4b-96cells-b64-ctx8k-sink32-win256": ("ouro1.4b-96cells-b64-ctx8k", 32, 256)}
# Workloads small enough to stay in the caches: flushed between timed steps.
FLUSHED = {"one-layer-4loops-b8-ctx4k", "single-cell-b1-ctx256"}
# The paged serving batch: the 96-cell plan, 128 requests of uniform 1K..16K tokens in 16-token
# pages of a shuffled table; a step appends one token per request to every cell, then decodes it.
PAGED = "ouro1.4b-96cells-paged-b128"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_digest(texts) -> str:
    """Digest of C++ sources with comments removed and whitespace collapsed, so that only a
    change to the code itself changes it."""
    h = hashlib.sha256()
    for t in texts:
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
    return h.hexdigest()[:16]


def kernel_hash() -> str:
    """Identifies the decode kernel's code: the stored HBM-traffic counters apply only while it
    is unchanged."""
    return source_digest(open(os.path.join(ROOT, "quantized_kv_decode_amd", "csrc", f)).read()
                         for f in ["decode.hip", "loopkv_internal.h"])


def build_cache(name, seed, tau, plan_name="seeded", v_group=128, shuffle=True, split_override=None):
    import torch
    from quantized_kv_decode_amd import loopkv as L
    from quantized_kv_decode_amd import synth
    from quantized_kv_decode_amd.cache import LoopKVCache

    base, S, W = NEAR.get(name, (name, 0, 0))
    layers, loops, B, N, p4, pr, split, heavy = WORKLOADS[base]
    if split_override is not None:
        split = split_override
    if plan_name.startswith("knapsack"):
        plan = knapsack_plan(plan_name, layers, loops, seed, v_group)
    elif plan_name != "seeded":
        plan = synth.named_plan(plan_name, layers, loops)
    elif p4 == "single":
        plan = np.array([[4]], np.uint8)
    elif p4 is None:
        plan = np.array([[4], [4], [2], [4]], np.uint8)
    else:
        plan = synth.plan(layers, loops, seed, p4, pr)
    P = 32
    pages_per_seq = N // P
    max_splits = 64 if split == "auto" else (max(1, N // split) if split else 1)
    shape = L.make_shape(num_layers=layers, num_loops=loops, page_tokens=P, v_group=v_group, max_batch=B,
                         max_pages_per_seq=pages_per_seq, tail_tokens=64 if W == 0 else W + 64,
                         max_splits=max_splits, num_pages=B * pages_per_seq,
                         sink_tokens=S, window_tokens=W)
    cache = LoopKVCache(shape, plan)
    pt_np, _ = synth.page_table([N] * B, P, seed + 1, shuffle=shuffle)
    pt = torch.as_tensor(pt_np).cuda()
    auto = split == "auto"
    if auto:      # the library's own choice; decode is called with LOOPKV_SPLIT_AUTO
        split = cache.auto_split(B, pt)
        log(f"[bench] automatic split: {split} tokens per split")
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    t0 = time.time()
    for t in range(loops):
        for l in range(layers):
            if plan[t, l] == L.REUSE:
                continue
            cs = seed * 100003 + t * 1000 + l
            k = synth.keys(B, N, 16, 128, cs, device="cuda", heavy_tail=heavy)
            v = synth.values(B, N, 16, 128, cs, device="cuda")
            cache.append(l, t, k, v, zeros, pt)
            del k, v
    torch.cuda.synchronize()
    log(f"[bench] filled {int((plan != 0).sum())} own cells in {time.time() - t0:.1f}s; "
        f"arena {cache.bytes.arena_bytes / 2**30:.1f} GiB")
    # quantized history [S, he) and exact tokens (sink and window) per request
    he = max(S, (N - W) // 32 * 32)
    return cache, plan, pt, pt_np, dict(layers=layers, loops=loops, B=B, N=N, split=split, heavy=heavy,
                                        S=S, W=W, n_hist=he - S, n_exact=N - (he - S), auto_split=auto)


def knapsack_plan(name, layers, loops, seed, v_group):
    """A plan from the library's exact planner on a seeded synthetic damage table: read-optimized
    (damage budget 3x the all-INT4 damage, no storage budget) or memory-optimized (5x, and at most
    65% of the all-INT4 storage, the ratio of the paper's 156 KiB budget to KIVI-4's 240 KiB)."""
    from quantized_kv_decode_amd import loopkv as L
    from quantized_kv_decode_amd import synth

    d = synth.damage_table(layers, loops, seed)
    d4 = float(np.nansum(d[:, :, 0]))
    shape = L.make_shape(num_layers=layers, num_loops=loops, v_group=v_group, max_batch=1,
                         max_pages_per_seq=1, num_pages=1)
    all4 = L.loopkv_cache_bytes(shape, np.full((loops, layers), 4, np.uint8)).stored_bytes_per_token
    if name == "knapsack_r":
        plan, cost = L.loopkv_plan_solve(shape, d, max_damage=3.0 * d4)
    else:
        plan, cost = L.loopkv_plan_solve(shape, d, max_damage=5.0 * d4, max_stored_bytes=0.65 * all4)
    log(f"[bench] {name}: damage {cost.damage:.3f} (all-INT4 {d4:.3f}), stored "
        f"{cost.stored_bytes_per_token / 1024:.1f} KiB, read {cost.read_bytes_per_token / 1024:.1f} KiB per token")
    return plan


def run_step(cache, plan, qs, outs, seq, pt, tau, split, stats=None, events=None, stream=None):
    """One decode step: every cell's decode launch in model order (loop-major). With `events`
    (a list of len(cells) + 1), an event is recorded before the first launch and after each."""
    loops, layers = plan.shape
    i = 0
    if events is not None:
        events[0].record(stream)
    for t in range(loops):
        for l in range(layers):
            cache.decode(l, t, qs[i], seq, pt, tau=tau, split_tokens=split, out=outs[i],
                         stats=None if stats is None else stats[i])
            if events is not None:
                events[i + 1].record(stream)
            i += 1


def algorithmic_bytes(plan, hot_frac, B, N, H=16, n_split=1, v_group=128, n_hist=None, n_exact=0):
    """Bytes one decode step reads/writes by the path's definition: per history (token, head)
    116 + 32*h bytes for an INT4-read cell and 84 for an INT2-read cell, 512 per exact bf16
    (token, head) (sink and window), plus q, out, the page table, and split partials."""
    n_hist = N if n_hist is None else n_hist
    loops, layers = plan.shape
    total = 0.0
    per_cell = []
    i = 0
    for t in range(loops):
        for l in range(layers):
            src = plan[loops - 1, l] if plan[t, l] == 0 else plan[t, l]
            vsz = 4 * 128 / v_group - 4          # value scale/zero beyond the 128-channel case
            per_tok = INT4_BASE + vsz + INT4_LO * hot_frac[i] if src == 4 else INT2_BYTES + vsz
            b = B * n_hist * H * per_tok + B * n_exact * H * 512 + B * H * 128 * (2 + 4) + B * (N // 32) * 4
            if n_split > 1:
                b += 2 * B * H * n_split * 130 * 4
            per_cell.append(b)
            total += b
            i += 1
    return total, per_cell


def graph_time(step_fn, check_fn, steps, advance=None, eager_work=None):
    """Captures one step (`step_fn`, launches on torch's current stream) in a HIP graph, replays
    it three times with eager work (`eager_work()`) and synchronizations in between, checking
    each replay with `check_fn` (True = outputs equal the eager path's), then times `steps`
    replays with events around each. `advance()` runs eagerly before every replay (e.g. moving
    lengths on by the appended token). Returns the median replay time in ms, or None with the
    reason when capture or a check fails."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_fn()                       # warm-up on a side stream, as capture requires
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_fn()
        torch.cuda.synchronize()
    except Exception as e:                  # capture unsupported: report, keep eager timing
        return None, f"capture failed: {e}"
    for r in range(3):
        if eager_work is not None:
            eager_work()
        if advance is not None:
            advance()
        graph.replay()
        torch.cuda.synchronize()
        if not check_fn():
            return None, f"replay {r} differs from the eager path"
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        if advance is not None:
            advance()
        ev[i][0].record()
        graph.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])), "ok"


def _baseline_rows(cfg, plan, seed):
    """The CPU baseline's sample, built untimed: for one request of one INT4, one INT2 and one
    reusing cell, the oracle quantizes the same synthetic K/V the GPU was filled with and packs
    them into pages. Returns (cells, rows): cells = [(bits, packed pages)], rows = one per
    (cell, head): (cell index, head, queries [B, D], sink K, sink V, window K, window V)."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    from quantized_kv_decode_amd import synth

    loops, B, N = cfg["loops"], cfg["B"], cfg["N"]
    S, he = cfg["S"], cfg["S"] + cfg["n_hist"]   # sink [0, S), history [S, he), window [he, N)
    H = 16
    picked = []
    for code in (4, 2, 0):
        idx = np.argwhere(plan == code)
        if len(idx):
            picked.append(tuple(int(x) for x in idx[0]))
    cells, rows = [], []
    with threadpool_limits(limits=1):
        for (t, l) in picked:
            st, sl = (loops - 1, l) if plan[t, l] == 0 else (t, l)
            bits = int(plan[st, sl])
            cs = seed * 100003 + st * 1000 + sl
            # the generator of the GPU fill; request 0 copied to the host
            k = synth.keys(B, N, H, 128, cs, device="cuda", heavy_tail=cfg["heavy"])[0].double().cpu().numpy()
            v = synth.values(B, N, H, 128, cs, device="cuda")[0].double().cpu().numpy()
            q = synth.queries(B, H, 128, 777 + t * 100 + l, device="cuda").double().cpu().numpy()
            heads = [O.quantize_head(k[S:he, h], v[S:he, h], bits, 128) for h in range(H)]
            pt = np.arange(N // 32)[None, :]
            cells.append((bits, O.pack_pool(bits, 32, [heads], pt, N // 32, hist_start=S)))
            for h in range(H):
                rows.append((len(cells) - 1, h, np.ascontiguousarray(q[:, h]), k[:S, h].copy(),
                             v[:S, h].copy(), k[he:, h].copy(), v[he:, h].copy()))
    return cells, rows


def _time_rows(cells, rows, cfg, tau, budget_s, start=0):
    """Decodes the sampled rows one after another, on one core, until `budget_s` seconds of
    decoding are spent: read the packed pages back, dequantize, build the fetch mask, fp64
    softmax attention. Returns (seconds, rows decoded)."""
    from threadpoolctl import threadpool_limits

    import oracle as O

    B, N, S = cfg["B"], cfg["N"], cfg["S"]
    he = S + cfg["n_hist"]
    timed, done = 0.0, 0
    with threadpool_limits(limits=1):
        while timed < budget_s:
            i = start + done
            c, h, qs, sk, sv, wk, wv = rows[i % len(rows)]
            bits, pool = cells[c]
            t0 = time.perf_counter()
            qh = O.unpack_pool_head(bits, 32, pool, np.arange(N // 32), he - S, h, 16, hist_start=S)
            O.decode_head(qs[i % B], qh, wk, wv, sm_scale=1 / math.sqrt(128), tau=tau,
                          split_tokens=cfg["split"], sink_k=sk, sink_v=sv, hist_start=S)
            timed += time.perf_counter() - t0
            done += 1
    return timed, done


_POOL = None   # (cells, rows, cfg, tau, budget) of the pool child, inherited by its workers


def _pool_worker(i):
    cells, rows, cfg, tau, budget = _POOL
    return _time_rows(cells, rows, cfg, tau, budget, start=7 * i)


def cpu_pool_main(path):
    """Entry point of the CPU-baseline child process (it never touches the GPU): loads the sample
    written by cpu_baseline, times it in one worker process per available core (at most 16), and
    prints one JSON line {"workers": n, "runs": [[seconds, rows], ...]}."""
    global _POOL
    import multiprocessing as mp

    z = np.load(path, allow_pickle=False)
    meta = json.loads(str(z["meta"]))
    cells = [(int(b), z[f"pool{c}"]) for c, b in enumerate(z["bits"])]
    rows = [(int(z["row_cell"][i]), int(z["row_head"][i]), z[f"q{i}"], z[f"sk{i}"], z[f"sv{i}"],
             z[f"wk{i}"], z[f"wv{i}"]) for i in range(len(z["row_cell"]))]
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    _POOL = (cells, rows, meta["cfg"], meta["tau"], meta["budget"])
    with mp.get_context("fork").Pool(n) as pool:
        runs = pool.map(_pool_worker, range(n))
    print(json.dumps({"workers": n, "runs": runs}), flush=True)


def _write_sample(path, cells, rows, cfg, tau, budget_s):
    """The CPU baseline's sample and settings as one .npz (plain arrays, no pickled objects)."""
    arrays = {"bits": np.array([b for b, _ in cells], np.int32),
              "row_cell": np.array([r[0] for r in rows], np.int32),
              "row_head": np.array([r[1] for r in rows], np.int32),
              "meta": np.array(json.dumps({"cfg": {k: cfg[k] for k in ("B", "N", "S", "n_hist", "split")},
                                           "tau": tau, "budget": budget_s}))}
    for c, (_, pool) in enumerate(cells):
        arrays[f"pool{c}"] = pool
    for i, r in enumerate(rows):
        for name, a in zip(("q", "sk", "sv", "wk", "wv"), r[2:]):
            arrays[f"{name}{i}"] = a
    np.savez(path, **arrays)


def _run_pool(path, budget_s):
    """Runs cpu_pool_main on `path` in a child Python (which imports no GPU library); returns its
    JSON result or raises."""
    import subprocess

    code = f"import sys; sys.path.insert(0, {ROOT!r}); import bench; bench.cpu_pool_main(sys.argv[1])"
    out = subprocess.run([sys.executable, "-c", code, path], capture_output=True, text=True,
                         timeout=budget_s + 60, cwd=ROOT)
    if out.returncode != 0:
        raise RuntimeError((out.stderr.strip().splitlines() or [f"exit {out.returncode}"])[-1])
    return json.loads(out.stdout.strip().splitlines()[-1])


def cpu_baseline(cfg, plan, tau, seed, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the same workload, timed on the host.

    One core first, in this process. Then every available core (at most 16): a child Python
    process that imports no GPU library runs one worker per core on the same sample, each for
    `budget_s` seconds; the value reported is that aggregate rate, or the one-core rate if the
    child fails. Rates are extrapolated linearly in (request, head) rows to the whole step."""
    import tempfile

    layers, loops, B, N = cfg["layers"], cfg["loops"], cfg["B"], cfg["N"]
    H = 16
    cells, rows = _baseline_rows(cfg, plan, seed)
    timed, done = _time_rows(cells, rows, cfg, tau, budget_s)
    rows_step = loops * layers * B * H
    us_one = timed / done * rows_step * 1e6
    what = (f"(request, head) decodes of {N} tokens from {len(rows)} packed rows of {len(cells)} "
            f"cells (INT4 / INT2 / reuse) on {host_cpu()}")
    result = {"value": round(us_one, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
              "sample": f"{done} {what}, {timed:.1f} s on one core; extrapolated "
                        f"x{rows_step / done:.0f} to the {rows_step} rows of one step"}
    try:
        with tempfile.TemporaryDirectory() as tmp:
            path = os.path.join(tmp, "sample.npz")
            _write_sample(path, cells, rows, cfg, tau, budget_s)
            log(f"[bench] CPU baseline: one core {us_one:.4g} us/step; now every available core")
            pj = _run_pool(path, budget_s)
        rate = sum(d / t for t, d in pj["runs"])          # rows per second over all workers
        n_rows = sum(d for _, d in pj["runs"])
        result.update({"value": round(rows_step / rate * 1e6, 1), "cores": pj["workers"],
                       "sample": f"{n_rows} {what}, {pj['workers']} worker processes for "
                                 f"{budget_s:.0f} s each; extrapolated to the {rows_step} rows of one "
                                 f"step; one core alone: {us_one:.4g} us/step"})
    except Exception as e:   # the one-core figure stands
        log(f"[bench] CPU baseline on all cores unavailable: {e}")
    return result


def host_cpu() -> str:
    """The host's CPU model and how many cores this process may run on."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{len(os.sched_getaffinity(0))} available ({model})"


def run_paged(args):
    """The paged serving batch: per step and cell (model order), quantize_append of one token per
    request, then the cell's decode; appends and decodes are timed separately with events."""
    import torch
    from quantized_kv_decode_amd import loopkv as L
    from quantized_kv_decode_amd import synth
    from quantized_kv_decode_amd.cache import LoopKVCache

    layers, loops, B, P, H, D = 24, 4, 128, 16, 16, 128
    plan = synth.plan(layers, loops, args.seed, 0.40, 0.25)
    lens0 = np.random.default_rng(args.seed + 7).integers(1024, 16385, size=B).astype(np.int64)
    grow = args.warmup + 2 * args.steps + 8    # one token per step: stats, warm-up, eager, graph steps
    pt_np, npages = synth.page_table(lens0 + grow, P, args.seed + 1, shuffle=True)
    pt = torch.as_tensor(pt_np).cuda()
    shape = L.make_shape(num_layers=layers, num_loops=loops, page_tokens=P, v_group=128, max_batch=B,
                         max_pages_per_seq=pt_np.shape[1], tail_tokens=64, max_splits=1, num_pages=npages)
    cache = LoopKVCache(shape, plan)
    t0 = time.time()
    chunk = 4096
    total = int(lens0.max())
    for t in range(loops):
        for l in range(layers):
            done = np.zeros(B, np.int64)
            off = 0
            cs = args.seed * 100003 + t * 1000 + l
            while off < total:
                n = min(chunk, total - off)
                k = synth.keys(B, n, H, D, cs, device="cuda", token_offset=off)
                v = synth.values(B, n, H, D, cs, device="cuda", token_offset=off)
                m = np.clip(lens0 - off, 0, n).astype(np.int32)
                cache.append(l, t, k, v, torch.as_tensor(done.astype(np.int32)).cuda(), pt,
                             n_new=torch.as_tensor(m).cuda())
                done += m
                off += n
                del k, v
    torch.cuda.synchronize()
    log(f"[bench] filled {loops * layers} cells ({int(lens0.sum())} tokens per cell) in {time.time() - t0:.1f}s; "
        f"arena {cache.bytes.arena_bytes / 2**30:.1f} GiB")
    ncell = loops * layers
    cells = [(t, l) for t in range(loops) for l in range(layers)]
    knew = [synth.keys(B, 1, H, D, 900 + i, device="cuda") for i in range(ncell)]
    vnew = [synth.values(B, 1, H, D, 900 + i, device="cuda") for i in range(ncell)]
    qs = [synth.queries(B, H, D, 777 + i, device="cuda") for i in range(ncell)]
    outs = [torch.empty(B, H, D, dtype=torch.float32, device="cuda") for _ in range(ncell)]
    lens = lens0.copy()

    def step(events=None, stats=None):
        before = torch.as_tensor(lens.astype(np.int32)).cuda()
        after = torch.as_tensor((lens + 1).astype(np.int32)).cuda()
        if events is not None:
            events[0].record()
        for i, (t, l) in enumerate(cells):
            cache.append(l, t, knew[i], vnew[i], before, pt)
            if events is not None:
                events[2 * i + 1].record()
            cache.decode(l, t, qs[i], after, pt, tau=args.tau, out=outs[i],
                         stats=None if stats is None else stats[i])
            if events is not None:
                events[2 * i + 2].record()
        lens[:] += 1

    stats = torch.zeros(ncell, 4, dtype=torch.int64, device="cuda")
    step(stats=[stats[i] for i in range(ncell)])
    torch.cuda.synchronize()
    st = stats.cpu().numpy().astype(np.float64)
    gated = st[:, 2] > 0
    hot_frac = np.where(gated, st[:, 1] / np.maximum(st[:, 2], 1), 0.0)
    overall_hot = float(st[gated, 1].sum() / max(st[gated, 2].sum(), 1)) if gated.any() else 0.0
    assert cache.device_errors() == 0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * ncell + 1)] for _ in range(args.steps)]
    hist_tokens = []
    for i in range(args.steps):
        hist_tokens.append(lens + 1)
        step(events=ev[i])
    torch.cuda.synchronize()
    # The same step as one HIP graph: appends read `before_d`, decodes `after_d`, moved on by one
    # token before every replay; each checked replay is compared with eager decodes of the state
    # it leaves.
    graph_ms, graph_note = None, "off"
    if not args.no_graph:
        before_d = torch.as_tensor(lens.astype(np.int32)).cuda()
        after_d = before_d + 1
        outs_g = [torch.empty_like(o) for o in outs]
        outs_c = [torch.empty_like(o) for o in outs]

        def gstep():
            for i, (t, l) in enumerate(cells):
                cache.append(l, t, knew[i], vnew[i], before_d, pt)
                cache.decode(l, t, qs[i], after_d, pt, tau=args.tau, out=outs_g[i])

        def eager_decodes():
            for i, (t, l) in enumerate(cells):
                cache.decode(l, t, qs[i], after_d, pt, tau=args.tau, out=outs_c[i])

        # A reusing cell decodes before the final loop appends in the same step, so its eager
        # re-run after the step may see one more quantized group of its source: only cells with
        # their own storage are compared bit for bit.
        own = [i for i, (t, l) in enumerate(cells) if plan[t, l] != 0]

        def check():
            eager_decodes()
            torch.cuda.synchronize()
            return all(torch.equal(outs_g[i], outs_c[i]) for i in own)

        first = [True]

        def advance():
            if first[0]:            # the capture's warm-up step appended at the current lengths
                first[0] = False
                lens[:] += 1
            before_d.add_(1)
            after_d.add_(1)
            lens[:] += 1

        graph_ms, graph_note = graph_time(gstep, check, args.steps, advance=advance, eager_work=eager_decodes)
        assert cache.device_errors() == 0
        log(f"[bench] graph: {graph_note}, {graph_ms} ms/step")
    app_ms = np.array([[ev[i][2 * j].elapsed_time(ev[i][2 * j + 1]) for j in range(ncell)] for i in range(args.steps)])
    dec_ms = np.array([[ev[i][2 * j + 1].elapsed_time(ev[i][2 * j + 2]) for j in range(ncell)] for i in range(args.steps)])
    step_ms = np.array([ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps)])
    med = int(np.argsort(step_ms)[len(step_ms) // 2])
    for o in outs:
        assert torch.isfinite(o).all()
    assert cache.device_errors() == 0
    # algorithmic decode bytes of the median step: every token of every request, per cell
    ntok = float(hist_tokens[med].sum())
    src_bits = np.array([plan[loops - 1, l] if plan[t, l] == 0 else plan[t, l] for (t, l) in cells])
    per_cell = np.array([ntok * H * ((INT4_BASE + INT4_LO * hot_frac[i]) if src_bits[i] == 4 else INT2_BYTES)
                         + B * H * D * 6 + ntok / 32 * 4 for i in range(ncell)])
    dec_step = float(dec_ms[med].sum())
    kinds = {}
    for bits in (4, 2):
        sel = src_bits == bits
        if sel.any():
            dur = float(dec_ms[:, sel].mean())
            byt = float(per_cell[sel].mean())
            kinds[f"decode_int{bits}_read"] = dict(launches_per_step=int(sel.sum()), avg_us=round(dur * 1e3, 1),
                                                   bytes_per_launch=int(byt), GBps=round(byt / (dur / 1e3) / 1e9, 1))
    kinds["append_one_token"] = dict(launches_per_step=ncell, avg_us=round(float(app_ms.mean()) * 1e3, 1))
    dom = max((k for k in kinds if k.startswith("decode")), key=lambda k: kinds[k]["avg_us"] * kinds[k]["launches_per_step"])
    line = {
        "metric": "fused LoopKV decode attn: µs/step and achieved HBM TB/s vs peak, 1 MI355X",
        "value": round((graph_ms if graph_ms is not None else float(step_ms[med])) * 1e3, 1),
        "unit": "us/step",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(graph_ms if graph_ms is not None else float(step_ms[med]), 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8 codes; fp16 scales and value weights; f32 scores and accumulation",
        "data": "synthetic (seeded Gaussian K/V/q, 4 outlier key channels x10 per cell and head)",
        "config": {"workload": PAGED, "layers": layers, "loops": loops, "cells": ncell, "kv_heads": H,
                   "head_dim": D, "batch": B, "context": "uniform 1024..16384 per request",
                   "tokens_per_cell": int(hist_tokens[med].sum()), "tau": args.tau, "split_tokens": 0,
                   "page_tokens": P, "v_group": 128, "plan_seed": args.seed,
                   "plan_counts": {"int4": int((plan == 4).sum()), "int2": int((plan == 2).sum()),
                                   "reuse": int((plan == 0).sum())}},
        "eager_ms_per_step": round(float(step_ms[med]), 4),
        "graph": {"used": graph_ms is not None, "note": graph_note, "launches_per_step": 2 * ncell,
                  "ms_per_step": None if graph_ms is None else round(graph_ms, 4)},
        "decode_us_per_step": round(dec_step * 1e3, 1),
        "append_us_per_step": round(float(app_ms[med].sum()) * 1e3, 1),
        "achieved_TBps": round(float(per_cell.sum()) / (dec_step / 1e3) / 1e12, 3),
        "hot_fraction": round(overall_hot, 4),
        "alg_bytes_per_step": int(per_cell.sum()),
        "kernels": kinds,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kinds[dom]["GBps"], "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(kinds[dom]["GBps"] / PEAK_HBM_GBPS, 4), "traffic": None},
        "cpu_baseline": None,
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ouro1.4b-96cells-b64-ctx8k",
                    choices=sorted(WORKLOADS) + sorted(NEAR) + [PAGED],
                    help="workloads in FLUSHED evict the caches before every timed step")
    ap.add_argument("--tau", type=float, default=0.01)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--plan", default="seeded",
                    choices=["seeded", "kivi4", "kivi4_loop3_share", "int2_loops123", "loopkv_r", "loopkv_m",
                             "knapsack_r", "knapsack_m"],
                    help="the workload's seeded plan, or one of the paper's fixed plans")
    ap.add_argument("--v-group", type=int, default=128, choices=[128, 64, 32])
    ap.add_argument("--split", type=int, default=None,
                    help="split_tokens (a multiple of 32; 0 = one split per row) instead of the workload's")
    ap.add_argument("--pages", default="shuffled", choices=["shuffled", "in-order"],
                    help="physical page order of each request's pages (the paged serving batch is "
                         "always shuffled)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for {args.gpus}). "
              "Rows (request, head) are independent, so requests or heads would shard across GPUs "
              "with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_kv_decode_amd import synth

    torch.cuda.set_device(0)
    if args.workload == PAGED:
        return run_paged(args)
    cache, plan, pt, pt_np, cfg = build_cache(args.workload, args.seed, args.tau, args.plan, args.v_group,
                                              shuffle=args.pages == "shuffled", split_override=args.split)
    loops, layers = plan.shape
    B, N, split = cfg["B"], cfg["N"], cfg["split"]
    from quantized_kv_decode_amd import loopkv as L
    call_split = L.SPLIT_AUTO if cfg["auto_split"] else split   # what each decode call passes
    ncell = loops * layers
    qs = [synth.queries(B, 16, 128, 777 + t * 100 + l, device="cuda") for t in range(loops) for l in range(layers)]
    outs = [torch.empty(B, 16, 128, dtype=torch.float32, device="cuda") for _ in range(ncell)]
    seq = torch.full((B,), N, dtype=torch.int32, device="cuda")

    # Hot fractions (one pass with device counters, untimed).
    stats = torch.zeros(ncell, 4, dtype=torch.int64, device="cuda")
    run_step(cache, plan, qs, outs, seq, pt, args.tau, call_split, stats=[stats[i] for i in range(ncell)])
    torch.cuda.synchronize()
    st = stats.cpu().numpy().astype(np.float64)
    hot_frac = np.where(st[:, 2] > 0, st[:, 1] / np.maximum(st[:, 2], 1), 0.0)
    gated = st[:, 2] > 0
    overall_hot = float(st[gated, 1].sum() / max(st[gated, 2].sum(), 1)) if gated.any() else 0.0
    assert cache.device_errors() == 0

    if args.calibrate_copy:
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    # The library launches on torch's current stream, so its events bracket the kernels.
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        run_step(cache, plan, qs, outs, seq, pt, args.tau, call_split)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ncell + 1)] for _ in range(args.steps)]
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if args.workload in FLUSHED else None

    def flush():   # evicts L2 and the last-level cache before a timed step (untimed)
        if flush_buf is not None:
            flush_buf.zero_()

    t_wall = time.perf_counter()
    for i in range(args.steps):
        flush()
        run_step(cache, plan, qs, outs, seq, pt, args.tau, call_split, events=ev[i], stream=stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_ms = np.array([ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps)])
    launch_ms = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(ncell)]
                          for i in range(args.steps)])              # [step, cell]
    total_ms = ev[0][0].elapsed_time(ev[-1][-1])
    med_ms = float(np.median(step_ms))
    for o in outs:
        assert torch.isfinite(o).all()

    # The same step as one HIP graph (the library enqueues kernels only, so it is capturable).
    graph_ms, graph_note = None, "off"
    if not args.no_graph:
        outs_g = [torch.empty_like(o) for o in outs]

        def check():
            return all(torch.equal(a, b) for a, b in zip(outs_g, outs))

        graph_ms, graph_note = graph_time(
            lambda: run_step(cache, plan, qs, outs_g, seq, pt, args.tau, call_split), check, args.steps,
            advance=flush, eager_work=lambda: run_step(cache, plan, qs, outs, seq, pt, args.tau, call_split))
        log(f"[bench] graph: {graph_note}, {graph_ms} ms/step (eager {med_ms:.3f})")
    eager_ms = med_ms
    if graph_ms is not None and graph_ms < med_ms:   # the faster of the two launch modes
        med_ms = graph_ms

    n_split = (N + split - 1) // split if split else 1
    alg_bytes, per_cell_bytes = algorithmic_bytes(plan, hot_frac, B, N, n_split=n_split, v_group=args.v_group,
                                                  n_hist=cfg["n_hist"], n_exact=cfg["n_exact"])
    # Dominant kernel: the INT4-read decode (own INT4 cells and cells reusing an INT4 source).
    src_bits = np.array([plan[loops - 1, l] if plan[t, l] == 0 else plan[t, l]
                         for t in range(loops) for l in range(layers)])
    kinds = {}
    for bits in (4, 2):
        sel = src_bits == bits
        if sel.any():
            dur = float(launch_ms[:, sel].mean())                    # ms per launch
            byt = float(np.asarray(per_cell_bytes)[sel].mean())      # bytes per launch
            kinds[bits] = dict(launches_per_step=int(sel.sum()), avg_us=round(dur * 1e3, 1),
                               bytes_per_launch=int(byt), GBps=round(byt / (dur / 1e3) / 1e9, 1))
    dom = max(kinds, key=lambda b: kinds[b]["avg_us"] * kinds[b]["launches_per_step"])
    achieved = kinds[dom]["GBps"]

    # HBM traffic and kernel-trace durations come from stored rocprofv3 runs of this workload
    # (profiles/), used only while the decode sources match the ones they were taken on.
    traffic, traffic_src, trace_us, trace_src = None, None, None, None
    stored = (args.plan == "seeded" and args.v_group == 128 and args.split is None and args.pages == "shuffled"
              and args.tau == 0.01)
    tfile = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if stored and os.path.exists(tfile):
        tj = json.load(open(tfile))
        if tj.get("kernel_hash") == kernel_hash() and tj.get("workload") == args.workload:
            traffic = tj.get("hbm_bytes_per_launch")
            traffic_src = f"profiles/decode_traffic.json (rocprofv3 --pmc, kernel hash {tj['kernel_hash']})"
    kfile = os.path.join(ROOT, "profiles", "decode_kernel_trace.json")
    if stored and os.path.exists(kfile):
        kj = json.load(open(kfile))
        if kj.get("kernel_hash") == kernel_hash() and kj.get("workload") == args.workload:
            trace_us = kj.get("avg_us", {}).get(f"int{dom}_read")
            trace_src = f"profiles/decode_kernel_trace.json (rocprofv3 --kernel-trace --stats, kernel hash {kj['kernel_hash']})"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, plan, args.tau, args.seed, args.cpu_budget)

    line = {
        "metric": "fused LoopKV decode attn: µs/step and achieved HBM TB/s vs peak, 1 MI355X",
        "value": round(med_ms * 1e3, 1),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8 codes; fp16 scales and value weights; f32 scores and accumulation",
        "data": "synthetic (seeded Gaussian K/V/q, 4 outlier key channels x10 per cell and head)",
        "config": {"workload": args.workload, "layers": layers, "loops": loops, "cells": ncell,
                   "kv_heads": 16, "head_dim": 128, "batch": B, "context": N, "tau": args.tau,
                   "split_tokens": split, "split_auto": cfg["auto_split"],
                   "plan_counts": {"int4": int((plan == 4).sum()),
                                                          "int2": int((plan == 2).sum()),
                                                          "reuse": int((plan == 0).sum())},
                   "page_tokens": 32, "v_group": args.v_group, "plan": args.plan, "plan_seed": args.seed,
                   "sink_tokens": cfg["S"], "window_tokens": cfg["W"], "pages": args.pages},
        "achieved_TBps": round(alg_bytes / (med_ms / 1e3) / 1e12, 3),
        "hot_fraction": round(overall_hot, 4),
        "alg_bytes_per_step": int(alg_bytes),
        "mean_ms_per_step": round(total_ms / args.steps, 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "graph": {"used": graph_ms is not None and med_ms == graph_ms, "note": graph_note,
                  "launches_per_step": ncell, "ms_per_step": None if graph_ms is None else round(graph_ms, 4)},
        "wall_s_timed": round(t_wall, 3),
        "kernels": {f"decode_int{b}_read": v for b, v in kinds.items()},
        "roofline": {"bound": "hbm", "kernel": f"decode_kernel<{dom},...> (INT{dom}-read cells)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "avg_launch_us_events": kinds[dom]["avg_us"],
                     "avg_launch_us_kernel_trace": trace_us,
                     "frac_kernel_trace": (None if trace_us is None else
                                           round(kinds[dom]["bytes_per_launch"] / (trace_us * 1e-6) / 1e9
                                                 / PEAK_HBM_GBPS, 4)),
                     "traffic_source": traffic_src, "kernel_trace_source": trace_src},
        "cpu_baseline": cpu,
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
