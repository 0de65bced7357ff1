"""GPU parity at full per-cell sizes, on sampled rows.

Each case builds one layer of four loops at a workload's full per-cell shape (batch, context,
heads, page size, split), fills it through quantize_append, decodes every cell through the C ABI
in the launch configuration the benchmark times, and checks a seeded sample of (request, head)
rows against the fp64 oracle, computed row by row from the same generated K/V:
  - outputs: max |out - ref| over the sampled rows <= 2e-3 * max |ref| over those rows;
  - fetch masks of cells that read 4-bit history: equal except tokens within 1e-6 of tau.
Shapes: the 96-cell 8K batch-64 cache (32-token pages), the paged serving batch (128 requests of
1K..16K tokens, 16-token pages in a shuffled table, one appended token per request per cell
before the decode), and the long-context shape (batch 16, 32K tokens, heavy-tailed keys,
8K-token splits merged by log-sum-exp), and the 8K batch-64 shape again with a 32-token sink and a
256-token window kept exact, and with 32-channel value groups (the paper's KIVI groups)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth
from quantized_kv_decode_amd.cache import LoopKVCache
from tests.helpers import assert_ties_rare, OUT_RTOL, check_mask, log

pytestmark = pytest.mark.gpu

PLAN = np.array([[4], [2], [0], [4]], np.uint8)   # loop 3 reuses the final loop's KV


def _run_case(name, *, B, lens, P, split, heavy, seed, rows_per_cell, append_one, S=0, W=0, VG=128):
    H, D, tau = 16, 128, 0.01
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int64)
    hist_len = lens - (1 if append_one else 0)     # tokens present before the decode step
    pt_np, npages = synth.page_table(lens, P, seed + 1, shuffle=True)
    pt = torch.as_tensor(pt_np).cuda()
    max_splits = max(1, int(pt_np.shape[1] * P // split)) if split else 1
    shape = L.make_shape(num_layers=1, num_loops=4, num_kv_heads=H, page_tokens=P, v_group=VG,
                         max_batch=B, max_pages_per_seq=pt_np.shape[1],
                         tail_tokens=64 if W == 0 else W + 64, max_splits=max_splits,
                         num_pages=npages, sink_tokens=S, window_tokens=W)
    cache = LoopKVCache(shape, PLAN, zero_arena=True)
    sample = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(rows_per_cell)]
    chunk = 4096
    kv_rows = {}   # (t, b, h) -> (k [n, D] f64, v [n, D] f64): every token the cell holds
    for t in range(4):
        log(f"[{name}] fill loop {t}")
        done = np.zeros(B, np.int64)
        parts = {bh: ([], []) for bh in sample}
        off = 0
        total = int(lens.max())
        while off < total:
            n = min(chunk, total - off)
            cs = seed * 1000 + t * 100
            k = synth.keys(B, n, H, D, cs, device="cuda", heavy_tail=heavy, token_offset=off)
            v = synth.values(B, n, H, D, cs, device="cuda", token_offset=off)
            for (b, h) in sample:
                m = int(max(0, min(n, lens[b] - off)))
                parts[b, h][0].append(k[b, :m, h].float().cpu().double().numpy())
                parts[b, h][1].append(v[b, :m, h].float().cpu().double().numpy())
            # before the decode step each request holds hist_len tokens; the last one (when
            # append_one) is appended on its own below, as a decode step does
            m_new = np.clip(hist_len - off, 0, n).astype(np.int32)
            if m_new.any():
                cache.append(0, t, k.contiguous(), v.contiguous(), torch.as_tensor(done.astype(np.int32)).cuda(),
                             pt, n_new=torch.as_tensor(m_new).cuda())
                done += m_new
            del k, v
            off += n
        if append_one:
            # the decode step's own token (position hist_len) for every request
            k1 = torch.zeros(B, 1, H, D, dtype=torch.bfloat16)
            v1 = torch.zeros_like(k1)
            # regenerate the chunks holding each request's last token, copy that token
            starts = (hist_len // chunk) * chunk
            for c0 in sorted(set(starts.tolist())):
                n = min(chunk, total - c0)
                cs = seed * 1000 + t * 100
                k = synth.keys(B, n, H, D, cs, device="cuda", heavy_tail=heavy, token_offset=c0)
                v = synth.values(B, n, H, D, cs, device="cuda", token_offset=c0)
                for b in np.nonzero(starts == c0)[0]:
                    k1[b, 0] = k[b, int(hist_len[b] - c0)].cpu()
                    v1[b, 0] = v[b, int(hist_len[b] - c0)].cpu()
                del k, v
            cache.append(0, t, k1.cuda(), v1.cuda(), torch.as_tensor(done.astype(np.int32)).cuda(), pt)
            done += 1
        assert np.array_equal(done, lens)
        for (b, h) in sample:
            kv_rows[t, b, h] = (np.concatenate(parts[b, h][0]), np.concatenate(parts[b, h][1]))
    torch.cuda.synchronize()
    assert cache.device_errors() == 0

    seq = torch.as_tensor(lens.astype(np.int32)).cuda()
    for t in range(4):
        src = 3 if PLAN[t, 0] == L.REUSE else t
        bits = int(PLAN[src, 0])
        q = synth.queries(B, H, D, seed * 10 + t)
        mask = torch.full((B, H, pt_np.shape[1] * P), 0xEE, dtype=torch.uint8, device="cuda")
        log(f"[{name}] decode loop {t} (reads {bits}-bit history, split {split})")
        out = cache.decode(0, t, q.cuda(), seq, pt, tau=tau, split_tokens=split,
                           fetch_mask=mask if bits == 4 else None)
        out = out.cpu().double().numpy()
        mk = mask.cpu().numpy()
        q64 = q.float().double().numpy()
        errs, refmax, ties, compared = 0.0, 0.0, 0, 0
        for (b, h) in sample:
            n = int(lens[b])
            # sink [0, se), quantized history [S, he), exact tail [he, n)
            se, _, he = O.near_far_split(n, S, W)
            ks, vs = kv_rows[src, b, h]
            qh = O.quantize_head(ks[S:he], vs[S:he], bits, VG)
            kt, vt = kv_rows[t, b, h]
            ref, hot, s = O.decode_head(q64[b, h], qh, kt[he:n], vt[he:n], sm_scale=1 / math.sqrt(D),
                                        tau=tau, split_tokens=split, sink_k=kt[:se], sink_v=vt[:se],
                                        hist_start=S)
            errs = max(errs, float(np.abs(out[b, h] - ref).max()))
            refmax = max(refmax, float(np.abs(ref).max()))
            if bits == 4:
                m0 = float((kt[:se] @ q64[b, h]).max()) / math.sqrt(D) if se else -math.inf
                tie = O.tie_mask(s, m0, tau, split, start=S)
                ties += check_mask(mk[b, h, S:], hot, tie, f"[{name}] loop {t} b={b} h={h}")
                compared += hot.shape[0]
        assert_ties_rare(ties, compared, f"[{name}] loop {t}")
        log(f"[{name}] loop {t}: max err {errs:.3e}, max |ref| {refmax:.3e}, ties {ties}")
        assert errs <= OUT_RTOL * refmax, f"[{name}] loop {t}: {errs:.3e} > {OUT_RTOL} * {refmax:.3e}"
    assert cache.device_errors() == 0


def test_fullsize_ouro14b_b64_ctx8k():
    """The benchmark's per-cell shape: batch 64, 8192 tokens, 32-token pages, one split."""
    _run_case("b64-ctx8k", B=64, lens=[8192] * 64, P=32, split=0, heavy=False, seed=301,
              rows_per_cell=8, append_one=False)


def test_fullsize_paged_serving_batch():
    """Batch 128, lengths uniform in [1K, 16K], 16-token pages in a shuffled table, and one
    appended token per request per cell before the decode."""
    lens = np.random.default_rng(302).integers(1024, 16385, size=128)
    _run_case("paged-b128", B=128, lens=lens, P=16, split=0, heavy=False, seed=302,
              rows_per_cell=8, append_one=True)


def test_fullsize_long_context_splits():
    """Batch 16, 32768 tokens, heavy-tailed key outliers, 8192-token splits."""
    _run_case("b16-ctx32k", B=16, lens=[32768] * 16, P=32, split=8192, heavy=True, seed=303,
              rows_per_cell=4, append_one=False)


def test_fullsize_ouro14b_b64_ctx8k_sink_window():
    """The benchmark's per-cell shape in the paper's serving setting: a 32-token sink and a
    256-token window stay exact, the 7904 tokens between are quantized history."""
    _run_case("b64-ctx8k-sink-window", B=64, lens=[8192] * 64, P=32, split=0, heavy=False, seed=304,
              rows_per_cell=8, append_one=False, S=32, W=256)


def test_fullsize_ouro14b_b64_ctx8k_value_groups_32():
    """The benchmark's per-cell shape with 32-channel value groups (four value scales per token
    and head), as in the paper's KIVI configurations."""
    _run_case("b64-ctx8k-vg32", B=64, lens=[8192] * 64, P=32, split=0, heavy=False, seed=305,
              rows_per_cell=8, append_one=False, VG=32)
