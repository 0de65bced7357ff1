"""GPU parity for value magnitudes far from N(0, 1), the automatic split, and repeatability of
the sink + window + split path of a reusing cell.

Value scales are fp16 numbers of any size ("Loop-Aware KV Cache Compression for Serving Looped
Transformers", section 3.3 "Bit-plane V layout": a scale and a zero point per group), so decode
must stay finite and within tolerance for groups of magnitude 1e3 and 1e-3. With
split_tokens = LOOPKV_SPLIT_AUTO the library picks the split (section 3.4: up to 64 far blocks
per decode row, merged by the row's last block); the test reads the choice back through
loopkv_auto_split and gives the oracle the same split."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth
from tests.helpers import Workload, check_out, log

pytestmark = pytest.mark.gpu


def _mask_buf(w):
    return torch.full((w.B, w.H, w.page_table_np.shape[1] * w.P), 0xEE, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("scale", ["1e3", "1e-3", "mixed"])
def test_decode_value_magnitudes(bits, scale):
    """Values scaled by 1e3 (fp16 value scales up to ~500 for INT4 and ~2700 for INT2), by 1e-3,
    or per token by 10^U(-3, 3.5): outputs finite and within 2e-3 of the oracle's largest
    magnitude; fetch masks as the oracle's."""
    log(f"value magnitudes bits={bits} scale={scale}")
    plan = np.array([[bits]], np.uint8)
    w = Workload(plan, batch=3, lens=[700, 333, 1000], seed=71 + bits)
    v = w.v[0, 0].double()
    if scale == "mixed":
        g = torch.Generator().manual_seed(5)
        f = 10.0 ** (torch.rand(v.shape[0], v.shape[1], v.shape[2], 1, generator=g, dtype=torch.float64) * 6.5 - 3)
        v = v * f
    else:
        v = v * float(scale)
    w.v[0, 0] = v.to(torch.bfloat16)
    w.append_upto(w.lens, chunk=300)
    for tau, split in [(0.02, 0), (0.0, 128), (2.0, 0)]:
        q = synth.queries(3, 16, 128, 700 + bits).cuda()
        mask = _mask_buf(w)
        out = w.cache.decode(0, 0, q, w.seq_lens(0, 0), w.page_table, tau=tau, split_tokens=split,
                             fetch_mask=mask)
        ref, hot = w.oracle_decode(0, 0, q.cpu(), tau=tau, split_tokens=split)
        err = check_out(out, ref, f"bits {bits} scale {scale} tau {tau} split {split}")
        w.check_masks(mask, hot, 0, 0, q.cpu(), tau, split)
        log(f"  tau {tau} split {split}: relative error {err:.2e}, max |ref| {np.abs(ref).max():.3e}")
    assert w.cache.device_errors() == 0


def _expected_auto_split(batch, heads, ctx, cus, max_splits):
    """The rule loopkv.h states for LOOPKV_SPLIT_AUTO."""
    rows = batch * heads
    n = min(-(-4 * cus // rows), 64, max_splits, ctx // 1024)
    if n <= 1:
        return 0
    return -(-(-(-ctx // n)) // 32) * 32


@pytest.mark.parametrize("batch,n", [(1, 8192), (3, 6000), (40, 1000)])
def test_decode_auto_split(batch, n):
    """A decode with split_tokens = LOOPKV_SPLIT_AUTO equals the oracle at the split that
    loopkv_auto_split reports, for a plan with 4-bit, 2-bit and reusing cells; the reported split
    follows the stated rule."""
    log(f"auto split batch={batch} n={n}")
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    lens = np.full(batch, n, np.int32)
    lens[0] = max(n - 37, 1)
    w = Workload(plan, batch=batch, lens=lens, seed=83)
    w.append_upto(w.lens, chunk=4096)
    split = w.cache.auto_split(batch, w.page_table)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ctx = w.page_table_np.shape[1] * w.P
    assert split == _expected_auto_split(batch, 16, ctx, cus, 64), (split, cus, ctx)
    log(f"  auto split {split} tokens ({-(-ctx // split) if split else 1} splits per row, {cus} CUs)")
    for t in range(4):
        q = synth.queries(batch, 16, 128, 830 + t).cuda()
        mask = _mask_buf(w)
        out = w.cache.decode(0, t, q, w.seq_lens(t, 0), w.page_table, tau=0.01,
                             split_tokens=L.SPLIT_AUTO, fetch_mask=mask)
        ref, hot = w.oracle_decode(t, 0, q.cpu(), tau=0.01, split_tokens=split)
        check_out(out, ref, f"loop {t} auto split {split}")
        w.check_masks(mask, hot, t, 0, q.cpu(), 0.01, split)
        # the same call with the split spelled out is bit-identical
        out2 = w.cache.decode(0, t, q, w.seq_lens(t, 0), w.page_table, tau=0.01, split_tokens=split)
        assert torch.equal(out, out2)
    assert w.cache.device_errors() == 0


@pytest.mark.parametrize("split", [64, 128])
def test_sink_window_split_reuse_repeats(split):
    """The shape of the sink + window + split path of a reusing cell (4 ragged requests, 32-token
    sink, 256-token window, the reusing cell one token ahead of its INT4 source): three repeats
    of each decode are bit-identical, finite and equal to the oracle."""
    log(f"sink/window/split/reuse repeats split={split}")
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    lens = np.array([40, 330, 700, 1000], np.int32)
    w = Workload(plan, batch=4, lens=lens + 3, page_tokens=32, seed=71, sink_tokens=32,
                 window_tokens=256)
    w.append_upto(lens, chunk=128)
    for step in range(2):
        for t in range(4):
            w.append_upto(w.done[t, 0] + 1, cells=[(t, 0)])
            q = synth.queries(4, 16, 128, 900 + 10 * step + t)
            res = []
            for _ in range(3):
                mask = _mask_buf(w)
                out = w.cache.decode(0, t, q.cuda(), w.seq_lens(t, 0), w.page_table, tau=0.02,
                                     split_tokens=split, fetch_mask=mask)
                res.append((out.clone(), mask.clone()))
            for o, m in res[1:]:
                assert torch.equal(o, res[0][0]) and torch.equal(m, res[0][1]), (step, t)
            ref, hot = w.oracle_decode(t, 0, q, tau=0.02, split_tokens=split)
            check_out(res[0][0], ref, f"step {step} loop {t} split {split}")
            w.check_masks(res[0][1], hot, t, 0, q, 0.02, split)
        log(f"  step {step} ok")
    assert w.cache.device_errors() == 0


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("kind", ["spread", "zero_blocks"])
def test_decode_query_dynamic_range(bits, kind):
    """The history scores' query operand is rounded relative to the largest |q * s_K| of each
    32-channel block: queries whose channels span 10^-4 .. 10^1 (spread), or whose first and
    third 32-channel blocks are exactly zero for some heads (zero_blocks), still give outputs
    within 2e-3 of the oracle and its fetch masks."""
    log(f"query dynamic range bits={bits} kind={kind}")
    plan = np.array([[bits]], np.uint8)
    w = Workload(plan, batch=3, lens=[900, 417, 1200], seed=91 + bits)
    w.append_upto(w.lens, chunk=400)
    q = synth.queries(3, 16, 128, 910 + bits).double()
    g = torch.Generator().manual_seed(9 + bits)
    if kind == "spread":
        q = q * 10.0 ** (torch.rand(1, 1, 128, generator=g, dtype=torch.float64) * 5 - 4)
        q = q * 4.0   # keep the scores' spread like the unscaled queries'
    else:
        q[:, ::2, 0:32] = 0.0
        q[:, ::3, 64:96] = 0.0
    q = q.to(torch.bfloat16)
    for tau, split in [(0.01, 0), (0.02, 256)]:
        mask = _mask_buf(w)
        out = w.cache.decode(0, 0, q.cuda(), w.seq_lens(0, 0), w.page_table, tau=tau, split_tokens=split,
                             fetch_mask=mask)
        ref, hot = w.oracle_decode(0, 0, q, tau=tau, split_tokens=split)
        err = check_out(out, ref, f"bits {bits} {kind} tau {tau} split {split}")
        w.check_masks(mask, hot, 0, 0, q, tau, split)
        log(f"  tau {tau} split {split}: relative error {err:.2e}")
    assert w.cache.device_errors() == 0


def test_decode_max_splits():
    """The largest split count a row can take (64 splits of 32 tokens; the shorter request's last
    splits are empty), against the oracle for a 4-bit, a 2-bit and a reusing cell: every split's
    partials meet in the in-launch merge."""
    log("max splits")
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    lens = np.array([2048, 1500], np.int32)
    w = Workload(plan, batch=2, lens=lens, seed=131, max_splits=64)
    w.append_upto(lens, chunk=512)
    seq = torch.as_tensor(lens).cuda()
    for t in range(4):
        q = synth.queries(2, 16, 128, 1310 + t)
        mask = _mask_buf(w)
        out = w.cache.decode(0, t, q.cuda(), seq, w.page_table, tau=0.01, split_tokens=32, fetch_mask=mask)
        ref, hot = w.oracle_decode(t, 0, q, tau=0.01, split_tokens=32)
        check_out(out, ref, f"loop {t} split 32")
        w.check_masks(mask, hot, t, 0, q, 0.01, 32)
    assert w.cache.device_errors() == 0
