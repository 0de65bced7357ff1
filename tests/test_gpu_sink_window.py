"""GPU parity with an exact sink and window: the first 32 tokens stay bf16, the most recent
`window` tokens stay bf16, a 32-token page is quantized when it leaves the window, and the sink's
largest score seeds the running maximum of the history ("Loop-Aware KV Cache Compression for
Serving Looped Transformers", section 2.3 "Measuring KV damage", section 3.2, section 3.4
"The unified kernel").

Pools, sinks, rings and counters are compared byte for byte with the oracle's window rule and
packing; outputs within 2e-3 of the oracle's largest magnitude; fetch masks bit for bit except
tokens within 1e-6 of tau."""
import numpy as np
import pytest
import torch

import oracle as O
from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth
from tests.helpers import Workload, check_out, log, to64

pytestmark = pytest.mark.gpu


def _mask_buf(w):
    return torch.full((w.B, w.H, w.page_table_np.shape[1] * w.P), 0xEE, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("bits,P", [(4, 32), (2, 16), (4, 16)])
def test_window_exit_append_bytes(bits, P):
    """Prefill in uneven chunks, then one token per call: groups are quantized exactly when
    they leave the 256-token window, the sink holds the first 32 tokens, the ring the rest."""
    log(f"window-exit append bits={bits} P={P}")
    w = Workload([[bits]], batch=3, lens=[400, 333, 290], page_tokens=P, seed=61,
                 sink_tokens=32, window_tokens=256)
    w.append_upto([300, 250, 20], chunk=77)
    w.append_upto(w.lens, chunk=1)
    pool = w.cache.own_pool(0, 0).cpu().numpy()
    ref = O.pack_pool(bits, P, w.quant(0, 0), w.page_table_np, w.num_pages, 128, hist_start=32)
    diff = np.nonzero(pool != ref)
    assert diff[0].size == 0, f"{diff[0].size} bytes differ, first at page {diff[0][:3]} byte {diff[1][:3]}"
    qg = w.cache.qgroups(0, 0).cpu().numpy().tolist()
    assert qg == [O.near_far_split(n, 32, 256)[2] // 32 for n in w.lens] == [4, 2, 1]
    sk, sv = w.cache.sink(0, 0)
    assert torch.equal(sk.cpu(), w.k[0, 0][:, :32]) and torch.equal(sv.cpu(), w.v[0, 0][:, :32])
    tk, _ = w.cache.tail(0, 0)
    tk = tk.cpu()
    ring = tk.shape[1]
    for b, n in enumerate(w.lens):
        for pos in range(O.near_far_split(int(n), 32, 256)[2], n):
            assert torch.equal(tk[b, pos % ring], w.k[0, 0][b, pos]), (b, pos)
    assert w.cache.device_errors() == 0


@pytest.mark.parametrize("P", [32, 16])
def test_decode_steps_sink_window(P):
    """Plan [4, 2, REUSE, 4] over one layer; ragged requests (all-exact, one group of history,
    many groups), prefill then decode steps in model order (append the step's token, then decode),
    so the reusing cell runs one token ahead of its source; splits of 0 and 128 tokens; the
    sink seed on and off."""
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    lens = np.array([40, 330, 700, 1000], np.int32)
    w = Workload(plan, batch=4, lens=lens + 3, page_tokens=P, seed=71, sink_tokens=32,
                 window_tokens=256)
    w.append_upto(lens, chunk=128)
    for step in range(3):
        for t in range(4):
            w.append_upto(w.done[t, 0] + 1, cells=[(t, 0)])
            q = synth.queries(4, 16, 128, 500 + 10 * step + t)
            for split, sink_seed in [(0, True), (128, True), (0, False)]:
                mask = _mask_buf(w)
                out = w.cache.decode(0, t, q.cuda(), w.seq_lens(t, 0), w.page_table, tau=0.02,
                                     split_tokens=split, fetch_mask=mask, sink_seed=sink_seed)
                ref, hot = w.oracle_decode(t, 0, q, tau=0.02, split_tokens=split, sink_seed=sink_seed)
                check_out(out, ref, f"step {step} loop {t} split {split} sink_seed {sink_seed}")
                w.check_masks(mask, hot, t, 0, q, 0.02, split, sink_seed=sink_seed)
        log(f"  step {step} ok")
    assert w.cache.device_errors() == 0


def test_dominant_sink_seed_all_cold():
    """A sink token aligned with every query scores far above the history: with the sink
    maximum as the seed no history token reads its low plane, and the output still matches."""
    w = Workload([[4]], batch=2, lens=[800, 611], seed=81, sink_tokens=32, window_tokens=256)
    q = synth.queries(2, 16, 128, 81)
    k = w.k[0, 0]
    k[:, 5] = (torch.sign(q.float()) * 8).to(torch.bfloat16)
    w.append_upto(w.lens, chunk=200)
    mask = _mask_buf(w)
    out = w.cache.decode(0, 0, q.cuda(), w.seq_lens(0, 0), w.page_table, tau=0.01, fetch_mask=mask)
    ref, hot = w.oracle_decode(0, 0, q, tau=0.01)
    check_out(out, ref, "dominant sink")
    assert not any(h.any() for row in hot for h in row)
    mk = mask.cpu().numpy()
    for b, n in enumerate(w.lens):
        he = O.near_far_split(int(n), 32, 256)[2]
        assert he > 32 and not mk[b, :, 32:he].any()
    # without the seed each row's largest history score reads its low plane
    mask0 = _mask_buf(w)
    w.cache.decode(0, 0, q.cuda(), w.seq_lens(0, 0), w.page_table, tau=0.01, fetch_mask=mask0,
                   sink_seed=False)
    assert mask0.cpu().numpy()[0, :, 32:O.near_far_split(800, 32, 256)[2]].any(axis=1).all()


def test_short_rows_sink_only():
    """Rows shorter than the sink, exactly the sink, and shorter than sink + window: all exact."""
    w = Workload([[4]], batch=4, lens=[0, 7, 32, 250], seed=91, sink_tokens=32, window_tokens=256)
    w.append_upto(w.lens, chunk=100)
    q = synth.queries(4, 16, 128, 91)
    st = torch.zeros(4, dtype=torch.int64, device="cuda")
    out = w.cache.decode(0, 0, q.cuda(), w.seq_lens(0, 0), w.page_table, tau=0.01,
                         stats=st)
    ref, _ = w.oracle_decode(0, 0, q, tau=0.01)
    assert torch.all(out[0] == 0)
    check_out(out, ref, "short rows")
    s = st.cpu().numpy()
    assert s[0] == 0 and s[3] == 16 * (7 + 32 + 250)
    assert w.cache.qgroups(0, 0).cpu().numpy().tolist() == [1, 1, 1, 1]
    assert w.cache.device_errors() == 0


def test_sink_window_eight_wave_rows():
    """A small launch of long rows (2 requests, one head per workgroup, eight waves per row:
    the launch is a single generation and each split spans at least 1024 tokens) with a sink
    and a window: unsplit, 1024-token splits and the automatic split, against the oracle and
    its fetch masks, for a 4-bit, a 2-bit and a reusing cell."""
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    lens = np.array([2300, 1450], np.int32)
    w = Workload(plan, batch=2, lens=lens, seed=141, sink_tokens=32, window_tokens=256)
    w.append_upto(lens, chunk=700)
    seq = torch.as_tensor(lens).cuda()
    auto = w.cache.auto_split(2, w.page_table)
    assert auto >= 1024, auto
    for t in range(4):
        q = synth.queries(2, 16, 128, 1410 + t)
        for split in (0, 1024, L.SPLIT_AUTO):
            ref_split = auto if split == L.SPLIT_AUTO else split
            mask = _mask_buf(w)
            out = w.cache.decode(0, t, q.cuda(), seq, w.page_table, tau=0.01, split_tokens=split,
                                 fetch_mask=mask)
            ref, hot = w.oracle_decode(t, 0, q, tau=0.01, split_tokens=ref_split)
            check_out(out, ref, f"loop {t} split {split}")
            w.check_masks(mask, hot, t, 0, q, 0.01, ref_split)
    assert w.cache.device_errors() == 0
