"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Codes, planes, scales and rings must match byte for byte; fetch masks bit for bit except
tokens whose test value lies within 1e-6 of tau; outputs within 2e-3 of the oracle's largest
magnitude per call."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth
from tests.helpers import assert_ties_rare, Workload, check_mask, check_out, log, to64

pytestmark = pytest.mark.gpu


def _mask_buf(w):
    return torch.full((w.B, w.H, w.page_table_np.shape[1] * w.P), 0xEE, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("P", [32, 16])
@pytest.mark.parametrize("v_group", [128, 32])
def test_append_bytes_exact(bits, P, v_group):
    """Pool bytes after appends in uneven chunks (so groups straddle calls and read the ring)
    equal the oracle's packing of its own quantization."""
    log(f"append bits={bits} P={P} G={v_group}")
    w = Workload([[bits]], batch=3, lens=[256, 200, 45], page_tokens=P, v_group=v_group, seed=3)
    w.append_upto([100, 77, 45], chunk=37)
    w.append_upto(w.lens, chunk=61)
    pool = w.cache.own_pool(0, 0).cpu().numpy()
    qh = w.quant(0, 0)
    ref = O.pack_pool(bits, P, qh, w.page_table_np, w.num_pages, v_group)
    diff = np.nonzero(pool != ref)
    assert diff[0].size == 0, f"{diff[0].size} bytes differ, first at page {diff[0][:3]} byte {diff[1][:3]}"
    assert w.cache.qgroups(0, 0).cpu().numpy().tolist() == [8, 6, 1]
    tk, tv = w.cache.tail(0, 0)
    tk = tk.cpu()
    for b, n in enumerate(w.lens):
        for pos in range(max(0, n - 64), n):
            assert torch.equal(tk[b, pos % 64], w.k[0, 0][b, pos]), (b, pos)
    assert w.cache.device_errors() == 0


def test_append_scale_edge_values():
    """Constant groups (scale 0), fp16-subnormal minima (rounding ties to even) and a channel
    spanning a wide range quantize exactly as the oracle does."""
    log("append edge values")
    w = Workload([[4]], batch=1, lens=[64], seed=5)
    k = w.k[0, 0]
    k[0, :32, 0, :] = 0.75                      # constant group: s = 0
    k[0, :32, 1, 3] = torch.tensor(2.0 ** -25, dtype=torch.bfloat16)
    k[0, 7, 1, 3] = torch.tensor(2.0 ** -25 + 15 * 2.0 ** -20, dtype=torch.bfloat16)
    k[0, 32:, 2, 5] = torch.linspace(-300, 300, 32).to(torch.bfloat16)
    w.v[0, 0][0, 5, 3, :] = -1.25
    w.append_upto(w.lens)
    pool = w.cache.own_pool(0, 0).cpu().numpy()
    ref = O.pack_pool(4, 32, w.quant(0, 0), w.page_table_np, w.num_pages, 128)
    assert np.array_equal(pool, ref)


def test_decode_single_cell_int4():
    """One INT4 cell: batch 1, 16 heads x 128, 256 tokens, tau = 0.01, one bf16 query."""
    log("decode single cell")
    w = Workload([[4]], batch=1, lens=[256], seed=11)
    w.append_upto(w.lens)
    q = synth.queries(1, 16, 128, 11)
    for split in [0, 64]:
        mask = _mask_buf(w)
        out = w.cache.decode(0, 0, q.cuda(), torch.tensor([256], dtype=torch.int32, device="cuda"),
                             w.page_table, tau=0.01, split_tokens=split, fetch_mask=mask)
        ref, hot = w.oracle_decode(0, 0, q, tau=0.01, split_tokens=split)
        check_out(out, ref, f"split={split}")
        w.check_masks(mask, hot, 0, 0, q, 0.01, split)
        assert not all(h.all() for h in hot[0]) and any(h.any() for h in hot[0])


@pytest.mark.parametrize("variant", ["A", "B"])
def test_decode_one_layer_four_loops(variant):
    """One layer, 4 loops, plan [4, 4, 2, 4] (A) or loop 3 reusing loop 4 (B); batch 8, 16 x 128,
    4096 tokens; tau in {0, 0.005, 0.02, 2}; 1024-token splits."""
    plan = np.array([[4], [4], [2 if variant == "A" else 0], [4]], np.uint8)
    log(f"decode 1x4 plan {variant}")
    w = Workload(plan, batch=8, lens=[4096] * 8, seed=21)
    if variant == "B":
        # the reusing cell's descriptor reads the final loop's pool and stores nothing
        # (section 3.2, C2)
        reuse, src = w.cache.cell_info(0, 2), w.cache.cell_info(0, 3)
        assert reuse.code == 0 and reuse.own_pool_dev is None
        assert reuse.read_pool_dev == src.own_pool_dev == src.read_pool_dev
        assert (reuse.read_bits, reuse.gated, reuse.page_bytes) == (4, 1, src.page_bytes)
        assert reuse.qgroups_dev is None or reuse.qgroups_dev != src.qgroups_dev
    w.append_upto(w.lens)
    seq = torch.full((8,), 4096, dtype=torch.int32, device="cuda")
    for t in range(4):
        q = synth.queries(8, 16, 128, 100 + t)
        for tau in [0.0, 0.005, 0.02, 2.0]:
            mask = _mask_buf(w)
            out = w.cache.decode(0, t, q.cuda(), seq, w.page_table, tau=tau, split_tokens=1024, fetch_mask=mask)
            ref, hot = w.oracle_decode(t, 0, q, tau=tau, split_tokens=1024)
            check_out(out, ref, f"loop {t} tau {tau}")
            w.check_masks(mask, hot, t, 0, q, tau, 1024)
            log(f"  loop {t} tau {tau} ok")
    assert w.cache.device_errors() == 0


def test_decode_steps_with_tails_ragged_paged():
    """Ragged lengths, 16-token pages in a shuffled table, seeds, and decode steps that append one
    token per request per cell before decoding (own cells quantize each group as it completes;
    the reusing cell reads the final loop's groups and its own exact tail)."""
    plan = np.array([[4, 2], [0, 4], [4, 0], [2, 4]], np.uint8)
    lens = np.array([40, 97, 31, 130, 64], np.int32)
    w = Workload(plan, batch=5, lens=lens + 40, page_tokens=16, seed=31)
    w.append_upto(lens, chunk=50)
    m0 = synth.seeds(5, 16, 31).numpy().astype(np.float32).astype(np.float64)
    seed_dev = torch.as_tensor(m0, dtype=torch.float32).cuda()
    for step in range(3):
        # A decode step in model order: each cell appends the new token, then decodes. A
        # reusing cell (loops 1 and 2 here) runs before the final loop has appended.
        for t in range(4):
            for l in range(2):
                w.append_upto(w.done[t, l] + 1, cells=[(t, l)])
                q = synth.queries(5, 16, 128, 1000 * step + 10 * t + l)
                mask = _mask_buf(w)
                out = w.cache.decode(l, t, q.cuda(), w.seq_lens(t, l), w.page_table, tau=0.02,
                                     seed=seed_dev, fetch_mask=mask)
                ref, hot = w.oracle_decode(t, l, q, tau=0.02, m0=m0)
                check_out(out, ref, f"step {step} cell ({t},{l})")
                w.check_masks(mask, hot, t, l, q, 0.02, 0, m0)
        log(f"  step {step} ok")
    assert w.cache.device_errors() == 0


def test_decode_empty_and_tail_only_rows():
    """A request with no tokens gets zeros; requests shorter than one group are all tail."""
    w = Workload([[4]], batch=3, lens=[0, 5, 33], seed=41)
    w.append_upto(w.lens)
    q = synth.queries(3, 16, 128, 41)
    out = w.cache.decode(0, 0, q.cuda(), w.seq_lens(0, 0), w.page_table, tau=0.01)
    ref, _ = w.oracle_decode(0, 0, q, tau=0.01)
    assert torch.all(out[0] == 0)
    check_out(out, ref, "short rows")


def test_misaligned_inputs_rejected_before_launch():
    """k_new, v_new and q are read in 16-byte pieces: a pointer off that alignment is an
    argument error, and nothing is enqueued."""
    w = Workload([[4]], batch=2, lens=[40, 40], seed=52)
    w.append_upto([32, 32])
    before = w.cache.own_pool(0, 0).clone()
    kk = torch.zeros(2 * 8 * 16 * 128 + 8, dtype=torch.bfloat16, device="cuda")
    k_off = kk[1:1 + 2 * 8 * 16 * 128]                      # 2 bytes past an aligned base
    seq = w.seq_lens(0, 0)
    for args in [(k_off.data_ptr(), kk.data_ptr()), (kk.data_ptr(), k_off.data_ptr())]:
        with pytest.raises(L.LoopKVError) as e:
            L.loopkv_quantize_append(w.cache.handle, 0, 0, *args, 2, 8, None, seq.data_ptr(),
                                     w.page_table.data_ptr(), w.page_table.stride(0), 0)
        assert e.value.status == L.EINVAL
    q = torch.zeros(2 * 16 * 128 + 8, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(2, 16, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_decode_attention(w.cache.handle, 0, 0, q[1:].data_ptr(), 2, seq.data_ptr(),
                                  w.page_table.data_ptr(), w.page_table.stride(0), None,
                                  out.data_ptr(), 0)
    assert e.value.status == L.EINVAL
    torch.cuda.synchronize()
    assert torch.equal(w.cache.own_pool(0, 0), before) and torch.all(out == 0)
    assert w.cache.device_errors() == 0


def test_device_errors_flag_bad_lengths():
    w = Workload([[2]], batch=2, lens=[64, 64], seed=51)
    w.append_upto(w.lens)
    q = synth.queries(2, 16, 128, 51)
    assert w.cache.device_errors() == 0
    bad = torch.tensor([64, 10 ** 6], dtype=torch.int32, device="cuda")
    out = w.cache.decode(0, 0, q.cuda(), bad, w.page_table, tau=0.0)
    assert w.cache.device_errors() & L.ERR_LENGTH
    assert torch.all(out[1] == 0)
    assert w.cache.device_errors() == 0


@pytest.mark.parametrize("v_group", [64, 32])
def test_decode_value_groups(v_group):
    """64- and 32-channel value groups (two and four value scales per token and head): plan
    [4, 2, REUSE, 4], ragged lengths, splits of 0 and 256 tokens, tau in {0, 0.02}."""
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    w = Workload(plan, batch=3, lens=[700, 333, 64], v_group=v_group, seed=61 + v_group)
    w.append_upto(w.lens, chunk=200)
    for t in range(4):
        q = synth.queries(3, 16, 128, 300 + t)
        for tau, split in [(0.0, 0), (0.02, 0), (0.02, 256)]:
            mask = _mask_buf(w)
            out = w.cache.decode(0, t, q.cuda(), w.seq_lens(t, 0), w.page_table, tau=tau,
                                 split_tokens=split, fetch_mask=mask)
            ref, hot = w.oracle_decode(t, 0, q, tau=tau, split_tokens=split)
            check_out(out, ref, f"G={v_group} loop {t} tau {tau} split {split}")
            w.check_masks(mask, hot, t, 0, q, tau, split)
    assert w.cache.device_errors() == 0


@pytest.mark.parametrize("heads,batch", [(1, 3), (6, 3), (20, 52), (4, 1100)])
def test_decode_head_counts(heads, batch):
    """Head counts off the 16-head shape: 1 and 6 heads (one head per workgroup), 20 heads x
    52 requests (260 four-head workgroups on 256 CUs: more than one generation, so requests are
    taken longest first), and 4 heads x 1100 requests (above the batch the longest-first order
    covers: launch order). Plan [4, 2, REUSE, 4], ragged lengths, tau 0.02."""
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    rng = np.random.default_rng(300 + heads)
    lens = rng.integers(33, 230 if batch < 1000 else 100, size=batch).astype(np.int32)
    log(f"decode heads={heads} batch={batch}")
    w = Workload(plan, batch=batch, lens=lens, heads=heads, seed=91 + heads)
    w.append_upto(w.lens, chunk=100)
    for t in range(4):
        q = synth.queries(batch, heads, 128, 700 + 10 * heads + t)
        mask = _mask_buf(w)
        out = w.cache.decode(0, t, q.cuda(), w.seq_lens(t, 0), w.page_table, tau=0.02, fetch_mask=mask)
        ref, hot = w.oracle_decode(t, 0, q, tau=0.02)
        check_out(out, ref, f"heads {heads} loop {t}")
        w.check_masks(mask, hot, t, 0, q, 0.02, 0)
    assert w.cache.device_errors() == 0


@pytest.mark.parametrize("bits", [4, 2])
def test_append_half_step_ties(bits):
    """Values exactly half a step above a code, x = z + (k + 1/2) s, for scales 1, 3, 5, 7 and 3/8
    and zero points 0, -7 and 2 (all exact in bf16 / fp16): the rounding rule rounds them up.
    The kernel's fp32 estimate sits on the boundary there (and with an inexact reciprocal of s
    may fall on either side), so the fp64 rule must decide. Keys along channels' groups, values
    along tokens' channels; pool bytes must equal the oracle's."""
    levels = (1 << bits) - 1
    w = Workload([[bits]], batch=1, lens=[64], seed=57)
    cases = [(1.0, 0.0), (3.0, 0.0), (5.0, -7.0), (7.0, 2.0), (0.375, -7.0), (3.0, 2.0)]

    def pattern(step, zero, n):
        ties = [zero, zero + levels * step] + [zero + (k + 0.5) * step for k in range(levels)]
        return torch.tensor((ties * n)[:n], dtype=torch.float64).to(torch.bfloat16), ties

    for j, (step, zero) in enumerate(cases):
        col, ties = pattern(step, zero, 32)
        assert torch.equal(col.double(), torch.tensor((ties * 32)[:32], dtype=torch.float64))
        w.k[0, 0][0, :32, 1 + j % 3, 7 + 11 * j] = col
        row, _ = pattern(step, zero, 128)
        w.v[0, 0][0, 33 + 2 * j, 2, :] = row
    w.append_upto(w.lens)
    qh = w.quant(0, 0)
    for j, (step, zero) in enumerate(cases):
        kc = qh[0][1 + j % 3].k_codes[:32, 7 + 11 * j]
        assert list(kc[2:2 + levels]) == list(range(1, levels + 1)), (step, zero)
    pool = w.cache.own_pool(0, 0).cpu().numpy()
    ref = O.pack_pool(bits, 32, qh, w.page_table_np, w.num_pages, 128)
    assert np.array_equal(pool, ref)


def test_decode_argument_errors():
    """Each invalid decode argument is an error status before anything is enqueued: tau negative
    or not finite, a negative or non-finite score scale, split_tokens not a multiple of 32, a
    mask row shorter than the context, more splits than the workspace holds, a batch above the
    shape's, a cell outside the plan. The output buffer stays untouched."""
    w = Workload([[4]], batch=2, lens=[64, 64], seed=53, max_splits=2, stride_extra=2)
    w.append_upto(w.lens)
    q = synth.queries(2, 16, 128, 53).cuda()
    seq = w.seq_lens(0, 0)
    out = torch.full((2, 16, 128), 7.0, dtype=torch.float32, device="cuda")
    ctx = w.page_table_np.shape[1] * 32
    mask = torch.zeros((2, 16, ctx), dtype=torch.uint8, device="cuda")

    def call(layer=0, loop=0, batch=2, **o):
        opts = L.DecodeOpts(o.get("tau", 0.0), o.get("sm", 0.0), o.get("split", 0), o.get("stride", 0),
                            None, o.get("mask"), None, 0)
        L.loopkv_decode_attention(w.cache.handle, layer, loop, q.data_ptr(), batch, seq.data_ptr(),
                                  w.page_table.data_ptr(), w.page_table.stride(0), opts, out.data_ptr(), 0)

    cases = [(dict(tau=-0.1), L.EINVAL), (dict(tau=math.nan), L.EINVAL), (dict(tau=math.inf), L.EINVAL),
             (dict(sm=-1.0), L.EINVAL), (dict(sm=math.nan), L.EINVAL), (dict(split=48), L.EINVAL),
             (dict(split=-32), L.EINVAL), (dict(mask=mask.data_ptr(), stride=ctx - 1), L.EINVAL),
             (dict(split=32), L.ECAPACITY), (dict(batch=3), L.EINVAL), (dict(batch=0), L.EINVAL),
             (dict(layer=1), L.EINVAL), (dict(loop=1), L.EINVAL), (dict(loop=-1), L.EINVAL)]
    for kw, status in cases:
        with pytest.raises(L.LoopKVError) as e:
            call(**kw)
        assert e.value.status == status, kw
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(mask == 0)
    call(split=32 * (ctx // 64 + 1))                 # two splits: within the workspace
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out)) and not torch.all(out == 7.0)
    assert w.cache.device_errors() == 0


def test_append_argument_errors():
    """Invalid append arguments are error statuses with nothing enqueued (a batch above the
    shape's, more new tokens than a row can hold, a cell outside the plan, a null pointer), and
    n_new == 0 is a no-op."""
    w = Workload([[4]], batch=2, lens=[64, 64], seed=54)
    w.append_upto([40, 40])
    before = [w.cache.own_pool(0, 0).clone(), *[t.clone() for t in w.cache.tail(0, 0)],
              w.cache.qgroups(0, 0).clone()]
    cap = w.page_table_np.shape[1] * 32
    kk = torch.zeros(3, cap + 32, 16, 128, dtype=torch.bfloat16, device="cuda")
    seq = w.seq_lens(0, 0)

    def call(layer=0, loop=0, batch=2, n_new=1, k=kk.data_ptr(), lens=seq.data_ptr()):
        L.loopkv_quantize_append(w.cache.handle, layer, loop, k, kk.data_ptr(), batch, n_new, None, lens,
                                 w.page_table.data_ptr(), w.page_table.stride(0), 0)

    for kw in [dict(batch=3), dict(batch=0), dict(n_new=cap + 1), dict(n_new=-1), dict(layer=1),
               dict(loop=1), dict(k=None), dict(lens=None)]:
        with pytest.raises(L.LoopKVError) as e:
            call(**kw)
        assert e.value.status == L.EINVAL, kw
    call(n_new=0)
    torch.cuda.synchronize()
    after = [w.cache.own_pool(0, 0), *w.cache.tail(0, 0), w.cache.qgroups(0, 0)]
    assert all(torch.equal(a, b) for a, b in zip(before, after))
    assert w.cache.device_errors() == 0


@pytest.mark.parametrize("split", [0, 128])
def test_decode_repeats_bit_identical(split):
    """The same decode call, repeated, gives bit-identical outputs and fetch masks: the kernels
    combine waves and splits in a fixed order and take no data-dependent schedule."""
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    w = Workload(plan, batch=4, lens=[700, 333, 1000, 64], seed=61)
    w.append_upto(w.lens, chunk=256)
    for t in range(4):
        q = synth.queries(4, 16, 128, 610 + t).cuda()
        res = []
        for _ in range(3):
            mask = _mask_buf(w)
            out = w.cache.decode(0, t, q, w.seq_lens(t, 0), w.page_table, tau=0.02, split_tokens=split,
                                 fetch_mask=mask)
            res.append((out.clone(), mask.clone()))
        for o, m in res[1:]:
            assert torch.equal(o, res[0][0]) and torch.equal(m, res[0][1]), f"loop {t} split {split}"
    assert w.cache.device_errors() == 0


def test_fetch_mask_contents_int2_and_tail():
    """The fetch mask as the header states it: 1 for every history token of a cell read at 2 bits,
    0 or 1 for a 4-bit cell's history, and the tail's entries (tokens not yet quantized) left as
    they were."""
    plan = np.array([[2, 4]], np.uint8)          # one loop, two layers: INT2 and INT4
    lens = np.array([100, 45, 257], np.int32)
    w = Workload(plan, batch=3, lens=lens, seed=63)
    w.append_upto(w.lens, chunk=50)
    q = synth.queries(3, 16, 128, 630).cuda()
    for layer, bits in [(0, 2), (1, 4)]:
        mask = _mask_buf(w)
        w.cache.decode(layer, 0, q, w.seq_lens(0, layer), w.page_table, tau=0.02, fetch_mask=mask)
        mk = mask.cpu().numpy()
        for b, n in enumerate(lens):
            hist = (int(n) // 32) * 32
            if bits == 2:
                assert (mk[b, :, :hist] == 1).all()
            else:
                assert np.isin(mk[b, :, :hist], [0, 1]).all()
            assert (mk[b, :, hist:] == 0xEE).all(), (layer, b)
    assert w.cache.device_errors() == 0


def test_stats_counters_match_oracle():
    """The optional counters as the header defines them, accumulated over two calls: history
    (token, head) pairs read, those whose low plane was read (the oracle's hot count, up to tokens
    within the tau tie band), pairs read from 4-bit pools, and exact pairs."""
    plan = np.array([[2, 4]], np.uint8)
    lens = np.array([300, 129, 64], np.int32)
    w = Workload(plan, batch=3, lens=lens, seed=64)
    w.append_upto(w.lens, chunk=100)
    q = synth.queries(3, 16, 128, 640)
    hist = sum((int(n) // 32) * 32 for n in lens) * 16
    exact = sum(int(n) % 32 for n in lens) * 16
    for layer, bits in [(0, 2), (1, 4)]:
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        for _ in range(2):
            w.cache.decode(layer, 0, q.cuda(), w.seq_lens(0, layer), w.page_table, tau=0.02, stats=st)
        s = st.cpu().numpy().tolist()
        assert s[0] == 2 * hist and s[3] == 2 * exact
        if bits == 2:
            assert s[1] == 0 and s[2] == 0
        else:
            _, hot = w.oracle_decode(0, layer, q, tau=0.02)
            n_hot = sum(int(h.sum()) for row in hot for h in row)
            qh = w.quant(0, layer, w.hist(0, layer))
            q64 = to64(q)
            n_tie = 0
            for b in range(3):
                for h in range(16):
                    kh = O.dequant_keys(qh[b][h].k_codes, qh[b][h].k_s, qh[b][h].k_z)
                    n_tie += int(O.tie_mask((kh @ q64[b, h]) / np.sqrt(128.0), -np.inf, 0.02, 0).sum())
            assert s[2] == 2 * hist
            assert abs(s[1] - 2 * n_hot) <= 2 * n_tie, (s[1], 2 * n_hot, n_tie)
            assert_ties_rare(n_tie, hist, "stats test")
    assert w.cache.device_errors() == 0
