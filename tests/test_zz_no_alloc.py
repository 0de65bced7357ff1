"""loopkv_decode_attention_static (the decode entry point whose split workspace is the
library's fixed per-GPU array, for callers that cannot allocate) against loopkv_decode_attention
on the same inputs: bit-identical outputs and fetch masks, on two calls in a row, the second with
a smaller input; both also equal the oracle. A call beyond the array's capacity is refused."""
import numpy as np
import pytest
import torch

from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth
from tests.helpers import Workload, check_out, log

pytestmark = pytest.mark.gpu


def _mask_buf(w, B):
    return torch.full((B, w.H, w.page_table_np.shape[1] * w.P), 0xEE, dtype=torch.uint8, device="cuda")


def test_static_workspace_decode_matches_arena_decode():
    plan = np.array([[4], [2], [0], [4]], np.uint8)
    lens = np.array([2000, 1333, 1700, 990], np.int32)
    w = Workload(plan, batch=4, lens=lens, seed=97, max_splits=64)
    w.append_upto(w.lens, chunk=512)
    # call 1: all four requests, 256-token splits; call 2: the first two requests, 512-token splits
    for batch, split in [(4, 256), (2, 512)]:
        for t in range(4):
            log(f"static workspace: batch {batch} split {split} loop {t}")
            q = synth.queries(4, 16, 128, 970 + t)[:batch].contiguous()
            seq = w.seq_lens(t, 0)[:batch].contiguous()
            pt = w.page_table[:batch]
            m_ref, m_st = _mask_buf(w, batch), _mask_buf(w, batch)
            ref = w.cache.decode(0, t, q.cuda(), seq, pt, tau=0.02, split_tokens=split, fetch_mask=m_ref)
            got = w.cache.decode(0, t, q.cuda(), seq, pt, tau=0.02, split_tokens=split, fetch_mask=m_st,
                                 static_workspace=True)
            assert torch.equal(got, ref) and torch.equal(m_st, m_ref), (batch, split, t)
            orc, _ = w.oracle_decode(t, 0, synth.queries(4, 16, 128, 970 + t), tau=0.02, split_tokens=split)
            check_out(got, orc[:batch], f"static workspace batch {batch} split {split} loop {t}")
    assert w.cache.device_errors() == 0
    # beyond the array: 8 requests x 16 heads x 128 splits of 32 tokens x 520 bytes > 4 MiB - 64 KiB
    # (refused on the host, before anything is enqueued; nothing needs to be appended)
    w2 = Workload(np.array([[4]], np.uint8), batch=8, lens=[4096] * 8, seed=98, max_splits=128)
    q = synth.queries(8, 16, 128, 979).cuda()
    with pytest.raises(L.LoopKVError) as e:
        w2.cache.decode(0, 0, q, w2.seq_lens(0, 0), w2.page_table, tau=0.02, split_tokens=32,
                        static_workspace=True)
    assert e.value.status == L.ECAPACITY


def test_static_workspace_small_launch():
    """A small launch (one request, automatic split: two 1024-token splits in one-head
    workgroups of eight waves) through the fixed array equals the arena entry point and the
    oracle."""
    plan = np.array([[4], [0], [4]], np.uint8)
    lens = np.array([2040], np.int32)
    w = Workload(plan, batch=1, lens=lens, seed=99, max_splits=64)
    w.append_upto(w.lens, chunk=1024)
    split = w.cache.auto_split(1, w.page_table)
    assert split >= 1024, split
    for t in range(3):
        q = synth.queries(1, 16, 128, 990 + t)
        seq = w.seq_lens(t, 0)
        m_ref, m_st = _mask_buf(w, 1), _mask_buf(w, 1)
        ref = w.cache.decode(0, t, q.cuda(), seq, w.page_table, tau=0.01, split_tokens=L.SPLIT_AUTO,
                             fetch_mask=m_ref)
        got = w.cache.decode(0, t, q.cuda(), seq, w.page_table, tau=0.01, split_tokens=L.SPLIT_AUTO,
                             fetch_mask=m_st, static_workspace=True)
        assert torch.equal(got, ref) and torch.equal(m_st, m_ref), t
        orc, _ = w.oracle_decode(t, 0, q, tau=0.01, split_tokens=split)
        check_out(got, orc, f"static workspace small launch loop {t}")
    assert w.cache.device_errors() == 0
