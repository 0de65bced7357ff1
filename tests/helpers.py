"""Shared helpers for the GPU parity tests: build caches through the C ABI, feed the same
seeded inputs to the oracle, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth
from quantized_kv_decode_amd.cache import LoopKVCache

OUT_RTOL = 2e-3   # max |out - ref| <= OUT_RTOL * max |ref| per call


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def check_out(out: torch.Tensor, ref: np.ndarray, what: str = "") -> float:
    o = out.detach().cpu().double().numpy()
    err = float(np.abs(o - ref).max()) if o.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    assert np.all(np.isfinite(o)), what
    assert err <= OUT_RTOL * max(scale, 1e-30), f"{what}: max err {err:.3e} vs {OUT_RTOL} * {scale:.3e}"
    return err / max(scale, 1e-30)


TIE_RATE = 1e-4   # near-tau ties the mask comparison may skip, as a share of compared tokens
TIE_FLOOR = 4     # small samples: a few ties are expected by chance (~5e-5 per token at tau 0.02)


def assert_ties_rare(n_ties: int, n_compared: int, what: str = "") -> None:
    """The tie band excuses only a sliver of the compared fetch decisions."""
    assert n_ties <= TIE_FLOOR + TIE_RATE * n_compared, f"{what}: {n_ties} ties among {n_compared} tokens"


def check_mask(mask_row: np.ndarray, hot: np.ndarray, tie: np.ndarray, what: str = "") -> int:
    n = hot.shape[0]
    got = mask_row[:n].astype(bool)
    bad = (got != hot) & ~tie
    assert not bad.any(), f"{what}: {int(bad.sum())} mask mismatches (first at {np.nonzero(bad)[0][:5]})"
    return int(tie.sum())


class Workload:
    """A seeded cache of T loops x L layers. Per cell, K and V are drawn on the CPU (bf16) and
    appended through the library; the oracle sees the same bf16 values."""

    def __init__(self, plan, *, batch, lens, page_tokens=32, v_group=128, heads=16, seed=0,
                 tail_tokens=None, max_splits=64, shuffle=True, heavy_tail=False, stride_extra=0,
                 sink_tokens=0, window_tokens=0):
        self.plan = np.asarray(plan, np.uint8)
        T, Lr = self.plan.shape
        self.T, self.L, self.B, self.H, self.D = T, Lr, batch, heads, 128
        self.P, self.v_group, self.seed = page_tokens, v_group, seed
        self.S, self.W = sink_tokens, window_tokens
        if tail_tokens is None:
            tail_tokens = 64 if window_tokens == 0 else window_tokens + 64
        self.lens = np.asarray(lens, np.int32)
        self.nmax = max(int(self.lens.max()) if len(self.lens) else 0, 1)
        ptab, npages = synth.page_table(self.lens, page_tokens, seed + 17, shuffle=shuffle)
        stride = max(ptab.shape[1], 1) + stride_extra
        pt = np.full((batch, stride), -1, np.int32)
        pt[:, :ptab.shape[1]] = ptab
        self.page_table_np = pt
        self.num_pages = max(npages, 1)
        self.shape = L.make_shape(num_layers=Lr, num_loops=T, num_kv_heads=heads, page_tokens=page_tokens,
                                  v_group=v_group, max_batch=batch, max_pages_per_seq=stride,
                                  tail_tokens=tail_tokens, max_splits=max_splits, num_pages=self.num_pages,
                                  sink_tokens=sink_tokens, window_tokens=window_tokens)
        self.cache = LoopKVCache(self.shape, self.plan, zero_arena=True)
        self.page_table = torch.as_tensor(pt).cuda()
        self.k, self.v = {}, {}
        for t in range(T):
            for l in range(Lr):
                cs = seed * 1000 + t * 100 + l
                self.k[t, l] = synth.keys(batch, self.nmax, heads, 128, cs, heavy_tail=heavy_tail)
                self.v[t, l] = synth.values(batch, self.nmax, heads, 128, cs)
        self.done = {(t, l): np.zeros(batch, np.int64) for t in range(T) for l in range(Lr)}

    def source(self, t, l):
        return (self.T - 1, l) if self.plan[t, l] == L.REUSE else (t, l)

    def append_upto(self, upto, chunk=None, cells=None):
        """Appends to the given cells (default all) the tokens [done_b, upto_b) of each request,
        in calls of at most `chunk` tokens (None = one call), one call covering the whole batch."""
        upto = np.minimum(np.asarray(upto, np.int64), self.lens)
        cells = cells or [(t, l) for t in range(self.T) for l in range(self.L)]
        for (t, l) in cells:
            cur = self.done[t, l].copy()
            while (cur < upto).any():
                rem = upto - cur
                n = int(rem.max()) if chunk is None else int(min(chunk, rem.max()))
                m = np.minimum(rem, n).astype(np.int32)
                kk = torch.zeros(self.B, n, self.H, self.D, dtype=torch.bfloat16)
                vv = torch.zeros_like(kk)
                for b in range(self.B):
                    if m[b]:
                        kk[b, :m[b]] = self.k[t, l][b, cur[b]:cur[b] + m[b]]
                        vv[b, :m[b]] = self.v[t, l][b, cur[b]:cur[b] + m[b]]
                self.cache.append(l, t, kk.cuda(), vv.cuda(), torch.as_tensor(cur.astype(np.int32)).cuda(),
                                  self.page_table, n_new=torch.as_tensor(m).cuda())
                cur += m
            self.done[t, l] = cur
        torch.cuda.synchronize()

    def seq_lens(self, t, l) -> torch.Tensor:
        return torch.as_tensor(self.done[t, l].astype(np.int32)).cuda()

    # Oracle views ------------------------------------------------------------------------
    def qend(self, n):
        """End of the quantized history (in tokens) of a request holding n tokens."""
        return O.near_far_split(int(n), self.S, self.W)[2]

    def hist(self, t, l):
        """End (in tokens) of the history decode reads for cell (t, l): the source's quantized
        history, never past the cell's own window. The history starts at the sink length."""
        st, sl = self.source(t, l)
        return np.array([min(self.qend(self.done[st, sl][b]), self.qend(self.done[t, l][b]))
                         for b in range(self.B)], np.int64)

    def quant(self, t, l, hist=None):
        """Oracle QuantHead per (b, h) of storage cell (t, l): its tokens [S, hist[b])
        (default: everything its own appends have quantized so far)."""
        bits = int(self.plan[t, l])
        if hist is None:
            hist = np.array([self.qend(n) for n in self.done[t, l]], np.int64)
        k64, v64 = to64(self.k[t, l]), to64(self.v[t, l])
        S = self.S
        return [[O.quantize_head(k64[b, S:max(hist[b], S), h], v64[b, S:max(hist[b], S), h], bits,
                                 self.v_group)
                 for h in range(self.H)] for b in range(self.B)]

    def oracle_decode(self, t, l, q, *, tau, split_tokens=0, m0=None, sm_scale=None, sink_seed=True):
        """The oracle's decode of cell (t, l) after the appends so far: the cell's own sink, history
        from the source cell's quantized groups, tail = the cell's own remaining exact tokens.
        Returns (out [B, H, D], hot[b][h])."""
        st, sl = self.source(t, l)
        hist = self.hist(t, l)
        qh = self.quant(st, sl, hist)
        done = self.done[t, l]
        k64, v64 = to64(self.k[t, l]), to64(self.v[t, l])
        q64 = to64(q)
        sm = 1.0 / np.sqrt(self.D) if sm_scale is None else sm_scale
        out = np.zeros((self.B, self.H, self.D))
        hot = [[None] * self.H for _ in range(self.B)]
        for b in range(self.B):
            se = min(int(done[b]), self.S)
            he = max(int(hist[b]), self.S) if done[b] > 0 else 0
            for h in range(self.H):
                seed = -np.inf if m0 is None else float(m0[b, h])
                out[b, h], hot[b][h], _ = O.decode_head(
                    q64[b, h], qh[b][h], k64[b, he:done[b], h], v64[b, he:done[b], h], sm_scale=sm,
                    tau=tau, m0=seed, split_tokens=split_tokens, sink_k=k64[b, :se, h],
                    sink_v=v64[b, :se, h], hist_start=self.S, sink_seed=sink_seed)
        return out, hot

    def check_masks(self, mask, hot, t, l, q, tau, split, m0=None, sink_seed=True):
        """Fetch masks of an INT4-read cell against the oracle's, except near-tau ties."""
        st, sl = self.source(t, l)
        if self.plan[st, sl] != L.INT4:
            return 0
        hist = self.hist(t, l)
        qh = self.quant(st, sl, hist)
        mk = mask.cpu().numpy()
        q64 = to64(q)
        k64 = to64(self.k[t, l])
        ties = compared = 0
        for b in range(self.B):
            for h in range(self.H):
                n = qh[b][h].k_codes.shape[0]
                if n == 0:
                    continue
                compared += n
                kh = O.dequant_keys(qh[b][h].k_codes, qh[b][h].k_s, qh[b][h].k_z)
                s = (kh @ q64[b, h]) / np.sqrt(128.0)
                seed = -np.inf if m0 is None else float(m0[b, h])
                se = min(int(self.done[t, l][b]), self.S)
                if sink_seed and se > 0:
                    seed = max(seed, float((k64[b, :se, h] @ q64[b, h]).max() / np.sqrt(128.0)))
                tie = O.tie_mask(s, seed, tau, split, start=self.S)
                ties += check_mask(mk[b, h, self.S:], hot[b][h], tie, f"mask b={b} h={h} tau={tau}")
        assert_ties_rare(ties, compared, f"masks of cell ({t}, {l}) tau={tau} split={split}")
        return ties
