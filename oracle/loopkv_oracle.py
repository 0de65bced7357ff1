"""Plain fp64 CPU oracle for LoopKV's decode-attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link this
module: only the tests, the package smoke check and the benchmark's CPU-baseline leg do.
It shares no code, header, table or constant with the HIP library.

Source: "Loop-Aware KV Cache Compression for Serving Looped Transformers" (the LoopKV
paper). Each function names the section it follows. Where the paper is silent or its
extracted text lost a formula, the reading adopted is stated at the function.

Every quantity is computed in float64 from the exact bf16 inputs. Scales and zero points
are rounded once to fp16 (round to nearest even): the paper keeps a scale and a zero point
per quantization group next to the codes (§3.3, "Bit-plane V layout") and this library
stores each as an fp16.

Functions and what pins them (tests/test_oracle_pins.py):
  quantize_keys / quantize_values  -- closed-form ramps, constant groups, brute-force
                                      nearest-grid search, the half-step error bound
  split_planes / dequant_*          -- bijection c = 4*hi + lo, cold error (1.5 - lo)*s,
                                      cold value = the nearest 2-bit grid point (bucket middle)
  fetch_mask                        -- tau=0 all hot, tau>1 all cold, conservativeness
                                      against the global row max (Proposition 1's proof),
                                      a non-streaming brute force on tiny rows (also with
                                      the history starting after a sink)
  tie_mask                          -- hand-placed scores at exp(s - m) = tau +- 5e-7 (ties)
                                      and tau +- 2e-6 (not), within a split, across a split
                                      reset, after a sink; rare on benchmark-like scores
  near_far_split                    -- token-by-token enumeration of the window rule
  decode_head with a sink           -- library attention over sink + history + window,
                                      closed-form all-cold row under a dominant sink,
                                      seed monotonicity
  attention_row / decode_cell       -- library softmax attention (torch SDPA in fp64) at
                                      tau=0 and tau>1, one token, zero query, the
                                      Proposition-1 error bound, split and page invariance
  pack_head_block / unpack          -- round trip, hand-placed single codes
  pack_pool                         -- hand-derived byte positions of head blocks > 0 in
                                      shuffled pages, history after a 32-token sink
  cache_bytes_ref                   -- the paper's KiB-per-token figures (32-channel
                                      value groups)
  plan_exhaustive / plan_milp       -- each other (enumeration of every plan vs an integer
                                      program solved by scipy's HiGHS), closed-form optima
                                      with no budget and with a zero damage budget,
                                      monotonicity in the budgets
No function here is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

INT2, INT4, REUSE = 2, 4, 0
K_GROUP = 32          # tokens per key quantization group: one 32-token page (§3.4 "Layout")


# --------------------------------------------------------------------------------------
# fp16 rounding
# --------------------------------------------------------------------------------------
def fp16_rne(x):
    """Round float64 values to the nearest fp16 (ties to even); returns float64.

    numpy's float64 -> float16 cast rounds once, directly from the double."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def fp16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------------------
# KIVI-style asymmetric quantization (§5.1 "Baselines": KIVI-4 / KIVI-2, groups; §3.4
# "Layout": keys per channel over a 32-token page, values per token)
# --------------------------------------------------------------------------------------
def _quantize(x, mn, mx, bits):
    """Shared asymmetric rounding rule for one group.

    s = fp16(( max - min) / (2^b - 1)), z = fp16(min), code = clamp(floor((x - z)/s + 1/2)).
    A group with s == 0 gets code 0 everywhere (it dequantizes to z).
    """
    levels = (1 << bits) - 1
    s = fp16_rne((mx - mn) / levels)
    z = fp16_rne(mn)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.floor((x - z) / s + 0.5)
    c = np.where(s == 0, 0.0, c)
    c = np.clip(c, 0, levels).astype(np.int64)
    return c, s, z


def quantize_keys(k, bits):
    """Keys of one (request, head) over whole 32-token groups.

    k: float64 [n_tokens, D] with n_tokens a multiple of 32.
    Returns codes int64 [n_tokens, D], s and z float64 [n_tokens // 32, D]: one scale and
    zero point per (group, channel), constant over the group's 32 tokens.
    """
    k = np.asarray(k, dtype=np.float64)
    n, d = k.shape
    assert n % K_GROUP == 0
    g = k.reshape(n // K_GROUP, K_GROUP, d)
    mn = g.min(axis=1, keepdims=True)
    mx = g.max(axis=1, keepdims=True)
    c, s, z = _quantize(g, mn, mx, bits)
    return c.reshape(n, d), s[:, 0, :], z[:, 0, :]


def quantize_values(v, bits, v_group):
    """Values of one (request, head): per token, per group of `v_group` channels.

    v: float64 [n_tokens, D]. Returns codes int64 [n_tokens, D], s and z float64
    [n_tokens, D // v_group].
    """
    v = np.asarray(v, dtype=np.float64)
    n, d = v.shape
    assert d % v_group == 0
    g = v.reshape(n, d // v_group, v_group)
    mn = g.min(axis=2, keepdims=True)
    mx = g.max(axis=2, keepdims=True)
    c, s, z = _quantize(g, mn, mx, bits)
    return c.reshape(n, d), s[:, :, 0], z[:, :, 0]


# --------------------------------------------------------------------------------------
# Bit planes and dequantization (§3.3 "Bit-plane V layout", "Read-time V precision")
# --------------------------------------------------------------------------------------
def split_planes(codes4):
    """A 4-bit value code c splits into a high plane c >> 2 and a low plane c & 3."""
    codes4 = np.asarray(codes4, dtype=np.int64)
    return codes4 >> 2, codes4 & 3


def dequant_keys(codes, s, z):
    """K^ = s * code + z with the group's per-channel s, z broadcast over its 32 tokens."""
    n = codes.shape[0]
    rep = lambda a: np.repeat(a, K_GROUP, axis=0)[:n]
    return rep(s) * codes + rep(z)


def _rep_v(a, d):
    v_group = d // a.shape[1]
    return np.repeat(a, v_group, axis=1)


def dequant_values_full(codes, s, z):
    """Full-precision value: s * c + z (a hot INT4 token, or any INT2 token)."""
    d = codes.shape[1]
    return _rep_v(s, d) * codes + _rep_v(z, d)


def dequant_values_cold(codes4, s, z):
    """A cold INT4 token reads only its high plane and decodes to the midpoint of the
    bucket {4*hi, ..., 4*hi + 3}: s * (4*hi + 1.5) + z.

    Reading: the paper's formula for the midpoint is lost in extraction; 4*hi + 1.5 is
    the midpoint of the four codes sharing the high plane, and equals the 2-bit value the
    high plane encodes on the 4-bit grid."""
    hi, _ = split_planes(codes4)
    d = codes4.shape[1]
    return _rep_v(s, d) * (4.0 * hi + 1.5) + _rep_v(z, d)


# --------------------------------------------------------------------------------------
# Read-time V precision mask (§3.3; §3.4 "The unified kernel"; Appendix "Proof of
# Proposition 1")
# --------------------------------------------------------------------------------------
def _split_groups(n, start, split_tokens, group):
    """Yields (g0, g1, new_split) for the 32-token groups of a history slice of n scores whose
    first score is absolute token `start`; new_split marks the first group of each split.
    Splits are runs of split_tokens tokens counted from token 0 of the request (0: one split)."""
    prev = None
    for g0 in range(0, n, group):
        sp = (start + g0) // split_tokens if split_tokens else 0
        yield g0, min(g0 + group, n), sp != prev
        prev = sp


def fetch_mask(scores, m0, tau, split_tokens=0, group=K_GROUP, start=0):
    """Which history tokens read the low plane (True = hot).

    scores: float64 [n] (n a multiple of `group`), the attention logits of the history
    tokens start, start + 1, ... of one row (start a multiple of `group`: 0, or the sink
    length when a sink precedes the history). The request is cut into splits of
    `split_tokens` tokens from token 0 (0 means one split). Within a split, a running
    maximum starts at the seed m0 (-inf when there is none) and, group by group in order,
    first absorbs the group's largest score, then tests the group's tokens: a token is cold
    iff exp(s_j - m) < tau.

    Reading: the paper ties the running maximum to the kernel's stream order, and the kernel
    has every key code of a page (hence every score of the page) before it touches the
    page's values, so the page's own scores join the maximum before its tokens are tested. Strict '<' makes tau = 0 read every lo plane (KIVI-4) and
    any tau > 1 read none.
    """
    scores = np.asarray(scores, dtype=np.float64)
    hot = np.ones(scores.shape[0], dtype=bool)
    m = m0
    for g0, g1, new_split in _split_groups(scores.shape[0], start, split_tokens, group):
        if new_split:
            m = m0
        m = max(m, float(scores[g0:g1].max()))
        hot[g0:g1] = ~(np.exp(scores[g0:g1] - m) < tau)
    return hot


def tie_mask(scores, m0, tau, split_tokens=0, group=K_GROUP, band=1e-6, start=0):
    """Tokens whose test value exp(s_j - m) lies within `band` of tau: their hot/cold
    decision may differ between fp64 and a kernel's fp32 arithmetic.

    At tau <= 0 there are none: the cold test exp(s_j - m) < tau is false for every token in
    any precision (a weight is never negative), so no decision can differ."""
    scores = np.asarray(scores, dtype=np.float64)
    tie = np.zeros(scores.shape[0], dtype=bool)
    if tau <= 0:
        return tie
    m = m0
    for g0, g1, new_split in _split_groups(scores.shape[0], start, split_tokens, group):
        if new_split:
            m = m0
        m = max(m, float(scores[g0:g1].max()))
        tie[g0:g1] = np.abs(np.exp(scores[g0:g1] - m) - tau) <= band
    return tie


# --------------------------------------------------------------------------------------
# Sink and window (§2.3 "Measuring KV damage"; §3.2 "Cross-loop KV sharing"; §3.4 "The
# unified kernel", "Layout")
# --------------------------------------------------------------------------------------
def near_far_split(n, sink_tokens=0, window_tokens=0, group=K_GROUP):
    """Which positions of a request holding n tokens are quantized history and which stay
    exact (bf16).

    The first `sink_tokens` positions are the sink and stay exact. A `group`-token page past
    the sink is quantized once it has left the window, i.e. once none of its tokens is among
    the last `window_tokens` positions; until then it is exact. With no sink and no window
    this is "quantize a group as soon as it is complete".
    Returns (sink_end, hist_begin, hist_end): the sink is [0, sink_end), the quantized history
    [hist_begin, hist_end) (whole groups, possibly empty), the exact rest [hist_end, n) when
    n > hist_end.
    """
    assert sink_tokens % group == 0 and window_tokens % group == 0
    hs = sink_tokens // group
    he = max(hs, (n - window_tokens) // group)
    return min(n, sink_tokens), hs * group, he * group


# --------------------------------------------------------------------------------------
# Attention (§3.4: the log-sum-exp merge of split partials gives the exact softmax, so the
# oracle takes one softmax over history and tail)
# --------------------------------------------------------------------------------------
def attention_row(scores, vhat):
    """out = sum_j softmax(scores)_j * vhat_j in float64; an empty row gives zeros."""
    scores = np.asarray(scores, dtype=np.float64)
    if scores.size == 0:
        return np.zeros(vhat.shape[1], dtype=np.float64)
    p = np.exp(scores - scores.max())
    return (p[:, None] * vhat).sum(axis=0) / p.sum()


@dataclass
class QuantHead:
    """Quantized history of one (request, head) of one storage cell."""
    bits: int
    k_codes: np.ndarray   # int64 [n, D]
    k_s: np.ndarray       # [n/32, D]
    k_z: np.ndarray
    v_codes: np.ndarray   # int64 [n, D]
    v_s: np.ndarray       # [n, D/v_group]
    v_z: np.ndarray


def quantize_head(k, v, bits, v_group):
    """Quantize one (request, head)'s history (whole 32-token groups) to `bits`."""
    kc, ks, kz = quantize_keys(k, bits)
    vc, vs, vz = quantize_values(v, bits, v_group)
    return QuantHead(bits, kc, ks, kz, vc, vs, vz)


def decode_head(q, qh: QuantHead | None, tail_k, tail_v, *, sm_scale, tau, m0=-math.inf,
                split_tokens=0, sink_k=None, sink_v=None, hist_start=0, sink_seed=True):
    """One (request, head) of one decode call.

    q: float64 [D] (exact bf16 query values). qh: the quantized history the cell reads
    (its own, or for a cell that reuses the final loop's KV, the final loop's at the same
    layer -- §3.2: it attends with its own query over that history), covering the tokens
    hist_start, hist_start + 1, ... tail_k/tail_v: float64 [t, D], exact bf16 tokens after
    the history (the window, or the tokens not quantized yet). sink_k/sink_v: float64
    [s, D], the exact sink tokens before the history, or None.

    Scores s_j = sm_scale * q . K^_j. INT4 history reads values at full precision for hot
    tokens and at the bucket midpoint for cold ones (fetch_mask); INT2 history has no mask.
    The running maximum of the mask starts at m0 joined with the largest sink score (§3.4:
    the near part publishes the sink maximum as the far part's seed; sink_seed=False keeps
    m0 alone). Reading: the pages fall back to -inf when the published maximum is late; here
    it is always used, so the mask is deterministic.
    Returns (out [D], hot [n_hist] bool, scores [n_hist]).
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[0]
    sink_k = np.zeros((0, d)) if sink_k is None else np.asarray(sink_k, dtype=np.float64).reshape(-1, d)
    sink_v = np.zeros((0, d)) if sink_v is None else np.asarray(sink_v, dtype=np.float64).reshape(-1, d)
    s_sink = sm_scale * (sink_k @ q)
    seed = m0
    if sink_seed and s_sink.size:
        seed = max(seed, float(s_sink.max()))
    if qh is not None and qh.k_codes.shape[0] > 0:
        khat = dequant_keys(qh.k_codes, qh.k_s, qh.k_z)
        s_hist = sm_scale * (khat @ q)
        if qh.bits == INT4:
            hot = fetch_mask(s_hist, seed, tau, split_tokens, start=hist_start)
            vfull = dequant_values_full(qh.v_codes, qh.v_s, qh.v_z)
            vcold = dequant_values_cold(qh.v_codes, qh.v_s, qh.v_z)
            vhat = np.where(hot[:, None], vfull, vcold)
        else:
            hot = np.ones(s_hist.shape[0], dtype=bool)
            vhat = dequant_values_full(qh.v_codes, qh.v_s, qh.v_z)
    else:
        s_hist = np.zeros(0)
        hot = np.zeros(0, dtype=bool)
        vhat = np.zeros((0, d))
    tail_k = np.asarray(tail_k, dtype=np.float64).reshape(-1, d)
    tail_v = np.asarray(tail_v, dtype=np.float64).reshape(-1, d)
    s_tail = sm_scale * (tail_k @ q)
    out = attention_row(np.concatenate([s_sink, s_hist, s_tail]),
                        np.concatenate([sink_v, vhat, tail_v]))
    return out, hot, s_hist


# --------------------------------------------------------------------------------------
# Page layout (§3.3 "Bit-plane V layout"; §3.4 "Layout")
#
# The paper fixes the contents of a page -- 32 tokens of one cell; keys as interleaved
# 4-bit codes; an INT4 cell's values as two contiguous 2-bit planes (hi, lo) followed by
# scales and zero points; an INT2 cell's own 2-bit codes -- but not the byte order. This
# library's order, per head block of a page of P tokens (P = 32, or 16 with two pages per
# key group), D channels, value groups of G channels (NVG = D / G):
#
#   KSZ  4*D bytes      fp16 (s, z) per channel for the key group that starts in this page
#                       (unused in a page that does not start a group)
#   KC   P*D*b/8 bytes  key codes, token-major 32-bit words W[t][w] at word t*(D*b/32) + w:
#                       INT4: word w holds channels 8w..8w+7; channel 8w + i (i < 4) in bits
#                             8i..8i+3 and channel 8w + 4 + i in bits 8i+4..8i+7
#                       INT2: word w holds channels 16w..16w+15; channel 16w + 4k + i
#                             (k, i < 4) in bits 8i+2k..8i+2k+1
#                       (masking a word's nibbles -- or 2-bit fields -- into bytes leaves four
#                       consecutive channels in each 32-bit register)
#   VC   P*D/4 bytes    INT4 high plane, or INT2 value codes: W[cb][t] at word cb*P + t,
#                       channel 16*cb + i in bits 2i..2i+1
#   VSZ  4*P*NVG bytes  fp16 (s, z) per (token, value group), token-major
#   VLO  P*D/4 bytes    INT4 only: low plane, token-major W[t][cb] at word t*(D/16) + cb,
#                       channel 16*cb + i in bits 2i..2i+1 -- one token's low plane is
#                       D/4 contiguous bytes, fetched only when the token is hot
#
# A page is H head blocks, head-major; page id p of a pool starts at p * page_bytes.
# --------------------------------------------------------------------------------------
def head_block_layout(bits, page_tokens, d=128, v_group=128):
    """Byte offsets and sizes of the regions of one head block."""
    p = page_tokens
    nvg = d // v_group
    regions = [("ksz", 4 * d), ("kc", p * d * bits // 8), ("vc", p * d // 4),
               ("vsz", 4 * p * nvg)]
    if bits == INT4:
        regions.append(("vlo", p * d // 4))
    off, out = 0, {}
    for name, size in regions:
        out[name] = (off, size)
        off += size
    out["total"] = (0, off)
    return out


def _pack_words_colmajor(codes, per_word, width):
    """codes [P, D] -> uint32 words [D/per_word, P], channel per_word*cb + i at bits width*i."""
    p, d = codes.shape
    c = codes.astype(np.uint64).reshape(p, d // per_word, per_word)
    shifts = (np.arange(per_word, dtype=np.uint64) * width)
    words = (c << shifts).sum(axis=2).astype(np.uint32)       # [P, D/per_word]
    return words.T.copy()                                     # [cb, t]


def _kc_field_channels(bits):
    """Channel (within its word) held by each field of a key-code word, low field first."""
    if bits == INT4:
        return np.array([(f % 2) * 4 + f // 2 for f in range(8)])
    return np.array([4 * (f % 4) + f // 4 for f in range(16)])


def _pack_kc(codes, bits):
    """Key codes [P, D] -> token-major uint32 words [P, D*bits/32] (the KC field order above)."""
    p, d = codes.shape
    per_word = 32 // bits
    ch = _kc_field_channels(bits)
    c = codes.astype(np.uint64).reshape(p, d // per_word, per_word)[:, :, ch]   # field order
    shifts = np.arange(per_word, dtype=np.uint64) * bits
    return (c << shifts).sum(axis=2).astype(np.uint32)


def _unpack_kc(words, bits):
    """Inverse of _pack_kc: uint32 [P, D*bits/32] -> codes [P, D]."""
    per_word = 32 // bits
    fields = _unpack_words(words, per_word, bits).reshape(words.shape[0], -1, per_word)
    out = np.empty_like(fields)
    out[:, :, _kc_field_channels(bits)] = fields
    return out.reshape(words.shape[0], -1)


def _unpack_words(words, per_word, width):
    """uint32 words [..., n] -> codes [..., n*per_word]."""
    w = words.astype(np.uint64)[..., None]
    shifts = np.arange(per_word, dtype=np.uint64) * width
    c = (w >> shifts) & np.uint64((1 << width) - 1)
    return c.reshape(*words.shape[:-1], words.shape[-1] * per_word).astype(np.int64)


def _fp16_pairs(s, z):
    """Interleave fp16 (s, z) pairs -> uint16 [..., 2]."""
    return np.stack([fp16_bits(s), fp16_bits(z)], axis=-1)


def pack_head_block(bits, page_tokens, k_codes, v_codes, v_s, v_z, k_s=None, k_z=None,
                    v_group=128):
    """Bytes of one head block of one page.

    k_codes, v_codes: int [P, D] for the page's tokens (rows past a partial page are
    zero codes). v_s, v_z: [P, D/v_group]. k_s, k_z: [D] for the key group starting in
    this page, or None to leave KSZ zero.
    """
    p = page_tokens
    d = k_codes.shape[1]
    lay = head_block_layout(bits, p, d, v_group)
    buf = np.zeros(lay["total"][1], dtype=np.uint8)

    def put(name, arr):
        off, size = lay[name]
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert b.size == size, (name, b.size, size)
        buf[off:off + size] = b

    if k_s is not None:
        put("ksz", _fp16_pairs(k_s, k_z))
    if bits == INT4:
        put("kc", _pack_kc(k_codes, INT4))
        hi, lo = split_planes(v_codes)
        put("vc", _pack_words_colmajor(hi, 16, 2))
        put("vlo", _pack_words_colmajor(lo, 16, 2).T.copy())   # token-major
    else:
        put("kc", _pack_kc(k_codes, INT2))
        put("vc", _pack_words_colmajor(v_codes, 16, 2))
    put("vsz", _fp16_pairs(v_s, v_z))
    return buf


def unpack_head_block(bits, page_tokens, buf, d=128, v_group=128):
    """Inverse of pack_head_block: returns dict of k_codes, v_codes [P, D], v_s, v_z
    [P, NVG], k_s, k_z [D] (all float64 / int64)."""
    p = page_tokens
    lay = head_block_layout(bits, p, d, v_group)

    def get(name, dtype):
        off, size = lay[name]
        return buf[off:off + size].view(dtype)

    ksz = get("ksz", np.uint16).reshape(d, 2).view(np.float16).astype(np.float64)
    nvg = d // v_group
    vsz = get("vsz", np.uint16).reshape(p, nvg, 2).view(np.float16).astype(np.float64)
    if bits == INT4:
        k_codes = _unpack_kc(get("kc", np.uint32).reshape(p, d // 8), INT4)
        hw = get("vc", np.uint32).reshape(d // 16, p).T
        lw = get("vlo", np.uint32).reshape(p, d // 16)
        v_codes = 4 * _unpack_words(hw, 16, 2) + _unpack_words(lw, 16, 2)
    else:
        k_codes = _unpack_kc(get("kc", np.uint32).reshape(p, d // 16), INT2)
        vw = get("vc", np.uint32).reshape(d // 16, p).T
        v_codes = _unpack_words(vw, 16, 2)
    return dict(k_codes=k_codes, v_codes=v_codes, k_s=ksz[:, 0], k_z=ksz[:, 1],
                v_s=vsz[:, :, 0], v_z=vsz[:, :, 1])


def pack_pool(bits, page_tokens, heads_q: list[list[QuantHead]], page_table, num_pages,
              v_group=128, hist_start=0):
    """The expected bytes of one cell's pool.

    heads_q[b][h]: the quantized history of request b, head h (whole groups) covering the
    tokens hist_start, hist_start + 1, ... (hist_start a multiple of 32: the sink length).
    page_table: int [B, stride], logical page -> physical page id. Pages never written stay
    zero. Returns uint8 [num_pages, page_bytes].
    """
    nb = len(heads_q)
    nh = len(heads_q[0]) if nb else 0
    d = heads_q[0][0].k_codes.shape[1] if nb else 128
    hb = head_block_layout(bits, page_tokens, d, v_group)["total"][1]
    pool = np.zeros((num_pages, nh * hb), dtype=np.uint8)
    for b in range(nb):
        for h in range(nh):
            qh = heads_q[b][h]
            n = qh.k_codes.shape[0]
            for lp in range(n // page_tokens):
                t0 = lp * page_tokens
                rows = slice(t0, t0 + page_tokens)
                starts = t0 % K_GROUP == 0
                g = t0 // K_GROUP
                blk = pack_head_block(bits, page_tokens, qh.k_codes[rows], qh.v_codes[rows],
                                      qh.v_s[rows], qh.v_z[rows],
                                      qh.k_s[g] if starts else None,
                                      qh.k_z[g] if starts else None, v_group)
                pid = int(page_table[b][(hist_start + t0) // page_tokens])
                pool[pid, h * hb:(h + 1) * hb] = blk
    return pool


def unpack_pool_head(bits, page_tokens, pool, page_table_row, n_tokens, h, num_heads,
                     d=128, v_group=128, hist_start=0) -> QuantHead:
    """Read one (request, head)'s quantized history (n_tokens, whole groups, starting at token
    hist_start) back out of a pool's bytes through its page-table row."""
    hb = head_block_layout(bits, page_tokens, d, v_group)["total"][1]
    kc, vc, vs, vz, ks, kz = [], [], [], [], [], []
    for lp in range(n_tokens // page_tokens):
        pid = int(page_table_row[(hist_start + lp * page_tokens) // page_tokens])
        blk = pool[pid, h * hb:(h + 1) * hb]
        u = unpack_head_block(bits, page_tokens, blk, d, v_group)
        kc.append(u["k_codes"]); vc.append(u["v_codes"]); vs.append(u["v_s"]); vz.append(u["v_z"])
        if (lp * page_tokens) % K_GROUP == 0:
            ks.append(u["k_s"]); kz.append(u["k_z"])
    cat = lambda a, shape: np.concatenate(a) if a else np.zeros(shape)
    nvg = d // v_group
    return QuantHead(bits, cat(kc, (0, d)).astype(np.int64), cat([x[None] for x in ks], (0, d)),
                     cat([x[None] for x in kz], (0, d)), cat(vc, (0, d)).astype(np.int64),
                     cat(vs, (0, nvg)), cat(vz, (0, nvg)))


# --------------------------------------------------------------------------------------
# Byte model (§1, §2.2, §3.1, §3.3; Table 5; Table 13)
# --------------------------------------------------------------------------------------
def token_head_bytes(bits, d=128, v_group=128, k_group=K_GROUP):
    """Stored bytes of one (token, head) by region: key codes, the token's share of the
    key group's fp16 (s, z), value codes (INT4: hi and lo planes), value (s, z)."""
    kc = d * bits / 8
    ksz = 4 * d / k_group
    vsz = 4 * (d // v_group)
    if bits == INT4:
        return dict(kc=kc, ksz=ksz, vhi=d / 4, vlo=d / 4, vsz=vsz)
    return dict(kc=kc, ksz=ksz, vc=d / 4, vsz=vsz)


def cache_bytes_ref(plan, num_kv_heads=16, d=128, v_group=128):
    """KV bytes per token over all cells of a plan (uint8 [loops, layers], REUSE cells read
    the final loop's cell at the same layer, §3.2).

    stored: bytes kept (REUSE cells store none). read_all_hot: bytes one decode step reads
    per token with every lo plane fetched (tau = 0). read_hi_only: with no lo plane fetched
    (tau > 1) -- the lo plane is the part C3 skips for cold tokens.
    """
    plan = np.asarray(plan)
    T = plan.shape[0]
    stored = read_all = read_hi = 0.0
    for t in range(T):
        for layer in range(plan.shape[1]):
            code = int(plan[t, layer])
            src = int(plan[T - 1, layer]) if code == REUSE else code
            r = token_head_bytes(src, d, v_group)
            tot = sum(r.values()) * num_kv_heads
            if code != REUSE:
                stored += tot
            read_all += tot
            read_hi += tot - r.get("vlo", 0.0) * num_kv_heads
    return dict(stored=stored, read_all_hot=read_all, read_hi_only=read_hi)


def bf16_bytes_per_token(num_cells, num_kv_heads=16, d=128):
    """Unquantized BF16 K and V of every cell: 2 tensors * 2 bytes per element."""
    return num_cells * num_kv_heads * d * 2 * 2


# --------------------------------------------------------------------------------------
# Cell level: a batch of (request, head) rows of one (loop, layer) cell
# --------------------------------------------------------------------------------------
def quantize_cell(k, v, hist_lens, bits, v_group=128):
    """k, v: float64 [B, N, H, D] exact bf16 values; hist_lens[b]: quantized tokens of
    request b (a multiple of 32). Returns heads_q[b][h]."""
    B, _, H, _ = k.shape
    out = []
    for b in range(B):
        n = int(hist_lens[b])
        out.append([quantize_head(k[b, :n, h], v[b, :n, h], bits, v_group) for h in range(H)])
    return out


def decode_cell(q, heads_q, tail_k, tail_v, *, tau, sm_scale=None, m0=None, split_tokens=0):
    """One decode call of one cell.

    q: float64 [B, H, D]; heads_q[b][h] or None (no history); tail_k/tail_v: per request a
    float64 [t_b, H, D] array of exact tokens (or None). m0: [B, H] seeds or None (-inf).
    Returns out float64 [B, H, D] and hot[b][h] bool arrays.
    """
    B, H, D = q.shape
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    out = np.zeros((B, H, D))
    hot = [[None] * H for _ in range(B)]
    for b in range(B):
        for h in range(H):
            qh = heads_q[b][h] if heads_q is not None else None
            tk = np.zeros((0, D)) if tail_k is None or tail_k[b] is None else tail_k[b][:, h]
            tv = np.zeros((0, D)) if tail_v is None or tail_v[b] is None else tail_v[b][:, h]
            seed = -math.inf if m0 is None else float(m0[b, h])
            o, hm, _ = decode_head(q[b, h], qh, tk, tv, sm_scale=sm, tau=tau, m0=seed,
                                   split_tokens=split_tokens)
            out[b, h] = o
            hot[b][h] = hm
    return out, hot


# --------------------------------------------------------------------------------------
# Planner (§1; §3 "System Design"; §3.1 "Allocation"; §2.4: single-cell damages add up;
# §3.2: a shared cell stores nothing and reads the final loop's pages)
#
# A plan gives every cell one option: INT4, INT2, or (loops before the last) REUSE of the final
# loop's KV at the same layer. The planner minimises the bytes read per decode step subject to
# a damage budget (the sum of the chosen options' single-cell damages) and a storage budget
# (stored bytes per token). Among plans with the fewest read bytes, the oracle prefers the
# least damage, then the least storage (reading: the paper names only the objective and the
# budgets; this order makes the optimum's cost unique).
# --------------------------------------------------------------------------------------
PLAN_OPTIONS = (INT4, INT2, REUSE)   # order of the damage table's last axis


def plan_cost(plan, damage, num_kv_heads=16, d=128, v_group=128, hot_fraction=1.0):
    """(damage, stored bytes per token, read bytes per token) of a plan uint8 [T, L].
    damage: [T, L, 3] per option in PLAN_OPTIONS order. Reads count each INT4-read cell's low
    plane with weight hot_fraction (1: every plane read)."""
    plan = np.asarray(plan)
    T, L = plan.shape
    dmg = 0.0
    for t in range(T):
        for layer in range(L):
            dmg += float(damage[t, layer, PLAN_OPTIONS.index(int(plan[t, layer]))])
    b = cache_bytes_ref(plan, num_kv_heads, d, v_group)
    read = b["read_hi_only"] + hot_fraction * (b["read_all_hot"] - b["read_hi_only"])
    return dmg, b["stored"], read


def _layer_choices(T):
    """Every option tuple of one layer's T cells (the final loop cannot reuse)."""
    import itertools
    opts = [PLAN_OPTIONS] * (T - 1) + [(INT4, INT2)]
    return list(itertools.product(*opts))


def _feasible(cost, max_damage, max_stored):
    dmg, sto, _ = cost
    return (max_damage < 0 or dmg <= max_damage) and (max_stored <= 0 or sto <= max_stored)


def plan_exhaustive(damage, max_damage=-1.0, max_stored=0.0, num_kv_heads=16, d=128,
                    v_group=128, hot_fraction=1.0):
    """Every plan, costed with plan_cost; returns (plan, cost) of the best feasible plan by
    (reads, damage, storage), or (None, None). For tiny T x L only."""
    import itertools
    damage = np.asarray(damage, dtype=np.float64)
    T, L, _ = damage.shape
    best, best_cost = None, None
    for cols in itertools.product(_layer_choices(T), repeat=L):
        plan = np.array(cols, dtype=np.uint8).T          # [T, L]
        cost = plan_cost(plan, damage, num_kv_heads, d, v_group, hot_fraction)
        if not _feasible(cost, max_damage, max_stored):
            continue
        key = (round(cost[2], 6), cost[0], cost[1])
        if best is None or key < best:
            best, best_cost, best_plan = key, cost, plan
    return (best_plan, best_cost) if best is not None else (None, None)


def plan_milp(damage, max_damage=-1.0, max_stored=0.0, num_kv_heads=16, d=128, v_group=128,
              hot_fraction=1.0):
    """The same choice as an integer program: one binary per (layer, option tuple of its
    cells), exactly one per layer, the budgets as linear constraints; scipy's milp (HiGHS)
    minimises the reads, then, with the reads fixed, the damage. Returns (plan, cost) or
    (None, None) when infeasible."""
    from scipy.optimize import Bounds, LinearConstraint, milp
    damage = np.asarray(damage, dtype=np.float64)
    T, L, _ = damage.shape
    ch = _layer_choices(T)
    K = len(ch)
    rd = np.zeros(L * K)
    st = np.zeros(L * K)
    dm = np.zeros(L * K)
    for layer in range(L):
        for k, opts in enumerate(ch):
            col = np.array(opts, dtype=np.uint8)[:, None]
            cd, cs, cr = plan_cost(col, damage[:, layer:layer + 1], num_kv_heads, d, v_group,
                                   hot_fraction)
            rd[layer * K + k], st[layer * K + k], dm[layer * K + k] = cr, cs, cd
    one = np.zeros((L, L * K))
    for layer in range(L):
        one[layer, layer * K:(layer + 1) * K] = 1
    cons = [LinearConstraint(one, 1, 1)]
    if max_damage >= 0:
        cons.append(LinearConstraint(dm[None], -np.inf, max_damage))
    if max_stored > 0:
        cons.append(LinearConstraint(st[None], -np.inf, max_stored))
    opt = {"mip_rel_gap": 0.0}
    ints = np.ones(L * K)
    r1 = milp(rd, constraints=cons, integrality=ints, bounds=Bounds(0, 1), options=opt)
    if r1.x is None:
        return None, None
    r_best = float(rd @ np.round(r1.x))
    cons2 = cons + [LinearConstraint(rd[None], -np.inf, r_best + 1e-6 * max(r_best, 1.0))]
    r2 = milp(dm, constraints=cons2, integrality=ints, bounds=Bounds(0, 1), options=opt)
    x = np.round(r2.x if r2.x is not None else r1.x)
    plan = np.zeros((T, L), dtype=np.uint8)
    for layer in range(L):
        k = int(np.argmax(x[layer * K:(layer + 1) * K]))
        plan[:, layer] = ch[k]
    return plan, plan_cost(plan, damage, num_kv_heads, d, v_group, hot_fraction)
