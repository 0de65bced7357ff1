"""Pins for the fp64 oracle: each test checks the oracle against something other than itself
(IEEE rounding facts, closed forms, exhaustive searches, a library softmax attention, the
paper's printed byte figures, hand-derived byte positions, stated invariants)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from quantized_kv_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def rand_bf16(rng, *shape, scale=1.0):
    return bf16(rng.standard_normal(shape) * scale)


# ------------------------------------------------------------------ fp16 rounding (IEEE 754)
@pytest.mark.parametrize("x,bits", [
    (1.0 / 3.0, 0x3555), (0.1, 0x2E66), (65504.0, 0x7BFF), (65520.0, 0x7C00),
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (3 * 2.0 ** -26, 0x0001),
    (1 + 2.0 ** -11, 0x3C00), (1 + 3 * 2.0 ** -11, 0x3C02), (-2.5, 0xC100),
    (2.0 ** -14, 0x0400), (2.0 ** -14 - 2.0 ** -25, 0x0400),
])
def test_fp16_rne_ieee_values(x, bits):
    assert int(O.fp16_bits(x)) == bits


# ------------------------------------------------------------------ quantizer
@pytest.mark.parametrize("bits", [2, 4])
def test_quantize_ramp_closed_form(bits):
    """A group whose values sit exactly on the grid z + k*s (fp16- and bf16-exact) and that
    contains its min and max gets codes k, scale s and zero z."""
    L = (1 << bits) - 1
    s, z = 0.25, -1.0
    k = np.arange(32) % (L + 1)
    x = z + k * s
    col = np.stack([x, x[::-1]], axis=1)              # two channels
    codes, ks, kz = O.quantize_keys(col, bits)
    assert np.all(ks == s) and np.all(kz == z)
    assert np.array_equal(codes[:, 0], k) and np.array_equal(codes[:, 1], k[::-1])
    # values: per token over one group of channels
    row = np.tile(z + np.arange(L + 1) * s, 128 // (L + 1))[None, :]
    vc, vs, vz = O.quantize_values(row, bits, 128)
    assert vs[0, 0] == s and vz[0, 0] == z
    assert np.array_equal(vc[0], np.tile(np.arange(L + 1), row.shape[1] // (L + 1)))


@pytest.mark.parametrize("bits", [2, 4])
def test_quantize_constant_group(bits):
    x = np.full((32, 4), bf16(0.3)[()])
    codes, s, z = O.quantize_keys(x, bits)
    assert np.all(s == 0) and np.all(codes == 0)
    assert np.allclose(O.dequant_keys(codes, s, z), O.fp16_rne(x))


@pytest.mark.parametrize("bits", [2, 4])
def test_quantize_matches_nearest_grid_point(bits):
    """Brute force: each code is the grid point s*c + z nearest to x (ties to the upper
    point, as round-half-up does), searched over every code."""
    rng = np.random.default_rng(1)
    L = (1 << bits) - 1
    x = rand_bf16(rng, 64, 16)
    x[:, 3] *= 10
    codes, s, z = O.quantize_keys(x, bits)
    sr = np.repeat(s, 32, axis=0)
    zr = np.repeat(z, 32, axis=0)
    grid = np.arange(L + 1)[None, None, :] * sr[..., None] + zr[..., None]
    err = np.abs(x[..., None] - grid)
    best = err.min(axis=-1, keepdims=True)
    brute = np.where(err == best, np.arange(L + 1), -1).max(axis=-1)
    assert np.array_equal(codes, brute)
    v = rand_bf16(rng, 8, 128)
    vc, vs, vz = O.quantize_values(v, bits, 32)
    sr = np.repeat(vs, 32, axis=1)
    zr = np.repeat(vz, 32, axis=1)
    grid = np.arange(L + 1)[None, None, :] * sr[..., None] + zr[..., None]
    err = np.abs(v[..., None] - grid)
    best = err.min(axis=-1, keepdims=True)
    brute = np.where(err == best, np.arange(L + 1), -1).max(axis=-1)
    assert np.array_equal(vc, brute)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantize_error_bound(bits):
    """|x - x^| <= s/2 away from clamping; in general within s/2 plus the fp16 rounding of
    the group's end points."""
    rng = np.random.default_rng(2)
    L = (1 << bits) - 1
    x = rand_bf16(rng, 32 * 8, 128, scale=3.0)
    codes, s, z = O.quantize_keys(x, bits)
    xh = O.dequant_keys(codes, s, z)
    g = x.reshape(-1, 32, 128)
    mn, mx = g.min(1), g.max(1)
    slack = np.abs(mn - z) + np.abs(mx - (z + L * s))
    bound = np.repeat(s / 2 + slack, 32, axis=0) * (1 + 1e-12)
    assert np.all(np.abs(x - xh) <= bound)
    assert codes.min() == 0 and codes.max() == L


def test_quantize_fp16_subnormal_zero_point():
    """A group minimum of 2^-25 is a tie between fp16 0 and 2^-24 and rounds to even (0)."""
    x = np.zeros((32, 1))
    x[:, 0] = 2.0 ** -25
    x[5, 0] = 2.0 ** -25 + 15 * 2.0 ** -20
    _, s, z = O.quantize_keys(x, 4)
    assert z[0, 0] == 0.0
    assert s[0, 0] == O.fp16_rne(2.0 ** -20)


# ------------------------------------------------------------------ planes
def test_planes_bijection_and_cold_error():
    c = np.arange(16)
    hi, lo = O.split_planes(c)
    assert np.array_equal(4 * hi + lo, c) and hi.max() == 3 and lo.max() == 3
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, size=(5, 128))
    s = O.fp16_rne(rng.uniform(0.1, 2, size=(5, 1)))
    z = O.fp16_rne(rng.standard_normal((5, 1)))
    full = O.dequant_values_full(codes, s, z)
    cold = O.dequant_values_cold(codes, s, z)
    _, lo = O.split_planes(codes)
    assert np.allclose(cold - full, (1.5 - lo) * s, atol=0, rtol=1e-15)
    assert np.all(np.abs(cold - full) <= 1.5 * s)


# ------------------------------------------------------------------ mask
def _brute_mask(scores, m0, tau, split, group=32, start=0):
    """Non-streaming: history token j sits at absolute position start + j; its reference
    maximum is the seed joined with every history score of its split (runs of `split` tokens
    from position 0) up to the end of its own group."""
    n = len(scores)
    hot = np.zeros(n, dtype=bool)
    for j in range(n):
        a = start + j
        s_lo, s_hi = ((a // split) * split, (a // split + 1) * split) if split else (0, start + n)
        g_hi = (a // group + 1) * group
        lo = max(s_lo, start) - start
        hi = min(g_hi, s_hi, start + n) - start
        m = max([m0] + list(scores[lo:hi]))
        hot[j] = math.exp(scores[j] - m) >= tau
    return hot


@pytest.mark.parametrize("split", [0, 32, 64, 96])
@pytest.mark.parametrize("tau", [0.0, 0.005, 0.02, 0.3, 1.0, 2.0])
@pytest.mark.parametrize("m0", [-math.inf, 0.5, 9.0])
def test_mask_matches_non_streaming_brute_force(split, tau, m0):
    rng = np.random.default_rng(4)
    scores = rng.standard_normal(192) * 3
    assert np.array_equal(O.fetch_mask(scores, m0, tau, split), _brute_mask(scores, m0, tau, split))


@pytest.mark.parametrize("start", [32, 96])
@pytest.mark.parametrize("split", [0, 64, 128])
def test_mask_after_sink_matches_brute_force(start, split):
    """History that starts after a sink: splits still count from token 0, so the first split
    holds fewer history groups."""
    rng = np.random.default_rng(41)
    scores = rng.standard_normal(256) * 3
    for tau in [0.01, 0.1]:
        got = O.fetch_mask(scores, -math.inf, tau, split, start=start)
        assert np.array_equal(got, _brute_mask(scores, -math.inf, tau, split, start=start))


def test_mask_identities_and_conservativeness():
    rng = np.random.default_rng(5)
    for trial in range(20):
        scores = rng.standard_normal(32 * 12) * rng.uniform(0.5, 6)
        split = [0, 32, 128, 256][trial % 4]
        m0 = [-math.inf, float(scores.min()), float(np.median(scores))][trial % 3]
        assert O.fetch_mask(scores, m0, 0.0, split).all()             # tau = 0: KIVI-4
        assert not O.fetch_mask(scores, m0, 2.0, split).any()         # tau > 1: hi only
        prev = None
        for tau in [0.001, 0.01, 0.05, 0.2, 0.9]:
            hot = O.fetch_mask(scores, m0, tau, split)
            # Proposition 1: the running max never exceeds the row max (seed <= row max
            # here), so every cold token's weight is below tau times the row's largest.
            p = np.exp(scores - scores.max())
            assert np.all(p[~hot] < tau)
            if prev is not None:
                assert np.all(hot <= prev)                          # monotone in tau
            prev = hot
    scores = rng.standard_normal(96)
    assert np.array_equal(O.fetch_mask(scores, -math.inf, 0.05, 0),
                          O.fetch_mask(scores, -math.inf, 0.05, 4096))



def _tie_case(tau, m, offsets):
    """Scores whose test value exp(s - m) sits at tau + offset for a known running maximum m."""
    return [m + math.log(tau + o) for o in offsets]


@pytest.mark.parametrize("tau", [0.01, 0.02])
def test_tie_mask_hand_placed(tau):
    """Tokens placed at exp(s - m) = tau +- 5e-7 are ties, tokens at tau +- 2e-6 are not: within
    one split, after a split reset (the second split's maximum starts again at the seed), and
    with the history starting after a 32-token sink (splits still count from token 0)."""
    far = -40.0                                   # exp(far - m) is nowhere near tau
    # one split, seed below the group maximum 0
    s = np.full(128, far)
    s[0] = 0.0
    s[3:7] = _tie_case(tau, 0.0, [5e-7, -5e-7, 2e-6, -2e-6])
    s[40:42] = _tie_case(tau, 0.0, [-4e-7, 1.5e-6])   # a later group: the maximum is still 0
    t = O.tie_mask(s, -math.inf, tau, 0)
    assert set(np.nonzero(t)[0]) == {3, 4, 40}
    # a seed above every score sets the maximum
    s2 = np.full(64, far)
    s2[10:13] = _tie_case(tau, 2.5, [3e-7, -9e-7, 3e-6])
    assert set(np.nonzero(O.tie_mask(s2, 2.5, tau, 0))[0]) == {10, 11}
    # split reset: 64-token splits, the second split's largest score is -3
    s3 = np.full(128, far)
    s3[0] = 0.0
    s3[64] = -3.0
    s3[70:72] = _tie_case(tau, -3.0, [5e-7, 2e-6])
    s3[72] = math.log(tau + 5e-7)                 # a tie only against the first split's maximum
    s3[20] = math.log(tau - 5e-7)                 # a tie in the first split
    assert set(np.nonzero(O.tie_mask(s3, -math.inf, tau, 64))[0]) == {20, 70}
    # history after a sink: history token j is token 32 + j; 64-token splits from token 0 put
    # history group 0 (tokens 32..63) in split 0 and history group 1 (64..95) in split 1
    s4 = np.full(96, far)
    s4[0] = 0.0
    s4[32] = -3.0
    s4[40:42] = _tie_case(tau, -3.0, [5e-7, -2e-6])
    s4[15] = math.log(tau - 5e-7)                 # history group 0, maximum 0
    assert set(np.nonzero(O.tie_mask(s4, -math.inf, tau, 64, start=32))[0]) == {15, 40}
    # at tau = 0 every token is hot in any precision: no ties, however small the weights
    tiny = np.array([0.0] + [-30.0] * 31)
    assert not O.tie_mask(tiny, -math.inf, 0.0, 0).any()
    assert O.fetch_mask(tiny, -math.inf, 0.0, 0).all()
    # the tie band covers both sides of every fetch decision the kernel could take differently
    for sc, m0, sp, st in [(s, -math.inf, 0, 0), (s3, -math.inf, 64, 0), (s4, -math.inf, 64, 32)]:
        hot = O.fetch_mask(sc, m0, tau, sp, start=st)
        tie = O.tie_mask(sc, m0, tau, sp, start=st)
        assert hot[tie].any() and (~hot[tie]).any()


def test_tie_band_is_rare_on_benchmark_like_scores():
    """On scores of the benchmark's distribution the tie band holds well under 1e-4 of the
    tokens, so excluding it from the mask comparison leaves the comparison nearly complete."""
    rng = np.random.default_rng(12)
    n_tie = n = 0
    for trial in range(64):
        k, _, qh = _head(rng, 1024, 4)
        q = rand_bf16(rng, 128)
        sc = (O.dequant_keys(qh.k_codes, qh.k_s, qh.k_z) @ q) / math.sqrt(128)
        for tau in [0.005, 0.01, 0.02]:
            n_tie += int(O.tie_mask(sc, -math.inf, tau, [0, 256][trial % 2]).sum())
            n += sc.size
    assert n_tie <= 1e-4 * n


# ------------------------------------------------------------------ cold value = 2-bit rounding
def test_cold_value_is_nearest_bucket_midpoint():
    """A cold INT4 token decodes to the middle of its high-plane bucket, which is the point of
    the 2-bit grid {1.5, 5.5, 9.5, 13.5} (in 4-bit steps) nearest to its 4-bit code: the
    high-plane dequantization is the 2-bit rounding of the 4-bit code."""
    mids = np.array([1.5, 5.5, 9.5, 13.5])
    rng = np.random.default_rng(13)
    s = O.fp16_rne(rng.uniform(0.01, 3, size=(16, 1)))
    z = O.fp16_rne(rng.standard_normal((16, 1)))
    codes = np.tile(np.arange(16), (16, 8))          # every code, every channel position
    cold = O.dequant_values_cold(codes, s, z)
    for c in range(16):
        d = np.abs(c - mids)
        nearest = mids[np.argmin(d)]
        assert np.sum(d == d.min()) == 1              # never a tie between two midpoints
        sel = codes == c
        assert np.all(cold[sel] == (np.broadcast_to(s, codes.shape) * nearest
                                    + np.broadcast_to(z, codes.shape))[sel])
    # and in value terms: the cold value is the nearest point of the 2-bit grid z + s*(1.5 + 4k)
    full = O.dequant_values_full(codes, s, z)
    grid = z[:, :, None] + s[:, :, None] * mids[None, None, :]
    pick = np.take_along_axis(grid.repeat(codes.shape[1], 1),
                              np.argmin(np.abs(full[:, :, None] - grid), axis=2)[:, :, None], 2)[:, :, 0]
    assert np.allclose(cold, pick, rtol=1e-15, atol=0)

# ------------------------------------------------------------------ attention
def _sdpa(q, k, v):
    """torch's scaled-dot-product attention in float64 (library routine, default 1/sqrt(D))."""
    t = lambda a: torch.as_tensor(a, dtype=torch.float64)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q)[:, :, None], t(k), t(v))[0, 0, 0].numpy()


def _head(rng, n, bits, v_group=128, d=128, outliers=True):
    k = rand_bf16(rng, n, d)
    if outliers:
        k[:, rng.choice(d, 4, replace=False)] *= 10
    v = rand_bf16(rng, n, d)
    return k, v, O.quantize_head(k, v, bits, v_group)


@pytest.mark.parametrize("bits,tau", [(4, 0.0), (4, 2.0), (2, 0.01), (2, 0.0)])
@pytest.mark.parametrize("v_group", [128, 32])
def test_attention_reduces_to_library_sdpa(bits, tau, v_group):
    """tau = 0 on INT4 is full INT4 attention; tau > 1 is hi-only attention; INT2 has no
    mask. Each equals a library softmax attention over the dequantized keys and values,
    with the exact bf16 tail appended."""
    rng = np.random.default_rng(6)
    _, _, qh = _head(rng, 96, bits, v_group)
    q = rand_bf16(rng, 128)
    tk, tv = rand_bf16(rng, 7, 128), rand_bf16(rng, 7, 128)
    out, hot, _ = O.decode_head(q, qh, tk, tv, sm_scale=1 / math.sqrt(128), tau=tau)
    khat = O.dequant_keys(qh.k_codes, qh.k_s, qh.k_z)
    if bits == 4 and tau > 1:
        vhat = O.dequant_values_cold(qh.v_codes, qh.v_s, qh.v_z)
        assert not hot.any()
    else:
        vhat = O.dequant_values_full(qh.v_codes, qh.v_s, qh.v_z)
        assert hot.all()
    ref = _sdpa(q, np.concatenate([khat, tk]), np.concatenate([vhat, tv]))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    _, _, qh = _head(rng, 32, 4)
    # a single exact token: the output is that token's value
    v1 = rand_bf16(rng, 1, 128)
    out, _, _ = O.decode_head(rand_bf16(rng, 128), None, rand_bf16(rng, 1, 128), v1,
                              sm_scale=0.1, tau=0.01)
    assert np.allclose(out, v1[0], rtol=0, atol=1e-15)
    # zero query: every score is 0, every token hot (exp(0) = 1 >= tau), output = mean
    out, hot, _ = O.decode_head(np.zeros(128), qh, np.zeros((0, 128)), np.zeros((0, 128)),
                                sm_scale=0.1, tau=0.5)
    assert hot.all()
    assert np.allclose(out, O.dequant_values_full(qh.v_codes, qh.v_s, qh.v_z).mean(0), rtol=1e-13)
    # empty row: zeros by definition
    out, _, _ = O.decode_head(np.ones(128), None, np.zeros((0, 128)), np.zeros((0, 128)),
                              sm_scale=0.1, tau=0.5)
    assert np.all(out == 0)


@pytest.mark.parametrize("v_group", [128, 32])
def test_proposition1_error_bound(v_group):
    """Weights are those of the full INT4 reader; a cold token moves the output by at most
    1.5 * s * p_j per channel."""
    rng = np.random.default_rng(8)
    _, _, qh = _head(rng, 256, 4, v_group)
    q = rand_bf16(rng, 128)
    sm = 1 / math.sqrt(128)
    o0, _, s0 = O.decode_head(q, qh, np.zeros((0, 128)), np.zeros((0, 128)), sm_scale=sm, tau=0.0)
    for tau in [0.005, 0.02, 0.2, 2.0]:
        ot, hot, st = O.decode_head(q, qh, np.zeros((0, 128)), np.zeros((0, 128)), sm_scale=sm, tau=tau)
        assert np.array_equal(s0, st)
        p = np.exp(st - st.max()); p /= p.sum()
        sch = np.repeat(qh.v_s, v_group, axis=1)                  # [n, D]
        bound = 1.5 * ((~hot)[:, None] * p[:, None] * sch).sum(0)
        assert np.all(np.abs(ot - o0) <= bound * (1 + 1e-9) + 1e-15)
        assert (~hot).sum() > 0


def test_split_invariance_at_identity_taus():
    rng = np.random.default_rng(9)
    _, _, qh = _head(rng, 256, 4)
    q = rand_bf16(rng, 128)
    e = np.zeros((0, 128))
    for tau in [0.0, 2.0]:
        outs = [O.decode_head(q, qh, e, e, sm_scale=0.09, tau=tau, split_tokens=s)[0]
                for s in [0, 32, 64, 160]]
        for o in outs[1:]:
            assert np.array_equal(o, outs[0])


# ------------------------------------------------------------------ layout
def test_layout_fixture_positions():
    fx = json.load(open(os.path.join(GOLDEN, "layout_single_codes.json")))
    for case in fx["cases"]:
        if "sizes" in case:
            for key, size in case["sizes"].items():
                bits = 4 if key.startswith("int4") else 2
                p = int(key.split("_")[1][1:])
                g = int(key.split("_")[2][1:])
                assert O.head_block_layout(bits, p, 128, g)["total"][1] == size
            continue
        P, bits = case["page_tokens"], case["bits"]
        kc = np.zeros((P, 128), dtype=np.int64)
        vc = np.zeros((P, 128), dtype=np.int64)
        (kc if case["tensor"] == "k" else vc)[case["token"], case["channel"]] = case["code"]
        buf = O.pack_head_block(bits, P, kc, vc, np.zeros((P, 1)), np.zeros((P, 1)))
        expect = case.get("bytes", [[case.get("byte"), case.get("value")]])
        nz = {int(i): int(buf[i]) for i in np.nonzero(buf)[0]}
        assert nz == {b: v for b, v in expect}, case["what"]


def test_pool_placement_fixture():
    """pack_pool puts each head block of each history page where the page table and the head
    index say, with the history starting after a 32-token sink (hand-derived positions)."""
    fx = json.load(open(os.path.join(GOLDEN, "pool_placement.json")))
    for case in fx["cases"]:
        bits, P, H, B, n = case["bits"], case["page_tokens"], case["heads"], case["batch"], case["hist_tokens"]
        heads = []
        for b in range(B):
            row = []
            for h in range(H):
                z = lambda *sh: np.zeros(sh)
                qh = O.QuantHead(bits, np.zeros((n, 128), np.int64), z(n // 32, 128), z(n // 32, 128),
                                 np.zeros((n, 128), np.int64), z(n, 1), z(n, 1))
                for st in case["sets"]:
                    if (st["b"], st["h"]) != (b, h):
                        continue
                    if st["kind"] == "k_code":
                        qh.k_codes[st["token"], st["channel"]] = st["value"]
                    elif st["kind"] == "v_code":
                        qh.v_codes[st["token"], st["channel"]] = st["value"]
                    else:
                        qh.k_s[st["group"], st["channel"]] = st["value"]
                row.append(qh)
            heads.append(row)
        pool = O.pack_pool(bits, P, heads, np.array(case["page_table"]), case["num_pages"], 128,
                           hist_start=case["hist_start"]).reshape(-1)
        nz = {int(i): int(pool[i]) for i in np.nonzero(pool)[0]}
        assert nz == {b: v for b, v in case["bytes"]}, case["what"]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("P", [16, 32])
@pytest.mark.parametrize("v_group", [128, 32])
def test_layout_round_trip(bits, P, v_group):
    rng = np.random.default_rng(10)
    L = (1 << bits) - 1
    kc = rng.integers(0, L + 1, size=(P, 128))
    vc = rng.integers(0, L + 1, size=(P, 128))
    nvg = 128 // v_group
    vs, vz = O.fp16_rne(rng.uniform(0, 1, (P, nvg))), O.fp16_rne(rng.standard_normal((P, nvg)))
    ks, kz = O.fp16_rne(rng.uniform(0, 1, 128)), O.fp16_rne(rng.standard_normal(128))
    buf = O.pack_head_block(bits, P, kc, vc, vs, vz, ks, kz, v_group)
    u = O.unpack_head_block(bits, P, buf, 128, v_group)
    assert np.array_equal(u["k_codes"], kc) and np.array_equal(u["v_codes"], vc)
    assert np.array_equal(u["v_s"], vs) and np.array_equal(u["v_z"], vz)
    assert np.array_equal(u["k_s"], ks) and np.array_equal(u["k_z"], kz)


@pytest.mark.parametrize("P", [16, 32])
def test_page_table_invariance(P):
    """Packing a history into pages through a shuffled table and reading it back gives
    the same quantized history, hence the same output."""
    rng = np.random.default_rng(11)
    H = 2
    heads = [[_head(rng, 96, 4)[2] for _ in range(H)] for _ in range(2)]
    n_lp = 96 // P
    perm = rng.permutation(2 * n_lp).reshape(2, n_lp)
    pool = O.pack_pool(4, P, heads, perm, 2 * n_lp)
    q = rand_bf16(rng, 128)
    for b in range(2):
        for h in range(H):
            back = O.unpack_pool_head(4, P, pool, perm[b], 96, h, H)
            for f in ["k_codes", "k_s", "k_z", "v_codes", "v_s", "v_z"]:
                assert np.array_equal(getattr(back, f), getattr(heads[b][h], f))
            o1 = O.decode_head(q, back, np.zeros((0, 128)), np.zeros((0, 128)), sm_scale=.09, tau=.01)[0]
            o2 = O.decode_head(q, heads[b][h], np.zeros((0, 128)), np.zeros((0, 128)), sm_scale=.09, tau=.01)[0]
            assert np.array_equal(o1, o2)


# ------------------------------------------------------------------ byte model
def _plan(name, layers, loops):
    names = {"all_int4": "kivi4", "int4_loop3_reuse": "kivi4_loop3_share", "int2_loops123": "int2_loops123",
             "loopkv_r": "loopkv_r", "loopkv_m": "loopkv_m"}
    return synth.named_plan(names[name], layers, loops)


def test_cache_bytes_match_paper_figures():
    fx = json.load(open(os.path.join(GOLDEN, "page_kib_per_token.json")))
    for c in fx["cases"]:
        if c["plan"] == "bf16":
            assert O.bf16_bytes_per_token(c["layers"] * c["loops"]) / 1024 == c["stored"]
            continue
        r = O.cache_bytes_ref(_plan(c["plan"], c["layers"], c["loops"]), 16, 128, 32)
        assert r["stored"] / 1024 == c["stored"], c["name"]
        if "read" in c:
            assert r["read_all_hot"] / 1024 == c["read"], c["name"]
    vp = fx["v_precision"]
    lo, hi = vp["full_precision_fraction_range"]
    for name in ["loopkv_r", "loopkv_m"]:
        r = O.cache_bytes_ref(_plan(name, 24, 4), 16, 128, 32)
        n_int4_read = (r["read_all_hot"] - r["read_hi_only"]) / 1024 / vp["lo_plane_kib_per_token_and_layer"]
        assert n_int4_read == int(n_int4_read)
        read = lambda f: (r["read_hi_only"] + f * (r["read_all_hot"] - r["read_hi_only"])) / 1024
        assert read(lo) <= vp[name]["read_with_v_precision"] + 0.5
        assert read(hi) >= vp[name]["read_with_v_precision"] - 0.5


def test_cache_bytes_baseline_shapes():
    """128-channel value groups: 148 B per INT4 (token, head), 84 B per INT2."""
    assert sum(O.token_head_bytes(4).values()) == 148
    assert sum(O.token_head_bytes(2).values()) == 84
    r = O.cache_bytes_ref(np.array([[4], [2], [0], [4]], dtype=np.uint8))
    assert r["stored"] == 16 * (148 + 84 + 148)
    assert r["read_all_hot"] == 16 * (148 + 84 + 148 + 148)
    assert r["read_all_hot"] - r["read_hi_only"] == 16 * 32 * 3


# ------------------------------------------------------------------ sink and window
def _brute_quantized_groups(n, S, W):
    """Token by token: a 32-token group past the sink is quantized iff it is complete and none
    of its tokens is among the last W positions."""
    return {g for g in range(S // 32, n // 32)
            if all(p < n and p < n - W for p in range(32 * g, 32 * g + 32))}


@pytest.mark.parametrize("S", [0, 32])
@pytest.mark.parametrize("W", [0, 32, 64, 256])
def test_near_far_split_enumeration(S, W):
    for n in range(0, 640):
        sink_end, hb, he = O.near_far_split(n, S, W)
        assert sink_end == min(n, S)
        groups = _brute_quantized_groups(n, S, W)
        assert set(range(hb // 32, he // 32)) == groups
        if groups:
            assert hb == S and W <= n - he <= W + 31
        else:
            assert he == hb == S


def _sink_row(rng, n_sink, n_hist, n_win, bits, outliers=True):
    ks, vs = rand_bf16(rng, n_sink, 128), rand_bf16(rng, n_sink, 128)
    _, _, qh = _head(rng, n_hist, bits, outliers=outliers)
    kw, vw = rand_bf16(rng, n_win, 128), rand_bf16(rng, n_win, 128)
    return ks, vs, qh, kw, vw


@pytest.mark.parametrize("bits,tau", [(4, 0.0), (4, 2.0), (2, 0.05)])
def test_sink_window_attention_reduces_to_library_sdpa(bits, tau):
    """Sink, history and window together: at the identity taus (and on INT2) the output is a
    library softmax attention over [sink exact; history dequantized; window exact]."""
    rng = np.random.default_rng(42)
    ks, vs, qh, kw, vw = _sink_row(rng, 32, 128, 37, bits)
    q = rand_bf16(rng, 128)
    out, hot, _ = O.decode_head(q, qh, kw, vw, sm_scale=1 / math.sqrt(128), tau=tau,
                                sink_k=ks, sink_v=vs, hist_start=32)
    khat = O.dequant_keys(qh.k_codes, qh.k_s, qh.k_z)
    if bits == 4 and tau > 1:
        vhat = O.dequant_values_cold(qh.v_codes, qh.v_s, qh.v_z)
        assert not hot.any()
    else:
        vhat = O.dequant_values_full(qh.v_codes, qh.v_s, qh.v_z)
        assert hot.all()
    ref = _sdpa(q, np.concatenate([ks, khat, kw]), np.concatenate([vs, vhat, vw]))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # a window that covers the whole request: exact attention over every token
    out2, hot2, _ = O.decode_head(q, None, kw, vw, sm_scale=1 / math.sqrt(128), tau=tau,
                                  sink_k=ks, sink_v=vs, hist_start=32)
    assert hot2.size == 0
    assert np.allclose(out2, _sdpa(q, np.concatenate([ks, kw]), np.concatenate([vs, vw])),
                       rtol=1e-12, atol=1e-12)


def test_dominant_sink_seed_makes_history_cold():
    """A sink key aligned with the query scores far above every history token, so with the
    sink maximum as the seed every history token is cold (exp(s_j - m) < tau from the first
    group on); without it each split's largest score is hot."""
    rng = np.random.default_rng(43)
    ks, vs, qh, kw, vw = _sink_row(rng, 32, 192, 5, 4, outliers=False)
    q = np.zeros(128)
    q[:8] = 1.0
    ks[3] = 0.0
    ks[3, :8] = 64.0                      # score 512 / sqrt(128) = 45.25 vs |history| < 10
    sm = 1 / math.sqrt(128)
    _, hot, s_hist = O.decode_head(q, qh, kw, vw, sm_scale=sm, tau=0.01, sink_k=ks, sink_v=vs,
                                   hist_start=32, split_tokens=64)
    assert s_hist.max() < 45.25 + math.log(0.01)
    assert not hot.any()
    _, hot0, _ = O.decode_head(q, qh, kw, vw, sm_scale=sm, tau=0.01, sink_k=ks, sink_v=vs,
                               hist_start=32, split_tokens=64, sink_seed=False)
    # splits of 64 from token 0 with the history at 32..223: splits [32,64), [64,128),
    # [128,192), [192,224); each has its largest score hot
    for lo, hi in [(0, 32), (32, 96), (96, 160), (160, 192)]:
        assert hot0[lo + int(np.argmax(s_hist[lo:hi]))]


def test_sink_seed_monotone_and_proposition1():
    """A larger seed only turns hot tokens cold; with the sink maximum as the seed every cold
    token still weighs less than tau times the largest weight of the whole row."""
    rng = np.random.default_rng(44)
    for trial in range(12):
        ks, vs, qh, kw, vw = _sink_row(rng, 32, 256, 40, 4)
        q = rand_bf16(rng, 128) * rng.uniform(0.5, 3)
        sm = 1 / math.sqrt(128)
        split = [0, 64, 128][trial % 3]
        kw_ = dict(sm_scale=sm, tau=0.02, sink_k=ks, sink_v=vs, hist_start=32, split_tokens=split)
        _, hot_s, s_hist = O.decode_head(q, qh, kw, vw, **kw_)
        _, hot_n, _ = O.decode_head(q, qh, kw, vw, sink_seed=False, **kw_)
        assert np.all(hot_s <= hot_n)
        row_max = max(s_hist.max(), sm * (ks @ q).max(), sm * (kw @ q).max())
        assert np.all(np.exp(s_hist[~hot_s] - row_max) < 0.02)


# ------------------------------------------------------------------ planner
def _tiny_damage(rng, T, L):
    d = rng.lognormal(-3, 1.0, size=(T, L, 3))
    d[:, :, 1] += d[:, :, 0]          # 2-bit codes cost more than 4-bit ones
    d[T - 1, :, 2] = np.nan
    return d


@pytest.mark.parametrize("T,L", [(2, 2), (3, 2), (2, 3)])
def test_planner_exhaustive_matches_integer_program(T, L):
    """Two independent exact methods -- enumerating every plan, and scipy's MILP solver over
    one binary per (layer, option tuple) -- agree on the optimum's reads and damage."""
    rng = np.random.default_rng(100 + 10 * T + L)
    for trial in range(4):
        d = _tiny_damage(rng, T, L)
        d4 = float(d[:, :, 0].sum())
        all4 = O.plan_cost(np.full((T, L), 4, np.uint8), d)[1]
        # storage budgets below the all-INT2 plan's (0.57 of all-INT4) force reusing cells
        md = [-1.0, d4 * rng.uniform(1.2, 4.0), -1.0, d4 * rng.uniform(3.0, 8.0)][trial]
        ms = [0.0, 0.0, all4 * 0.5, all4 * 0.55][trial]
        if trial == 3:
            # a binding storage budget: 2-bit codes are too damaging, so every cell reads 4 bits,
            # and only reusing cells can bring the storage under 80% of the all-INT4 plan's
            d[:, :, 0], d[:, :, 1], d[:, :, 2] = 0.01, 1.0, 0.02
            d[T - 1, :, 2] = np.nan
            md, ms = 0.5, all4 * 0.8
        pe, ce = O.plan_exhaustive(d, md, ms)
        pm, cm = O.plan_milp(d, md, ms)
        assert (pe is None) == (pm is None)
        if pe is None:
            continue
        assert ce[2] == cm[2] and abs(ce[0] - cm[0]) <= 1e-12 * max(1.0, ce[0])
        assert (pe[T - 1] != O.REUSE).all()


def test_planner_closed_form_optima():
    """No budget: every cell reads 2-bit bytes (reusing a 2-bit final loop reads the same), so
    the reads are those of the all-INT2 plan. A zero damage budget with free 4-bit codes forces
    the all-INT4 plan."""
    rng = np.random.default_rng(7)
    T, L = 3, 2
    d = _tiny_damage(rng, T, L)
    all2 = np.full((T, L), 2, np.uint8)
    p, c = O.plan_exhaustive(d)
    assert c[2] == O.plan_cost(all2, d)[2]
    assert all(int(p[t, l]) == 2 or (int(p[t, l]) == 0 and int(p[T - 1, l]) == 2)
               for t in range(T) for l in range(L))
    d0 = d.copy()
    d0[:, :, 0] = 0.0
    p, c = O.plan_exhaustive(d0, max_damage=0.0)
    assert (p == 4).all() and c[0] == 0.0
    assert O.plan_milp(d0, max_damage=0.0)[1][2] == O.plan_cost(np.full((T, L), 4, np.uint8), d0)[2]


def test_planner_monotone_in_budgets():
    rng = np.random.default_rng(8)
    d = _tiny_damage(rng, 3, 2)
    d4 = float(d[:, :, 0].sum())
    prev = None
    for f in [1.0, 1.5, 2.5, 4.0, 8.0]:
        _, c = O.plan_exhaustive(d, max_damage=d4 * f)
        assert c is not None
        if prev is not None:
            assert c[2] <= prev
        prev = c[2]


# --------------------------------------------------------------------------------------
# End to end against a scalar pure-Python decode (no NumPy in the computation)
# --------------------------------------------------------------------------------------
def _half(x):
    """Nearest fp16 value of a Python float, ties to even (struct's 'e' format rounds so)."""
    import struct
    return struct.unpack("<e", struct.pack("<e", x))[0]


def _scalar_quant(xs, bits):
    levels = (1 << bits) - 1
    mn, mx = min(xs), max(xs)
    s, z = _half((mx - mn) / levels), _half(mn)
    codes = [0 if s == 0 else min(max(math.floor((x - z) / s + 0.5), 0), levels) for x in xs]
    return codes, s, z


def _scalar_decode(q, k, v, tail_k, tail_v, bits, v_group, sm, tau, m0, split):
    """Quantize (keys per channel over 32-token groups, values per token over v_group channels),
    dequantize (cold 4-bit values at the middle of their high-plane bucket), stream the fetch
    test (running maximum per split, updated per group before its tokens are tested), softmax
    over history and exact tail, weighted sum of values. Lists and loops only."""
    n, d = len(k), len(q)
    khat = [[0.0] * d for _ in range(n)]
    for g0 in range(0, n, 32):
        for c in range(d):
            codes, s, z = _scalar_quant([k[t][c] for t in range(g0, g0 + 32)], bits)
            for i, t in enumerate(range(g0, g0 + 32)):
                khat[t][c] = s * codes[i] + z
    vfull, vcold = [[0.0] * d for _ in range(n)], [[0.0] * d for _ in range(n)]
    for t in range(n):
        for c0 in range(0, d, v_group):
            codes, s, z = _scalar_quant(v[t][c0:c0 + v_group], bits)
            for i, c in enumerate(range(c0, c0 + v_group)):
                vfull[t][c] = s * codes[i] + z
                vcold[t][c] = s * (4 * (codes[i] >> 2) + 1.5) + z
    score = [sm * sum(q[c] * khat[t][c] for c in range(d)) for t in range(n)]
    hot = [True] * n
    if bits == 4:
        span = split if split else n
        for a in range(0, n, span):
            m = m0
            for g0 in range(a, min(a + span, n), 32):
                m = max(m, max(score[g0:g0 + 32]))
                for t in range(g0, g0 + 32):
                    hot[t] = math.exp(score[t] - m) >= tau
    vals = [vfull[t] if hot[t] else vcold[t] for t in range(n)] + [list(r) for r in tail_v]
    allsc = score + [sm * sum(q[c] * r[c] for c in range(d)) for r in tail_k]
    mx = max(allsc)
    w = [math.exp(x - mx) for x in allsc]
    tot = sum(w)
    out = [sum(w[j] * vals[j][c] for j in range(len(w))) / tot for c in range(d)]
    return out, hot


@pytest.mark.parametrize("bits,tau,split,m0", [(4, 0.05, 0, -math.inf), (4, 0.2, 64, -math.inf),
                                               (4, 0.01, 32, 0.8), (2, 0.05, 0, -math.inf)])
def test_decode_matches_scalar_python(bits, tau, split, m0):
    """The whole oracle decode (quantize, dequantize, fetch mask, softmax attention) against the
    scalar loops above on tiny rows (D = 8, 8-channel value groups, 96 history tokens and 5 exact
    ones): the hot set exactly, the output to 1e-12 relative. Intermediate tau values, so hot
    and cold tokens mix in the output."""
    rng = np.random.default_rng(900 + bits + int(tau * 1000) + split)
    d, n = 8, 96
    k = np.round(rng.normal(size=(n, d)) * 64) / 64
    k[:, 3] *= 6.0                              # one outlier channel concentrates attention
    v = np.round(rng.normal(size=(n, d)) * 64) / 64
    tk, tv = np.round(rng.normal(size=(5, d)) * 64) / 64, np.round(rng.normal(size=(5, d)) * 64) / 64
    q = np.round(rng.normal(size=d) * 64) / 64
    sm = 1 / math.sqrt(d)
    ref, hot_ref = _scalar_decode(q.tolist(), k.tolist(), v.tolist(), tk.tolist(), tv.tolist(),
                                  bits, 8, sm, tau, m0, split)
    qh = O.quantize_head(k, v, bits, 8)
    out, hot, _ = O.decode_head(q, qh, tk, tv, sm_scale=sm, tau=tau, m0=m0, split_tokens=split)
    assert list(hot) == hot_ref
    if bits == 4:
        assert 0 < sum(hot_ref) < n                  # both kinds of token present
    assert np.allclose(out, ref, rtol=0, atol=1e-12 * max(abs(x) for x in ref))
