"""Plant plausible mistakes in the oracle (on the CPU only) and check that a pin catches each.

Every mutant below is a one-line slip a careful reader could make -- a dropped half-step, a
swapped plane, '<=' for '<', the wrong midpoint, a transposed word order -- and each must make
at least one pin of tests/test_oracle_pins.py fail."""
import math

import numpy as np
import pytest

import oracle as O
import oracle.loopkv_oracle as M
from tests import test_oracle_pins as P


def _fails(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except AssertionError:
        return True
    return False


def _quantize_no_half(x, mn, mx, bits):
    L = (1 << bits) - 1
    s = O.fp16_rne((mx - mn) / L); z = O.fp16_rne(mn)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.floor((x - z) / s)
    return np.clip(np.where(s == 0, 0, c), 0, L).astype(np.int64), s, z


def _quantize_scale_by_levels_plus_one(x, mn, mx, bits):
    L = (1 << bits) - 1
    s = O.fp16_rne((mx - mn) / (L + 1)); z = O.fp16_rne(mn)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.floor((x - z) / s + 0.5)
    return np.clip(np.where(s == 0, 0, c), 0, L).astype(np.int64), s, z


def _planes_swapped(c):
    c = np.asarray(c, dtype=np.int64)
    return c & 3, c >> 2


def _cold_midpoint_2(codes4, s, z):
    hi = np.asarray(codes4) >> 2
    return M._rep_v(s, codes4.shape[1]) * (4.0 * hi + 2.0) + M._rep_v(z, codes4.shape[1])


def _mask_le(scores, m0, tau, split_tokens=0, group=32, start=0):
    scores = np.asarray(scores, dtype=np.float64)
    n = len(scores); hot = np.ones(n, dtype=bool); step = split_tokens or max(n, 1)
    for s0 in range(0, n, step):
        m = m0
        for g0 in range(s0, min(s0 + step, n), group):
            g1 = min(g0 + group, s0 + step, n)
            m = max(m, float(scores[g0:g1].max()))
            hot[g0:g1] = ~(np.exp(scores[g0:g1] - m) <= tau)
    return hot


def _mask_max_after_test(scores, m0, tau, split_tokens=0, group=32, start=0):
    scores = np.asarray(scores, dtype=np.float64)
    n = len(scores); hot = np.ones(n, dtype=bool); step = split_tokens or max(n, 1)
    for s0 in range(0, n, step):
        m = m0
        for g0 in range(s0, min(s0 + step, n), group):
            g1 = min(g0 + group, s0 + step, n)
            with np.errstate(invalid="ignore"):
                hot[g0:g1] = ~(np.exp(scores[g0:g1] - m) < tau)
            m = max(m, float(scores[g0:g1].max()))
    return hot


def _mask_no_split_reset(scores, m0, tau, split_tokens=0, group=32, start=0):
    return M.__dict__["_orig_fetch_mask"](scores, m0, tau, 0, group)


def _mask_splits_from_history_start(scores, m0, tau, split_tokens=0, group=32, start=0):
    return M.__dict__["_orig_fetch_mask"](scores, m0, tau, split_tokens, group, start=0)


def _window_exit_when_page_starts_leaving(n, sink_tokens=0, window_tokens=0, group=32):
    hs = sink_tokens // group
    he = max(hs, (n - window_tokens + group - 1) // group)
    return min(n, sink_tokens), hs * group, he * group


def _decode_head_sink_not_seeding(*a, **kw):
    kw["sink_seed"] = False
    return M.__dict__["_orig_decode_head"](*a, **kw)


def _decode_head_sink_dropped(*a, **kw):
    kw["sink_k"] = kw["sink_v"] = None
    return M.__dict__["_orig_decode_head"](*a, **kw)


def _plan_cost_reuse_reads_nothing(plan, damage, num_kv_heads=16, d=128, v_group=128, hot_fraction=1.0):
    dmg, sto, read = M.__dict__["_orig_plan_cost"](plan, damage, num_kv_heads, d, v_group, hot_fraction)
    plan = np.asarray(plan)
    T = plan.shape[0]
    for t in range(T):
        for layer in range(plan.shape[1]):
            if plan[t, layer] == 0:
                src = int(plan[T - 1, layer])
                read -= sum(M.token_head_bytes(src, d, v_group).values()) * num_kv_heads
    return dmg, sto, read


def _feasible_ignores_storage(cost, max_damage, max_stored):
    return max_damage < 0 or cost[0] <= max_damage


def _pack_rowmajor(codes, per_word, width):
    p, d = codes.shape
    c = codes.astype(np.uint64).reshape(p, d // per_word, per_word)
    return (c << (np.arange(per_word, dtype=np.uint64) * width)).sum(axis=2).astype(np.uint32)


def _dequant_keys_sign(codes, s, z):
    n = codes.shape[0]
    rep = lambda a: np.repeat(a, 32, axis=0)[:n]
    return rep(s) * codes - rep(z)


def _attention_no_max_sub(scores, vhat):
    # keeps the softmax but forgets to normalise by the sum
    if np.asarray(scores).size == 0:
        return np.zeros(vhat.shape[1])
    p = np.exp(scores - np.max(scores))
    return (p[:, None] * vhat).sum(0)


def _token_bytes_no_ksz(bits, d=128, v_group=128, k_group=32):
    r = M.__dict__["_orig_token_head_bytes"](bits, d, v_group, k_group)
    r["ksz"] = 0.0
    return r


def _tie_band_x1000(scores, m0, tau, split_tokens=0, group=32, band=1e-6, start=0):
    return M.__dict__["_orig_tie_mask"](scores, m0, tau, split_tokens, group, band * 1000, start)


def _tie_no_split_reset(scores, m0, tau, split_tokens=0, group=32, band=1e-6, start=0):
    return M.__dict__["_orig_tie_mask"](scores, m0, tau, 0, group, band, start)


def _tie_splits_from_history_start(scores, m0, tau, split_tokens=0, group=32, band=1e-6, start=0):
    return M.__dict__["_orig_tie_mask"](scores, m0, tau, split_tokens, group, band, 0)


def _tie_band_log_units(scores, m0, tau, split_tokens=0, group=32, band=1e-6, start=0):
    scores = np.asarray(scores, dtype=np.float64)
    tie = np.zeros(scores.shape[0], dtype=bool)
    m = m0
    for g0, g1, new_split in M._split_groups(scores.shape[0], start, split_tokens, group):
        if new_split:
            m = m0
        m = max(m, float(scores[g0:g1].max()))
        tie[g0:g1] = np.abs(scores[g0:g1] - m - math.log(tau)) <= band
    return tie


def _tie_band_at_tau_zero(scores, m0, tau, split_tokens=0, group=32, band=1e-6, start=0):
    scores = np.asarray(scores, dtype=np.float64)
    tie = np.zeros(scores.shape[0], dtype=bool)
    m = m0
    for g0, g1, new_split in M._split_groups(scores.shape[0], start, split_tokens, group):
        if new_split:
            m = m0
        m = max(m, float(scores[g0:g1].max()))
        tie[g0:g1] = np.abs(np.exp(scores[g0:g1] - m) - tau) <= band
    return tie


def _tie_own_group_max(scores, m0, tau, split_tokens=0, group=32, band=1e-6, start=0):
    scores = np.asarray(scores, dtype=np.float64)
    tie = np.zeros(scores.shape[0], dtype=bool)
    for g0, g1, _ in M._split_groups(scores.shape[0], start, split_tokens, group):
        m = max(m0, float(scores[g0:g1].max()))
        tie[g0:g1] = np.abs(np.exp(scores[g0:g1] - m) - tau) <= band
    return tie


def _pack_pool_ignores_sink(bits, page_tokens, heads_q, page_table, num_pages, v_group=128, hist_start=0):
    return M.__dict__["_orig_pack_pool"](bits, page_tokens, heads_q, page_table, num_pages, v_group, 0)


def _pack_pool_heads_reversed(bits, page_tokens, heads_q, page_table, num_pages, v_group=128, hist_start=0):
    rev = [list(reversed(row)) for row in heads_q]
    return M.__dict__["_orig_pack_pool"](bits, page_tokens, rev, page_table, num_pages, v_group, hist_start)


def _kc_fields_in_channel_order(bits):
    return np.arange(32 // bits)


MUTANTS = {
    "key-code words packed in plain channel order": ("_kc_field_channels", _kc_fields_in_channel_order,
                                                     [P.test_layout_fixture_positions], []),
    "pool pages placed from token 0 despite a sink": ("pack_pool", _pack_pool_ignores_sink,
                                                      [P.test_pool_placement_fixture], []),
    "pool head blocks in reverse order": ("pack_pool", _pack_pool_heads_reversed,
                                          [P.test_pool_placement_fixture], []),
    "tie band 1000x too wide": ("tie_mask", _tie_band_x1000, [P.test_tie_mask_hand_placed], [0.01]),
    "tie band without the per-split reset": ("tie_mask", _tie_no_split_reset,
                                             [P.test_tie_mask_hand_placed], [0.01]),
    "tie band splits counted from the history start": ("tie_mask", _tie_splits_from_history_start,
                                                       [P.test_tie_mask_hand_placed], [0.02]),
    "tie band counting tiny weights at tau = 0": ("tie_mask", _tie_band_at_tau_zero,
                                                  [P.test_tie_mask_hand_placed], [0.01]),
    "tie band in log units": ("tie_mask", _tie_band_log_units, [P.test_tie_mask_hand_placed], [0.01]),
    "tie band against the group's own maximum": ("tie_mask", _tie_own_group_max,
                                                 [P.test_tie_mask_hand_placed], [0.01]),
    "round half dropped": ("_quantize", _quantize_no_half,
                           [P.test_quantize_matches_nearest_grid_point, P.test_quantize_ramp_closed_form], [4]),
    "scale over 2^b levels": ("_quantize", _quantize_scale_by_levels_plus_one,
                              [P.test_quantize_ramp_closed_form], [4]),
    "planes swapped": ("split_planes", _planes_swapped, [P.test_planes_bijection_and_cold_error], []),
    "cold midpoint 2": ("dequant_values_cold", _cold_midpoint_2, [P.test_cold_value_is_nearest_bucket_midpoint], []),
    "cold test <=": ("fetch_mask", _mask_le, [P.test_mask_matches_non_streaming_brute_force], [0, 1.0, 0.5]),
    "max joined after test": ("fetch_mask", _mask_max_after_test,
                              [P.test_mask_matches_non_streaming_brute_force], [0, 0.02, -math.inf]),
    "split ignored": ("fetch_mask", _mask_no_split_reset,
                      [P.test_mask_matches_non_streaming_brute_force], [32, 0.02, -math.inf]),
    "word order transposed": ("_pack_words_colmajor", _pack_rowmajor, [P.test_layout_fixture_positions], []),
    "key zero subtracted": ("dequant_keys", _dequant_keys_sign,
                            [P.test_quantize_error_bound], [4]),
    "softmax unnormalised": ("attention_row", _attention_no_max_sub,
                             [P.test_attention_special_cases], []),
    "key scale bytes dropped": ("token_head_bytes", _token_bytes_no_ksz,
                                [P.test_cache_bytes_match_paper_figures], []),
    "splits counted from the history start": ("fetch_mask", _mask_splits_from_history_start,
                                              [P.test_mask_after_sink_matches_brute_force], [32, 64]),
    "page quantized when it starts leaving the window": (
        "near_far_split", _window_exit_when_page_starts_leaving,
        [P.test_near_far_split_enumeration], [32, 256]),
    "sink maximum not used as the seed": ("decode_head", _decode_head_sink_not_seeding,
                                          [P.test_dominant_sink_seed_makes_history_cold], []),
    "sink left out of the softmax": ("decode_head", _decode_head_sink_dropped,
                                     [P.test_sink_window_attention_reduces_to_library_sdpa], [4, 0.0]),
    "a reusing cell reads nothing": ("plan_cost", _plan_cost_reuse_reads_nothing,
                                     [P.test_planner_closed_form_optima], []),
    "enumeration ignores the storage budget": ("_feasible", _feasible_ignores_storage,
                                               [P.test_planner_exhaustive_matches_integer_program], [3, 2]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, mutant, pins, args = MUTANTS[name]
    monkeypatch.setitem(M.__dict__, "_orig_fetch_mask", M.fetch_mask)
    monkeypatch.setitem(M.__dict__, "_orig_token_head_bytes", M.token_head_bytes)
    monkeypatch.setitem(M.__dict__, "_orig_decode_head", M.decode_head)
    monkeypatch.setitem(M.__dict__, "_orig_plan_cost", M.plan_cost)
    monkeypatch.setitem(M.__dict__, "_orig_tie_mask", M.tie_mask)
    monkeypatch.setitem(M.__dict__, "_orig_pack_pool", M.pack_pool)
    monkeypatch.setattr(M, attr, mutant)
    monkeypatch.setattr(O, attr, mutant, raising=False)
    caught = []
    for pin in pins:
        nargs = pin.__code__.co_argcount
        caught.append(_fails(pin, *args[:nargs]))
    assert any(caught), f"no pin caught mutant: {name}"
