"""The library's planner (loopkv_plan_solve, host C++) against the oracle's exact planners.

Tiny instances: the full (reads, damage, storage) optimum of the oracle's enumeration of every
plan. The paper's cell grids (24 x 4 = 96 and 48 x 4 = 192 cells) on synthetic damage tables:
the optimum reads and damage of the oracle's integer program (scipy's HiGHS). Every returned
plan is checked against its own budgets with the oracle's cost function."""
import math

import numpy as np
import pytest

import oracle as O
from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth


def _shape(layers, loops, v_group=128):
    return L.make_shape(num_layers=layers, num_loops=loops, v_group=v_group, max_batch=1,
                        max_pages_per_seq=1, num_pages=1)


def _check_valid(plan, cost, d, md, ms, v_group=128, h=1.0):
    T = plan.shape[0]
    assert set(np.unique(plan)) <= {0, 2, 4} and (plan[T - 1] != 0).all()
    c = O.plan_cost(plan, d, v_group=v_group, hot_fraction=h)
    assert abs(c[0] - cost.damage) <= 1e-9 * max(1.0, c[0])
    assert c[1] == cost.stored_bytes_per_token and abs(c[2] - cost.read_bytes_per_token) <= 1e-6
    assert md < 0 or c[0] <= md
    assert ms <= 0 or c[1] <= ms
    return c


@pytest.mark.parametrize("T,Lr", [(2, 2), (3, 2), (2, 3), (4, 1)])
def test_tiny_instances_match_enumeration(T, Lr):
    rng = np.random.default_rng(200 + 10 * T + Lr)
    for trial in range(6):
        d = rng.lognormal(-3, 1.0, size=(T, Lr, 3))
        d[:, :, 1] += d[:, :, 0]
        d[T - 1, :, 2] = np.nan
        d4 = float(d[:, :, 0].sum())
        all4 = O.plan_cost(np.full((T, Lr), 4, np.uint8), d)[1]
        md = [-1.0, d4 * 1.5, d4 * 3.0, -1.0, 0.5, d4 * 2.0][trial]
        ms = [0.0, 0.0, all4 * 0.6, all4 * 0.5, all4 * 0.8, 0.0][trial]
        if trial == 4:                      # 4-bit reads forced, storage binding
            d[:, :, 0], d[:, :, 1], d[:, :, 2] = 0.01, 1.0, 0.02
            d[T - 1, :, 2] = np.nan
        h = [1.0, 0.25][trial % 2]
        pe, ce = O.plan_exhaustive(d, md, ms, hot_fraction=h)
        if pe is None:
            with pytest.raises(L.LoopKVError) as e:
                L.loopkv_plan_solve(_shape(Lr, T), d, md, ms, h)
            assert e.value.status == L.EINFEASIBLE
            continue
        plan, cost = L.loopkv_plan_solve(_shape(Lr, T), d, md, ms, h)
        c = _check_valid(plan, cost, d, md, ms, h=h)
        assert abs(c[2] - ce[2]) <= 1e-6 and abs(c[0] - ce[0]) <= 1e-12 * max(1.0, ce[0])
        assert c[1] == ce[1]


@pytest.mark.parametrize("layers,v_group", [(24, 32), (24, 128), (48, 128)])
def test_paper_grids_match_integer_program(layers, v_group):
    """Read-optimized (damage budget only) and memory-optimized (damage and storage budgets)
    plans on the 96- and 192-cell grids, at full and at 20% low-plane reads."""
    d = synth.damage_table(layers, 4, 11 + layers)
    d4 = float(np.nansum(d[:, :, 0]))
    all4 = O.plan_cost(np.full((4, layers), 4, np.uint8), d, v_group=v_group)[1]
    for md, ms, h in [(d4 * 3.0, 0.0, 1.0), (d4 * 5.0, all4 * 0.62, 1.0), (d4 * 4.0, 0.0, 0.2),
                      (d4 * 8.0, all4 * 0.5, 1.0)]:
        plan, cost = L.loopkv_plan_solve(_shape(layers, 4, v_group), d, md, ms, h)
        c = _check_valid(plan, cost, d, md, ms, v_group, h)
        pm, cm = O.plan_milp(d, md, ms, v_group=v_group, hot_fraction=h)
        assert pm is not None
        assert abs(c[2] - cm[2]) <= 1e-6, (c, cm)
        assert abs(c[0] - cm[0]) <= 1e-7 * max(1.0, cm[0]), (c, cm)


def test_sharing_only_when_storage_binds():
    """With reads minimised and no storage budget, a reusing cell never reads INT4 pages when
    reusing is more damaging than an own INT4 copy (true of every cell of this table): it would
    read as much as the own copy for no saving (the paper's read-optimized plan shares no cell
    for this reason). Reusing a 2-bit final loop reads as little as 2-bit codes and may win."""
    d = synth.damage_table(24, 4, 5)
    assert (d[:3, :, 2] > d[:3, :, 0]).all()
    d4 = float(np.nansum(d[:, :, 0]))
    for f in [1.5, 2.5, 4.0]:
        plan, _ = L.loopkv_plan_solve(_shape(24, 4), d, d4 * f)
        reuse = np.argwhere(plan == 0)
        assert all(plan[3, l] == 2 for _, l in reuse)


def test_invalid_and_infeasible():
    d = synth.damage_table(4, 3, 1)
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_plan_solve(_shape(4, 3), d, max_damage=0.0)
    assert e.value.status == L.EINFEASIBLE
    bad = d.copy()
    bad[0, 0, 1] = math.inf
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_plan_solve(_shape(4, 3), bad)
    assert e.value.status == L.EINVAL
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_plan_solve(_shape(4, 3), d, hot_fraction=1.5)
    assert e.value.status == L.EINVAL
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_plan_solve(_shape(2, 6), synth.damage_table(2, 6, 1))
    assert e.value.status == L.ENOTSUP


@pytest.mark.parametrize("T,Lr", [(1, 3), (5, 1)])
def test_loop_count_limits_match_enumeration(T, Lr):
    """One loop (every cell is the final loop: no reuse option) and five loops (the largest
    supported: 2 * 3^4 whole-layer choices), against the oracle's enumeration of every plan."""
    rng = np.random.default_rng(500 + T)
    d = rng.lognormal(-3, 1.0, size=(T, Lr, 3))
    d[:, :, 1] += d[:, :, 0]
    d[T - 1, :, 2] = np.nan
    d4 = float(d[:, :, 0].sum())
    all4 = O.plan_cost(np.full((T, Lr), 4, np.uint8), d)[1]
    for md, ms in [(-1.0, 0.0), (d4 * 2.0, 0.0), (d4 * 3.0, all4 * 0.7)]:
        pe, ce = O.plan_exhaustive(d, md, ms)
        if pe is None:
            with pytest.raises(L.LoopKVError):
                L.loopkv_plan_solve(_shape(Lr, T), d, md, ms)
            continue
        plan, cost = L.loopkv_plan_solve(_shape(Lr, T), d, md, ms)
        c = _check_valid(plan, cost, d, md, ms)
        assert abs(c[2] - ce[2]) <= 1e-6 and abs(c[0] - ce[0]) <= 1e-12 * max(1.0, ce[0])
        if T == 1:
            assert (plan != 0).all()
