"""HIP-graph capture of a serving step: the library only enqueues kernels on the caller's stream
("Loop-Aware KV Cache Compression for Serving Looped Transformers", section 3.4, "The unified
kernel": fixed device addresses make the step capturable).

One step appends one token per request to every cell, then decodes every cell, in model order.
Two caches are filled identically; one runs the step as a captured graph, the other eagerly.
Each of several replays runs after eager work and a synchronisation, and its outputs, pools,
rings and counters must equal the eager cache's bit for bit; the last step is also checked
against the oracle."""
import numpy as np
import pytest
import torch

from quantized_kv_decode_amd import loopkv as L
from quantized_kv_decode_amd import synth
from tests.helpers import Workload, check_out, log

pytestmark = pytest.mark.gpu


def _cells(w):
    return [(t, l) for t in range(w.T) for l in range(w.L)]


@pytest.mark.parametrize("P,sink,window,split", [(32, 0, 0, 0), (16, 32, 64, 0), (32, 0, 0, 64)])
def test_graph_replays_match_eager_step(P, sink, window, split):
    """split > 0: every decode is split, and the partials are merged inside the launch by the
    row group's last workgroup, whose counters must be back at zero for every replay."""
    plan = np.array([[4, 2], [2, 4], [0, 0], [4, 2]], np.uint8)
    lens0 = np.array([31, 96, 170, 257, 33], np.int32)
    steps = 4
    log(f"graph step P={P} sink={sink} window={window} split={split}")
    ws = [Workload(plan, batch=5, lens=lens0 + steps + 1, page_tokens=P, seed=123, sink_tokens=sink,
                   window_tokens=window) for _ in range(2)]
    g_w, e_w = ws
    for w in ws:
        w.append_upto(lens0, chunk=64)
    B, H, D = g_w.B, g_w.H, g_w.D
    q = {c: synth.queries(B, H, D, 900 + 10 * c[0] + c[1]).cuda() for c in _cells(g_w)}
    tau = 0.02

    def make_io():
        return dict(k={c: torch.empty(B, 1, H, D, dtype=torch.bfloat16, device="cuda") for c in _cells(g_w)},
                    v={c: torch.empty(B, 1, H, D, dtype=torch.bfloat16, device="cuda") for c in _cells(g_w)},
                    before=torch.empty(B, dtype=torch.int32, device="cuda"),
                    after=torch.empty(B, dtype=torch.int32, device="cuda"),
                    out={c: torch.empty(B, H, D, dtype=torch.float32, device="cuda") for c in _cells(g_w)})

    io = {"g": make_io(), "e": make_io()}

    def load_inputs(w, x):
        """The next token of every request: rows at each request's current length."""
        done = w.done[0, 0]
        for (t, l) in _cells(w):
            assert (w.done[t, l] == done).all()
            kk = torch.stack([w.k[t, l][b, done[b]] for b in range(B)])[:, None]
            vv = torch.stack([w.v[t, l][b, done[b]] for b in range(B)])[:, None]
            x["k"][t, l].copy_(kk)
            x["v"][t, l].copy_(vv)
        x["before"].copy_(torch.as_tensor(done.astype(np.int32)))
        x["after"].copy_(torch.as_tensor((done + 1).astype(np.int32)))

    def step(w, x):
        for (t, l) in _cells(w):
            w.cache.append(l, t, x["k"][t, l], x["v"][t, l], x["before"], w.page_table)
            w.cache.decode(l, t, q[t, l], x["after"], w.page_table, tau=tau, split_tokens=split,
                           out=x["out"][t, l])

    def advance(w):
        for c in _cells(w):
            w.done[c] += 1

    # One eager step on both caches first (loads every kernel the step uses), then capture.
    for w, k in [(g_w, "g"), (e_w, "e")]:
        load_inputs(w, io[k])
        step(w, io[k])
        advance(w)
    torch.cuda.synchronize()
    load_inputs(g_w, io["g"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(g_w, io["g"])
    torch.cuda.synchronize()
    # Capture enqueued nothing: the graph cache is still one step behind its inputs.
    for r in range(steps - 1):
        # eager work between replays: the other cache's step, and unrelated device work
        load_inputs(e_w, io["e"])
        step(e_w, io["e"])
        scratch = torch.randn(1 << 20, device="cuda")
        scratch.mul_(2.0).sum().item()
        torch.cuda.synchronize()
        load_inputs(g_w, io["g"])
        graph.replay()
        torch.cuda.synchronize()
        advance(g_w)
        advance(e_w)
        for (t, l) in _cells(g_w):
            assert torch.equal(io["g"]["out"][t, l], io["e"]["out"][t, l]), f"replay {r} cell {(t, l)} out"
            if plan[t, l] != L.REUSE:
                assert torch.equal(g_w.cache.own_pool(l, t), e_w.cache.own_pool(l, t)), f"replay {r} pool"
                assert torch.equal(g_w.cache.qgroups(l, t), e_w.cache.qgroups(l, t)), f"replay {r} counters"
            for a, b in zip(g_w.cache.tail(l, t), e_w.cache.tail(l, t)):
                assert torch.equal(a, b), f"replay {r} ring"
        log(f"  replay {r} equal to the eager step")
    for (t, l) in _cells(g_w):
        ref, _ = g_w.oracle_decode(t, l, q[t, l].cpu(), tau=tau, split_tokens=split)
        check_out(io["g"]["out"][t, l], ref, f"graph cell {(t, l)}")
    assert g_w.cache.device_errors() == 0 and e_w.cache.device_errors() == 0
