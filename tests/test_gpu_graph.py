"""A decode step captured in a HIP graph and replayed equals the same calls made eagerly.

The launch-bound shapes (GPT-2-sized caches: a few MB per step against a few
kernel launches) gain most from replaying a captured step.  The library makes no
allocation, no memset and no host read-back in a step, so the three calls of a
step (conf_attend, conf_confidence, conf_ema_evict_compact) capture as kernel
nodes.  Two caches take identical inputs: one runs eagerly, the other replays a
graph of ten steps five times, with eager work and synchronisations in between.
After every replay both caches, outputs, confidences and budgets must be
bit-identical (the same kernels on the same data).  The graph is captured from
one stream, and again with each step's confidence a branch on a second stream
beside its attention, joined before its eviction."""
import pytest
import torch

from adaptive_kv_cache_amd import binding, synth
from adaptive_kv_cache_amd.binding import Engine
from adaptive_kv_cache_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

SEED = 11
K = 10          # steps per graph
REPLAYS = 5


def _inputs(wl, steps0, n):
    return [(synth.logits(wl, s, SEED, device="cuda"), synth.q_new(wl, s, SEED, device="cuda"),
             *synth.kv_new(wl, s, SEED, device="cuda")) for s in range(steps0, steps0 + n)]


def _step(eng, wl, inp, out, c, budget, side=None):
    """One step; with `side` the confidence is a branch on that stream, forked
    before the attention and joined before the eviction."""
    z, q, k, v = inp
    if side is not None:
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            eng.confidence(z, c=c, budget=budget)
    eng.attend(-1, q, k, v, out=out)
    if side is not None:
        main.wait_stream(side)
    else:
        eng.confidence(z, c=c, budget=budget)
    eng.ema_evict_compact(-1, budget)


@pytest.mark.parametrize("fork", [False, True], ids=["one-stream", "forked-confidence"])
@pytest.mark.parametrize("name", ["gpt2_12layer_b8_pyramid", "gpt2_1layer_b1"])
def test_graph_replays_equal_eager_steps(name, fork):
    wl = WORKLOADS[name]
    eager, graph = Engine(wl), Engine(wl)
    L, B = wl.n_layers, wl.batch

    def bufs():
        return (torch.empty(L, B, wl.n_q_heads, wl.head_dim, dtype=torch.float32, device="cuda"),
                torch.empty(B, dtype=torch.float32, device="cuda"),
                torch.empty(B, L, dtype=torch.int32, device="cuda"))

    # both caches past their budgets first (eviction and demotion in every step)
    warm = _inputs(wl, 0, 400)
    for inp in warm:
        for eng in (eager, graph):
            _step(eng, wl, inp, *bufs())
    steps = _inputs(wl, 400, K)
    gout = [bufs() for _ in range(K)]
    eout = [bufs() for _ in range(K)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream() if fork else None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for inp, b in zip(steps, gout):
            _step(graph, wl, inp, *b, side=side)
    for r in range(REPLAYS):
        g.replay()
        for inp, b in zip(steps, eout):
            _step(eager, wl, inp, *b)
        torch.cuda.synchronize()
        for (o1, c1, b1), (o2, c2, b2) in zip(eout, gout):
            assert torch.equal(o1, o2) and torch.equal(c1, c2) and torch.equal(b1, b2), (name, r)
        for f in binding._CACHE_FIELDS:
            assert torch.equal(getattr(eager, "t_" + f), getattr(graph, "t_" + f)), (name, r, f)
        # the program's own eager work between replays
        torch.cuda.synchronize()
    assert eager.status() == 0 and graph.status() == 0
