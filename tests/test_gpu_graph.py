"""A decode step in per-layer form (rkv_advance, then rkv_decode_step once
per layer on a one-layer view of the cache) captured as a HIP graph and
replayed, against the same calls made eagerly: outputs, rings and states
equal after every replay, with the eager run's own launches and
synchronisations between the replays (re-base every 5 positions, a split
key range, several replays of each captured graph)."""
import numpy as np
import pytest
import torch

from gpu_util import device, rkv_mod, say

pytestmark = pytest.mark.gpu


def test_per_layer_step_graph_replays_match_eager_calls():
    rkv = rkv_mod()
    dev = device()
    L, S, W, dc, P, steps = 3, 4, 40, 5, 3, 60
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc)
    cfg1 = rkv.make_cfg(S, 1, rebase_chunk=dc, num_splits=3,      # split + merge launches
                        max_cap=W)
    origins = np.array([0, 2, 9, 31], np.int64)
    gen = torch.Generator().manual_seed(31)
    q = torch.randn((P, L, S, 16, 128), generator=gen).to(torch.bfloat16).to(dev)
    k = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    v = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    nb = rkv.rkv_workspace_bytes(cfg1, W)
    assert nb > 0

    def setup():
        cache = rkv.Cache(cfg, W, W, W, origins, device=dev)
        views = [rkv.kv_view(cache.k[l:l + 1], cache.v[l:l + 1]) for l in range(L)]
        ws = torch.zeros((nb + 3) // 4, dtype=torch.float32, device=dev)
        out = torch.zeros((L, S, 16, 128), dtype=torch.bfloat16, device=dev)
        return cache, views, ws, out

    def calls(ctx, j):
        cache, views, ws, out = ctx
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        for l in range(L):
            rkv.rkv_decode_step(cfg1, cache.plan, views[l], q[j][l], k[j][l], v[j][l], out[l], ws)

    a, b = setup(), setup()
    graphs = []
    torch.cuda.synchronize()
    for j in range(P):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls(b, j)
        graphs.append(g)
    torch.cuda.synchronize()
    # capturing ran nothing: b is still at its initial state
    assert torch.equal(a[0].state, b[0].state)
    rebased = 0
    for t in range(steps):
        j = t % P
        calls(a, j)
        torch.cuda.synchronize()
        graphs[j].replay()
        torch.cuda.synchronize()
        assert torch.equal(a[3], b[3]), f"output differs at step {t}"
        assert torch.equal(a[0].state, b[0].state), f"state differs at step {t}"
        if t % 10 == 9:
            assert torch.equal(a[0].buf, b[0].buf), f"rings differ at step {t}"
        rebased += int((a[0].plan_host()["rebase_delta"] != 0).sum())
    assert rebased > 0
    say(f"per-layer step graphs: {steps} replays of {P} graphs equal the eager calls "
        f"({rebased} stream re-bases)")
