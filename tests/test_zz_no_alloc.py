"""rkv_decode_step_noalloc -- the decode step whose key-range split partials
live in the library's own device array, for callers that cannot allocate --
against rkv_decode_step with a caller workspace (the same kernels): every
output and every ring byte must be identical.  Two runs in a row share the
array: the first with 2 layers x 2 streams at W = 375, re-based every step
with the residual (8 splits per item), the second smaller (1 layer, 1 stream,
W = 200, 4 splits), so its partials overwrite only part of what the first
left behind."""
import numpy as np
import pytest
import torch

from gpu_util import device, rkv_mod, say

pytestmark = pytest.mark.gpu


def _compare(rkv, dev, S, L, W, dc, flags, splits, seed, steps):
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc, flags=flags, num_splits=splits)
    need = rkv.rkv_workspace_bytes(cfg, W)
    say(f"no-alloc: S={S} L={L} W={W} dc={dc} flags={flags} splits={splits} "
        f"partials {need} bytes")
    assert 0 < need <= rkv.RKV_NOALLOC_SCRATCH_BYTES
    origins = np.arange(S, dtype=np.int64) * 3
    a = rkv.Cache(cfg, W, W, W, origins, device=dev)     # caller workspace
    b = rkv.Cache(cfg, W, W, W, origins, device=dev)     # library array
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((steps, L, S, 16, 128), generator=gen).to(torch.bfloat16).to(dev)
    k = torch.randn((steps, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    v = torch.randn((steps, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    oa = torch.zeros((steps, L, S, 16, 128), dtype=torch.bfloat16, device=dev)
    ob = torch.full_like(oa, float("nan"))
    for t in range(steps):
        rkv.rkv_advance(cfg, a.state, a.plan)
        rkv.rkv_decode_step(cfg, a.plan, a.kv, q[t], k[t], v[t], oa[t], a.workspace)
        rkv.rkv_advance(cfg, b.state, b.plan)
        rkv.rkv_decode_step_noalloc(cfg, b.plan, b.kv, q[t], k[t], v[t], ob[t])
    torch.cuda.synchronize()
    same = oa.view(torch.int16) == ob.view(torch.int16)
    say(f"  outputs identical: {int(same.sum())} of {same.numel()}")
    assert bool(same.all())
    assert torch.equal(a.buf.view(torch.int16), b.buf.view(torch.int16))
    assert bool(torch.isfinite(oa.float()).all())


def test_no_alloc_step_matches_workspace_step_twice():
    rkv = rkv_mod()
    dev = device()
    _compare(rkv, dev, 2, 2, 375, 1, rkv.RKV_F_COMPENSATED, 0, 41, 40)
    _compare(rkv, dev, 1, 1, 200, 5, 0, 4, 42, 30)
