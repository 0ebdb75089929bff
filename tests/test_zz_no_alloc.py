"""moe_route_noalloc, the allocation-free routing entry point, against moe_route (same kernels on a
caller workspace): two calls in a row through the C ABI, the second with a smaller routing, every
output compared bit for bit (integer results), sentinels catching unwritten entries."""
import numpy as np
import pytest
import torch

import mxfp8_quantized_moe_amd as fm
from mxfp8_quantized_moe_amd import synth
from gpu_helpers import DEV, note, host

pytestmark = pytest.mark.gpu

SENT = -7


def _outputs(T, k, E, pad):
    rows = fm.moe_route_rows_bound(T * k, E, pad)
    return tuple(torch.full((n,), SENT, dtype=torch.int32, device=DEV) for n in (E, E, T * k, rows))


def _check(ids_np, E, pad, what):
    T, k = ids_np.shape
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(DEV)
    note(f"moe_route_noalloc {what}: tokens={T} topk={k} experts={E} pad={pad}")
    got = fm.moe_route_noalloc(ids, E, _outputs(T, k, E, pad), pad)
    ref = fm.moe_route(ids, E, pad, out=_outputs(T, k, E, pad))
    for name, g, r in zip(("counts", "offs", "dest", "src"), got, ref):
        g, r = host(g), host(r)
        assert np.array_equal(g, r), f"{what}: {name} differs at {np.argwhere(g != r)[:4].ravel()}"
        assert not np.any(g == SENT), f"{what}: {name} has unwritten entries"


def test_noalloc_route_two_calls_then_smaller():
    ids3 = synth.routing_ids(3)                        # 8192 tokens x top-6 over 64 experts (Zipf)
    _check(ids3, 64, 32, "first call")
    rng = np.random.default_rng(5)
    small = rng.integers(-1, 17, size=(1000, 2)).astype(np.int32)   # 16 experts; -1 and 16 drop a slot
    _check(small, 16, 1, "second call, smaller")


def test_noalloc_route_rejects_beyond_scratch():
    # 2^20 slots over 1024 experts need 16 MiB of block histograms: rejected before any GPU work
    ids = torch.zeros((1 << 18, 4), dtype=torch.int32, device=DEV)
    out = tuple(torch.empty(1, dtype=torch.int32, device=DEV) for _ in range(4))
    with pytest.raises(fm.Fp8MoeError) as e:
        fm.moe_route_noalloc(ids, 1024, out)
    assert e.value.status == fm._lib.ERR_SCRATCH
