"""moe_route_dispatch_noalloc (the library's built-in per-GPU workspace)
against moe_route_dispatch with a caller workspace, through the C ABI.

Several calls in a row on the same GPU, each smaller or differently shaped
than the one before, so a later call runs on what an earlier one left in the
shared array: every output must be bit for bit that of moe_route_dispatch
(integer outputs, the copied rows and the fp32 weights alike -- the same
kernels run on the same inputs).
"""
import numpy as np
import pytest
import torch

from moe_token_routing_router_amd import _lib as L
from moe_token_routing_router_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.library()


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _outputs(N, H, E, K, tdt, fill):
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(ids=torch.full((N, K), fill, **i32),
                w=torch.full((N, K), float(fill), dtype=torch.float32, device="cuda"),
                counts=torch.full((E,), fill, **i32), offsets=torch.full((E + 1,), fill, **i32),
                perm=torch.full((N * K,), fill, **i32), inv=torch.full((N * K,), fill, **i32),
                x_perm=torch.full((N * K, H), fill, dtype=tdt, device="cuda"))


def _bits(t):
    if t.dtype in (torch.bfloat16, torch.float32):
        return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    return t.cpu().numpy()


def _run_pair(d):
    N, H, E, K, dt = d["N"], d["H"], d["E"], d["K"], d["dtype"]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    x, gw = _dev(d["x"], dt), _dev(d["gate_w"], dt)
    b = None if d["bias"] is None else torch.from_numpy(d["bias"]).cuda()
    need = L.moe_route_dispatch_workspace_size(N, H, E, K, tdt)
    assert need <= 8 << 20
    ref = _outputs(N, H, E, K, tdt, -7)
    ws = torch.full((max(1, need),), 0x5A, dtype=torch.uint8, device="cuda")
    L.moe_route_dispatch(x, gw, b, K, ref["ids"], ref["w"], ref["counts"], ref["offsets"],
                         ref["perm"], ref["inv"], ref["x_perm"], ws)
    got = _outputs(N, H, E, K, tdt, -3)
    L.moe_route_dispatch_noalloc(x, gw, b, K, got["ids"], got["w"], got["counts"],
                                 got["offsets"], got["perm"], got["inv"], got["x_perm"])
    torch.cuda.synchronize()
    for k in ref:
        assert np.array_equal(_bits(got[k]), _bits(ref[k])), f"{k} differs (N={N} H={H} E={E} K={K})"
    # sanity: the reference itself is a valid dispatch of its ids
    counts = ref["counts"].cpu().numpy()
    assert counts.sum() == N * K
    assert np.array_equal(np.bincount(ref["ids"].cpu().numpy().ravel(), minlength=E), counts)


def test_noalloc_equals_route_dispatch_consecutive_calls():
    print("noalloc: headline shape, then smaller inputs", flush=True)
    cases = [
        I.make_inputs("h4096-bf16", with_y=False),                       # 0.7 MiB of scratch
        I.random_case(11, 3001, 1024, 128, 8, "bf16", bias=True, with_y=False),
        I.random_case(12, 777, 512, 64, 2, "bf16", with_y=False),        # smaller again
        I.random_case(13, 300, 256, 16, 2, "f32", bias=True, with_y=False),
    ]
    for d in cases:
        print(f"  N={d['N']} H={d['H']} E={d['E']} K={d['K']} {d['dtype']}", flush=True)
        _run_pair(d)


def test_noalloc_zipf128_then_small():
    # the largest of the five workloads' scratch (1.8 MiB), then a tiny call
    print("noalloc: zipf128 then small", flush=True)
    _run_pair(I.make_inputs("zipf128-bf16", with_y=False))
    _run_pair(I.random_case(14, 65, 64, 20, 3, "bf16", bias=True, with_y=False))


def test_noalloc_rejects_oversize_and_keeps_empty_calls():
    N, H, E, K = 600000, 8192, 256, 2   # needs > 8 MiB of scratch
    tdt = torch.bfloat16
    assert L.moe_route_dispatch_workspace_size(N, H, E, K, tdt) > 8 << 20
    lib = L.library()
    fake = 0x7F0000000000  # never dereferenced: rejected before any launch
    st = lib.moe_route_dispatch_noalloc(fake, fake, None, N, H, E, K, L.MOE_BF16, fake, fake,
                                        fake, fake, fake, fake, fake, None)
    assert st == 4  # MOE_ERR_WORKSPACE_TOO_SMALL
    # N = 0: counts and offsets zero-filled
    out = _outputs(0, 64, 8, 2, tdt, -1)
    out["counts"].fill_(5)
    out["offsets"].fill_(5)
    x = torch.empty((0, 64), dtype=tdt, device="cuda")
    gw = torch.zeros((64, 8), dtype=tdt, device="cuda")
    L.moe_route_dispatch_noalloc(x, gw, None, 2, out["ids"], out["w"], out["counts"],
                                 out["offsets"], out["perm"], out["inv"], out["x_perm"])
    torch.cuda.synchronize()
    assert not out["counts"].any() and not out["offsets"].any()
