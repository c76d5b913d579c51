"""The forward path captured in a HIP graph and replayed.

The library enqueues only kernels on the caller's stream (no allocation, no
memset, no synchronisation), so one fused moe_route_dispatch + moe_combine
step, or the three separate calls, can be captured once and replayed; for the
small workloads the replay removes the per-call launch overhead.  Each test
replays the graph several times with the program's own eager work and
synchronisations in between, changes the inputs in place between replays, and
checks every replay bit for bit against the eager calls on the same inputs
(themselves checked against the oracle by the parity tests); the first
replay is also compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

from moe_token_routing_router_amd import _lib as L
from moe_token_routing_router_amd import inputs as I
from oracle import oracle as O
from tests.parity import check_combine, check_route, from_dev, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.library()


class Step:
    """Static buffers of one forward step (route, dispatch, combine)."""

    def __init__(self, name, fused):
        d = I.make_inputs(name)
        self.d, self.fused = d, fused
        N, H, E, K = d["x"].shape[0], d["x"].shape[1], d["E"], d["K"]
        self.N, self.H, self.E, self.K = N, H, E, K
        self.x = to_dev(d["x"], d["dtype"])
        self.gw = to_dev(d["gate_w"], d["dtype"])
        self.bias = None if d["bias"] is None else torch.from_numpy(d["bias"]).cuda()
        self.y = to_dev(d["y"], d["dtype"])
        dev, dt = self.x.device, self.x.dtype
        i32 = dict(dtype=torch.int32, device=dev)
        self.ids = torch.empty((N, K), **i32)
        self.w = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.counts, self.offsets = torch.empty((E,), **i32), torch.empty((E + 1,), **i32)
        self.perm, self.inv = torch.empty((N * K,), **i32), torch.empty((N * K,), **i32)
        self.x_perm = torch.empty((N * K, H), dtype=dt, device=dev)
        self.out = torch.empty((N, H), dtype=dt, device=dev)
        if fused:
            nws = L.moe_route_dispatch_workspace_size(N, H, E, K, dt)
            self.ws = torch.empty((max(1, nws),), dtype=torch.uint8, device=dev)
        else:
            nrw = L.moe_route_workspace_size(H, E, dt)
            self.rws = torch.empty((nrw,), dtype=torch.uint8, device=dev) if nrw else None
            self.dws = torch.empty((L.moe_dispatch_workspace_size(N, E, K),),
                                   dtype=torch.uint8, device=dev)

    def run(self):
        if self.fused:
            L.moe_route_dispatch(self.x, self.gw, self.bias, self.K, self.ids, self.w,
                                 self.counts, self.offsets, self.perm, self.inv, self.x_perm,
                                 self.ws)
        else:
            L.moe_route(self.x, self.gw, self.bias, self.K, self.ids, self.w, None, self.rws)
            L.moe_dispatch(self.ids, self.x, self.E, self.counts, self.offsets, self.perm,
                           self.inv, self.x_perm, self.dws)
        L.moe_combine(self.y, self.inv, self.w, self.out)

    def outputs(self):
        return [t.clone() for t in (self.ids, self.w, self.counts, self.offsets, self.perm,
                                    self.inv, self.x_perm, self.out)]

    def scramble(self):
        for t in (self.ids, self.counts, self.offsets, self.perm, self.inv):
            t.fill_(-7)
        self.w.fill_(float("nan"))
        self.x_perm.fill_(3.0)
        self.out.fill_(-3.0)


def same(a, b):
    return all(torch.equal(u.view(torch.uint8) if u.is_floating_point() else u,
                           v.view(torch.uint8) if v.is_floating_point() else v)
               for u, v in zip(a, b))


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "three-call"])
@pytest.mark.parametrize("name", ["tiny-fp32", "small-bf16", "biased-bf16"])
def test_graph_replay_matches_eager(name, fused):
    st = Step(name, fused)
    # inputs for alternate replays: the same shapes, other values
    x_alt = st.x.flip(0).contiguous()
    y_alt = st.y.flip(0).contiguous()
    x0, y0 = st.x.clone(), st.y.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the library up off the capture
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()

    for rep in range(REPLAYS):
        src_x, src_y = (x0, y0) if rep % 2 == 0 else (x_alt, y_alt)
        st.x.copy_(src_x)
        st.y.copy_(src_y)
        torch.cuda.synchronize()
        st.run()  # eager reference on the same inputs
        torch.cuda.synchronize()
        want = st.outputs()
        st.scramble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = st.outputs()
        assert same(got, want), f"{name} fused={fused}: replay {rep} differs from eager"
        if rep == 0:
            # the first replay against the oracle as well: the routing with
            # the parity tests' margin rule, the dispatch of the replay's own
            # ids exactly, and the combine of its own inv and weights
            d = st.d
            ids_o, w_o, logits_o, _ = O.route(d["x"], d["gate_w"], d["bias"], d["K"], d["dtype"])
            ids_g, w_g = from_dev(got[0]), from_dev(got[1])
            check_route(ids_g, w_g, ids_o, w_o, logits_o, d["K"], d["dtype"])
            counts, offsets, perm, inv = O.dispatch(ids_g, d["E"])
            for k, ref in ((2, counts), (3, offsets), (4, perm), (5, inv)):
                np.testing.assert_array_equal(from_dev(got[k]), ref)
            check_combine(from_dev(got[7]), O.combine(d["y"], inv, w_g, d["dtype"]), d["dtype"])
    del g
