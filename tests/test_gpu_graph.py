"""moe_forward inside a captured HIP graph: it launches kernels only (no host
synchronisation, no memset nodes, no allocation), so one capture replays the
whole layer.  Every replay, with other eager work and synchronisations in
between, must reproduce the eager result bit for bit (both combine forms are
deterministic for these shapes)."""
import numpy as np
import pytest

from moe_synth import Workload, custom_config
from tests.parity import gpu_forward

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_bincount_amd as m
    return m


@pytest.mark.parametrize("T,E,k,cf,shared,overflow", [
    (600, 8, 2, None, True, "drop"),       # grouped output + combine kernel
    (64, 8, 2, None, False, "drop"),       # decode-sized: atomic combine
    (800, 16, 2, 0.75, True, "reroute"),   # re-routing rounds inside the graph
    (500, 8, 2, 1.0, True, "shared")])
def test_forward_graph_replays(moe, T, E, k, cf, shared, overflow):
    print(f"[graph] T={T} E={E} k={k} cf={cf} shared={shared} {overflow}", flush=True)
    cfg = custom_config(T, 256, E, k, 256, cf=cf, shared=shared, seed=T + E,
                        router_bias="zipf1.5" if cf else None)
    wl = Workload(cfg)
    rounds = 2 if overflow == "reroute" else 0
    out, layer, dev = gpu_forward(wl, overflow=overflow, rounds=rounds)
    eager = layer.y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer(dev["x"])                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(dev["x"])
    for rep in range(3):
        layer.y.fill_(float("nan"))          # the replay must overwrite every element
        _ = (torch.randn(1 << 16, device="cuda") * 2).sum().item()   # eager work in between
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, eager), f"replay {rep} differs from the eager result"
    assert np.array_equal(layer.counts.cpu().numpy(), out["counts"])
