"""GPU parity of the device-side expert placement with hot-expert
replication (moe_eplb_plan) against the oracle: integer work, bit-exact."""
import json
import os

import numpy as np
import pytest

import oracle
from moe_synth import Workload, custom_config
from tests.conftest import GOLDEN
from tests.parity import gpu_forward

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_bincount_amd as m
    return m


def _gpu_plan(moe, load, D, extra):
    E = len(load)
    counts = torch.tensor(np.asarray(load, dtype=np.int32), device="cuda")
    replicas = torch.full((E,), -5, dtype=torch.int32, device="cuda")
    slot_device = torch.full((E + extra,), -5, dtype=torch.int32, device="cuda")
    slot_load = torch.full((E + extra,), -5, dtype=torch.int32, device="cuda")
    device_load = torch.full((D,), -5, dtype=torch.int64, device="cuda")
    moe.moe_eplb_plan(counts, D, extra, replicas, slot_device, slot_load, device_load)
    torch.cuda.synchronize()
    return (replicas.cpu().numpy(), slot_device.cpu().numpy(), slot_load.cpu().numpy(),
            device_load.cpu().numpy())


def _check(moe, load, D, extra):
    r, sd, sl, dl = _gpu_plan(moe, load, D, extra)
    p = oracle.eplb_plan(load, D, extra)
    S = int(p["replicas"].sum())
    assert np.array_equal(r, p["replicas"]), "replicas differ"
    assert np.array_equal(sl[:S], p["slot_load"]), "slot loads differ"
    assert np.array_equal(sd[:S], p["slot_device"]), "slot devices differ"
    assert np.array_equal(dl, p["device_load"]), "device loads differ"
    assert np.all(sd[S:] == -1) and np.all(sl[S:] == 0)
    return p


def test_eplb_hand_worked_examples(moe):
    with open(os.path.join(GOLDEN, "eplb_replication_examples.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        print(f"[eplb golden] {c['name']}", flush=True)
        r, sd, sl, dl = _gpu_plan(moe, c["load"], c["devices"], c["extra"])
        assert r.tolist() == c["replicas"]
        assert sd.tolist() == c["slot_device"] and sl.tolist() == c["slot_load"]
        assert dl.tolist() == c["device_load"]


@pytest.mark.parametrize("E,D,extra,dist", [
    (4, 2, 0, "tutorial"), (8, 8, 0, "zipf"), (64, 8, 8, "zipf"), (256, 8, 32, "zipf"),
    (256, 8, 32, "ties"), (1024, 64, 1024, "zipf"), (1024, 1, 0, "uniform"),
    (3, 4, 20, "zipf"),           # more extra than E*(D-1): unused slots
    (100, 7, 50, "zeros"), (17, 5, 9, "ties")])
def test_eplb_bit_exact(moe, E, D, extra, dist):
    print(f"[eplb] E={E} D={D} extra={extra} {dist}", flush=True)
    rng = np.random.default_rng(E + 13 * D + extra)
    if dist == "tutorial":
        load = np.array([38, 34, 29, 27])
    elif dist == "zipf":
        load = np.minimum(rng.zipf(1.5, size=E) * 7, 100000)
    elif dist == "ties":
        load = rng.integers(0, 4, size=E) * 16
    elif dist == "zeros":
        load = np.zeros(E, dtype=np.int64)
        load[::9] = rng.integers(1, 50, size=load[::9].size)
    else:
        load = rng.integers(0, 1000, size=E)
    _check(moe, load, D, extra)


def test_eplb_from_forward_counts(moe):
    """The online form: the plan from the counts moe_forward wrote on the
    device in the same step (256 experts, top-8, 8 devices, 32 extra
    replicas)."""
    cfg = custom_config(1024, 256, 256, 8, 128, router_bias="zipf1.5", seed=71)
    out, layer, _ = gpu_forward(Workload(cfg))
    E, D, extra = 256, 8, 32
    replicas = torch.empty(E, dtype=torch.int32, device="cuda")
    slot_device = torch.empty(E + extra, dtype=torch.int32, device="cuda")
    slot_load = torch.empty(E + extra, dtype=torch.int32, device="cuda")
    device_load = torch.empty(D, dtype=torch.int64, device="cuda")
    moe.moe_eplb_plan(layer.counts, D, extra, replicas, slot_device, slot_load, device_load)
    torch.cuda.synchronize()
    p = oracle.eplb_plan(out["counts"], D, extra)
    assert np.array_equal(replicas.cpu().numpy(), p["replicas"])
    assert np.array_equal(slot_device.cpu().numpy(), p["slot_device"])
    assert np.array_equal(device_load.cpu().numpy(), p["device_load"])
    plain = oracle.lpt_pack(out["counts"], D)[1]
    print(f"  device loads max {p['device_load'].max()} (plain LPT {plain.max()}, "
          f"mean {out['counts'].sum() / D:.0f})", flush=True)
