"""moe_forward_noalloc: the layer with the library's fixed device scratch in
place of a caller workspace.  On the GPU it must give moe_forward's result
(routing, counts and offsets bit for bit; y within fp32 summation order,
since the fused combine adds with atomics) and the oracle's within the bf16
bound, on two calls in a row, the second with a smaller input, in both
combine forms.  On the host, shapes past the scratch size are refused before
anything is launched."""
import numpy as np
import pytest

from moe_synth import Workload, custom_config
from tests.parity import check_forward, gpu_forward, rel_err

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_bincount_amd as m
    return m


def _noalloc(moe, layer, dev):
    s = layer.shape
    T, d, E, k = s.T, s.d, s.E, s.top_k
    y = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    W_g = layer.W_g_packed if layer.W_g_packed is not None else dev["W_g"]
    moe.moe_forward_noalloc(s, dev["x"], W_g, dev["b_g"], layer.weights, y, idx, w,
                            counts, offsets)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), idx=idx.cpu().numpy(), w=w.cpu().numpy(),
                counts=counts.cpu().numpy(), offsets=offsets.cpu().numpy())


@pytest.mark.gpu
@pytest.mark.parametrize("combine", ["fused", "grouped"])
def test_noalloc_matches_forward_twice(moe, combine):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # decode-sized then smaller; a shared expert and a capacity in the first
    for T, shared, cf, seed in ((96, True, 1.0, 11), (40, False, None, 12)):
        print(f"[noalloc] combine={combine} T={T} shared={shared} cf={cf}", flush=True)
        cfg = custom_config(T, 1024, 8, 2, 2048, shared=shared, cf=cf, seed=seed)
        wl = Workload(cfg)
        ref, layer, dev = gpu_forward(wl, combine=combine)
        got = _noalloc(moe, layer, dev)
        for key in ("idx", "counts", "offsets"):
            assert np.array_equal(got[key], ref[key]), key
        assert np.array_equal(got["w"], ref["w"])
        assert not np.isnan(got["y"]).any()
        err = rel_err(got["y"], ref["y"])
        assert err <= 1e-5, err
        if combine == "grouped":  # slot-order sums: bit-identical
            assert np.array_equal(got["y"], ref["y"])
        rep = check_forward(wl, got)
        print(f"  vs moe_forward {err:.2e}, vs oracle {rep['err']:.3e}", flush=True)


@pytest.mark.cpu
def test_noalloc_refuses_shapes_past_its_scratch(moe):
    # the Mixtral-shaped prefill needs hundreds of MiB of workspace
    s = moe.make_shape(4096, 4096, 8, 2, 14336)
    assert moe.moe_workspace_bytes(s) > moe.NOALLOC_SCRATCH_BYTES
    fake = 256  # never dereferenced: the size check comes first
    with pytest.raises(moe.MoEError, match="scratch") as ei:
        moe.moe_forward_noalloc(s, fake, fake, None, moe.make_weights(W1=fake, W3=fake, W2=fake),
                                fake, fake, fake, fake, fake, stream=0)
    assert ei.value.status == 2
    # shape validation still comes first
    with pytest.raises(moe.MoEError, match="E="):
        moe.moe_forward_noalloc(moe.make_shape(16, 256, 0, 2, 128), fake, fake, None,
                                moe.make_weights(W1=fake, W3=fake, W2=fake), fake, fake, fake,
                                fake, fake, stream=0)
