"""The host-side helpers of the GPU parity tests: the expert stream that
feeds the oracle decoded weights ahead of its loop gives the oracle exactly
the result it computes from the generator directly (same arithmetic, only
moved to other threads), for every weight format."""
import numpy as np
import pytest

import oracle
from moe_synth import Workload, custom_config
from tests.parity import ExpertStream, expert_bytes_f64

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("w,shared,cf", [("bf16", True, None), ("fp8_e4m3", False, 1.0),
                                         ("int8", True, 0.75), ("int4", False, None)])
def test_expert_stream_equals_direct_generation(w, shared, cf):
    cfg = custom_config(96, 128, 12, 3, 128, w=w, shared=shared, cf=cf, seed=5)
    wl = Workload(cfg)
    C = oracle.capacity(cfg.T, cfg.E, cfg.k, cfg.cf)
    sh = wl.shared if shared else None
    direct = oracle.forward(wl.x(), wl.W_g(), wl.b_g(), cfg.k, cfg.E, wl.expert, C=C, shared=sh)
    stream = ExpertStream(wl.expert, cfg.E, expert_bytes_f64(cfg), workers=3,
                          budget_bytes=4 * expert_bytes_f64(cfg))
    try:
        via = oracle.forward(wl.x(), wl.W_g(), wl.b_g(), cfg.k, cfg.E, stream, C=C, shared=sh)
    finally:
        stream.close()
    assert np.array_equal(direct["y"], via["y"])


def test_expert_stream_out_of_order_and_skips():
    """Requests may skip experts (empty segments) and may go back; each answer
    is that expert's decoded weights."""
    cfg = custom_config(16, 64, 10, 2, 128, seed=9)
    wl = Workload(cfg)
    stream = ExpertStream(wl.expert, cfg.E, expert_bytes_f64(cfg), workers=2,
                          budget_bytes=3 * expert_bytes_f64(cfg))
    try:
        for e in (0, 3, 4, 9, 2):
            got = stream(e)
            ref = wl.expert(e)
            for n in ("W1", "W3", "W2"):
                assert np.array_equal(got[n], oracle.moe_oracle._weight(ref, n))
    finally:
        stream.close()
