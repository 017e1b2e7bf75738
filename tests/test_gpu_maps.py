"""The device copy of the index-map arithmetic (the window function the
readout and the softmax branch use) against the host maps and the oracle's
brute-force set enumeration, bit for bit, through vda_index_map_device."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu


def _device_maps(desc):
    import torch
    n = desc.frames - 2 * desc.anchors
    C = -(-n // desc.chunk) if n > 0 else 0
    rows = torch.full((C, 7), -7, dtype=torch.int32, device="cuda")
    fc = torch.full((desc.frames,), -7, dtype=torch.int32, device="cuda")
    vda.vda_index_map_device(desc, rows, fc)
    torch.cuda.synchronize()
    return rows.cpu().numpy(), fc.cpu().numpy()


@pytest.mark.parametrize("cfg", inp.CONFIGS, ids=lambda c: c.name)
def test_device_maps_equal_host_and_oracle(cfg):
    print(f"[maps] {cfg.name}", flush=True)
    d = vda.desc_for(cfg)
    rows, fc = _device_maps(d)
    hr, hf = vda.vda_index_map(d)
    rr, ff = orc.index_maps(cfg.frames, cfg.chunk, cfg.window, cfg.anchors)
    assert np.array_equal(rows, hr) and np.array_equal(fc, hf)
    assert np.array_equal(rows, rr) and np.array_equal(fc, ff)


def test_device_maps_random_shapes():
    print("[maps] 300 random shapes", flush=True)
    g = np.random.default_rng(21)
    for _ in range(300):
        P = int(g.integers(1, 8))
        anchors = int(g.integers(0, 2))
        w = int(g.integers(-1, 5))
        n = int(g.integers(0, 30)) * (P if w >= 0 else 1)
        T = n + 2 * anchors
        d = vda.make_desc(1, T, 4, 16, chunk=P, anchors=anchors, window=w)
        rows, fc = _device_maps(d)
        rr, ff = orc.index_maps(T, P, w, anchors)
        assert np.array_equal(rows, rr) and np.array_equal(fc, ff), (T, P, w, anchors)
