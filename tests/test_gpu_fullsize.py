"""GPU parity at the full workload sizes, through the entry point the
benchmark times (vda_forward), against the float64 oracle on every head.

Heads are independent in the linear branch, so the oracle checks whole heads
one by one.  The H3-shaped workload runs with all 24 heads, exactly as
benchmarked.  The long-video (202 frames) and high-resolution (402 frames,
U = 2016) workloads run at their full per-head shape with fewer heads, to keep
input generation and host memory small.
"""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_STATE = 1e-3


def _oracle(cfg, h_in):
    f = h_in.f64
    text = cfg.text_tokens > 0
    return orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"), f("beta"),
                        f("alpha"), f("kt") if text else None, f("vt") if text else None,
                        f("bt") if text else None)


def _run_and_check(cfg, sample_heads, chunk_scan=False):
    print(f"[fullsize] {cfg.name}: H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} "
          f"chunk_scan={chunk_scan}: drawing inputs", flush=True)
    heads_in = inp.all_heads(cfg)
    print("[fullsize] running vda_forward", flush=True)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=True, chunk_scan=chunk_scan)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    import torch
    a = cfg.anchors
    out = bufs.out
    # every head: finite output, zero anchor rows
    assert bool(torch.isfinite(out.float()).all())
    if a:
        assert not bool(out[:, 0].any()) and not bool(out[:, -1].any())
    sf = bufs.states_f
    sr = bufs.states_r
    for h in sample_heads:
        print(f"[fullsize] oracle head {h}", flush=True)
        ref = _oracle(cfg, heads_in[h])
        O = out[h].float().cpu().numpy().astype(np.float64)
        sl = slice(a, cfg.frames - a)
        r_o = orc.rel_l2(O[sl], ref["O"][sl])
        r_f = orc.rel_l2(sf[h].cpu().numpy(), ref["states_f"])
        r_r = orc.rel_l2(sr[h].cpu().numpy(), ref["states_r"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_o <= TOL_O
        assert r_f <= TOL_STATE and r_r <= TOL_STATE


@pytest.mark.timeout(900)
def test_h3_full_size_all_heads():
    _run_and_check(inp.CONFIG_BY_NAME["h3"], sample_heads=range(24))


@pytest.mark.timeout(900)
def test_long_video_full_shape():
    _run_and_check(inp.scaled(inp.CONFIG_BY_NAME["long"], heads=2), sample_heads=(0, 1))


@pytest.mark.timeout(900)
def test_high_resolution_full_shape():
    _run_and_check(inp.scaled(inp.CONFIG_BY_NAME["hires"], heads=2), sample_heads=(0, 1))


@pytest.mark.timeout(900)
def test_h3_full_size_chunk_scan():
    """The same workload with the scans at chunk level (VDA_CHUNK_SCAN)."""
    _run_and_check(inp.CONFIG_BY_NAME["h3"], sample_heads=range(24), chunk_scan=True)


@pytest.mark.timeout(900)
def test_long_video_chunk_scan():
    _run_and_check(inp.scaled(inp.CONFIG_BY_NAME["long"], heads=2), sample_heads=(0, 1), chunk_scan=True)
