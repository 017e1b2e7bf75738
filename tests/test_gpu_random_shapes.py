"""A seeded sweep of small random workloads through the whole linear-branch
path on the GPU, each checked against the float64 oracle: every head size,
ragged token counts, chunk lengths 1 .. 6, windows -1 .. 2, with and without
anchors and text, both scan levels, every output dtype.  The shapes are drawn
once from a fixed seed, so the sweep is the same on every run."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_STATE = 1e-3
TOL_O = {"f32": 1e-3, "f16": 1.5e-3, "bf16": 2e-3}


def _draw_cases(n=14, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = (16, 32, 64, 128)[i % 4]
        chunk = int(rng.integers(1, 7))
        anchors = int(rng.integers(0, 2))
        window = int(rng.integers(-1, 3))
        if window >= 0:  # windowed readout: whole chunks only
            scanned = chunk * int(rng.integers(1, 7))
        else:
            scanned = int(rng.integers(1, 31))
        cfg = inp.Config(
            name=f"rand{i}", heads=int(rng.integers(1, 3)), d=d, frames=scanned + 2 * anchors,
            tokens=int(rng.integers(1, 150)), chunk=chunk, anchors=anchors, window=window,
            text_tokens=int(rng.choice([0, 8, 37])), in_dtype=str(rng.choice(["bf16", "f32"])),
            out_dtype=str(rng.choice(["f32", "f16", "bf16"])), alpha_lo=float(rng.uniform(0.8, 0.99)),
            seed=5000 + i)
        chunk_scan = window >= 0 and bool(rng.integers(0, 2))
        cases.append((cfg, chunk_scan))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("cfg,chunk_scan", CASES, ids=[c.name for c, _ in CASES])
def test_random_shape_matches_oracle(cfg, chunk_scan):
    print(f"[random] {cfg} chunk_scan={chunk_scan}", flush=True)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, chunk_scan=chunk_scan)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    O = runner.out_f64(bufs)
    sf = bufs.states_f.cpu().numpy()
    sr = bufs.states_r.cpu().numpy()
    text = cfg.text_tokens > 0
    a = cfg.anchors
    for h in range(cfg.heads):
        f = heads_in[h].f64
        ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"), f("beta"),
                           f("alpha"), f("kt") if text else None, f("vt") if text else None,
                           f("bt") if text else None, text_init_scale=0.5)
        r_f = orc.rel_l2(sf[h], ref["states_f"])
        r_r = orc.rel_l2(sr[h], ref["states_r"])
        r_o = orc.rel_l2(O[h][a:cfg.frames - a], ref["O"][a:cfg.frames - a])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_f <= TOL_STATE and r_r <= TOL_STATE
        assert r_o <= TOL_O[cfg.out_dtype]
        if a:
            assert not O[h, 0].any() and not O[h, -1].any()
