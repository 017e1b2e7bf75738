"""A seeded sweep of the path's options in combination on the GPU, each run
checked against the float64 oracle: the fused prep, the readout without the
decay bridge, the chunk-level scan, the Newton-iteration inverse and the
SANA-WM comparator, through the separate calls or through vda_forward, over
random small workloads (every head size, ragged token counts, chunk lengths
1 .. 6, windows -1 .. 2, with and without anchors and text, every output
dtype).  The cases are drawn once from a fixed seed, so the sweep is the
same on every run."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_STATE = 1e-3
TOL_O = {"f32": 1e-3, "f16": 1.5e-3, "bf16": 2e-3}
EPS_N = 1e-6  # the normalisation epsilon of VDA_PREP

# frame-write variants: (descriptor flags, oracle update)
MODES = {
    "vda": ({}, "vda"),
    "chunk": (dict(chunk_scan=True), "vda"),
    "newton": (dict(newton=True), "vda"),
    "chunk+newton": (dict(chunk_scan=True, newton=True), "vda"),
    "sana": (dict(sana_wm=True), "sana"),
}


def _draw_cases(n=15, seed=4242):
    rng = np.random.default_rng(seed)
    names = list(MODES)
    cases = []
    for i in range(n):
        mode = names[i % len(names)]
        d = (16, 32, 64, 128)[(i + i // len(names)) % 4]
        chunk = int(rng.integers(1, 7))
        anchors = int(rng.integers(0, 2))
        lo = 0 if "chunk" in mode else -1  # the chunk-level scan needs a window
        window = int(rng.integers(lo, 3))
        scanned = chunk * int(rng.integers(1, 7)) if window >= 0 else int(rng.integers(1, 31))
        prep = bool(rng.integers(0, 2))
        bridge = window < 0 or bool(rng.integers(0, 2))
        fused = bool(rng.integers(0, 2))
        cfg = inp.Config(
            name=f"flags{i}-{mode}", heads=int(rng.integers(1, 3)), d=d, frames=scanned + 2 * anchors,
            tokens=int(rng.integers(1, 150)), chunk=chunk, anchors=anchors, window=window,
            text_tokens=int(rng.choice([0, 8, 37])), in_dtype=str(rng.choice(["bf16", "f32"])),
            out_dtype=str(rng.choice(["f32", "f16", "bf16"])), alpha_lo=float(rng.uniform(0.8, 0.99)),
            seed=7000 + i)
        cases.append((cfg, mode, prep, bridge, fused))
    return cases


CASES = _draw_cases()


def _ref(cfg, x, update, prep, bridge):
    f = x.f64
    text = cfg.text_tokens > 0
    q, k, b, a = f("q"), f("k"), f("beta"), f("alpha")
    kt, bt = (f("kt"), f("bt")) if text else (None, None)
    if prep:
        q, k, b, a, kt, bt = orc.prep(q, k, b, a, kt, bt, eps=EPS_N)
    return orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, q, k, f("v"), b, a, kt,
                        f("vt") if text else None, bt, bridge=bridge, update=update)


@pytest.mark.parametrize("cfg,mode,prep,bridge,fused", CASES, ids=[c[0].name for c in CASES])
def test_option_combination_matches_oracle(cfg, mode, prep, bridge, fused):
    flags, update = MODES[mode]
    print(f"[flags] {cfg} mode={mode} prep={prep} bridge={bridge} fused={fused}", flush=True)
    heads_in = inp.all_raw_heads(cfg) if prep else inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=fused, prep=prep, bridge=bridge, **flags)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    O = runner.out_f64(bufs)
    sf, sr = bufs.states_f.cpu().numpy(), bufs.states_r.cpu().numpy()
    a = cfg.anchors
    sl = slice(a, cfg.frames - a)
    for h in range(cfg.heads):
        ref = _ref(cfg, heads_in[h], update, prep, bridge)
        r_o = orc.rel_l2(O[h][sl], ref["O"][sl])
        r_f = orc.rel_l2(sf[h], ref["states_f"])
        r_r = orc.rel_l2(sr[h], ref["states_r"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_f <= TOL_STATE and r_r <= TOL_STATE
        assert r_o <= TOL_O[cfg.out_dtype]
        if a:
            assert not O[h, 0].any() and not O[h, -1].any()
