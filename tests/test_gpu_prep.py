"""GPU parity of the fused prep (VDA_PREP: raw q/k L2-normalised and the
beta/alpha gates taken as sigmoid of logits inside the kernels) against the
float64 oracle's prep followed by the oracle's branch, through the C ABI."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_STATE = 1e-3
EPS_N = 1e-6  # the normalisation epsilon of VDA_PREP


def _ref(cfg, h_in):
    f = h_in.f64
    text = cfg.text_tokens > 0
    q, k, b, a, kt, bt = orc.prep(f("q"), f("k"), f("beta"), f("alpha"), f("kt") if text else None,
                                  f("bt") if text else None, eps=EPS_N)
    return orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, q, k, f("v"), b, a, kt,
                        f("vt") if text else None, bt), a


def _check(cfg, fused=False):
    print(f"[prep] {cfg.name} H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} window={cfg.window} "
          f"in={cfg.in_dtype} fused={fused}", flush=True)
    heads_in = inp.all_raw_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=fused, prep=True)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    O = runner.out_f64(bufs)
    sf, sr = bufs.states_f.cpu().numpy(), bufs.states_r.cpu().numpy()
    a = cfg.anchors
    for h in range(cfg.heads):
        ref, _ = _ref(cfg, heads_in[h])
        r_o = orc.rel_l2(O[h][a:cfg.frames - a], ref["O"][a:cfg.frames - a])
        r_f = orc.rel_l2(sf[h], ref["states_f"])
        r_r = orc.rel_l2(sr[h], ref["states_r"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_o <= TOL_O and r_f <= TOL_STATE and r_r <= TOL_STATE
        if a:
            assert not O[h, 0].any() and not O[h, -1].any()
    return heads_in, desc, dev, bufs


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),                                                  # d = 16, f32 inputs
    ("scan_only", {}),                                             # d = 64, per-frame readout, no text
    ("h3", dict(heads=2, frames=17, tokens=300)),                  # d = 128, bf16, text, ragged tiles
    ("h3", dict(heads=1, frames=12, tokens=37, d=32)),             # d = 32
])
def test_prep_matches_oracle(name, over):
    _check(inp.scaled(inp.CONFIG_BY_NAME[name], **over))


def test_prep_through_vda_forward():
    _check(inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=12, tokens=200), fused=True)


def test_prep_equals_prepared_inputs():
    """VDA_PREP on raw inputs against the plain path on inputs that were
    prepared on the host in float32 and stored in the same dtype: agreement to
    the rounding of those stored inputs."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=128, in_dtype="f32", out_dtype="f32")
    heads_in = inp.all_raw_heads(cfg)
    _, _, b_prep = runner.run(cfg, heads_in, prep=True)
    h = heads_in[0]
    f = h.f64
    q, k, b, a, kt, bt = orc.prep(f("q"), f("k"), f("beta"), f("alpha"), f("kt"), f("bt"), eps=EPS_N)
    ready = inp.HeadInputs(dtype="f32", q=q.astype(np.float32), k=k.astype(np.float32), v=h.v,
                           beta=b.astype(np.float32), alpha=a.astype(np.float32), kt=kt.astype(np.float32),
                           vt=h.vt, bt=bt.astype(np.float32))
    _, _, b_plain = runner.run(cfg, [ready])
    r = orc.rel_l2(runner.out_f64(b_prep), runner.out_f64(b_plain))
    print(f"  prep vs host-prepared: {r:.3e}", flush=True)
    assert r <= 1e-3


def test_prep_with_gated_readout():
    """Both next-step rows together: raw inputs and the readout epilogue."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=200)
    heads_in, desc, dev, bufs = _check(cfg)
    epi = [inp.epilogue_inputs(cfg, 0)]
    gate, w = runner.upload_epilogue(cfg, epi)
    y = runner.readout_gated(desc, dev, bufs, gate, w, 1e-6, "f32").cpu().numpy().astype(np.float64)
    ref, _ = _ref(cfg, heads_in[0])
    y_ref = orc.rmsnorm_gate(ref["O"], epi[0].f64("weight"), epi[0].f64("gate"), 1e-6)
    a = cfg.anchors
    r = orc.rel_l2(y[0][a:cfg.frames - a], y_ref[a:cfg.frames - a])
    print(f"  gated with prep: {r:.3e}", flush=True)
    assert r <= TOL_O
