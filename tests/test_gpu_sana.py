"""GPU parity of the SANA-WM comparator (VDA_SANA_WM: the batched additive
frame update S_bar (I - A/U) + B/sqrt(U) in place of the VDA write) against
the float64 oracle's additive update, through the C ABI, and the expansion
that the additive transition shows when lambda_max(A/U) > 2 while the VDA
write of the same frames stays non-expansive."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_STATE = 1e-3


def _ref(cfg, x, prep=False):
    f = x.f64
    text = cfg.text_tokens > 0
    q, k, b, a, kt, bt = f("q"), f("k"), f("beta"), f("alpha"), f("kt") if text else None, f("bt") if text else None
    if prep:
        q, k, b, a, kt, bt = orc.prep(q, k, b, a, kt, bt, eps=1e-6)
    return orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, q, k, f("v"), b, a, kt,
                        f("vt") if text else None, bt, update="sana")


def _check(cfg, fused=False, prep=False):
    print(f"[sana] {cfg.name} H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} w={cfg.window} "
          f"text={cfg.text_tokens} in={cfg.in_dtype} fused={fused} prep={prep}", flush=True)
    heads_in = inp.all_raw_heads(cfg) if prep else inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=fused, sana_wm=True, prep=prep)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    O = runner.out_f64(bufs)
    sf, sr = bufs.states_f.cpu().numpy(), bufs.states_r.cpu().numpy()
    a = cfg.anchors
    for h in range(cfg.heads):
        ref = _ref(cfg, heads_in[h], prep)
        sl = slice(a, cfg.frames - a)
        r_o = orc.rel_l2(O[h][sl], ref["O"][sl])
        r_f = orc.rel_l2(sf[h], ref["states_f"])
        r_r = orc.rel_l2(sr[h], ref["states_r"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_o <= TOL_O and r_f <= TOL_STATE and r_r <= TOL_STATE
    return heads_in, bufs


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),                                                   # d = 16, f32 inputs
    ("scan_only", {}),                                              # d = 64, per-frame states, no text
    ("h3", dict(heads=3, frames=22, tokens=300)),                   # d = 128, text, ragged tiles
    ("h3", dict(heads=1, frames=17, tokens=37, d=32, window=0)),    # d = 32, own chunk only
])
def test_sana_wm_matches_oracle(name, over):
    _check(inp.scaled(inp.CONFIG_BY_NAME[name], **over))


def test_sana_wm_through_vda_forward_and_prep():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=12, tokens=200)
    _check(cfg, fused=True)
    _check(cfg, prep=True)


def test_sana_wm_expands_where_vda_does_not():
    """Every token of a frame carries the same key, of squared norm 8, with
    beta = 1/2: A/U = 4 k k^T/|k|^2, so I - A/U maps the key direction to -3
    times itself and the inherited state triples every frame (alpha = 1,
    no values); the VDA write of the same frames shrinks it.  Eight frames
    keep the grown state inside the f16 range of the scan's MFMA operands
    (an expanding state leaves it after about ten frames and turns
    non-finite)."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=8, tokens=64, d=64, text_tokens=16,
                     window=-1, anchors=0)
    h = inp.all_heads(cfg)[0]
    g = np.random.default_rng(41)
    kdir = g.standard_normal(64)
    kdir *= np.sqrt(8.0) / np.linalg.norm(kdir)
    k = np.broadcast_to(kdir, (cfg.frames, cfg.tokens, 64))
    x = inp.HeadInputs(**{**h.__dict__})
    x.k = inp.store(k, "bf16")
    x.v = inp.store(np.zeros((cfg.frames, cfg.tokens, 64)), "bf16")
    x.beta = np.full((cfg.frames, cfg.tokens), 0.5, np.float32)
    x.alpha = np.ones((cfg.frames, 64), np.float32)
    x.kt = inp.store(np.broadcast_to(kdir, (16, 64)), "bf16")  # S^T along the key direction
    desc, dev, b_sana = runner.run(cfg, [x], sana_wm=True)
    _, _, b_vda = runner.run(cfg, [x])
    ref = _ref(cfg, x)
    st = b_sana.states_f.cpu().numpy()[0].astype(np.float64)
    assert orc.rel_l2(st, ref["states_f"]) <= TOL_STATE
    kq = x.f64("k")[0, 0]
    growth = [np.linalg.norm(st[i + 1] @ kq) / np.linalg.norm(st[i] @ kq) for i in range(cfg.frames)]
    print(f"  SANA-WM growth per frame along k: {np.round(growth, 4)}", flush=True)
    expect = abs(1.0 - 0.5 * kq @ kq)  # 3, up to the bf16 rounding of k
    assert abs(expect - 3.0) < 0.01
    assert all(abs(gr - expect) < 1e-3 * expect for gr in growth)
    sv = b_vda.states_f.cpu().numpy()[0].astype(np.float64)
    assert all(np.linalg.norm(sv[i + 1], 2) <= np.linalg.norm(sv[i], 2) * (1 + 1e-4) for i in range(cfg.frames))
    assert torch.isfinite(b_sana.out.float()).all()
