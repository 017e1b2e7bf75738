"""GPU parity of the chunk-level scan (VDA_CHUNK_SCAN: vda_compose_chunks,
then S <- S M_c + J_c per chunk) against the float64 oracle, through the C
ABI: the composed maps themselves, the recorded states and the output, over
head sizes, chunk lengths, windows, text, prep and an explicit initial state,
plus bitwise checks between entry points and under time reversal."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O = 2e-3       # output, relative L2 (bf16 output rounding is 1.66e-3 of it)
TOL_STATE = 1e-3   # recorded states
TOL_MAP = 2e-3     # M_c, J_c: f16 N_t and B_t composed in float32, then stored as f16


def _oracle(cfg, h_in, scale=0.5, S0=None, prep=False):
    f = h_in.f64
    text = cfg.text_tokens > 0
    if prep:  # raw inputs: the oracle's prep, then the branch
        q, k, b, a, kt, bt = orc.prep(f("q"), f("k"), f("beta"), f("alpha"), f("kt") if text else None,
                                      f("bt") if text else None, eps=1e-6)
        return orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, q, k, f("v"), b, a, kt,
                            f("vt") if text else None, bt, text_init_scale=scale)
    if S0 is None:
        return orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"),
                            f("beta"), f("alpha"), f("kt") if text else None, f("vt") if text else None,
                            f("bt") if text else None, text_init_scale=scale)
    rows, fc = orc.index_maps(cfg.frames, cfg.chunk, cfg.window, cfg.anchors)
    order = orc.scanned_frames(cfg.frames, cfg.anchors)
    st_f = orc.scan(order, f("k"), f("v"), f("beta"), f("alpha"), scale * S0, cfg.chunk)
    st_r = orc.scan(order[::-1], f("k"), f("v"), f("beta"), f("alpha"), scale * S0, cfg.chunk)
    return dict(states_f=st_f, states_r=st_r, O=orc.readout_windowed(f("q"), f("alpha"), st_f, st_r, rows, fc))


def _check(cfg, fused=False, heads_in=None, prep=False, **over):
    print(f"[chunk] {cfg.name} H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} P={cfg.chunk} "
          f"w={cfg.window} text={cfg.text_tokens} fused={fused} prep={prep} {over}", flush=True)
    if heads_in is None:
        heads_in = inp.all_raw_heads(cfg) if prep else inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=fused, chunk_scan=True, prep=prep, **over)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    O = runner.out_f64(bufs)
    sf, sr = bufs.states_f.cpu().numpy(), bufs.states_r.cpu().numpy()
    a = cfg.anchors
    for h in range(cfg.heads):
        ref = _oracle(cfg, heads_in[h], prep=prep)
        sl = slice(a, cfg.frames - a)
        r_o = orc.rel_l2(O[h][sl], ref["O"][sl])
        r_f = orc.rel_l2(sf[h], ref["states_f"])
        r_r = orc.rel_l2(sr[h], ref["states_r"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_o <= TOL_O
        assert r_f <= TOL_STATE and r_r <= TOL_STATE
        if a:
            assert not O[h, 0].any() and not O[h, -1].any()
    return desc, bufs, heads_in


def _maps(bufs, desc):
    """Decode the chunk maps from the workspace: [H][2][C] (M_c, J_c)."""
    d, H, P = desc.d_k, desc.heads, desc.chunk
    n = desc.frames - 2 * desc.anchors
    C = n // P
    n_eff = n + (1 if desc.text_tokens else 0)
    off = 256 + H * n_eff * 8 * d * d
    raw = bufs.ws.cpu().numpy()[off:off + H * 2 * C * 4 * d * d].reshape(H, 2, C, 4 * d * d)
    # M_c in the fragment order of N: the chunk ntile_chunk(d, j, c) holds M_c[8c .. 8c+7][j]
    KS, LG = max(1, d // 32), min(4, d // 8)
    j = np.arange(d)[:, None]
    c = np.arange(d // 8)[None, :]
    chunk = (((j // 16) * KS + c // 4) * LG + c % 4) * 16 + j % 16
    idx = (chunk[:, :, None] * 8 + np.arange(8)[None, None, :]).reshape(d, d)  # [j][8c + e]
    Mf = raw[..., :2 * d * d].copy().view(np.float16).reshape(H, 2, C, d * d)[..., idx]
    M = np.swapaxes(Mf, -1, -2).astype(np.float64)
    # J_c in accumulator order: the f16x4 (R * d/16 + ct) * 64 + l holds
    # J_c[16R + 4(l // 16) + e][16 ct + l % 16]
    Jf = raw[..., 2 * d * d:].copy().view(np.float16).reshape(H, 2, C, d // 16, d // 16, 4, 16, 4)
    # axes: R, ct, l // 16, l % 16, e  ->  rows 16R + 4(l//16) + e, columns 16ct + l%16
    J = Jf.transpose(0, 1, 2, 3, 5, 7, 4, 6).reshape(H, 2, C, d, d).astype(np.float64)
    return M, J


@pytest.mark.parametrize("d,tokens,chunk,text", [
    (16, 40, 5, 8),
    (32, 64, 3, 16),
    (64, 100, 5, 0),
    (128, 300, 5, 64),
])
def test_composed_maps_match_oracle(d, tokens, chunk, text):
    """Each chunk's forward map composes its frames in increasing order and
    the reverse map in decreasing order (method steps, step (4))."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=2 + 3 * chunk, tokens=tokens, d=d,
                     chunk=chunk, text_tokens=text)
    desc, bufs, heads_in = _check(cfg)
    M, J = _maps(bufs, desc)
    order = orc.scanned_frames(cfg.frames, cfg.anchors)
    worst = 0.0
    for h in range(cfg.heads):
        f = heads_in[h].f64
        for c in range(3):
            fr = order[chunk * c:chunk * (c + 1)]
            for dr, frs in ((0, fr), (1, fr[::-1])):
                Mr, Jr = orc.chunk_map(frs, f("k"), f("v"), f("beta"), f("alpha"))
                rm, rj = orc.rel_l2(M[h, dr, c], Mr), orc.rel_l2(J[h, dr, c], Jr)
                worst = max(worst, rm, rj)
                assert rm <= TOL_MAP and rj <= TOL_MAP, (h, dr, c, rm, rj)
    print(f"  maps: worst rel {worst:.3e}", flush=True)


@pytest.mark.parametrize("name", ["tiny"])
@pytest.mark.parametrize("fused", [False, True])
def test_tiny_config_chunk_scan(name, fused):
    _check(inp.CONFIG_BY_NAME[name], fused=fused)


@pytest.mark.parametrize("over", [
    dict(heads=4, frames=22, tokens=300, d=128),                   # reduced H3
    dict(heads=2, frames=27, tokens=64, d=64, window=0),            # own chunk only, odd C
    dict(heads=2, frames=22, tokens=48, d=32, window=3),            # window wider than the sequence
    dict(heads=2, frames=12, tokens=40, d=64, chunk=1),             # unit chunks: a map per frame
    dict(heads=2, frames=30, tokens=37, d=64, anchors=0, text_tokens=0),  # no anchors, no text
    dict(heads=1, frames=7, tokens=64, d=128),                       # C = 1
])
def test_chunk_scan_matches_oracle(over):
    _check(inp.scaled(inp.CONFIG_BY_NAME["h3"], **over))


def test_chunk_scan_with_prep():
    """Raw q, k and logit gates (VDA_PREP): compose applies sigmoid to alpha."""
    _check(inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=22, tokens=200, d=128), prep=True)


def test_chunk_scan_entry_points_agree_bitwise():
    """vda_forward and the step calls (prepare, compose, two scans, readout)
    run the same kernels: identical bits."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=3, frames=32, tokens=300)
    heads_in = inp.all_heads(cfg)
    _, _, b1 = runner.run(cfg, heads_in, chunk_scan=True)
    _, _, b2 = runner.run(cfg, heads_in, fused=True, chunk_scan=True)
    assert torch.equal(b1.states_f, b2.states_f)
    assert torch.equal(b1.states_r, b2.states_r)
    assert torch.equal(b1.out.view(torch.int16), b2.out.view(torch.int16))


def test_chunk_scan_reverse_is_forward_on_reversed_time():
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=22, tokens=300)
    heads_in = inp.all_heads(cfg)
    _, _, b1 = runner.run(cfg, heads_in, chunk_scan=True)
    rev = []
    for h in heads_in:
        r = inp.HeadInputs(**{**h.__dict__})
        for name in ("q", "k", "v", "beta", "alpha"):
            setattr(r, name, np.ascontiguousarray(getattr(h, name)[::-1]))
        rev.append(r)
    _, _, b2 = runner.run(cfg, rev, chunk_scan=True)
    assert torch.equal(b1.states_r, b2.states_f)
    assert torch.equal(b1.states_f, b2.states_r)


def test_chunk_scan_close_to_frame_scan():
    """Both scan levels reach the same states up to the f16 storage of the
    maps."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=3, frames=52, tokens=300)
    heads_in = inp.all_heads(cfg)
    _, _, b1 = runner.run(cfg, heads_in)
    _, _, b2 = runner.run(cfg, heads_in, chunk_scan=True)
    for a, b in ((b1.states_f, b2.states_f), (b1.states_r, b2.states_r)):
        r = orc.rel_l2(b.cpu().numpy(), a.cpu().numpy())
        print(f"  chunk vs frame states: {r:.3e}", flush=True)
        assert r <= TOL_STATE


def test_chunk_scan_explicit_initial_state():
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=12, tokens=64, d=64, text_tokens=0)
    heads_in = inp.all_heads(cfg)
    S0 = np.random.default_rng(5).standard_normal((2, 64, 64)).astype(np.float32)
    desc, dev, bufs = runner.run(cfg, heads_in, s_init=torch.from_numpy(S0).cuda(), chunk_scan=True)
    O = runner.out_f64(bufs)
    for h in range(2):
        ref = _oracle(cfg, heads_in[h], S0=S0[h].astype(np.float64))
        assert orc.rel_l2(bufs.states_f.cpu().numpy()[h], ref["states_f"]) <= TOL_STATE
        assert orc.rel_l2(bufs.states_r.cpu().numpy()[h], ref["states_r"]) <= TOL_STATE
        assert orc.rel_l2(O[h][1:-1], ref["O"][1:-1]) <= TOL_O


def test_chunk_scan_no_scanned_frames():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=2, tokens=40, d=64)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, chunk_scan=True)
    assert not bufs.out.float().cpu().numpy().any()
    for h in range(2):
        ref = _oracle(cfg, heads_in[h])
        assert orc.rel_l2(bufs.states_f.cpu().numpy()[h, 0], ref["states_f"][0]) <= TOL_STATE
