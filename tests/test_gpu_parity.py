"""GPU parity of the libvda HIP path against the float64 oracle, at sizes the
oracle finishes in seconds (several MFMA tiles, ragged token tails, every
supported head size), plus the path's edge cases.  All calls go through the
C ABI."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O = 2e-3       # output, relative L2 (bf16 inputs, float32 state)
TOL_STATE = 1e-3   # recorded states, relative L2
TOL_N = 6e-4       # N = (I + A)^-1 stored as f16: rounding alone is <= 2^-11 per entry
TOL_J = 6e-4       # J = B N stored as f16, formed from f16 beta*V and K


def _oracle(cfg, h_in, bridge=True, scale=0.5):
    f = h_in.f64
    text = cfg.text_tokens > 0
    return orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"),
                        f("beta"), f("alpha"), f("kt") if text else None, f("vt") if text else None,
                        f("bt") if text else None, text_init_scale=scale, bridge=bridge)


def _scanned_rel(O, ref, cfg):
    a = cfg.anchors
    sl = slice(a, cfg.frames - a)
    return orc.rel_l2(O[sl], ref[sl])


def _check(cfg, heads=None, tol_o=TOL_O, bridge=True, fused=False, **over):
    print(f"[parity] {cfg.name} H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} fused={fused} {over}",
          flush=True)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, bridge=bridge, fused=fused, **over)
    O = runner.out_f64(bufs)
    sf = bufs.states_f.cpu().numpy()
    sr = bufs.states_r.cpu().numpy()
    assert vda.vda_device_status(desc, bufs.ws) == 0
    worst = 0.0
    for h in (range(cfg.heads) if heads is None else heads):
        ref = _oracle(cfg, heads_in[h], bridge=bridge)
        r_o = _scanned_rel(O[h], ref["O"], cfg)
        r_f = orc.rel_l2(sf[h], ref["states_f"])
        r_r = orc.rel_l2(sr[h], ref["states_r"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_o <= tol_o
        assert r_f <= TOL_STATE and r_r <= TOL_STATE
        # anchors are exactly zero
        if cfg.anchors:
            assert not O[h, 0].any() and not O[h, -1].any()
        worst = max(worst, r_o)
    return desc, bufs, heads_in, worst


def _ws_frames(bufs, desc):
    """(N_t, J_t) of every slot, decoded from the workspace: N (f16) in the
    scan's operand fragment order at byte 0, J = B N (f16) in accumulator
    order at byte 2 d^2."""
    d = desc.d_k
    n = desc.frames - 2 * desc.anchors
    n_eff = n + (1 if desc.text_tokens else 0)
    raw = bufs.ws.cpu().numpy()[256:256 + desc.heads * n_eff * 2 * d * d * 4]
    slots = raw.reshape(desc.heads, n_eff, 8 * d * d)
    # N: chunk ((ct*KS + kk)*LG + lg)*16 + lr holds N[16 ct + lr][32 kk + 8 lg .. +7]
    KS, LG = max(1, d // 32), min(4, d // 8)
    j = np.arange(d)[:, None]
    c = np.arange(d // 8)[None, :]
    chunk = (((j // 16) * KS + c // 4) * LG + c % 4) * 16 + j % 16
    idx = (chunk[:, :, None] * 8 + np.arange(8)[None, None, :]).reshape(d, d)
    Nf = slots[..., :2 * d * d].copy().view(np.float16).reshape(desc.heads, n_eff, d * d)[..., idx]
    # J: the f16x4 at (R * RT + ct) * 64 + l holds J[16R + 4(l // 16) + e][16ct + l % 16]
    RT = d // 16
    r = np.arange(d)[:, None]
    col = np.arange(d)[None, :]
    jidx = (((r // 16) * RT + col // 16) * 64 + 16 * ((r % 16) // 4) + col % 16) * 4 + r % 4
    Jf = slots[..., 2 * d * d:4 * d * d].copy().view(np.float16).reshape(desc.heads, n_eff, d * d)[..., jidx]
    return np.stack([Nf.astype(np.float64), Jf.astype(np.float64)], axis=2)


def _check_slot(fr, K, V, beta):
    """The slot's N against (I + A)^-1 and J against B (I + A)^-1."""
    A, B = orc.frame_stats(K, V, beta)
    N = np.linalg.inv(np.eye(A.shape[0]) + A)
    assert orc.rel_l2(fr[0], N) <= TOL_N
    assert orc.rel_l2(fr[1], B @ N) <= TOL_J


def test_tiny_config():
    cfg = inp.CONFIG_BY_NAME["tiny"]
    desc, bufs, heads_in, _ = _check(cfg)
    # stage check: N_t = (I + A_t)^-1 and J_t = B_t N_t in the workspace
    fr = _ws_frames(bufs, desc)
    h = heads_in[0]
    for f in range(cfg.scanned):
        t = cfg.anchors + f
        _check_slot(fr[0, f], h.f64("k")[t], h.f64("v")[t], h.f64("beta")[t])
    _check_slot(fr[0, cfg.scanned], h.f64("kt"), h.f64("vt"), h.f64("bt"))


def test_scan_only_config():
    _check(inp.CONFIG_BY_NAME["scan_only"])


@pytest.mark.parametrize("name", ["tiny", "scan_only"])
def test_fused_entry_point_matches_oracle(name):
    _check(inp.CONFIG_BY_NAME[name], fused=True)


def test_fused_entry_point_equals_step_by_step():
    """vda_forward runs the same kernels as the four calls: identical bits."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=3, frames=32, tokens=300)
    heads_in = inp.all_heads(cfg)
    _, _, b1 = runner.run(cfg, heads_in)
    _, _, b2 = runner.run(cfg, heads_in, fused=True)
    assert torch.equal(b1.states_f, b2.states_f)
    assert torch.equal(b1.states_r, b2.states_r)
    assert torch.equal(b1.out.view(torch.int16), b2.out.view(torch.int16))


@pytest.mark.parametrize("frames,d,window,text,anchors", [
    (32, 64, 1, 16, 1),    # C = 6
    (27, 32, 1, 16, 1),    # C = 5: odd, the reverse half is one chunk shorter
    (7, 32, 1, 16, 1),     # C = 1
    (42, 128, 2, 0, 1),    # C = 8, wide window, no text
    (30, 64, 0, 16, 0),    # window = own chunk only, no anchors
    (23, 64, -1, 16, 0),   # per-frame readout, ragged group sizes
])
def test_fused_schedule_equals_step_by_step(frames, d, window, text, anchors):
    """vda_forward (every kernel on the caller's stream) gives the same bits
    as the step calls (the reverse scan on a second stream), over chunk
    counts, windows, text and anchor settings."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=3, d=d, frames=frames, tokens=64, window=window,
                     text_tokens=text, anchors=anchors)
    print(f"[parity] fused schedule T={frames} d={d} w={window} text={text} anchors={anchors}", flush=True)
    heads_in = inp.all_heads(cfg)
    _, _, b1 = runner.run(cfg, heads_in)
    _, _, b2 = runner.run(cfg, heads_in, fused=True)
    assert torch.equal(b1.states_f, b2.states_f)
    assert torch.equal(b1.states_r, b2.states_r)
    assert torch.equal(b1.out.view(torch.int16), b2.out.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "scan_only"])
def test_bidirectional_scan_equals_two_scans(name):
    """vda_scan_bidir (one launch) records the same bits as vda_scan_fwd and
    vda_scan_rev, also with an explicit initial state."""
    import torch
    cfg = inp.CONFIG_BY_NAME[name]
    heads_in = inp.all_heads(cfg)
    desc, dev, b1 = runner.run(cfg, heads_in)
    sf, sr = torch.empty_like(b1.states_f), torch.empty_like(b1.states_r)
    vda.vda_scan_bidir(desc, b1.ws, dev.alpha, None, sf, sr)
    torch.cuda.synchronize()
    assert torch.equal(sf, b1.states_f) and torch.equal(sr, b1.states_r)
    g = np.random.default_rng(7)
    s0 = torch.from_numpy(g.standard_normal((cfg.heads, cfg.d, cfg.d)).astype(np.float32)).cuda()
    f1, r1 = torch.empty_like(sf), torch.empty_like(sr)
    vda.vda_scan_fwd(desc, b1.ws, dev.alpha, s0, f1)
    vda.vda_scan_rev(desc, b1.ws, dev.alpha, s0, r1)
    vda.vda_scan_bidir(desc, b1.ws, dev.alpha, s0, sf, sr)
    torch.cuda.synchronize()
    assert torch.equal(sf, f1) and torch.equal(sr, r1)


def test_forward_replays_from_a_hip_graph():
    """vda_forward enqueues only kernels on the caller's stream (no memsets,
    no other streams), so it can be captured in a HIP graph.  Every replay,
    with eager work on the same buffers between replays, gives the eager
    result bit for bit."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=22, tokens=96)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=True)
    ref = [bufs.out.clone(), bufs.states_f.clone(), bufs.states_r.clone()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fw = runner.Forward(desc, dev, bufs)
        fw.main = s
        fw.enqueue()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fw.enqueue()
    torch.cuda.synchronize()
    for i in range(3):
        bufs.out.zero_()
        bufs.states_f.fill_(float("nan"))
        bufs.states_r.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[parity] graph replay {i}", flush=True)
        assert torch.equal(bufs.out.view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(bufs.states_f, ref[1]) and torch.equal(bufs.states_r, ref[2])
        assert vda.vda_device_status(desc, bufs.ws) == 0


def test_fused_without_reverse_states():
    """window = -1 with states_rev = NULL: the reverse scan is skipped."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["scan_only"], heads=2, frames=13, tokens=40)
    heads_in = inp.all_heads(cfg)
    _, dev, b1 = runner.run(cfg, heads_in)
    desc = vda.desc_for(cfg)
    b2 = runner.allocate(desc, cfg.out_dtype, "cuda")
    vda.vda_forward(desc, dev.q, dev.k, dev.v, dev.beta, dev.alpha, None, None, None, b2.ws, b2.states_f,
                    None, b2.out, ws_bytes=b2.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(b1.states_f, b2.states_f)
    assert torch.equal(b1.out.view(torch.int16), b2.out.view(torch.int16))


def test_h3_shape_reduced_frames():
    """H3 frame shape (U = 1008, d = 128, 512 text tokens), 2 heads, 4 chunks."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=22)
    desc, bufs, heads_in, _ = _check(cfg)
    fr = _ws_frames(bufs, desc)
    h = heads_in[1]
    for f in (0, 7, 19):
        t = cfg.anchors + f
        _check_slot(fr[1, f], h.f64("k")[t], h.f64("v")[t], h.f64("beta")[t])
    _check_slot(fr[1, cfg.scanned], h.f64("kt"), h.f64("vt"), h.f64("bt"))  # text slot


@pytest.mark.parametrize("d,U", [(16, 5), (32, 70), (64, 100), (128, 37), (128, 1000)])
def test_head_sizes_and_ragged_tokens(d, U):
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=3, frames=17, tokens=U, d=d, text_tokens=13)
    _check(cfg)


@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
def test_output_dtypes(out_dtype):
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=200, out_dtype=out_dtype)
    _, _, _, worst = _check(cfg)
    assert worst <= 5e-4  # no bf16 rounding of the output


def test_float32_inputs_d128():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=100, in_dtype="f32",
                     out_dtype="f32")
    _, _, _, worst = _check(cfg)
    assert worst <= 5e-4


def test_without_bridge():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=27, tokens=64, d=64)
    _check(cfg, bridge=False)


def test_wide_window_and_unit_chunks():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=14, tokens=48, d=32, chunk=3, window=2,
                     text_tokens=0)
    _check(cfg)
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=9, tokens=48, d=32, chunk=1, window=1,
                     anchors=0)
    _check(cfg)


def test_reverse_scan_is_forward_scan_on_reversed_time():
    """Same kernels, same frame data in the opposite order: bitwise equal."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=22, tokens=300)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in)
    rev = []
    for h in heads_in:
        r = inp.HeadInputs(**{**h.__dict__})
        for name in ("q", "k", "v", "beta", "alpha"):
            setattr(r, name, np.ascontiguousarray(getattr(h, name)[::-1]))
        rev.append(r)
    _, _, bufs2 = runner.run(cfg, rev)
    assert torch.equal(bufs.states_r, bufs2.states_f)
    assert torch.equal(bufs.states_f, bufs2.states_r)


def test_no_scanned_frames():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=2, tokens=40, d=64)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in)
    assert not bufs.out.float().cpu().numpy().any()
    sf = bufs.states_f.cpu().numpy()
    for h in range(2):
        ref = _oracle(cfg, heads_in[h])
        assert orc.rel_l2(sf[h, 0], ref["states_f"][0]) <= TOL_STATE


def test_zero_tokens_is_pure_decay():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=0, d=64, text_tokens=20)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in)
    ref = _oracle(cfg, heads_in[0])
    assert orc.rel_l2(bufs.states_f.cpu().numpy()[0], ref["states_f"]) <= TOL_STATE
    assert orc.rel_l2(bufs.states_r.cpu().numpy()[0], ref["states_r"]) <= TOL_STATE


def test_explicit_initial_state():
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=12, tokens=64, d=64, text_tokens=0)
    heads_in = inp.all_heads(cfg)
    S0 = np.random.default_rng(5).standard_normal((2, 64, 64)).astype(np.float32)
    s_init = torch.from_numpy(S0).cuda()
    desc, dev, bufs = runner.run(cfg, heads_in, s_init=s_init)
    O = runner.out_f64(bufs)
    for h in range(2):
        f = heads_in[h].f64
        rows, fc = orc.index_maps(cfg.frames, cfg.chunk, cfg.window, cfg.anchors)
        order = orc.scanned_frames(cfg.frames, cfg.anchors)
        S_0 = 0.5 * S0[h].astype(np.float64)
        st_f = orc.scan(order, f("k"), f("v"), f("beta"), f("alpha"), S_0, cfg.chunk)
        st_r = orc.scan(order[::-1], f("k"), f("v"), f("beta"), f("alpha"), S_0, cfg.chunk)
        ref = orc.readout_windowed(f("q"), f("alpha"), st_f, st_r, rows, fc)
        assert orc.rel_l2(bufs.states_f.cpu().numpy()[h], st_f) <= TOL_STATE
        assert _scanned_rel(O[h], ref, cfg) <= TOL_O


def test_device_status_flags_bad_data():
    """Non-positive-definite I + A (negative write gates) and NaN keys are
    reported through the status word; the kernels still run to completion."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=7, tokens=64, d=32, text_tokens=0)
    heads_in = inp.all_heads(cfg)
    h = heads_in[0]
    h.beta = (-50.0 * np.ones_like(h.beta)).astype(np.float32)
    desc, dev, bufs = runner.run(cfg, heads_in)
    assert vda.vda_device_status(desc, bufs.ws) & vda.VDA_DEV_PIVOT
    heads_in = inp.all_heads(cfg)
    k = inp.bf16_bits_to_f32(heads_in[0].k).copy()
    k[3, 5, 7] = np.nan
    heads_in[0].k = inp.f32_to_bf16_bits(k)
    desc, dev, bufs = runner.run(cfg, heads_in)
    assert vda.vda_device_status(desc, bufs.ws) & vda.VDA_DEV_NONFINITE
    # a clean run clears the word again
    desc, dev, bufs = runner.run(cfg, inp.all_heads(cfg))
    assert vda.vda_device_status(desc, bufs.ws) == 0
