"""Degenerate shapes through the C ABI on the GPU: no heads (every entry
point returns without touching memory), no frames (the states are the
scaled text state), the softmax branch with anchor frames only (no chunks)
and with no tokens."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu


def test_zero_heads_every_entry_point_is_a_no_op():
    import torch
    print("[edges] heads = 0", flush=True)
    sentinel = lambda: torch.full((64,), 7.0, device="cuda")
    bufs = [sentinel() for _ in range(12)]
    (q, k, v, beta, alpha, kt, vt, bt, sf, sr, out, gate) = bufs
    for flags in (dict(), dict(chunk_scan=True), dict(sana_wm=True), dict(newton=True), dict(prep=True)):
        d = vda.make_desc(0, 22, 16, 16, text_tokens=8, in_dtype="f32", out_dtype="f32", **flags)
        wsb = vda.vda_workspace_bytes(d)
        assert wsb == 256
        ws = torch.full((64,), 7.0, device="cuda")
        vda.vda_prepare_frames(d, k, v, beta, kt, vt, bt, ws, wsb)
        if flags.get("chunk_scan"):
            vda.vda_compose_chunks(d, ws, alpha, ws_bytes=wsb)
        vda.vda_scan_bidir(d, ws, alpha, None, sf, sr)
        vda.vda_readout(d, q, alpha, sf, sr, out)
        vda.vda_readout_gated(d, q, alpha, sf, sr, gate, beta, 1e-6, out)
        vda.vda_forward(d, q, k, v, beta, alpha, kt, vt, bt, ws, sf, sr, out, ws_bytes=wsb)
        torch.cuda.synchronize()
    db = vda.make_desc(0, 22, 16, 32, text_tokens=8, in_dtype="bf16", out_dtype="bf16")
    vda.vda_softmax_branch(db, q, k, v, kt, vt, 0.1, out)
    torch.cuda.synchronize()
    for b in bufs[8:]:  # states and outputs untouched (the clear-status kernel writes only ws)
        assert bool((b == 7.0).all())


@pytest.mark.parametrize("window", [1, -1])
def test_zero_frames_leaves_the_text_state(window):
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=0, anchors=0, tokens=40, d=64, text_tokens=30,
                     window=window)
    print(f"[edges] frames = 0, window = {window}", flush=True)
    heads_in = inp.all_heads(cfg)
    for fused in (False, True):
        desc, dev, bufs = runner.run(cfg, heads_in, fused=fused)
        assert vda.vda_device_status(desc, bufs.ws) == 0
        assert bufs.states_f.shape[1] == 1
        for h in range(cfg.heads):
            f = heads_in[h].f64
            ST = orc.text_state(f("kt"), f("vt"), f("bt"), 64, 64)
            assert orc.rel_l2(bufs.states_f[h, 0].cpu().numpy(), 0.5 * ST) <= 1e-3
            if window >= 0:
                assert orc.rel_l2(bufs.states_r[h, 0].cpu().numpy(), 0.5 * ST) <= 1e-3


def _softmax(cfg, v_dtype="bf16"):
    import torch
    ins = [inp.softmax_inputs(cfg, h) for h in range(cfg.heads)]
    dev = lambda name: runner._dev(np.stack([getattr(x, name) for x in ins]), "cuda")
    q, k, v = dev("q"), dev("k"), dev("v")
    kt, vt = (dev("kt"), dev("vt")) if cfg.text_tokens else (None, None)
    desc = vda.desc_for(cfg, in_dtype="bf16", out_dtype="f32")
    out = torch.full((cfg.heads, cfg.frames, cfg.tokens, cfg.d), 7.0, device="cuda")
    scale = 1.0 / np.sqrt(cfg.d)
    vda.vda_softmax_branch(desc, q, k, v, kt, vt, scale, out)
    torch.cuda.synchronize()
    return ins, out.cpu().numpy().astype(np.float64), scale


def test_softmax_anchor_frames_only():
    """frames = 2 with anchors: no chunks; both anchor frames see both frames
    and the text."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=2, tokens=150, d=64, text_tokens=40)
    print("[edges] softmax, anchors only", flush=True)
    ins, O, scale = _softmax(cfg)
    for h in range(cfg.heads):
        x = ins[h]
        ref = orc.softmax_branch(x.f64("q"), x.f64("k"), x.f64("v"), x.f64("kt"), x.f64("vt"), cfg.frames,
                                 cfg.chunk, cfg.window, cfg.anchors, scale)
        r = orc.rel_l2(O[h], ref)
        print(f"  head {h}: rel {r:.3e}", flush=True)
        assert r <= 5e-4  # float32 output: only P's f16 rounding


def test_softmax_single_chunk_without_anchors_or_text():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=5, anchors=0, tokens=70, d=128, text_tokens=0)
    print("[edges] softmax, one chunk, no anchors, no text", flush=True)
    ins, O, scale = _softmax(cfg)
    x = ins[0]
    ref = orc.softmax_branch(x.f64("q"), x.f64("k"), x.f64("v"), None, None, cfg.frames, cfg.chunk, cfg.window,
                             cfg.anchors, scale)
    r = orc.rel_l2(O[0], ref)
    print(f"  rel {r:.3e}", flush=True)
    assert r <= 5e-4


def test_softmax_zero_tokens_is_a_no_op():
    import torch
    print("[edges] softmax, tokens = 0", flush=True)
    d = vda.make_desc(2, 12, 0, 64, text_tokens=16, in_dtype="bf16", out_dtype="bf16")
    t = torch.zeros((16,), dtype=torch.bfloat16, device="cuda")
    vda.vda_softmax_branch(d, t, t, t, t, t, 0.125, t)
    torch.cuda.synchronize()
    assert not bool(t.any())
