"""GPU parity of the softmax window + anchor + text branch
(vda_softmax_branch) against the float64 oracle, through the C ABI: every
supported head size, ragged query and key tiles, with and without anchors and
text, several window widths and all output types."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL = 2e-3   # relative L2; P is rounded to f16 and a bf16 output adds its own rounding


def _run(cfg, out_dtype="bf16", scale=None, v_dtype="bf16"):
    import torch
    print(f"[softmax] {cfg.name} H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} window={cfg.window} "
          f"anchors={cfg.anchors} text={cfg.text_tokens} out={out_dtype}", flush=True)
    ins = [inp.softmax_inputs(cfg, h) for h in range(cfg.heads)]
    dev = lambda name: runner._dev(np.stack([getattr(x, name) for x in ins]), "cuda")
    q, k, v = dev("q"), dev("k"), dev("v")
    kt, vt = (dev("kt"), dev("vt")) if cfg.text_tokens else (None, None)
    if v_dtype == "f16":  # the same bf16 values, stored as f16 (exact)
        v = v.view(torch.bfloat16).to(torch.float16)
        vt = None if vt is None else vt.view(torch.bfloat16).to(torch.float16)
    desc = vda.desc_for(cfg, in_dtype="bf16", out_dtype=out_dtype)
    out = torch.empty((cfg.heads, cfg.frames, cfg.tokens, cfg.d), device="cuda",
                      dtype={"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype])
    scale = 1.0 / np.sqrt(cfg.d) if scale is None else scale
    vda.vda_softmax_branch(desc, q, k, v, kt, vt, scale, out, v_dtype=v_dtype)
    torch.cuda.synchronize()
    return ins, out.float().cpu().numpy().astype(np.float64), scale


def _check(cfg, out_dtype="bf16", heads=None, frames=None, scale=None, v_dtype="bf16"):
    ins, O, scale = _run(cfg, out_dtype, scale, v_dtype)
    for h in (range(cfg.heads) if heads is None else heads):
        x = ins[h]
        text = cfg.text_tokens > 0
        ref = orc.softmax_branch(x.f64("q"), x.f64("k"), x.f64("v"), x.f64("kt") if text else None,
                                 x.f64("vt") if text else None, cfg.frames, cfg.chunk, cfg.window, cfg.anchors,
                                 scale)
        sl = slice(None) if frames is None else frames
        r = orc.rel_l2(O[h][sl], ref[sl])
        print(f"  head {h}: rel {r:.3e}", flush=True)
        assert r <= TOL


@pytest.mark.parametrize("over", [
    dict(heads=2, frames=12, tokens=100, text_tokens=64),              # C = 2, anchors, text, ragged tiles
    dict(heads=1, frames=17, tokens=37, text_tokens=5),                # C = 3, tiny frames, 5 text tokens
    dict(heads=1, frames=22, tokens=64, d=64, text_tokens=100),        # d = 64
    dict(heads=1, frames=22, tokens=48, d=32, text_tokens=0),          # d = 32, no text
    dict(heads=1, frames=20, tokens=40, anchors=0, text_tokens=16),    # no anchors
    dict(heads=1, frames=27, tokens=30, window=0, text_tokens=16),     # own chunk only
    dict(heads=1, frames=27, tokens=30, window=3, text_tokens=16),     # window wider than the sequence
])
def test_softmax_branch_matches_oracle(over):
    _check(inp.scaled(inp.CONFIG_BY_NAME["h3"], **over))


@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
def test_softmax_branch_output_dtypes(out_dtype):
    _check(inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=70, text_tokens=20), out_dtype)


@pytest.mark.parametrize("over", [
    dict(heads=2, frames=12, tokens=100, text_tokens=64),
    dict(heads=1, frames=22, tokens=64, d=64, text_tokens=100),
])
def test_softmax_branch_f16_values(over):
    """V given as f16 (the bf16 draws, exactly representable) skips the
    conversion in the kernel and gives the same result."""
    _check(inp.scaled(inp.CONFIG_BY_NAME["h3"], **over), v_dtype="f16")


def test_softmax_branch_other_scale():
    _check(inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=70, text_tokens=20), "f32", scale=0.3)


@pytest.mark.timeout(900)
def test_softmax_branch_h3_full_size_sampled_frames():
    """The H3-shaped workload at full size (24 heads, 102 frames, U = 1008,
    512 text tokens), checked by the oracle's softmax branch on sampled query
    frames of three heads: the first frame of the first chunk, a frame of
    chunk 1, a middle chunk's frame, the last two chunks' frames, and on one
    head also both anchor frames (which see every frame)."""
    cfg = inp.CONFIG_BY_NAME["h3"]
    ins, O, scale = _run(cfg, v_dtype="f16")
    samples = {0: (1, 7, 48, 93, 100), 11: (0, 3, 52, 97, 101), 23: (2, 6, 50, 99)}
    for h, frames in samples.items():
        f = ins[h].f64
        ref = orc.softmax_branch(f("q"), f("k"), f("v"), f("kt"), f("vt"), cfg.frames, cfg.chunk, cfg.window,
                                 cfg.anchors, scale, query_frames=frames)
        for t in frames:
            r = orc.rel_l2(O[h][t], ref[t])
            print(f"  head {h} frame {t}: rel {r:.3e}", flush=True)
            assert r <= TOL
