"""GPU parity of the readout epilogue (vda_readout_gated: RMSNorm over the
value channels, then a sigmoid gate) against the float64 oracle, through the
C ABI, on every head size, ragged token tails, both readout modes and all
output types."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_Y = 2e-3      # gated output, relative L2 (16-bit output rounding dominates)
TOL_EPI = 2e-5    # f32 gated output vs the oracle epilogue applied to the GPU's own f32 readout
EPS = 1e-6


def _run(cfg, eps=EPS, out_dtypes=("bf16",)):
    print(f"[epilogue] {cfg.name} H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} "
          f"window={cfg.window} in={cfg.in_dtype} out={out_dtypes}", flush=True)
    heads_in = inp.all_heads(cfg)
    epi_in = [inp.epilogue_inputs(cfg, h) for h in range(cfg.heads)]
    desc, dev, bufs = runner.run(cfg, heads_in, out_dtype="f32")
    gate, weight = runner.upload_epilogue(cfg, epi_in)
    outs = {od: runner.readout_gated(desc, dev, bufs, gate, weight, eps, od) for od in out_dtypes}
    return heads_in, epi_in, bufs, outs


def _check_against_oracle(cfg, heads_in, epi_in, outs, eps=EPS, tol=TOL_Y):
    a = cfg.anchors
    for h in range(cfg.heads):
        f = heads_in[h].f64
        text = cfg.text_tokens > 0
        ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"), f("beta"),
                           f("alpha"), f("kt") if text else None, f("vt") if text else None,
                           f("bt") if text else None)
        Y_ref = orc.rmsnorm_gate(ref["O"], epi_in[h].f64("weight"), epi_in[h].f64("gate"), eps)
        for od, out in outs.items():
            Y = out[h].float().cpu().numpy().astype(np.float64)
            r = orc.rel_l2(Y[a:cfg.frames - a], Y_ref[a:cfg.frames - a])
            print(f"  head {h} out {od}: rel {r:.3e}", flush=True)
            assert r <= tol
            if a:
                assert not Y[0].any() and not Y[-1].any()


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),                                                   # d = 16, f32 in
    ("scan_only", {}),                                              # d = 64, per-frame readout
    ("h3", dict(heads=2, frames=17, tokens=300)),                   # d = 128, bf16, 3 chunks, ragged tile
    ("h3", dict(heads=1, frames=12, tokens=37, d=32)),              # d = 32, one partial tile
    ("h3", dict(heads=1, frames=7, tokens=1000, d=128, window=0)),  # own-chunk window, 16 tiles
])
def test_gated_readout_matches_oracle(name, over):
    cfg = inp.scaled(inp.CONFIG_BY_NAME[name], **over)
    heads_in, epi_in, _, outs = _run(cfg, out_dtypes=("bf16", "f16", "f32"))
    _check_against_oracle(cfg, heads_in, epi_in, outs)


def test_epilogue_arithmetic_on_the_gpu_readout():
    """The gated kernel's epilogue equals the oracle's epilogue applied to the
    plain readout's own float32 output: this isolates the RMSNorm and gate
    from the readout error."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=12, tokens=200)
    heads_in, epi_in, bufs, outs = _run(cfg, out_dtypes=("f32",))
    O = runner.out_f64(bufs)  # plain readout, f32 output
    for h in range(cfg.heads):
        Y_cpu = orc.rmsnorm_gate(O[h], epi_in[h].f64("weight"), epi_in[h].f64("gate"), EPS)
        Y = outs["f32"][h].cpu().numpy().astype(np.float64)
        r = orc.rel_l2(Y, Y_cpu)
        print(f"  head {h}: epilogue rel {r:.3e}", flush=True)
        assert r <= TOL_EPI


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_epsilon_is_applied(eps):
    """A large eps visibly shrinks the normalised rows; both follow the oracle."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=64)
    heads_in, epi_in, _, outs = _run(cfg, eps=eps, out_dtypes=("f32",))
    _check_against_oracle(cfg, heads_in, epi_in, outs, eps=eps)


def test_gated_readout_without_scanned_frames():
    """Only anchors: every output row is zero."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["tiny"], frames=2)
    heads_in, _, _, outs = _run(cfg, out_dtypes=("f32",))
    assert not bool(torch.any(outs["f32"] != 0))
