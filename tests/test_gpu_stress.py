"""Badly conditioned frames on the default path: keys drawn from a rank-r
subspace plus a little noise, so that I + A_t has r eigenvalues near
1 + U mean(beta) / r and the rest near 1 (condition number about 65 at
r = 8 and 110 at r = 4 with U = 1008).  The states and the output must stay
within the same bars as on the well-conditioned workloads: the rounding
sites of the path must not be amplified by the conditioning."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O, TOL_STATE = 2e-3, 1e-3


def subspace_keys(cfg, rank, seed=5, noise=0.05):
    """[T, U, d] unit keys: N(0, 1) coordinates in a random rank-r subspace
    plus noise * N(0, 1) in every channel, normalised per token, as bf16."""
    g = np.random.default_rng(seed)
    basis = np.linalg.qr(g.standard_normal((cfg.d, rank)))[0].T
    k = g.standard_normal((cfg.frames, cfg.tokens, rank)) @ basis \
        + noise * g.standard_normal((cfg.frames, cfg.tokens, cfg.d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return inp.store(k, cfg.in_dtype)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rank", [8, 4])
def test_default_path_on_low_rank_keys(rank):
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=22)
    print(f"[stress] rank-{rank} keys, H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d}", flush=True)
    heads_in = inp.all_heads(cfg)
    for h, x in enumerate(heads_in):
        x.k = subspace_keys(cfg, rank, seed=5 + h)
    f = heads_in[0].f64
    A, _ = orc.frame_stats(f("k")[3], f("v")[3], f("beta")[3])
    ev = np.linalg.eigvalsh(np.eye(cfg.d) + A)
    print(f"  kappa(I + A) of frame 3: {ev[-1] / ev[0]:.0f}", flush=True)
    assert ev[-1] / ev[0] > 40
    for fused in (False, True):
        desc, dev, bufs = runner.run(cfg, heads_in, fused=fused)
        assert vda.vda_device_status(desc, bufs.ws) == 0
        O = runner.out_f64(bufs)
        for h in range(cfg.heads):
            g = heads_in[h].f64
            ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, g("q"), g("k"), g("v"),
                               g("beta"), g("alpha"), g("kt"), g("vt"), g("bt"))
            r_o = orc.rel_l2(O[h][1:-1], ref["O"][1:-1])
            r_s = max(orc.rel_l2(bufs.states_f[h].cpu().numpy(), ref["states_f"]),
                      orc.rel_l2(bufs.states_r[h].cpu().numpy(), ref["states_r"]))
            print(f"  fused={fused} head {h}: O {r_o:.3e}  states {r_s:.3e}", flush=True)
            assert r_o <= TOL_O and r_s <= TOL_STATE


def test_out_of_range_values_are_reported():
    """|beta v| beyond the f16 range of the statistics' operands (here
    v = 1e6) cannot be represented: the run completes and the device status
    word reports a non-finite statistic; a run on in-range data is clean."""
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=7, tokens=64, d=32, text_tokens=0)
    print("[stress] v = 1e6 in one frame", flush=True)
    heads_in = inp.all_heads(cfg)
    v = inp.bf16_bits_to_f32(heads_in[0].v).copy()
    v[2] = 1e6
    heads_in[0].v = inp.f32_to_bf16_bits(v)
    desc, dev, bufs = runner.run(cfg, heads_in)
    assert vda.vda_device_status(desc, bufs.ws) & vda.VDA_DEV_NONFINITE
    desc, dev, bufs = runner.run(cfg, inp.all_heads(cfg))
    assert vda.vda_device_status(desc, bufs.ws) == 0
