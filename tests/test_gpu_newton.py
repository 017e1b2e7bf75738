"""GPU parity of the Newton-iteration inverse (VDA_NEWTON: N_t = (I + A_t)^-1
by X <- X + (I - G X) X in place of Gauss-Jordan) against the float64
oracle, through the C ABI: the factors in the workspace against the exact
inverse and the oracle's Newton iteration, and the whole path's states and
output, alone and with the other modes, up to the full H3-shaped size."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_STATE = 1e-3
TOL_N = 6e-4  # N stored as f16: rounding alone is <= 2^-11 per entry; the iteration stops at <= 1e-6


def _factors(bufs, desc):
    """N_t of every head and slot, decoded from the workspace's fragment order."""
    d = desc.d_k
    n = desc.frames - 2 * desc.anchors
    n_eff = n + (1 if desc.text_tokens else 0)
    raw = bufs.ws.cpu().numpy()[256:256 + desc.heads * n_eff * 2 * d * d * 4]
    slots = raw.reshape(desc.heads, n_eff, 8 * d * d)
    KS, LG = max(1, d // 32), min(4, d // 8)
    j = np.arange(d)[:, None]
    c = np.arange(d // 8)[None, :]
    chunk = (((j // 16) * KS + c // 4) * LG + c % 4) * 16 + j % 16
    idx = (chunk[:, :, None] * 8 + np.arange(8)[None, None, :]).reshape(d, d)
    return slots[..., :2 * d * d].copy().view(np.float16).reshape(desc.heads, n_eff, d * d)[..., idx].astype(np.float64)


def _check(cfg, fused=False, heads_in=None, **over):
    print(f"[newton] {cfg.name} H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d} w={cfg.window} "
          f"text={cfg.text_tokens} fused={fused} {over}", flush=True)
    if heads_in is None:
        heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=fused, newton=True, **over)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    O = runner.out_f64(bufs)
    sf, sr = bufs.states_f.cpu().numpy(), bufs.states_r.cpu().numpy()
    a = cfg.anchors
    text = cfg.text_tokens > 0
    for h in range(cfg.heads):
        f = heads_in[h].f64
        ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"), f("beta"),
                           f("alpha"), f("kt") if text else None, f("vt") if text else None,
                           f("bt") if text else None)
        sl = slice(a, cfg.frames - a)
        r_o = orc.rel_l2(O[h][sl], ref["O"][sl])
        r_f = orc.rel_l2(sf[h], ref["states_f"])
        r_r = orc.rel_l2(sr[h], ref["states_r"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}  states_r {r_r:.3e}", flush=True)
        assert r_o <= TOL_O and r_f <= TOL_STATE and r_r <= TOL_STATE
    return desc, bufs, heads_in


@pytest.mark.parametrize("d,tokens", [(16, 40), (32, 64), (64, 100), (128, 300)])
def test_newton_factors_match_the_inverse(d, tokens):
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=12, tokens=tokens, d=d, text_tokens=24)
    desc, bufs, heads_in = _check(cfg)
    N = _factors(bufs, desc)
    worst = 0.0
    for h in range(cfg.heads):
        f = heads_in[h].f64
        for s in range(cfg.scanned + 1):
            if s < cfg.scanned:
                t = cfg.anchors + s
                A, _ = orc.frame_stats(f("k")[t], f("v")[t], f("beta")[t])
            else:
                A, _ = orc.frame_stats(f("kt"), f("vt"), f("bt"))
            G = np.eye(d) + A
            inv = np.linalg.solve(G, np.eye(d))
            X, k = orc.newton_schulz_inverse(G, tol=1e-6)
            r_inv, r_ns = orc.rel_l2(N[h, s], inv), orc.rel_l2(N[h, s], X)
            worst = max(worst, r_inv)
            assert r_inv <= TOL_N and r_ns <= TOL_N, (h, s, k, r_inv, r_ns)
    print(f"  factors: worst rel vs the inverse {worst:.3e}", flush=True)


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("scan_only", {}),
    ("h3", dict(heads=3, frames=22, tokens=300)),
])
def test_newton_path_matches_oracle(name, over):
    _check(inp.scaled(inp.CONFIG_BY_NAME[name], **over))


def test_newton_with_chunk_scan_and_fused_entry_point():
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=22, tokens=200)
    _check(cfg, fused=True)
    _check(cfg, chunk_scan=True)


def test_newton_on_badly_conditioned_frames():
    """Keys from a rank-4 subspace with large write gates: I + A has a wide
    eigenvalue range (kappa ~ 60), so the iteration runs longer.  The
    factors still match the inverse to their f16 storage.  The Newton
    comparator keeps B_t (f16) and forms (S Diag(alpha) + B_t) N_t, whose f16
    roundings the conditioning amplifies (states ~1.5e-3, bound 2.5e-3); the
    default path, which keeps J_t = B_t N_t instead, stays within the 1e-3
    bar on the same input."""
    import torch
    cfg = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=1, frames=12, tokens=256, d=64, text_tokens=0)
    h = inp.all_heads(cfg)[0]
    g = np.random.default_rng(51)
    basis = np.linalg.qr(g.standard_normal((64, 4)))[0].T
    k = g.standard_normal((cfg.frames, cfg.tokens, 4)) @ basis + 0.05 * g.standard_normal((cfg.frames, cfg.tokens, 64))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    x = inp.HeadInputs(**{**h.__dict__})
    x.k = inp.store(k, "bf16")
    x.beta = np.full((cfg.frames, cfg.tokens), 0.9, np.float32)
    f = x.f64
    desc, _, b_ns = runner.run(cfg, [x], newton=True)
    _, _, b_gj = runner.run(cfg, [x])
    assert vda.vda_device_status(desc, b_ns.ws) == 0
    N = _factors(b_ns, desc)
    worst_k = 0
    for s_ in range(cfg.scanned):
        A, _ = orc.frame_stats(f("k")[1 + s_], f("v")[1 + s_], f("beta")[1 + s_])
        G = np.eye(64) + A
        ev = np.linalg.eigvalsh(G)
        _, kk = orc.newton_schulz_inverse(G, tol=1e-6)
        worst_k = max(worst_k, kk)
        r = orc.rel_l2(N[0, s_], np.linalg.solve(G, np.eye(64)))
        assert ev[-1] / ev[0] > 30 and r <= TOL_N, (s_, ev[-1] / ev[0], r)
    ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"), f("beta"),
                       f("alpha"))
    errs = {}
    for name, b in (("newton", b_ns), ("default", b_gj)):
        errs[name] = max(orc.rel_l2(b.states_f[0].cpu().numpy(), ref["states_f"]),
                         orc.rel_l2(b.states_r[0].cpu().numpy(), ref["states_r"]))
    print(f"  up to {worst_k} Newton steps; states vs oracle: {errs}", flush=True)
    assert errs["newton"] <= 2.5e-3
    assert errs["default"] <= 1e-3
    assert bool(torch.isfinite(b_ns.out.float()).all())


@pytest.mark.timeout(900)
def test_newton_h3_full_size():
    cfg = inp.CONFIG_BY_NAME["h3"]
    print("[newton] full-size H3: drawing inputs", flush=True)
    heads_in = inp.all_heads(cfg)
    desc, dev, bufs = runner.run(cfg, heads_in, fused=True, newton=True)
    assert vda.vda_device_status(desc, bufs.ws) == 0
    O = runner.out_f64(bufs)
    for h in (0, 17):
        f = heads_in[h].f64
        ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"), f("beta"),
                           f("alpha"), f("kt"), f("vt"), f("bt"))
        r_o = orc.rel_l2(O[h][1:-1], ref["O"][1:-1])
        r_f = orc.rel_l2(bufs.states_f[h].cpu().numpy(), ref["states_f"])
        print(f"  head {h}: O {r_o:.3e}  states_f {r_f:.3e}", flush=True)
        assert r_o <= TOL_O and r_f <= TOL_STATE
