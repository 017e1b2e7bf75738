"""vda_forward_noalloc (the path with the library's own device workspace,
for callers that cannot allocate) against vda_forward on the same inputs:
two calls in a row, the second with a smaller workload, each bit for bit
equal to vda_forward and within the parity bars of the float64 oracle."""
import numpy as np
import pytest

from frame_wise_delta_amd import inputs as inp
from frame_wise_delta_amd import runner, vda
from oracle import vda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_O, TOL_STATE = 2e-3, 1e-3


def _noalloc(cfg, heads_in, dev):
    import torch
    desc = vda.desc_for(cfg)
    cnt = vda.vda_state_count(desc)
    H, d = cfg.heads, cfg.d
    sf = torch.full((H, cnt, d, d), 7.0, dtype=torch.float32, device="cuda")
    sr = torch.full_like(sf, 7.0)
    out = torch.full((H, cfg.frames, cfg.tokens, d), 7.0, device="cuda").to(torch.bfloat16)
    status = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    vda.vda_forward_noalloc(desc, dev.q, dev.k, dev.v, dev.beta, dev.alpha, dev.kt, dev.vt, dev.bt, sf, sr, out,
                            status=status)
    torch.cuda.synchronize()
    return sf, sr, out, int(status[0])


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_equals_forward_on_two_calls(order):
    import torch
    big = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=3, frames=22, tokens=300)
    small = inp.scaled(inp.CONFIG_BY_NAME["h3"], heads=2, frames=12, tokens=100, d=64, text_tokens=40)
    for cfg in (big, small):
        print(f"[noalloc] H={cfg.heads} T={cfg.frames} U={cfg.tokens} d={cfg.d}", flush=True)
        heads_in = inp.all_heads(cfg)
        desc, dev, ref = runner.run(cfg, heads_in, fused=True)
        assert vda.vda_device_status(desc, ref.ws) == 0
        sf, sr, out, status = _noalloc(cfg, heads_in, dev)
        assert status == 0
        assert torch.equal(sf, ref.states_f) and torch.equal(sr, ref.states_r)
        assert torch.equal(out.view(torch.int16), ref.out.view(torch.int16))
        f = heads_in[0].f64
        o = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, f("q"), f("k"), f("v"), f("beta"),
                         f("alpha"), f("kt"), f("vt"), f("bt"))
        O = out.float().cpu().numpy().astype(np.float64)[0]
        assert orc.rel_l2(O[1:-1], o["O"][1:-1]) <= TOL_O
        assert orc.rel_l2(sf[0].cpu().numpy(), o["states_f"]) <= TOL_STATE
