"""bench.py on the host: the one-GPU contract and the work counts its
throughput and roofline figures are computed from (no GPU needed)."""
import importlib.util
import os
import subprocess
import sys

import pytest

from frame_wise_delta_amd import inputs as inp
from oracle import vda_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    bm = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bm)
    return bm


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration it does not run


@pytest.mark.parametrize("name,over", [
    ("h3", {}),
    ("tiny", {}),
    ("h3", dict(frames=27, window=3)),      # window wider than the sequence
    ("h3", dict(frames=20, anchors=0)),     # no anchors
    ("h3", dict(frames=22, window=0)),      # own chunk only
])
def test_softmax_work_counts_the_oracles_key_sets(name, over):
    """The closed-form count of (query, key) pairs behind the softmax
    branch's TFLOP/s equals the pairs of the oracle's visible key frames
    (built from sets), plus every query against every text token."""
    bm = _bench()
    cfg = inp.scaled(inp.CONFIG_BY_NAME[name], **over)
    keys = orc.softmax_key_frames(cfg.frames, cfg.chunk, cfg.window, cfg.anchors)
    pairs = sum(len(k) for k in keys) * cfg.tokens * cfg.tokens + cfg.frames * cfg.tokens * cfg.text_tokens
    flops, nbytes = bm.softmax_work(cfg)
    assert flops == 4 * cfg.d * pairs * cfg.heads
    assert nbytes == cfg.heads * (4 * cfg.frames * cfg.tokens * cfg.d * 2 + 2 * cfg.text_tokens * cfg.d * 2)


def test_h3_work_figures():
    """The H3-shaped workload's figures quoted with the measurements.  FLOPs
    per step: the statistics, solves, both scan directions and the text
    state, with the readout counted as one product per frame with the merged
    operand W_t (264.0 GFLOP), and with the forward and reverse reads
    counted as two products (343.2 GFLOP, the count the measurement plan
    states).  The prepare kernel's 1,254,647,808 algorithmic bytes (K, V
    bf16 and beta of 24 x 100 frames of 1008 tokens plus 512 text tokens per
    head) and the readout's 1.252 GB (Q bf16, alpha, and every output row in
    bf16, anchors included)."""
    bm = _bench()
    cfg = inp.CONFIG_BY_NAME["h3"]
    flops, _, flops_two = bm.algorithmic_work(cfg)
    U, d, Nt = 1008, 128, 512
    common = (2 * U * d * d      # A = K^T Diag(beta) K
              + 2 * U * d * d    # B = V^T Diag(beta) K
              + d ** 3           # N = (I + A)^-1
              + 2 * 2 * d ** 3)  # the frame write in the forward and the reverse scan
    merged = common + 2 * d * d + 2 * U * d * d      # W_t formed, then one product with Q
    two = common + 2 * 2 * U * d * d                 # the forward and reverse state products
    per_text = 4 * Nt * d * d + d ** 3 + 2 * d ** 3  # A_T, B_T, their solve, S^T = B_T N_T
    assert flops == 24 * (100 * merged + per_text)
    assert flops_two == 24 * (100 * two + per_text)
    assert round(flops_two / 1e9, 1) == 343.2
    assert round(flops / 1e9, 1) == 264.0
    kb = bm.kernel_bytes(cfg)
    frame_bytes = 1008 * 128 * 2 * 2 + 1008 * 4
    text_bytes = 512 * 128 * 2 * 2 + 512 * 4
    assert kb["frame_kernel"] == kb["stats_kernel"] == 24 * (100 * frame_bytes + text_bytes) == 1_254_647_808
    assert kb["readout_kernel"] == 24 * (100 * (1008 * 128 * 2 + 128 * 4) + 102 * 1008 * 128 * 2)
    assert round(kb["readout_kernel"] / 1e9, 3) == 1.252


def test_kernel_code_hash_ignores_comments_only():
    """The traffic table is keyed by a hash of each kernel's code: comments
    and blank lines do not change it, a change of code does."""
    bm = _bench()
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n"
    assert bm._code_only(code) == bm._code_only("/* a header\n   comment */\n" + code.replace("// one more", "// else"))
    assert bm._code_only(code) == bm._code_only(code.replace("\n", "\n\n"))
    assert bm._code_only(code) != bm._code_only(code.replace("a + 1", "a + 2"))
    assert bm._code_only("x = 1; /* a */ y = 2;") == "x = 1;  y = 2;"
