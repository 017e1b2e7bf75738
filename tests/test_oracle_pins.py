"""Pins of the float64 oracle against facts fixed by the Video DeltaNet summary
page and by the mathematics, independent of the oracle's own formulas.

Each pin is chosen so that a plausible slip in the oracle (a dropped term,
decay on the wrong side, a transposed cross term, a wrong bridge range, a
window off by one chunk) fails at least one of them.  CPU only.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import vda_oracle as orc
from frame_wise_delta_amd import inputs as inp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(g, shape):
    x = g.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _frame(g, U, d):
    K = _unit(g, (U, d))
    V = g.standard_normal((U, d))
    beta = 1 / (1 + np.exp(-g.standard_normal(U)))
    alpha = 0.9 + 0.1 * g.random(d)
    S_prev = g.standard_normal((d, d))
    return S_prev, K, V, beta, alpha


def _objective_grad(S, S_bar, K, V, beta):
    """Gradient of 1/2||S - S_bar||^2 + sum_u beta_u/2 ||S k_u - v_u||^2,
    written token by token from the joint objective (核心方法 para 2)."""
    g = S - S_bar
    for u in range(K.shape[0]):
        g = g + beta[u] * np.outer(S @ K[u] - V[u], K[u])
    return g


# ------------------------------------------------ frame update (a1 + a2) --

@pytest.mark.parametrize("U,d", [(1, 4), (7, 5), (40, 16), (300, 64)])
def test_closed_form_is_stationary_point_of_objective(U, d):
    """The oracle's S_t zeroes the gradient of the joint objective, i.e. it
    satisfies the normal equations S_t(I + A_t) = S_bar_t + B_t."""
    g = np.random.default_rng([1, U, d])
    S_prev, K, V, beta, alpha = _frame(g, U, d)
    S = orc.frame_update(S_prev, K, V, beta, alpha)
    S_bar = S_prev * alpha[None, :]
    grad = _objective_grad(S, S_bar, K, V, beta)
    assert np.abs(grad).max() <= 1e-12 * max(1.0, np.abs(S).max())


def test_gradient_descent_reaches_the_same_minimiser():
    """Brute-force minimisation of the joint objective on tiny inputs."""
    for seed in range(5):
        g = np.random.default_rng([2, seed])
        d, U = 3 + seed, 5 + 3 * seed
        S_prev, K, V, beta, alpha = _frame(g, U, d)
        S_bar = S_prev * alpha[None, :]
        # step 1/L with L >= lambda_max of the Hessian (trace bound)
        step = 1.0 / (1.0 + float(np.sum(beta * np.sum(K * K, axis=1))))
        S = S_bar.copy()
        for _ in range(200000):
            grad = _objective_grad(S, S_bar, K, V, beta)
            if np.abs(grad).max() < 1e-13:
                break
            S = S - step * grad
        ref = orc.frame_update(S_prev, K, V, beta, alpha)
        assert np.abs(S - ref).max() <= 1e-10


def test_single_token_equals_implicit_delta_step():
    """U = 1: the frame write is the implicit token delta step
    S_bar + beta (v - S_bar k) k^T / (1 + beta ||k||^2)  (Delta 规则)."""
    g = np.random.default_rng(3)
    for d in (2, 8, 64):
        S_prev = g.standard_normal((d, d))
        k = g.standard_normal(d)          # not normalised on purpose
        v = g.standard_normal(d)
        beta = float(g.random()) * 3
        alpha = 0.5 + 0.5 * g.random(d)
        S_bar = S_prev * alpha[None, :]
        expect = S_bar + beta * np.outer(v - S_bar @ k, k) / (1 + beta * k @ k)
        got = orc.frame_update(S_prev, k[None], v[None], np.array([beta]), alpha)
        assert np.abs(got - expect).max() <= 1e-13 * max(1, np.abs(expect).max())


def test_correlation_awareness_saturation():
    """Repeated key U times -> read weight U beta/(1 + U beta); orthonormal
    keys -> beta/(1 + beta) each (技术新颖性, appendix A.2 summary)."""
    g = np.random.default_rng(4)
    d, U, beta = 16, 9, 0.37
    k = _unit(g, (d,))
    v = g.standard_normal(d)
    K = np.tile(k, (U, 1))
    V = np.tile(v, (U, 1))
    S = orc.frame_update(np.zeros((d, d)), K, V, np.full(U, beta), np.ones(d))
    assert np.abs(S @ k - U * beta / (1 + U * beta) * v).max() <= 1e-14
    # with a non-zero decayed state: S k = (S_bar k + U beta v)/(1 + U beta)
    S_prev = g.standard_normal((d, d))
    alpha = 0.9 + 0.1 * g.random(d)
    S = orc.frame_update(S_prev, K, V, np.full(U, beta), alpha)
    S_bar = S_prev * alpha[None, :]
    assert np.abs(S @ k - (S_bar @ k + U * beta * v) / (1 + U * beta)).max() <= 1e-13
    # orthonormal keys
    Qm, _ = np.linalg.qr(g.standard_normal((d, d)))
    Ko = Qm.T[:6]
    Vo = g.standard_normal((6, d))
    S = orc.frame_update(np.zeros((d, d)), Ko, Vo, np.full(6, beta), np.ones(d))
    for u in range(6):
        assert np.abs(S @ Ko[u] - beta / (1 + beta) * Vo[u]).max() <= 1e-14


def test_exact_rational_two_by_two():
    """d = 2, U = 2 with rational data, solved exactly (Cramer's rule on the
    normal equations in exact fractions) against the float64 oracle."""
    F = Fraction
    K = [[F(1, 2), F(1, 3)], [F(-1, 4), F(2, 3)]]
    V = [[F(3, 2), F(-1)], [F(1, 5), F(2)]]
    beta = [F(1, 2), F(3, 4)]
    alpha = [F(9, 10), F(4, 5)]
    S_prev = [[F(1), F(-2)], [F(1, 2), F(3)]]
    S_bar = [[S_prev[i][j] * alpha[j] for j in range(2)] for i in range(2)]
    G = [[(1 if i == j else 0) + sum(beta[u] * K[u][i] * K[u][j] for u in range(2))
          for j in range(2)] for i in range(2)]
    Y = [[S_bar[i][j] + sum(beta[u] * V[u][i] * K[u][j] for u in range(2))
          for j in range(2)] for i in range(2)]
    det = G[0][0] * G[1][1] - G[0][1] * G[1][0]
    Ginv = [[G[1][1] / det, -G[0][1] / det], [-G[1][0] / det, G[0][0] / det]]
    S_exact = [[sum(Y[i][m] * Ginv[m][j] for m in range(2)) for j in range(2)] for i in range(2)]
    f = lambda M: np.array([[float(x) for x in r] for r in M])
    got = orc.frame_update(f(S_prev), f(K), f(V), np.array([float(b) for b in beta]),
                           np.array([float(a) for a in alpha]))
    assert np.abs(got - f(S_exact)).max() <= 2e-15


def test_transition_is_non_expansive():
    """Proposition 1: ||S_bar (I + A)^{-1}||_2 <= ||S_bar||_2 and
    ||Diag(alpha)(I + A)^{-1}||_2 <= 1 without commutation (核心方法 para 2,
    技术新颖性).  Counter-check: the batched additive transition I - A of
    SANA-WM expands when lambda_max(A) > 2 (核心方法 para 2)."""
    g = np.random.default_rng(5)
    for trial in range(40):
        d, U = (16, 16) if trial < 20 else (8, 64)
        S_prev, K, V, beta, alpha = _frame(g, U, d)
        S_bar = S_prev * alpha[None, :]
        # V = 0 isolates the inherited-state transition S_bar -> S_bar N
        S = orc.frame_update(S_prev, K, np.zeros_like(V), beta, alpha)
        assert np.linalg.norm(S, 2) <= np.linalg.norm(S_bar, 2) * (1 + 1e-12)
        # M = Diag(alpha) N is the image of S_prev = I
        M = orc.frame_update(np.eye(d), K, np.zeros_like(V), beta, alpha)
        assert np.linalg.norm(M, 2) <= 1 + 1e-12
    # SANA-WM comparator: many aligned tokens make lambda_max(A) > 2
    k = _unit(g, (8,))
    K = np.tile(k, (10, 1))
    A = K.T @ (0.5 * K)
    assert np.linalg.eigvalsh(A).max() > 2
    assert np.linalg.norm(np.eye(8) - A, 2) > 1
    M = orc.frame_update(np.eye(8), K, np.zeros_like(K), np.full(10, 0.5), np.ones(8))
    assert np.linalg.norm(M, 2) <= 1 + 1e-12


# ----------------------------------------------------------------- scans --

def _small_cfg_inputs(seed=6, T=17, U=12, d=8, anchors=1, nt=5):
    g = np.random.default_rng(seed)
    q = _unit(g, (T, U, d))
    k = _unit(g, (T, U, d))
    v = g.standard_normal((T, U, d))
    beta = 1 / (1 + np.exp(-g.standard_normal((T, U))))
    alpha = 0.9 + 0.1 * g.random((T, d))
    kt = _unit(g, (nt, d))
    vt = g.standard_normal((nt, d))
    bt = 1 / (1 + np.exp(-g.standard_normal(nt)))
    return q, k, v, beta, alpha, kt, vt, bt


def test_reverse_scan_equals_forward_scan_on_reversed_time():
    q, k, v, beta, alpha, kt, vt, bt = _small_cfg_inputs()
    T = k.shape[0]
    r = orc.run_head(T, 5, 1, 1, q, k, v, beta, alpha, kt, vt, bt)
    rr = orc.run_head(T, 5, 1, 1, q[::-1], k[::-1], v[::-1], beta[::-1], alpha[::-1], kt, vt, bt)
    assert np.array_equal(r["states_r"], rr["states_f"])
    assert np.array_equal(r["states_f"], rr["states_r"])


def test_no_writes_gives_pure_decay():
    """beta = 0: S = S_0 Diag(prod alpha); alpha = 1 too: S = S_0."""
    g = np.random.default_rng(7)
    T, U, d = 12, 6, 5
    k = _unit(g, (T, U, d))
    v = g.standard_normal((T, U, d))
    alpha = 0.8 + 0.2 * g.random((T, d))
    S0 = g.standard_normal((d, d))
    order = list(range(1, T - 1))
    st = orc.scan(order, k, v, np.zeros((T, U)), alpha, S0, 1)
    for i in range(len(order) + 1):
        decay = np.ones(d)
        for t in order[:i]:
            decay = decay * alpha[t]
        assert np.abs(st[i] - S0 * decay[None, :]).max() <= 1e-14
    st = orc.scan(order, k, v, np.zeros((T, U)), np.ones((T, d)), S0, 1)
    assert np.array_equal(st[-1], S0)


def test_scan_records_every_chunk_boundary():
    q, k, v, beta, alpha, *_ = _small_cfg_inputs(T=22)
    order = list(range(1, 21))
    per_frame = orc.scan(order, k, v, beta, alpha, np.zeros((8, 8)), 1)
    per_chunk = orc.scan(order, k, v, beta, alpha, np.zeros((8, 8)), 5)
    assert np.array_equal(per_chunk, per_frame[::5])


# ------------------------------------------------ chunk composition (a3) --

@pytest.mark.parametrize("P", [1, 3, 5, 7])
def test_chunk_scan_equals_frame_scan_at_every_boundary(P):
    """S_out = S_in M_chunk + J_chunk (方法步骤详情 step (4)) reaches the
    frame-by-frame states at each chunk boundary, forward and reverse,
    including a shorter last run (20 frames in runs of 3 or 7)."""
    q, k, v, beta, alpha, kt, vt, bt = _small_cfg_inputs(T=22)
    order = list(range(1, 21))
    S0 = 0.5 * orc.text_state(kt, vt, bt, 8, 8)
    for o in (order, order[::-1]):
        ref = orc.scan(o, k, v, beta, alpha, S0, P)
        got = orc.scan_chunked(o, k, v, beta, alpha, S0, P)
        assert got.shape == ref.shape
        assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_frame_map_satisfies_the_normal_equations():
    """M_t (I + A_t) = Diag(alpha_t) and J_t (I + A_t) = B_t, with A_t and
    B_t summed token by token (方法步骤详情 step (3))."""
    g = np.random.default_rng(21)
    for U, d in ((1, 4), (9, 6), (50, 16)):
        _, K, V, beta, alpha = _frame(g, U, d)
        A = sum(beta[u] * np.outer(K[u], K[u]) for u in range(U))
        B = sum(beta[u] * np.outer(V[u], K[u]) for u in range(U))
        M, J = orc.frame_map(K, V, beta, alpha)
        G = np.eye(d) + A
        assert np.abs(M @ G - np.diag(alpha)).max() <= 1e-12
        assert np.abs(J @ G - B).max() <= 1e-12 * max(1.0, np.abs(B).max())


def test_chunk_map_without_writes_is_pure_decay_and_non_expansive():
    """beta = 0: M_chunk = Diag(prod alpha) and J_chunk = 0.  With writes,
    ||M_chunk||_2 <= 1 (a product of non-expansive transitions, 核心方法
    para 2)."""
    q, k, v, beta, alpha, *_ = _small_cfg_inputs(T=12)
    frames = [3, 4, 5, 6, 7]
    M, J = orc.chunk_map(frames, k, v, np.zeros_like(beta), alpha)
    assert np.abs(M - np.diag(np.prod(alpha[frames], axis=0))).max() <= 1e-15
    assert np.abs(J).max() == 0.0
    for fr in (frames, frames[::-1], [2]):
        M, _ = orc.chunk_map(fr, k, v, beta, alpha)
        assert np.linalg.norm(M, 2) <= 1 + 1e-12


def test_chunk_map_order_matters_and_reverse_matches_reversed_time():
    """The reverse scan composes a chunk last frame first; on time-reversed
    input it is the forward composition."""
    q, k, v, beta, alpha, *_ = _small_cfg_inputs(T=12)
    fr = [3, 4, 5, 6, 7]
    Mf, Jf = orc.chunk_map(fr, k, v, beta, alpha)
    Mr, Jr = orc.chunk_map(fr[::-1], k, v, beta, alpha)
    assert np.abs(Mf - Mr).max() > 1e-6  # the transitions do not commute
    T = k.shape[0]
    rev = [T - 1 - t for t in fr[::-1]]
    M2, J2 = orc.chunk_map(rev, k[::-1], v[::-1], beta[::-1], alpha[::-1])
    assert np.array_equal(M2, Mr) and np.array_equal(J2, Jr)


# ---------------------------------------------------------------- maps ----

def _closed_form_rows(T, P, w, anchors):
    a = 1 if anchors else 0
    n = T - 2 * a
    C = -(-n // P)
    w = max(w, 0)
    rows = []
    for c in range(C):
        lo, hi = max(0, c - w), min(C - 1, c + w)
        ws = a + P * lo
        we = min(a + P * (hi + 1) - 1, a + n - 1)
        rows.append((c, lo, hi, ws, we, lo, C - 1 - hi))
    return np.array(rows, dtype=np.int32)


def test_maps_match_hand_derived_tiny_table():
    rows, fc = orc.index_maps(22, 5, 1, 1)
    table, fcg = [], None
    with open(os.path.join(GOLDEN, "tiny_maps.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            if line.startswith("frame_chunk"):
                fcg = np.array([int(x) for x in line.split()[1:]], dtype=np.int32)
            else:
                table.append([int(x) for x in line.split()])
    assert np.array_equal(rows, np.array(table, dtype=np.int32))
    assert np.array_equal(fc, fcg)


@pytest.mark.parametrize("cfg", inp.CONFIGS, ids=lambda c: c.name)
def test_maps_closed_form_and_partition(cfg):
    _check_maps(cfg.frames, cfg.chunk, cfg.window, cfg.anchors)


def test_maps_random_shapes():
    g = np.random.default_rng(8)
    for _ in range(200):
        P = int(g.integers(1, 8))
        n = int(g.integers(1, 12)) * P
        anchors = int(g.integers(0, 2))
        w = int(g.integers(0, 4))
        _check_maps(n + 2 * anchors, P, w, anchors)


def _check_maps(T, P, w, anchors):
    rows, fc = orc.index_maps(T, P, w, anchors)
    assert np.array_equal(rows, _closed_form_rows(T, P, w, anchors))
    a = 1 if anchors else 0
    scanned = set(range(a, T - a))
    C = len(rows)
    for c, lo, hi, ws, we, F, R in rows:
        fwd = {f for f in scanned if fc[f] < F}
        win = set(range(ws, we + 1))
        rev = {f for f in scanned if fc[f] >= C - R}
        # forward frames, window and reverse frames partition the scanned frames
        assert fwd | win | rev == scanned
        assert not (fwd & win) and not (win & rev) and not (fwd & rev)
        # the query chunk lies inside its window and the window spans 2w+1
        # chunks unless clipped at an end
        own = {f for f in scanned if fc[f] == c}
        assert own <= win
        if w >= 0 and P * (2 * w + 1) <= len(scanned):
            assert len(win) == P * (hi - lo + 1)


def test_h3_maps_sample_rows():
    rows, _ = orc.index_maps(102, 5, 1, 1)
    assert tuple(rows[0][3:]) == (1, 10, 0, 18)
    assert tuple(rows[10][3:]) == (46, 60, 9, 8)
    assert tuple(rows[19][3:]) == (91, 100, 18, 0)
    # 15-frame window for interior chunks (核心方法 para 1)
    assert all(r[4] - r[3] + 1 == 15 for r in rows[1:-1])


# ------------------------------------------------------------- readout ----

def test_text_is_counted_once_when_video_writes_nothing():
    """beta = 0, alpha = 1 in the video: both reads see 1/2 S^T, so the output
    is exactly S^T q (nothing counted twice, 核心方法 para 1)."""
    q, k, v, beta, alpha, kt, vt, bt = _small_cfg_inputs(T=22)
    r = orc.run_head(22, 5, 1, 1, q, k, v, np.zeros_like(beta), np.ones_like(alpha), kt, vt, bt)
    ST = r["S_text"]
    for t in range(1, 21):
        assert np.abs(r["O"][t] - q[t] @ ST.T).max() <= 1e-14
    assert not r["O"][0].any() and not r["O"][21].any()


def test_bridge_continues_the_decay_through_the_window():
    """With beta = 0 everywhere in the video the scans only decay.  The bridged
    windowed read of frame t must then equal the read of the decay-only
    states carried all the way to t from both ends (bridge inclusive of t)."""
    q, k, v, beta, alpha, kt, vt, bt = _small_cfg_inputs(T=22, seed=9)
    r = orc.run_head(22, 5, 1, 1, q, k, v, np.zeros_like(beta), alpha, kt, vt, bt)
    S0 = 0.5 * r["S_text"]
    for t in range(1, 21):
        df = np.prod(alpha[1:t + 1], axis=0)
        dr = np.prod(alpha[t:21], axis=0)
        expect = q[t] @ (S0 * df[None, :]).T + q[t] @ (S0 * dr[None, :]).T
        assert np.abs(r["O"][t] - expect).max() <= 1e-14


def test_text_state_satisfies_its_normal_equations():
    q, k, v, beta, alpha, kt, vt, bt = _small_cfg_inputs(nt=30)
    ST = orc.text_state(kt, vt, bt, 8, 8)
    grad = _objective_grad(ST, np.zeros((8, 8)), kt, vt, bt)
    assert np.abs(grad).max() <= 1e-12


def test_full_forward_readout_uses_state_after_own_write():
    q, k, v, beta, alpha, *_ = _small_cfg_inputs(T=9, anchors=0)
    r = orc.run_head(9, 5, -1, 0, q, k, v, beta, alpha)
    S = np.zeros((8, 8))
    for t in range(9):
        S = orc.frame_update(S, k[t], v[t], beta[t], alpha[t])
        assert np.abs(r["O"][t] - q[t] @ S.T).max() <= 1e-14


def test_readout_is_linear_in_q():
    q, k, v, beta, alpha, kt, vt, bt = _small_cfg_inputs(T=22, seed=10)
    q2 = np.random.default_rng(11).standard_normal(q.shape)
    o1 = orc.run_head(22, 5, 1, 1, q, k, v, beta, alpha, kt, vt, bt)["O"]
    o2 = orc.run_head(22, 5, 1, 1, q2, k, v, beta, alpha, kt, vt, bt)["O"]
    o3 = orc.run_head(22, 5, 1, 1, q + 2 * q2, k, v, beta, alpha, kt, vt, bt)["O"]
    assert np.abs(o3 - (o1 + 2 * o2)).max() <= 1e-12


# -------------------------------------------------------------- inputs ----

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1e-3, 3.0e5], dtype=np.float32)
    b = inp.bf16_bits_to_f32(inp.f32_to_bf16_bits(x))
    assert b[0] == 1.0 and b[1] == 1.0 and b[2] == 1.0 + 4 * 2**-8 and b[3] == -2.5
    assert abs(b[4] - 1e-3) <= 1e-3 * 2**-8
    assert abs(b[5] - 3.0e5) <= 3.0e5 * 2**-8


def test_inputs_are_deterministic_per_head():
    cfg = inp.CONFIG_BY_NAME["tiny"]
    a = inp.head_inputs(cfg, 0)
    b = inp.head_inputs(cfg, 0)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.alpha, b.alpha)
    k = a.f64("k")
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-6)
    assert ((a.alpha >= 0.9) & (a.alpha < 1.0)).all()


# ----------------------------------------------------- readout epilogue (f1) --

def test_epilogue_hand_worked_example():
    """o = (3, 4): the mean square over the two channels is 12.5, so with
    eps = 0 the normalised row is (3, 4) / sqrt(12.5) = (3, 4) * sqrt(2) / 5.
    Weight (2, 1/2), gate logits (0, 0) -> sigmoid 1/2:
    y = (3 sqrt(2) / 5, 4 sqrt(2) / 5) * (2, 1/2) * 1/2 = (3 sqrt(2) / 5, sqrt(2) / 5)."""
    O = np.array([[[3.0, 4.0]]])
    y = orc.rmsnorm_gate(O, np.array([2.0, 0.5]), np.zeros((1, 1, 2)), 0.0)
    r2 = np.sqrt(2.0)
    np.testing.assert_allclose(y[0, 0], [3 * r2 / 5, r2 / 5], rtol=1e-15)
    # large logits saturate the gate: sigmoid(40) = 1 - 4.2e-18, sigmoid(-40) = 4.2e-18
    y = orc.rmsnorm_gate(O, np.ones(2), np.array([[[40.0, -40.0]]]), 0.0)
    np.testing.assert_allclose(y[0, 0, 0], 3 * r2 / 5, rtol=1e-15)
    assert 0 < y[0, 0, 1] < 1e-17


def test_epilogue_unit_rms_and_epsilon():
    """With unit weight and an open gate, every output row has root mean
    square sqrt(m / (m + eps)), m the row's mean square (1 for eps = 0)."""
    g = np.random.default_rng(7)
    O = g.standard_normal((3, 5, 16)) * np.exp(g.standard_normal((3, 5, 1)))
    m = np.mean(O * O, axis=-1)
    open_gate = np.full(O.shape, 60.0)
    for eps in (0.0, 1e-6, 0.3):
        y = orc.rmsnorm_gate(O, np.ones(16), open_gate, eps)
        rms = np.sqrt(np.mean(y * y, axis=-1))
        np.testing.assert_allclose(rms, np.sqrt(m / (m + eps)), rtol=1e-12)


def test_epilogue_scale_sign_and_gate_symmetry():
    """eps = 0: positive rescaling of a row does not change the output and
    negation negates it; sigmoid(x) + sigmoid(-x) = 1, so the outputs for
    opposite logits add up to the normalised, weighted row."""
    g = np.random.default_rng(8)
    O = g.standard_normal((2, 4, 8))
    w = 1 + 0.1 * g.standard_normal(8)
    z = g.standard_normal(O.shape)
    y = orc.rmsnorm_gate(O, w, z, 0.0)
    np.testing.assert_allclose(orc.rmsnorm_gate(3.7 * O, w, z, 0.0), y, rtol=1e-13)
    np.testing.assert_allclose(orc.rmsnorm_gate(-O, w, z, 0.0), -y, rtol=1e-13)
    both = y + orc.rmsnorm_gate(O, w, -z, 0.0)
    norm = O / np.sqrt(np.mean(O * O, axis=-1, keepdims=True))
    np.testing.assert_allclose(both, norm * w, rtol=1e-13)


def test_epilogue_keeps_zero_rows():
    """Anchor rows of the linear branch are zero and stay zero."""
    O = np.zeros((1, 3, 4))
    y = orc.rmsnorm_gate(O, np.ones(4), np.zeros(O.shape), 1e-6)
    assert not y.any()


def test_epilogue_inputs_are_deterministic_per_head():
    cfg = inp.CONFIG_BY_NAME["tiny"]
    a, b = inp.epilogue_inputs(cfg, 0), inp.epilogue_inputs(cfg, 0)
    assert np.array_equal(a.gate, b.gate) and np.array_equal(a.weight, b.weight)
    c = inp.epilogue_inputs(cfg, 1) if cfg.heads > 1 else inp.epilogue_inputs(inp.scaled(cfg, seed=cfg.seed + 1), 0)
    assert not np.array_equal(a.gate, c.gate)
    assert a.gate.shape == (cfg.frames, cfg.tokens, cfg.d) and a.weight.shape == (cfg.d,)


# ------------------------------------------------------------ prep (f2) --

def test_prep_hand_worked_example():
    """(3, 4) normalises to (0.6, 0.8) with eps = 0; sigmoid(0) = 1/2 and
    sigmoid(log 3) = 3/4."""
    q, k, b, a, _, _ = orc.prep(np.array([[3.0, 4.0]]), np.array([[0.0, 2.0]]), np.array([0.0]),
                                np.array([np.log(3.0)]), eps=0.0)
    np.testing.assert_allclose(q, [[0.6, 0.8]], rtol=1e-15)
    np.testing.assert_allclose(k, [[0.0, 1.0]], rtol=1e-15)
    np.testing.assert_allclose(b, [0.5], rtol=1e-15)
    np.testing.assert_allclose(a, [0.75], rtol=1e-15)


def test_prep_norms_and_gate_ranges():
    g = np.random.default_rng(11)
    X = g.standard_normal((5, 7, 16)) * 3
    for eps in (0.0, 1e-6, 2.0):
        Y = orc.l2_normalise(X, eps)
        n2 = np.sum(X * X, axis=-1)
        np.testing.assert_allclose(np.sum(Y * Y, axis=-1), n2 / (n2 + eps), rtol=1e-13)
    z = g.standard_normal(100) * 5
    s = orc.sigmoid(z)
    assert np.all((s > 0) & (s < 1))
    np.testing.assert_allclose(s + orc.sigmoid(-z), 1.0, rtol=1e-15)


def test_prep_makes_the_branch_invariant_to_q_k_scale():
    """With normalisation (eps = 0), rescaling the raw q and k rows by any
    positive factors leaves the whole branch unchanged."""
    cfg = inp.CONFIG_BY_NAME["tiny"]
    h = inp.raw_head_inputs(cfg, 0)
    f = h.f64
    g = np.random.default_rng(12)
    cq = np.exp(g.standard_normal((cfg.frames, cfg.tokens, 1)))
    ck = np.exp(g.standard_normal((cfg.frames, cfg.tokens, 1)))
    ckt = np.exp(g.standard_normal((cfg.text_tokens, 1)))
    runs = []
    for sq, sk, skt in ((1.0, 1.0, 1.0), (cq, ck, ckt)):
        q, k, b, a, kt, bt = orc.prep(sq * f("q"), sk * f("k"), f("beta"), f("alpha"), skt * f("kt"), f("bt"),
                                      eps=0.0)
        runs.append(orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, q, k, f("v"), b, a, kt, f("vt"),
                                 bt)["O"])
    np.testing.assert_allclose(runs[1], runs[0], rtol=1e-10, atol=1e-12)


def test_raw_inputs_are_the_usual_draws_before_prep():
    """raw_head_inputs draws the same numbers as head_inputs: after the
    oracle's prep (eps = 0) the gates match to float32 rounding and the
    normalised keys match the stored unit keys to their rounding."""
    cfg = inp.CONFIG_BY_NAME["tiny"]
    raw, ref = inp.raw_head_inputs(cfg, 0), inp.head_inputs(cfg, 0)
    _, _, b, a, _, bt = orc.prep(raw.f64("q"), raw.f64("k"), raw.f64("beta"), raw.f64("alpha"),
                                 raw.f64("kt"), raw.f64("bt"), eps=0.0)
    np.testing.assert_allclose(b, ref.f64("beta"), rtol=1e-6)
    np.testing.assert_allclose(a, ref.f64("alpha"), rtol=1e-6)
    np.testing.assert_allclose(bt, ref.f64("bt"), rtol=1e-6)


# ------------------------------------------------------ softmax branch (f3) --

def test_softmax_key_frames_match_hand_derived_tiny_table():
    table = {}
    with open(os.path.join(GOLDEN, "tiny_softmax_keys.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            xs = [int(x) for x in line.split()]
            table[xs[0]] = xs[1:]
    keys = orc.softmax_key_frames(22, 5, 1, 1)
    assert len(keys) == 22
    for t in range(22):
        assert keys[t] == table[t], t


def test_softmax_key_frames_without_anchors_and_wide_window():
    """No anchors: every frame is a query of some chunk and nothing is seen
    globally; a window wider than the sequence sees every frame."""
    keys = orc.softmax_key_frames(20, 5, 0, 0)
    assert keys[0] == list(range(5)) and keys[19] == list(range(15, 20))
    keys = orc.softmax_key_frames(22, 5, 9, 1)
    assert all(kf == list(range(22)) for kf in keys)


def test_softmax_branch_uniform_scores_average_the_visible_values():
    """q = 0 makes every score equal, so each output is the plain mean of the
    visible values; with v = the key's frame number (and text v = -1) that
    mean is fixed by the key sets: chunk 0 of the tiny layout sees frames
    {0, ..., 10, 21} with 2 tokens each and 3 text tokens."""
    T, U, d = 22, 2, 4
    q = np.zeros((T, U, d))
    k = np.random.default_rng(3).standard_normal((T, U, d))
    v = np.broadcast_to(np.arange(T, dtype=np.float64)[:, None, None], (T, U, d)).copy()
    kt = np.random.default_rng(4).standard_normal((3, d))
    vt = -np.ones((3, d))
    O = orc.softmax_branch(q, k, v, kt, vt, T, 5, 1, 1)
    expect = (2 * (sum(range(11)) + 21) - 3) / (2 * 12 + 3)
    np.testing.assert_allclose(O[1], expect, rtol=1e-14)
    expect_anchor = (2 * sum(range(22)) - 3) / (2 * 22 + 3)
    np.testing.assert_allclose(O[0], expect_anchor, rtol=1e-14)


def test_softmax_branch_dominant_key_and_shift_invariance():
    """A key far more aligned with the query than the others takes all the
    weight; adding one vector c to every key (video and text) shifts all
    scores of a query by the same q.c and leaves the output unchanged."""
    g = np.random.default_rng(5)
    T, U, d = 7, 3, 8
    q = g.standard_normal((T, U, d))
    k = g.standard_normal((T, U, d)) * 0.01
    v = g.standard_normal((T, U, d))
    k[3, 1] = 500 * q[4, 0] / np.linalg.norm(q[4, 0])   # frame 3 is in frame 4's window (chunk 0)
    O = orc.softmax_branch(q, k, v, None, None, T, 5, 1, 1)
    np.testing.assert_allclose(O[4, 0], v[3, 1], rtol=1e-9)
    k = g.standard_normal((T, U, d))
    kt, vt = g.standard_normal((4, d)), g.standard_normal((4, d))
    c = g.standard_normal(d)
    O1 = orc.softmax_branch(q, k, v, kt, vt, T, 5, 1, 1)
    O2 = orc.softmax_branch(q, k + c, v, kt + c, vt, T, 5, 1, 1)
    np.testing.assert_allclose(O2, O1, rtol=1e-10, atol=1e-12)


# ------------------------------------------- variants: SANA-WM and Newton --

def test_sana_wm_single_token_hand_worked():
    """One token, key scale 1 (U = 1): the explicit token delta rule.
    S_prev = [[1, 2], [3, 4]], alpha = (1/2, 1), k = (1, 0), v = (1, 1),
    beta = 1/2: S_bar = [[1/2, 2], [3/2, 4]], S_bar k = (1/2, 3/2), the
    residual is (1/2, -1/2), so S = [[3/4, 2], [5/4, 4]]."""
    S = orc.sana_wm_update(np.array([[1.0, 2.0], [3.0, 4.0]]), np.array([[1.0, 0.0]]),
                           np.array([[1.0, 1.0]]), np.array([0.5]), np.array([0.5, 1.0]))
    assert np.array_equal(S, np.array([[0.75, 2.0], [1.25, 4.0]]))


def test_sana_wm_frame_size_key_scale_hand_worked():
    """Four copies of one token at the default key scale 1/sqrt(4) = 1/2:
    k' = (1/2, 0), S_bar = [[1/2, 2], [3/2, 4]] as above, beta = 1/2.  Each
    residual is v - S_bar k' = (1, 1) - (1/4, 3/4) = (3/4, 1/4); the four
    corrections sum to 4 * 1/2 * (3/4, 1/4) k'^T, i.e. (3/4, 1/4) in the
    first column: S = [[5/4, 2], [7/4, 4]]."""
    K = np.tile([1.0, 0.0], (4, 1))
    V = np.tile([1.0, 1.0], (4, 1))
    S = orc.sana_wm_update(np.array([[1.0, 2.0], [3.0, 4.0]]), K, V, np.full(4, 0.5), np.array([0.5, 1.0]))
    assert np.array_equal(S, np.array([[1.25, 2.0], [1.75, 4.0]]))


def test_sana_wm_orthonormal_keys_and_pure_decay():
    """Orthonormal keys at key scale 1: each key direction moves to
    (1 - beta_u) S_bar k_u + beta_u v_u independently; beta = 0 is decay."""
    g = np.random.default_rng(31)
    d = 6
    Q, _ = np.linalg.qr(g.standard_normal((d, d)))
    K = Q.T                                   # rows are orthonormal keys
    V = g.standard_normal((d, d))
    beta = g.random(d)
    alpha = 0.9 + 0.1 * g.random(d)
    S_prev = g.standard_normal((d, d))
    S = orc.sana_wm_update(S_prev, K, V, beta, alpha, key_scale=1.0)
    S_bar = S_prev * alpha[None, :]
    for u in range(d):
        expect = (1 - beta[u]) * (S_bar @ K[u]) + beta[u] * V[u]
        assert np.abs(S @ K[u] - expect).max() <= 1e-13
    S0 = orc.sana_wm_update(S_prev, K, V, np.zeros(d), alpha)
    assert np.abs(S0 - S_bar).max() == 0.0


def test_sana_wm_expands_where_vda_does_not():
    """Ten aligned tokens with beta = 1/2 at key scale 1 give
    lambda_max(A) = 5 > 2: the additive transition I - A maps the key
    direction to -4 times itself, so the inherited state grows four-fold
    (核心方法 para 2); the VDA write of the same frame does not expand.
    With the frame-size scale 1/sqrt(U) and beta < 1 the additive update is
    non-expansive too."""
    g = np.random.default_rng(32)
    d, U = 8, 10
    k = _unit(g, (d,))
    K = np.tile(k, (U, 1))
    V = np.zeros((U, d))
    beta = np.full(U, 0.5)
    S_prev = np.outer(g.standard_normal(d), k)  # inherited state along k
    one = np.ones(d)
    S_sana = orc.sana_wm_update(S_prev, K, V, beta, one, key_scale=1.0)
    assert np.linalg.norm(S_sana, 2) == pytest.approx(4.0 * np.linalg.norm(S_prev, 2), rel=1e-12)
    S_vda = orc.frame_update(S_prev, K, V, beta, one)
    assert np.linalg.norm(S_vda, 2) <= np.linalg.norm(S_prev, 2)
    for trial in range(20):
        S_prev, K, _, beta, alpha = _frame(g, 64, 16)
        S = orc.sana_wm_update(S_prev, K, np.zeros((64, 16)), beta, alpha)
        assert np.linalg.norm(S, 2) <= np.linalg.norm(S_prev * alpha[None, :], 2) * (1 + 1e-12)


def test_sana_wm_branch_runs_the_additive_rule_everywhere():
    """run_head(update="sana") applies the additive rule to the text write
    and to every scanned frame; with beta = 0 on the video both rules give
    the same (pure decay) states from their own text state."""
    q, k, v, beta, alpha, kt, vt, bt = _small_cfg_inputs(T=12)
    r = orc.run_head(12, 5, 1, 1, q, k, v, np.zeros_like(beta), alpha, kt, vt, bt, update="sana")
    ST = orc.sana_wm_update(np.zeros((8, 8)), kt, vt, bt, np.ones(8))
    assert np.abs(r["S_text"] - ST).max() == 0.0
    decay = np.prod(alpha[1:6], axis=0)
    assert np.abs(r["states_f"][1] - 0.5 * ST * decay[None, :]).max() <= 1e-15


def test_newton_schulz_hand_worked():
    """G = diag(1, 3): g = 3, c = 1/2, r = 1/2; X_1 = diag(3/4, 1/4),
    X_2 = diag(15/16, 5/16); a tolerance of 0.1 needs k = 2 (r^4 = 1/16)."""
    X, k = orc.newton_schulz_inverse(np.diag([1.0, 3.0]), tol=0.1)
    assert k == 2
    assert np.array_equal(X, np.diag([15 / 16, 5 / 16]))


def test_newton_schulz_residual_is_a_power_of_the_start():
    """From X_0 = c I the residual I - G X_k equals (I - c G)^(2^k), checked
    through the eigendecomposition of G; it is within the tolerance, and
    one step fewer would not be."""
    g = np.random.default_rng(33)
    for U, d in ((40, 16), (300, 32)):
        _, K, _, beta, _ = _frame(g, U, d)
        G = np.eye(d) + K.T @ (beta[:, None] * K)
        tol = 1e-6
        X, k = orc.newton_schulz_inverse(G, tol=tol)
        gmax = np.abs(G).sum(axis=1).max()
        c = 2 / (1 + gmax)
        lam, Q = np.linalg.eigh(G)
        R = (Q * (1 - c * lam) ** (2 ** k)) @ Q.T
        assert np.abs((np.eye(d) - G @ X) - R).max() <= 1e-12
        r = (gmax - 1) / (gmax + 1)
        assert np.linalg.norm(np.eye(d) - G @ X, 2) <= r ** (2 ** k) * (1 + 1e-9) + 1e-12
        assert r ** (2 ** k) <= tol < r ** (2 ** (k - 1))
        assert np.abs(X - X.T).max() <= 1e-12


# ------------------------------------------------- the comparison and scale --

def test_rel_l2_hand_values():
    """The measure every parity test uses: ||x - ref|| / ||ref||, with both
    norms over all elements.  ref = (3, 4), x = (3, 5): |x - ref| = 1 and
    |ref| = 5, so 0.2; swapping the roles gives 1 / sqrt(34)."""
    assert orc.rel_l2(np.array([3.0, 5.0]), np.array([3.0, 4.0])) == pytest.approx(0.2, rel=1e-15)
    assert orc.rel_l2(np.array([3.0, 4.0]), np.array([3.0, 5.0])) == pytest.approx(1 / np.sqrt(34), rel=1e-15)
    assert orc.rel_l2(np.array([3.0, 4.0]), np.array([3.0, 4.0])) == 0.0


def test_rel_l2_runs_over_every_axis():
    """A 2 x 3 x 4 reference of ones has norm sqrt(24); one element off by
    0.5 gives 0.5 / sqrt(24) wherever it sits (a norm per row or per slice,
    or a ravel of one axis only, would give another value), and a uniform
    relative error e of every element gives e."""
    ref = np.ones((2, 3, 4))
    for idx in [(0, 0, 0), (1, 2, 3), (1, 0, 2)]:
        x = ref.copy()
        x[idx] += 0.5
        assert orc.rel_l2(x, ref) == pytest.approx(0.5 / np.sqrt(24), rel=1e-14)
    g = np.random.default_rng(9)
    ref = g.standard_normal((3, 5, 7))
    assert orc.rel_l2(ref * (1 + 3e-4), ref) == pytest.approx(3e-4, rel=1e-9)
    assert orc.rel_l2(-ref, ref) == pytest.approx(2.0, rel=1e-14)


def test_rel_l2_zero_reference_and_dtypes():
    """A zero reference leaves the absolute norm; 16-bit and integer inputs
    are compared in float64."""
    assert orc.rel_l2(np.array([0.0, 3.0, 4.0]), np.zeros(3)) == pytest.approx(5.0, rel=1e-15)
    assert orc.rel_l2(np.array([3, 5], dtype=np.int32), np.array([3.0, 4.0], dtype=np.float16)) \
        == pytest.approx(0.2, rel=1e-15)


def _two_key_case():
    """One frame (no anchors, one chunk) of two tokens in d = 2: keys (1, 0)
    and (0, 0), values (1, 0) and (0, 1); query 0 is (1, 0), query 1 is 0."""
    q = np.array([[[1.0, 0.0], [0.0, 0.0]]])
    k = np.array([[[1.0, 0.0], [0.0, 0.0]]])
    v = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    return q, k, v


@pytest.mark.parametrize("scale", [2.0, 0.5, None])
def test_softmax_branch_scale_hand_worked(scale):
    """Query 0 scores s = scale * (1, 0).(1, 0) against key 0 and 0 against
    key 1, so its weights are e^s / (1 + e^s) and 1 / (1 + e^s) and its
    output is that pair (the values are the unit vectors); query 1 scores 0
    against both and averages them.  The default scale is 1 / sqrt(d) =
    1 / sqrt(2).  Dropping, squaring or inverting the scale changes
    query 0's output."""
    q, k, v = _two_key_case()
    O = orc.softmax_branch(q, k, v, None, None, 1, 1, 0, 0, scale)
    s = 1 / np.sqrt(2) if scale is None else scale
    w = np.exp(s) / (1 + np.exp(s))
    np.testing.assert_allclose(O[0, 0], [w, 1 - w], rtol=1e-14)
    np.testing.assert_allclose(O[0, 1], [0.5, 0.5], rtol=1e-14)
    for wrong in (1.0, s * s, 1 / s):
        wx = np.exp(wrong) / (1 + np.exp(wrong))
        assert abs(wx - w) > 1e-3


def test_softmax_branch_text_tokens_join_the_softmax():
    """Adding one text token with key (1, 0) and value (0, 0) to the same
    frame: query 0 now weighs e^s, 1, e^s over keys 0, 1 and the text key,
    so its output is (e^s, 1) / (2 e^s + 1)."""
    q, k, v = _two_key_case()
    s = 0.75
    O = orc.softmax_branch(q, k, v, np.array([[1.0, 0.0]]), np.array([[0.0, 0.0]]), 1, 1, 0, 0, s)
    np.testing.assert_allclose(O[0, 0], np.array([np.exp(s), 1.0]) / (2 * np.exp(s) + 1), rtol=1e-14)


def test_softmax_branch_query_frame_subset():
    """Computing only some query frames gives exactly those rows of the full
    result and zeros elsewhere."""
    g = np.random.default_rng(12)
    T, U, d = 12, 3, 8
    q, k, v = (g.standard_normal((T, U, d)) for _ in range(3))
    kt, vt = g.standard_normal((2, d)), g.standard_normal((2, d))
    full = orc.softmax_branch(q, k, v, kt, vt, T, 5, 1, 1)
    part = orc.softmax_branch(q, k, v, kt, vt, T, 5, 1, 1, query_frames=[0, 4, 11])
    for t in range(T):
        if t in (0, 4, 11):
            assert np.array_equal(part[t], full[t])
        else:
            assert not part[t].any()
