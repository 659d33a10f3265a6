"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what it pins. The pages print no worked example and no formula, so
the pins are: brute force on tiny inputs (pure Python loops), the quadratic closed
form of linear attention, exact rational arithmetic, textbook special cases,
invariants, and one independent library routine (torch's scaled_dot_product_attention
in float64 on the CPU).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from hla_inputs import WORKLOADS, layer_inputs, custom

RNG_SEED = 1234


def rand(shape, seed=RNG_SEED, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ----------------------------------------------------------------------------
# pure-Python brute force: the per-token definitions, written with scalar loops
# ----------------------------------------------------------------------------

def _sig(x):
    if x == -math.inf:
        return 0.0
    if x == math.inf:
        return 1.0
    return 1.0 / (1.0 + math.exp(-x))


def brute_linear(q, k, v, g, eps):
    """O_n = sig(G_n) * sum_m w_nm V_m / (sum_m w_nm + eps), w_nm = phi(Q_n).phi(K_m)."""
    N, D = len(q), len(q[0])
    out = [[0.0] * D for _ in range(N)]
    for n in range(N):
        w = []
        for m in range(N):
            s = 0.0
            for d in range(D):
                s += max(q[n][d], 0.0) * max(k[m][d], 0.0)
            w.append(s)
        den = sum(w) + eps
        for j in range(D):
            num = 0.0
            for m in range(N):
                num += w[m] * v[m][j]
            out[n][j] = _sig(g[n][j]) * num / den
    return out


def brute_softmax(q, k, v, g, scale):
    """O_n = sig(G_n) * sum_m exp(l_nm - max) V_m / sum_m exp(l_nm - max), l = s Q_n.K_m."""
    N, M, D = len(q), len(k), len(q[0])
    out = [[0.0] * D for _ in range(N)]
    for n in range(N):
        logits = []
        for m in range(M):
            s = 0.0
            for d in range(D):
                s += q[n][d] * k[m][d]
            logits.append(scale * s)
        mx = max(logits)
        e = [math.exp(x - mx) for x in logits]
        tot = sum(e)
        for j in range(D):
            acc = 0.0
            for m in range(M):
                acc += e[m] * v[m][j]
            out[n][j] = _sig(g[n][j]) * acc / tot
    return out


def _close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / scale <= tol


# ----------------------------------------------------------------------------
# brute force on tiny inputs (P2)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N,D,eps", [(1, 4, 1e-6), (5, 3, 1e-6), (17, 8, 0.25), (64, 16, 1e-6)])
def test_linear_matches_brute_force(N, D, eps):
    q, k, v, g = (rand((N, D), RNG_SEED + i) for i in range(4))
    got = oracle.gated_linear(q, k, v, g, eps)
    ref = brute_linear(q.tolist(), k.tolist(), v.tolist(), g.tolist(), eps)
    assert _close(got, ref, 1e-12)


@pytest.mark.parametrize("N,D,scale", [(1, 4, 0.5), (7, 3, 1 / math.sqrt(3)), (33, 8, 0.125), (64, 16, 0.25)])
def test_softmax_matches_brute_force(N, D, scale):
    q, k, v, g = (rand((N, D), RNG_SEED + 10 + i) for i in range(4))
    got = oracle.gated_softmax(q[None, None], k[None, None], v[None, None], g[None, None], scale)[0, 0]
    ref = brute_softmax(q.tolist(), k.tolist(), v.tolist(), g.tolist(), scale)
    assert _close(got, ref, 1e-12)


def test_softmax_block_split_and_rows_subset():
    # the row-blocking and the rows= spot-check path compute the same rows
    B, H, N, D = 1, 2, 300, 8
    q, k, v, g = (rand((B, H, N, D), 77 + i) for i in range(4))
    full = oracle.gated_softmax(q, k, v, g, 0.3)
    small_blocks = oracle.gated_softmax(q, k, v, g, 0.3, block=7)
    rows = np.array([0, 5, 299, 128])
    sub = oracle.gated_softmax(q, k, v, g, 0.3, rows=rows)
    assert _close(small_blocks, full, 1e-13)
    assert _close(sub, full[..., rows, :], 1e-13)
    brute = brute_softmax(q[0, 1].tolist(), k[0, 1].tolist(), v[0, 1].tolist(), g[0, 1].tolist(), 0.3)
    assert _close(full[0, 1], brute, 1e-12)


# ----------------------------------------------------------------------------
# quadratic closed form of linear attention (P1)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N,D", [(256, 32), (1000, 64), (4096, 32)])
def test_linear_equals_quadratic_closed_form(N, D):
    q, k, v, g = (rand((2, N, D), 99 + i) for i in range(4))
    eps = 1e-6
    got = oracle.gated_linear(q, k, v, g, eps)
    A = np.maximum(q, 0) @ np.swapaxes(np.maximum(k, 0), -1, -2)   # N x N association
    ref = oracle.sigmoid(g) * (A @ v) / (A.sum(-1, keepdims=True) + eps)
    assert _close(got, ref, 1e-12)


def test_linear_closed_form_tiny_workload():
    w = WORKLOADS[0]
    q, k, v, g = layer_inputs(w, 0)
    got = oracle.gated_linear(q, k, v, g, w.eps)
    Q, K, V, G = (oracle.as_f64(t) for t in (q, k, v, g))
    A = np.maximum(Q, 0) @ np.swapaxes(np.maximum(K, 0), -1, -2)
    ref = oracle.sigmoid(G) * (A @ V) / (A.sum(-1, keepdims=True) + w.eps)
    assert got.shape == (1, 2, 256, 32)
    assert _close(got, ref, 1e-12)


# ----------------------------------------------------------------------------
# exact rational arithmetic (G = 0 gives sigma = 1/2 exactly)
# ----------------------------------------------------------------------------

def test_linear_exact_rational_example():
    # integer inputs, gate 0 (sigma = 1/2), eps = 1/4: every step is exact in Q.
    q = [[1, -2, 3], [0, 0, 0], [-1, 2, 1], [2, 1, -3]]
    k = [[2, 1, -1], [-3, 4, 2], [1, 0, 5], [0, -2, 1]]
    v = [[1, 2, 3], [-4, 5, 0], [2, -1, 7], [3, 3, -2]]
    eps = Fraction(1, 4)
    N, D = 4, 3
    exact = []
    for n in range(N):
        w = [sum(Fraction(max(q[n][d], 0) * max(k[m][d], 0)) for d in range(D)) for m in range(N)]
        den = sum(w) + eps
        exact.append([Fraction(1, 2) * sum(w[m] * v[m][j] for m in range(N)) / den for j in range(D)])
    z = np.zeros((N, D))
    got = oracle.gated_linear(np.array(q, float), np.array(k, float), np.array(v, float), z, float(eps))
    for n in range(N):
        for j in range(D):
            assert abs(got[n][j] - float(exact[n][j])) <= 1e-15 * max(1.0, abs(float(exact[n][j])))
    # a zero feature row (phi(Q_n) = 0) gives exactly 0, not 0/0
    assert np.all(got[1] == 0.0)


def test_softmax_two_key_closed_form():
    # D=1, s=1, q=1, keys ln3 and 0: weights 3/4 and 1/4; gate 0 halves the result.
    q = np.array([[[[1.0]]]])
    k = np.array([[[[math.log(3.0)], [0.0]]]])
    v = np.array([[[[8.0], [-4.0]]]])
    g = np.zeros_like(q)
    got = oracle.gated_softmax(q, k, v, g, 1.0)
    assert abs(got[0, 0, 0, 0] - 0.5 * (0.75 * 8.0 + 0.25 * -4.0)) <= 1e-15


def test_softmax_equal_logits_is_mean():
    # identical keys: every logit equal, P uniform, O = sigma(G) * mean(V)
    N, D = 50, 6
    q = rand((1, 1, N, D), 5)
    k = np.tile(rand((1, 1, 1, D), 6), (1, 1, N, 1))
    v = rand((1, 1, N, D), 7)
    g = rand((1, 1, N, D), 8)
    got = oracle.gated_softmax(q, k, v, g, 0.7)
    ref = oracle.sigmoid(g) * v.mean(axis=-2, keepdims=True)
    assert _close(got, ref, 1e-13)


# ----------------------------------------------------------------------------
# invariants (P3-P10)
# ----------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    q, k = rand((3, 40, 16), 1), rand((3, 70, 16), 2)
    P = oracle.softmax_probs(q, k, 0.25)
    assert P.shape == (3, 40, 70)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-12
    assert np.all(P >= 0)


def test_softmax_large_logits_no_overflow():
    # logits ~ 1e4: a softmax without max subtraction overflows to inf/nan
    q, k, v, g = (rand((1, 1, 20, 8), 30 + i) for i in range(4))
    got = oracle.gated_softmax(q * 300.0, k * 300.0, v, g, 1.0)
    assert np.all(np.isfinite(got))
    ref = brute_softmax((q[0, 0] * 300).tolist(), (k[0, 0] * 300).tolist(), v[0, 0].tolist(), g[0, 0].tolist(), 1.0)
    assert _close(got[0, 0], ref, 1e-12)


def test_constant_v():
    N, D = 80, 8
    q, k, g = (rand((1, 1, N, D), 40 + i) for i in range(3))
    c = rand((D,), 44)
    v = np.tile(c, (1, 1, N, 1))
    o_s = oracle.gated_softmax(q, k, v, g, 0.35)
    assert _close(o_s, oracle.sigmoid(g) * c, 1e-13)
    eps = 1e-3
    o_l = oracle.gated_linear(q, k, v, g, eps)
    r = np.maximum(q, 0) @ np.maximum(k, 0).sum(-2)[..., None]   # phi(Q_n) . z
    assert _close(o_l, oracle.sigmoid(g) * c * r / (r + eps), 1e-13)


@pytest.mark.parametrize("which", ["linear", "softmax"])
def test_gate_values(which):
    N, D = 33, 8
    q, k, v, g = (rand((1, 1, N, D), 50 + i) for i in range(4))

    def run(gate):
        if which == "linear":
            return oracle.gated_linear(q, k, v, gate, 1e-6)
        return oracle.gated_softmax(q, k, v, gate, 0.3)

    ungated = run(np.full_like(g, np.inf))
    closed = run(np.full_like(g, -np.inf))
    assert np.all(closed == 0.0)
    assert np.all(run(np.full_like(g, -1e4)) == 0.0)
    assert np.array_equal(run(np.zeros_like(g)), 0.5 * ungated)
    # ungated output is the plain (sigma = 1) operator
    if which == "linear":
        S, z = oracle.linear_state(k, v)
        phq = np.maximum(q, 0)
        ref = (phq @ S) / ((phq @ z[..., None]) + 1e-6)
    else:
        ref = oracle.softmax_probs(q, k, 0.3) @ v
    assert _close(ungated, ref, 1e-13)
    # and the gate is sigma(G), elementwise, not sigma(-G)
    assert _close(run(g), oracle.sigmoid(g) * ungated, 1e-13)
    assert np.all(oracle.sigmoid(np.array([2.0])) > 0.5)


def test_softmax_vs_torch_sdpa():
    # independent library routine, float64 on the CPU, gate at +inf (sigma = 1)
    B, H, N, D = 2, 3, 96, 16
    q, k, v = (rand((B, H, N, D), 60 + i) for i in range(3))
    for scale in (D ** -0.5, 0.05):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
        got = oracle.gated_softmax(q, k, v, np.full_like(q, np.inf), scale)
        assert _close(got, ref, 1e-12)


@pytest.mark.parametrize("which", ["linear", "softmax"])
def test_token_permutation(which):
    N, D = 45, 8
    q, k, v, g = (rand((1, 2, N, D), 70 + i) for i in range(4))
    f = (lambda *a: oracle.gated_linear(*a, 1e-6)) if which == "linear" else (lambda *a: oracle.gated_softmax(*a, 0.3))
    base = f(q, k, v, g)
    p = np.random.default_rng(3).permutation(N)
    # permuting keys and values together leaves O unchanged (non-causal, no positions)
    assert _close(f(q, k[..., p, :], v[..., p, :], g), base, 1e-12)
    # permuting queries and gates permutes O
    assert _close(f(q[..., p, :], k, v, g[..., p, :]), base[..., p, :], 1e-12)


def test_softmax_shift_and_single_key():
    N, D = 40, 8
    q, k, v, g = (rand((1, 1, N, D), 80 + i) for i in range(4))
    u = rand((D,), 85)
    base = oracle.gated_softmax(q, k, v, g, 0.4)
    assert _close(oracle.gated_softmax(q, k + u, v, g, 0.4), base, 1e-12)
    one = oracle.gated_softmax(q, k[..., :1, :], v[..., :1, :], g, 0.4)
    assert _close(one, oracle.sigmoid(g) * v[..., :1, :], 1e-14)


def test_linear_homogeneity():
    N, D = 60, 8
    q, k, v, g = (rand((1, 1, N, D), 90 + i) for i in range(4))
    base = oracle.gated_linear(q, k, v, g, 0.0)
    assert _close(oracle.gated_linear(3.5 * q, 0.25 * k, v, g, 0.0), base, 1e-12)
    # with eps > 0, rescaling changes the result only through eps
    b1 = oracle.gated_linear(q, k, v, g, 10.0)
    b2 = oracle.gated_linear(2.0 * q, 2.0 * k, v, g, 40.0)
    assert _close(b1, b2, 1e-12)


@pytest.mark.parametrize("which", ["linear", "softmax"])
def test_linearity_in_v(which):
    N, D = 50, 8
    q, k, v1, v2, g = (rand((1, 1, N, D), 100 + i) for i in range(5))
    f = (lambda v: oracle.gated_linear(q, k, v, g, 1e-6)) if which == "linear" else (lambda v: oracle.gated_softmax(q, k, v, g, 0.3))
    assert _close(f(v1 + 2.5 * v2), f(v1) + 2.5 * f(v2), 1e-12)


# ----------------------------------------------------------------------------
# hybrid stack (P11)
# ----------------------------------------------------------------------------

def test_hybrid_kinds_three_to_one():
    assert oracle.hybrid_kinds(8) == [0, 0, 0, 1, 0, 0, 0, 1]
    assert WORKLOADS[3].kinds == tuple(oracle.hybrid_kinds(8))


def test_stack_composition_brute_force():
    N, D, L = 24, 4, 8
    kinds = oracle.hybrid_kinds(L)
    x0 = rand((1, 1, N, D), 200)
    layers = [tuple(rand((1, 1, N, D), 300 + 10 * l + t) for t in range(4)) for l in range(L)]
    got = oracle.hybrid_stack(x0, layers, kinds, 1e-6, 0.5)
    x = x0[0, 0].tolist()
    for kind, (q, k, v, g) in zip(kinds, layers):
        a = [t[0, 0].tolist() for t in (q, k, v, g)]
        o = brute_linear(*a, 1e-6) if kind == 0 else brute_softmax(*a, 0.5)
        x = [[x[n][j] + o[n][j] for j in range(D)] for n in range(N)]
    assert _close(got[0, 0], x, 1e-12)
    # the anchors sit at layers 4 and 8: swapping the kinds changes the result
    swapped = oracle.hybrid_stack(x0, layers, [1 - kd for kd in kinds], 1e-6, 0.5)
    assert not _close(swapped, got, 1e-6)


# ----------------------------------------------------------------------------
# inputs and the error metric
# ----------------------------------------------------------------------------

def test_bf16_upcast_is_exact():
    t = custom((1000,), 5, torch.bfloat16, n=1)[0]
    a = oracle.as_f64(t)
    assert np.array_equal(a.astype(np.float32), t.float().numpy())


def test_max_rel_error_metric():
    ref = np.zeros((1, 2, 4, 4))
    ref[0, 0] = 2.0
    ref[0, 1] = 100.0
    got = ref.copy()
    got[0, 0, 0, 0] += 0.02      # 1e-2 of slab 0's max
    got[0, 1, 0, 0] += 0.5       # 5e-3 of slab 1's max
    assert abs(oracle.max_rel_error(got, ref) - 1e-2) < 1e-15
    got[0, 1, 1, 1] = np.nan
    assert oracle.max_rel_error(got, ref) == float("inf")


# ----------------------------------------------------------------------------
# write-gated linear attention (beta_m = sigma(W_m) on each token's phi(K_m))
# ----------------------------------------------------------------------------

def brute_linear_write(q, k, v, g, w, eps):
    """O_n = sig(G_n) * sum_m b_m a_nm V_m / (sum_m b_m a_nm + eps), a_nm = phi(Q_n).phi(K_m)."""
    N, D = len(q), len(q[0])
    out = [[0.0] * D for _ in range(N)]
    for n in range(N):
        a = []
        for m in range(N):
            s = 0.0
            for d in range(D):
                s += max(q[n][d], 0.0) * max(k[m][d], 0.0)
            a.append(_sig(w[m]) * s)
        den = sum(a) + eps
        for j in range(D):
            num = 0.0
            for m in range(N):
                num += a[m] * v[m][j]
            out[n][j] = _sig(g[n][j]) * num / den
    return out


@pytest.mark.parametrize("N,D,eps", [(1, 4, 1e-6), (9, 5, 0.3), (40, 16, 1e-6)])
def test_write_gated_linear_matches_brute_force(N, D, eps):
    q, k, v, g = (rand((N, D), seed=60 + i) for i in range(4))
    w = rand((N,), seed=64, scale=2.0)
    ref = brute_linear_write(q.tolist(), k.tolist(), v.tolist(), g.tolist(), w.tolist(), eps)
    assert _close(oracle.gated_linear_write(q, k, v, g, w, eps), ref)


def test_write_gate_open_is_plain_gated_linear():
    # W = +inf writes every token in full (beta = 1): the plain operator
    q, k, v, g = (rand((2, 3, 50, 8), seed=70 + i) for i in range(4))
    w = np.full((2, 3, 50), np.inf)
    assert np.array_equal(oracle.gated_linear_write(q, k, v, g, w, 1e-6),
                          oracle.gated_linear(q, k, v, g, 1e-6))


def test_write_gate_closed_removes_tokens():
    # W = -inf (beta = 0) for a token is the same as leaving its K, V out
    q, k, v, g = (rand((1, 2, 30, 8), seed=80 + i) for i in range(4))
    keep = np.arange(30) % 3 != 1
    w = np.where(keep, np.inf, -np.inf)[None, None, :].repeat(2, axis=1)
    got = oracle.gated_linear_write(q, k, v, g, w, 1e-6)
    # queries keep all rows; keys and values only the written tokens
    phq = np.maximum(q, 0.0)
    phk = np.maximum(k[..., keep, :], 0.0)
    S = np.swapaxes(phk, -1, -2) @ v[..., keep, :]
    z = phk.sum(axis=-2)
    ref = (1 / (1 + np.exp(-g))) * (phq @ S) / ((phq @ z[..., :, None]) + 1e-6)
    assert _close(got, ref)


def test_write_gate_common_strength_scales_eps():
    # one beta for every token cancels between state and normaliser except against
    # eps: the result equals the plain operator with eps / beta
    q, k, v, g = (rand((1, 1, 64, 16), seed=90 + i) for i in range(4))
    wl = 0.7
    beta = 1 / (1 + math.exp(-wl))
    got = oracle.gated_linear_write(q, k, v, g, np.full((1, 1, 64), wl), 0.05)
    assert _close(got, oracle.gated_linear(q, k, v, g, 0.05 / beta))


def test_write_gated_quadratic_closed_form():
    # O = sig(G) (A V) / (A 1 + eps) with A = phi(Q) diag(beta) phi(K)^T
    q, k, v, g = (rand((2, 2, 300, 32), seed=100 + i) for i in range(4))
    w = rand((2, 2, 300), seed=104, scale=3.0)
    beta = 1 / (1 + np.exp(-w))
    A = np.maximum(q, 0) @ (beta[..., :, None] * np.maximum(k, 0)).swapaxes(-1, -2)
    ref = (1 / (1 + np.exp(-g))) * (A @ v) / (A.sum(axis=-1, keepdims=True) + 1e-6)
    assert _close(oracle.gated_linear_write(q, k, v, g, w, 1e-6), ref, tol=1e-11)


# ----------------------------------------------------------------------------
# block attention residuals: routing completed block summaries
# ----------------------------------------------------------------------------

def brute_attnres(x, summaries, w):
    """Per token n: q_j = sum_k x_k W[k][j]; a_i = sum_j q_j s_i[j] / sqrt(D);
    alpha = softmax over the blocks i; returns x + sum_i alpha_i s_i."""
    N, D, M = len(x), len(x[0]), len(summaries)
    out = []
    for n in range(N):
        q = [sum(x[n][k] * w[k][j] for k in range(D)) for j in range(D)]
        a = [sum(q[j] * summaries[i][n][j] for j in range(D)) / math.sqrt(D) for i in range(M)]
        top = max(a)
        e = [math.exp(ai - top) for ai in a]
        tot = sum(e)
        out.append([x[n][j] + sum(e[i] / tot * summaries[i][n][j] for i in range(M))
                    for j in range(D)])
    return out


@pytest.mark.parametrize("N,D,M", [(1, 4, 1), (5, 6, 3), (12, 16, 4)])
def test_attnres_route_matches_brute_force(N, D, M):
    x = rand((N, D), seed=90)
    w = rand((D, D), seed=91, scale=0.5)
    S = [rand((N, D), seed=92 + i) for i in range(M)]
    ref = brute_attnres(x.tolist(), [s.tolist() for s in S], w.tolist())
    assert _close(oracle.attnres_route(x, S, w), ref)


def test_attnres_one_block_adds_its_summary():
    # a single completed block gets weight 1 whatever the router computes
    x, s = rand((2, 3, 20, 8), seed=100), rand((2, 3, 20, 8), seed=101)
    w = rand((8, 8), seed=102, scale=5.0)
    assert _close(oracle.attnres_route(x, [s], w), x + s, tol=1e-15)


def test_attnres_zero_router_averages_the_blocks():
    x = rand((1, 2, 15, 8), seed=110)
    S = [rand((1, 2, 15, 8), seed=111 + i) for i in range(3)]
    assert _close(oracle.attnres_route(x, S, np.zeros((8, 8))), x + sum(S) / 3, tol=1e-14)


def test_attnres_block_order_and_identical_blocks():
    x = rand((1, 1, 25, 8), seed=120)
    S = [rand((1, 1, 25, 8), seed=121 + i) for i in range(4)]
    w = rand((8, 8), seed=125)
    assert _close(oracle.attnres_route(x, S, w), oracle.attnres_route(x, S[::-1], w), tol=1e-14)
    assert _close(oracle.attnres_route(x, [S[0]] * 3, w), x + S[0], tol=1e-14)


def test_attnres_no_completed_block_passes_the_stream():
    x = rand((1, 2, 7, 8), seed=130)
    out = oracle.attnres_route(x, [], np.eye(8))
    assert np.array_equal(out, x)


def test_attnres_dominant_block_is_selected():
    # W = 100 I makes q = 100 x; a block equal to x scores 100|x|^2/sqrt(D), one
    # equal to -x the negative: the gap is hundreds, so softmax is one-hot in fp64
    x = rand((1, 1, 10, 8), seed=140) + 2.0
    out = oracle.attnres_route(x, [-x, x], 100.0 * np.eye(8))
    assert _close(out, 2.0 * x, tol=1e-15)


def test_block_summary_is_the_blocks_layer_sum():
    # the summary of one 8-layer block (3:1 kinds) equals the sum of its layers' outputs
    B, H, N, D = 1, 1, 12, 4
    kinds = oracle.hybrid_kinds(oracle.ATTNRES_BLOCK)
    layers = [tuple(rand((B, H, N, D), seed=150 + 4 * l + i) for i in range(4)) for l in range(8)]
    x0 = rand((B, H, N, D), seed=190)
    x8 = oracle.hybrid_stack(x0, layers, kinds, 1e-6, D ** -0.5)
    ref = [brute_linear(*(t[0, 0].tolist() for t in L), 1e-6) if kd == oracle.LINEAR else
           brute_softmax(*(t[0, 0].tolist() for t in L), D ** -0.5) for kd, L in zip(kinds, layers)]
    assert _close(oracle.block_summary(x0, x8)[0, 0], np.sum(np.array(ref), axis=0), tol=1e-12)


def test_linear_state_adds_over_token_chunks():
    # the state is a sum over tokens: chunked sums reproduce it (the large-N GPU
    # test builds its reference this way)
    k, v = rand((1, 2, 1000, 8), seed=200), rand((1, 2, 1000, 8), seed=201)
    S, z = oracle.linear_state(k, v)
    parts = [oracle.linear_state(k[..., a:a + 300, :], v[..., a:a + 300, :]) for a in range(0, 1000, 300)]
    assert _close(sum(p[0] for p in parts), S, tol=1e-13)
    assert _close(sum(p[1] for p in parts), z, tol=1e-13)
    q, g = rand((1, 2, 1000, 8), seed=202), rand((1, 2, 1000, 8), seed=203)
    rows = [0, 17, 999]
    assert _close(oracle.linear_readout(q[..., rows, :], g[..., rows, :], S, z, 1e-6),
                  oracle.gated_linear(q, k, v, g, 1e-6)[..., rows, :], tol=1e-14)
