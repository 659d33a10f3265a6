"""Planted mistakes: each plausible error in the oracle must fail a pin (CPU only).

The mutants below are copies of the oracle's operators with one mistake each (a
dropped term, a wrong sign, a transposed operand, a wrong axis or scale). Every
mutant is run through the same independent checks the pins use -- pure-Python
brute force, exact special cases, torch's SDPA -- and at least one check must
reject it. This shows the pins are strong enough to catch such slips.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import brute_linear, brute_softmax, rand

sig = oracle.sigmoid
relu = oracle.relu


# --- linear mutants ---------------------------------------------------------

def lin_ok(q, k, v, g, eps):
    return oracle.gated_linear(q, k, v, g, eps)


def lin_no_eps(q, k, v, g, eps):
    return oracle.gated_linear(q, k, v, g, 0.0)


def lin_gate_sign(q, k, v, g, eps):
    return oracle.gated_linear(q, k, v, -g, eps)


def lin_state_transposed(q, k, v, g, eps):
    S = np.swapaxes(v, -1, -2) @ relu(k)   # S^T where S belongs
    z = relu(k).sum(-2)
    phq = relu(q)
    return sig(g) * (phq @ S) / ((phq @ z[..., None]) + eps)


def lin_z_wrong_axis(q, k, v, g, eps):
    S = np.swapaxes(relu(k), -1, -2) @ v
    z = relu(k).sum(-1).mean(-1, keepdims=True) * np.ones(k.shape[-1])
    phq = relu(q)
    return sig(g) * (phq @ S) / ((phq @ z[..., None]) + eps)


def lin_no_relu_on_q(q, k, v, g, eps):
    S = np.swapaxes(relu(k), -1, -2) @ v
    z = relu(k).sum(-2)
    return sig(g) * (q @ S) / ((q @ z[..., None]) + eps)


def lin_eps_in_numerator(q, k, v, g, eps):
    S = np.swapaxes(relu(k), -1, -2) @ v
    z = relu(k).sum(-2)
    phq = relu(q)
    return sig(g) * (phq @ S + eps) / ((phq @ z[..., None]) + eps)


# --- softmax mutants --------------------------------------------------------

def sm_ok(q, k, v, g, s):
    return oracle.gated_softmax(q, k, v, g, s)


def sm_no_scale(q, k, v, g, s):
    return oracle.gated_softmax(q, k, v, g, 1.0)


def sm_wrong_axis(q, k, v, g, s):
    L = s * q @ np.swapaxes(k, -1, -2)
    E = np.exp(L - L.max(-2, keepdims=True))
    return sig(g) * (E / E.sum(-2, keepdims=True)) @ v


def sm_no_max_sub(q, k, v, g, s):
    L = s * q @ np.swapaxes(k, -1, -2)
    with np.errstate(over="ignore", invalid="ignore"):
        E = np.exp(L)
        return sig(g) * (E / E.sum(-1, keepdims=True)) @ v


def sm_gate_before_pv(q, k, v, g, s):
    P = oracle.softmax_probs(q, k, s)
    return P @ (sig(g) * v)


def sm_transposed_v(q, k, v, g, s):
    P = oracle.softmax_probs(q, k, s)
    return sig(g) * (P @ np.swapaxes(v, -1, -2))


def sm_scale_sqrt_wrong(q, k, v, g, s):
    return oracle.gated_softmax(q, k, v, g, s * s)


# --- checks (the same independent references the pins use) -----------------

def linear_checks(f):
    fails = 0
    for (N, D, eps, seed) in [(9, 4, 0.3, 1), (16, 6, 1e-6, 2)]:
        q, k, v, g = (rand((N, D), 500 + seed * 10 + i) for i in range(4))
        try:
            got = f(q, k, v, g, eps)
            ref = np.array(brute_linear(q.tolist(), k.tolist(), v.tolist(), g.tolist(), eps))
            if got.shape != ref.shape or not np.allclose(got, ref, rtol=1e-10, atol=1e-12):
                fails += 1
        except Exception:
            fails += 1
    return fails


def softmax_checks(f):
    fails = 0
    for (N, D, s, mult, seed) in [(11, 4, 0.35, 1.0, 1), (16, 8, 0.2, 60.0, 2)]:
        q, k, v, g = (rand((1, 1, N, D), 600 + seed * 10 + i) for i in range(4))
        q = q * mult
        k = k * mult
        try:
            with np.errstate(all="ignore"):
                got = f(q, k, v, g, s)
            ref = np.array(brute_softmax(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), g[0, 0].tolist(), s))
            if got.shape[-2:] != ref.shape or not np.allclose(got[0, 0], ref, rtol=1e-10, atol=1e-12):
                fails += 1
        except Exception:
            fails += 1
    q, k, v = (rand((1, 2, 12, 8), 700 + i) for i in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=8 ** -0.5).numpy()
    try:
        got = f(q, k, v, np.full_like(q, np.inf), 8 ** -0.5)
        if not np.allclose(got, ref, rtol=1e-10, atol=1e-12):
            fails += 1
    except Exception:
        fails += 1
    return fails


def test_correct_oracle_passes_checks():
    assert linear_checks(lin_ok) == 0
    assert softmax_checks(sm_ok) == 0


@pytest.mark.parametrize("mutant", [lin_no_eps, lin_gate_sign, lin_state_transposed, lin_z_wrong_axis,
                                    lin_no_relu_on_q, lin_eps_in_numerator])
def test_linear_mutant_is_caught(mutant):
    # a mutant without eps divides 0 by 0 on all-zero feature rows: expected here
    with np.errstate(invalid="ignore", divide="ignore"):
        assert linear_checks(mutant) > 0, mutant.__name__


@pytest.mark.parametrize("mutant", [sm_no_scale, sm_wrong_axis, sm_no_max_sub, sm_gate_before_pv,
                                    sm_transposed_v, sm_scale_sqrt_wrong])
def test_softmax_mutant_is_caught(mutant):
    assert softmax_checks(mutant) > 0, mutant.__name__


# --- write-gated linear mutants -------------------------------------------------

from tests.test_oracle_pins import brute_linear_write  # noqa: E402


def wl_ok(q, k, v, g, w, eps):
    return oracle.gated_linear_write(q, k, v, g, w, eps)


def _wl(q, k, v, g, eps, bs, bz, bq=None):
    phk = relu(k)
    S = np.swapaxes(bs[..., :, None] * phk, -1, -2) @ v
    z = (bz[..., :, None] * phk).sum(-2)
    phq = relu(q) if bq is None else bq[..., :, None] * relu(q)
    return sig(g) * (phq @ S) / ((phq @ z[..., None]) + eps)


def wl_state_only(q, k, v, g, w, eps):       # beta in S, not in the normaliser
    return _wl(q, k, v, g, eps, sig(w), np.ones_like(w))


def wl_norm_only(q, k, v, g, w, eps):        # beta in the normaliser only
    return _wl(q, k, v, g, eps, np.ones_like(w), sig(w))


def wl_on_queries(q, k, v, g, w, eps):       # beta applied to the query rows
    return _wl(q, k, v, g, eps, np.ones_like(w), np.ones_like(w), sig(w))


def wl_no_sigmoid(q, k, v, g, w, eps):       # raw logits as strengths
    return _wl(q, k, v, g, eps, w, w)


def write_checks(f):
    fails = 0
    for (N, D, eps, seed) in [(9, 5, 0.3, 900), (20, 8, 1e-6, 910)]:
        q, k, v, g = (rand((1, 1, N, D), seed + i) for i in range(4))
        w = rand((1, 1, N), seed + 4, scale=2.0)
        try:
            with np.errstate(all="ignore"):
                got = f(q, k, v, g, w, eps)
            ref = np.array(brute_linear_write(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                              g[0, 0].tolist(), w[0, 0].tolist(), eps))
            if not np.allclose(got[0, 0], ref, rtol=1e-10, atol=1e-12):
                fails += 1
        except Exception:
            fails += 1
    return fails


def test_correct_write_gated_oracle_passes_checks():
    assert write_checks(wl_ok) == 0


@pytest.mark.parametrize("mutant", [wl_state_only, wl_norm_only, wl_on_queries, wl_no_sigmoid])
def test_write_gated_mutant_is_caught(mutant):
    assert write_checks(mutant) > 0, mutant.__name__


# --- block attention residual (routing) mutants -----------------------------

from tests.test_oracle_pins import brute_attnres  # noqa: E402


def _route(x, S, w, q_of=lambda x, w: x @ w, scale=True, axis=0, residual=True):
    D = x.shape[-1]
    St = np.stack(S)
    a = (q_of(x, w)[None] * St).sum(-1) / (np.sqrt(D) if scale else 1.0)
    a = a - a.max(axis=axis, keepdims=True)
    e = np.exp(a)
    al = e / e.sum(axis=axis, keepdims=True)
    r = (al[..., None] * St).sum(0)
    return x + r if residual else r


def ar_no_scale(x, S, w):
    return _route(x, S, w, scale=False)


def ar_router_transposed(x, S, w):
    return _route(x, S, w, q_of=lambda x, w: x @ w.T)


def ar_no_projection(x, S, w):
    return _route(x, S, w, q_of=lambda x, w: x)


def ar_softmax_over_tokens(x, S, w):
    return _route(x, S, w, axis=1)


def ar_no_residual(x, S, w):
    return _route(x, S, w, residual=False)


def attnres_checks(f):
    fails = 0
    for (N, D, M, seed) in [(6, 4, 3, 1), (9, 8, 2, 2)]:
        x = rand((N, D), 800 + seed * 10)
        w = rand((D, D), 801 + seed * 10, scale=0.7)
        S = [rand((N, D), 802 + seed * 10 + i) for i in range(M)]
        try:
            got = f(x, S, w)
            ref = np.array(brute_attnres(x.tolist(), [s.tolist() for s in S], w.tolist()))
            if got.shape != ref.shape or not np.allclose(got, ref, rtol=1e-10, atol=1e-12):
                fails += 1
        except Exception:
            fails += 1
    return fails


def test_correct_attnres_oracle_passes_checks():
    assert attnres_checks(oracle.attnres_route) == 0


@pytest.mark.parametrize("mutant", [ar_no_scale, ar_router_transposed, ar_no_projection,
                                     ar_softmax_over_tokens, ar_no_residual])
def test_attnres_mutant_is_caught(mutant):
    assert attnres_checks(mutant) > 0
