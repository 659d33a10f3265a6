"""Plain fp64 CPU oracle for SANA-Video 2.0's hybrid linear-softmax attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code with the HIP path.

What the pages state (SANA-Video 2.0, five web summaries of one paper):
  * the token mixer interleaves gated linear attention (O(N), a fixed-size state)
    with periodic gated-softmax "anchor" layers at a 3:1 ratio, every fourth layer
    being softmax (SANA-Video 2.0 abstract, thelatestinai.com listing; lode.cx
    article, "How It Works"; ai-papers.net summary, section on hybrid linear
    attention);
  * linear attention compresses the sequence into a fixed-size state matrix and
    costs O(N) (ai-papers.net summary, background section and hybrid linear
    attention section);
  * softmax anchors keep exact, full-rank token interactions (lode.cx article,
    "The Core Innovation").
The pages give no formula for either operator. The readings used here are:
  phi(x)   = max(x, 0)                         (ReLU feature map)
  sigma(x) = 1 / (1 + exp(-x))                 (sigmoid output gate, per channel)
  linear : S = phi(K)^T V, z = phi(K)^T 1,  O = sigma(G) * (phi(Q) S) / (phi(Q) z + eps)
  softmax: O = sigma(G) * softmax_rows(s Q K^T) V,  s = 1/sqrt(D), non-causal
  stack  : x_l = x_{l-1} + layer_l(Q_l, K_l, V_l, G_l), kinds L,L,L,S repeating
  write  : linear attention whose state takes beta_m = sigma(W_m) of each token's
           phi(K_m) (in S and in z), W one logit per token and head
  attnres: blocks of 8 layers; the summary of a completed block is its total
           update of the residual stream, s_i = x_end - x_start; a linear layer
           in a later block reads x + sum_i alpha_i s_i with, per token,
           alpha = softmax_i((x W) . s_i / sqrt(D)) and one router projection W
           shared by every layer (ai-papers.net summary, section on attention
           residuals: 8-layer blocks, block summaries routed to later linear
           layers, a depth-shared query router; lode.cx article and SANA-Video 2.0
           abstract: completed block summaries into later linear layers)
Every array is float64; bf16 or fp32 inputs are upcast exactly.
"""
from __future__ import annotations

import numpy as np

LINEAR = 0
SOFTMAX = 1


def as_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or CPU torch tensor to float64."""
    if hasattr(x, "detach"):  # torch tensor, without importing torch here
        x = x.detach().to("cpu")
        x = x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def relu(x: np.ndarray) -> np.ndarray:
    """Feature map phi(x) = max(x, 0), elementwise."""
    return np.maximum(x, 0.0)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic gate 1 / (1 + exp(-x)); exactly 0 at -inf and exactly 1 at +inf."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------
# gated linear attention (non-causal)
# ----------------------------------------------------------------------------

def linear_state(k, v):
    """Fixed-size per-head state of linear attention.

    S = phi(K)^T V  (D x D) and the normaliser z = sum_n phi(K_n) (D), over all N
    tokens; the "fixed-size state matrix" of the ai-papers.net summary (hybrid
    linear attention section). k, v: [..., N, D]. Returns S [..., D, D], z [..., D].
    """
    phk = relu(as_f64(k))
    v = as_f64(v)
    S = np.matmul(np.swapaxes(phk, -1, -2), v)
    z = phk.sum(axis=-2)
    return S, z


def linear_readout(q, g, S, z, eps: float):
    """Output rows of gated linear attention from its state (S, z).

    O_n = sigma(G_n) * (phi(Q_n) S) / (phi(Q_n) . z + eps); q, g: [..., R, D] (any
    R rows), S: [..., D, D], z: [..., D].
    """
    q = as_f64(q)
    g = as_f64(g)
    phq = relu(q)
    num = np.matmul(phq, as_f64(S))
    den = np.matmul(phq, as_f64(z)[..., :, None])[..., 0] + float(eps)
    return sigmoid(g) * num / den[..., None]


def gated_linear(q, k, v, g, eps: float):
    """Gated linear attention output O [..., N, D] in its O(N) (state) form.

    O_n = sigma(G_n) * (phi(Q_n) S) / (phi(Q_n) . z + eps)
    """
    S, z = linear_state(k, v)
    return linear_readout(q, g, S, z, eps)


def gated_linear_write(q, k, v, g, w, eps: float):
    """Gated linear attention with a write gate on the state (O(N) form).

    The ai-papers.net summary (section on hybrid linear attention) describes a
    gate that regulates how much each token writes into the fixed-size state;
    the pages give no formula. Reading used here: one write strength per token
    and head, beta_m = sigma(W_m), scales the token's key feature in both the
    state and the normaliser, so a token with beta = 0 is as if absent:
      S = sum_m beta_m phi(K_m)^T V_m,  z = sum_m beta_m phi(K_m)
      O_n = sigma(G_n) * (phi(Q_n) S) / (phi(Q_n) . z + eps)
    w: [..., N] (the gate logits W).
    """
    q = as_f64(q)
    g = as_f64(g)
    beta = sigmoid(as_f64(w))
    phk = beta[..., :, None] * relu(as_f64(k))
    S = np.matmul(np.swapaxes(phk, -1, -2), as_f64(v))
    z = phk.sum(axis=-2)
    phq = relu(q)
    num = np.matmul(phq, S)
    den = np.matmul(phq, z[..., :, None])[..., 0] + float(eps)
    return sigmoid(g) * num / den[..., None]


# ----------------------------------------------------------------------------
# gated softmax anchor (non-causal)
# ----------------------------------------------------------------------------

def softmax_probs(q_rows, k, scale: float):
    """Row-stochastic attention matrix P for a block of query rows.

    Exact two-pass softmax: logits, subtract each row's maximum, exponentiate,
    divide by the row sum. q_rows: [..., M, D], k: [..., N, D] -> P [..., M, N].
    """
    L = float(scale) * np.matmul(as_f64(q_rows), np.swapaxes(as_f64(k), -1, -2))
    L = L - L.max(axis=-1, keepdims=True)
    E = np.exp(L)
    return E / E.sum(axis=-1, keepdims=True)


def gated_softmax(q, k, v, g, scale: float, rows=None, block: int = 1024):
    """Gated softmax anchor O = sigma(G) * softmax(s Q K^T) V.

    q, k, v, g: [B, H, N, D]. ``rows`` (optional 1-D index array) restricts the
    output to those query rows, for spot checks at sizes where the full N x N
    product is too slow; the result then has shape [B, H, len(rows), D].
    Query rows are processed in blocks of ``block`` to bound memory.
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    g = as_f64(g)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[..., rows, :]
        g = g[..., rows, :]
    M = q.shape[-2]
    out = np.empty(q.shape[:-2] + (M, v.shape[-1]), dtype=np.float64)
    for r0 in range(0, M, block):
        r1 = min(M, r0 + block)
        P = softmax_probs(q[..., r0:r1, :], k, scale)
        out[..., r0:r1, :] = sigmoid(g[..., r0:r1, :]) * np.matmul(P, v)
    return out


# ----------------------------------------------------------------------------
# hybrid stack
# ----------------------------------------------------------------------------

def hybrid_kinds(n_layers: int, period: int = 4):
    """Layer kinds with a softmax anchor at every ``period``-th layer (1-based)."""
    return [SOFTMAX if (l + 1) % period == 0 else LINEAR for l in range(n_layers)]


def layer(kind: int, q, k, v, g, eps: float, scale: float):
    if kind == LINEAR:
        return gated_linear(q, k, v, g, eps)
    if kind == SOFTMAX:
        return gated_softmax(q, k, v, g, scale)
    raise ValueError(f"unknown layer kind {kind}")


def hybrid_stack(x0, layers, kinds, eps: float, scale: float):
    """Residual stack x_l = x_{l-1} + layer_l(Q_l, K_l, V_l, G_l); returns x_L.

    ``layers`` is a sequence of (q, k, v, g) per layer, ``kinds`` the layer kinds
    (LINEAR = 0, SOFTMAX = 1).
    """
    x = as_f64(x0).copy()
    for kind, (q, k, v, g) in zip(kinds, layers):
        x = x + layer(kind, q, k, v, g, eps, scale)
    return x


# ----------------------------------------------------------------------------
# block attention residuals (AttnRes)
# ----------------------------------------------------------------------------

ATTNRES_BLOCK = 8  # layers per block


def block_summary(x_start, x_end):
    """Summary of a completed block: what it added to the residual stream."""
    return as_f64(x_end) - as_f64(x_start)


def attnres_route(x, summaries, w):
    """Residual stream a later linear layer reads: x + sum_i alpha_i s_i.

    x: [..., N, D]; summaries: sequence of M arrays shaped like x (completed
    blocks, in any order); w: [D, D], the router projection shared across depth.
    Per token n: q = x_n W, a_i = q . s_i,n / sqrt(D), alpha = softmax over the
    M blocks. With no completed block the stream passes unchanged.
    """
    x = as_f64(x)
    if len(summaries) == 0:
        return x.copy()
    W = as_f64(w)
    D = x.shape[-1]
    S = np.stack([as_f64(si) for si in summaries])     # [M, ..., N, D]
    q = x @ W                                          # [..., N, D]
    a = (q[None] * S).sum(-1) / np.sqrt(D)             # [M, ..., N]
    a = a - a.max(axis=0, keepdims=True)
    e = np.exp(a)
    alpha = e / e.sum(axis=0, keepdims=True)
    return x + (alpha[..., None] * S).sum(0)


# ----------------------------------------------------------------------------
# error metric
# ----------------------------------------------------------------------------

def max_rel_error(got, ref, per_slab: bool = True) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i|, worst over the [b, h] slabs.

    NaN or Inf anywhere in ``got`` gives +inf.
    """
    got = as_f64(got)
    ref = as_f64(ref)
    if not np.all(np.isfinite(got)):
        return float("inf")
    if got.ndim < 3 or not per_slab:
        denom = np.max(np.abs(ref))
        return float(np.max(np.abs(got - ref)) / denom) if denom > 0 else float(np.max(np.abs(got - ref)))
    err = np.abs(got - ref).reshape(-1, *got.shape[-2:]).max(axis=(-1, -2))
    den = np.abs(ref).reshape(-1, *ref.shape[-2:]).max(axis=(-1, -2))
    den = np.where(den > 0, den, 1.0)
    return float(np.max(err / den))
