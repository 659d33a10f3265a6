"""GPU parity of the fp8-probability anchor (hla_softmax_anchor_fp8p_fwd).

The call rounds the softmax probabilities to OCP e4m3 before the P V product
(quantized inference: ai-papers.net summary, training and limitations sections,
which report quantization-aware training without a number format). Its error
against the fp64 oracle is therefore not the bf16 bar's; it is bounded per
output element as derived here.

Rounding. The kernel forms P_i = 2^(c s_i - m) with m its running row maximum,
which never exceeds the true row maximum M, so P_i = p_i 2^gamma with p_i the
probability relative to the true maximum (p_max = 1) and gamma >= 0; P_i <= 2^8.
e4m3 keeps 3 fraction bits: round to nearest even moves a normal value (>= 2^-6)
by at most 2^-4 of itself and a smaller one by at most 2^-10 (half the 2^-9
subnormal spacing; a value below 2^-10 rounds to 0 and moves by itself). In
units of p the error h_i is thus at most max(2^-4 p_i, min(p_i, 2^-10)) for
every gamma >= 0, and the same holds for each key-range piece of a split block
(its own maximum is below M).

Propagation. With rounded weights p~ the result is O~ = sum p~_i v_i / sum p~_i,
and exactly O~ - O = sum_i (p~_i - p_i)(v_i - O) / sum p~_i. Hence
  worst case:  |O~_d - O_d| <= sum_i h_i |v_id - O_d| / L,
  L = max(sum p - sum h, (1 - 2^-4) sum_{p_i >= 2^-6} p_i) <= sum p~;
and, the roundings of different keys being independent and zero-mean (their
values are continuous draws), the error has standard deviation at most
  sigma_d = sqrt(sum_i h_i^2 (v_id - O_d)^2 / 3) / L
(a uniform rounding error of half-width h has variance h^2 / 3). The test bound
per element is min(worst case, 6 sigma_d) times the gate, plus 2^-8 of the
reference (the bf16 output rounding and the fp32 sums) and 1e-4 of the slab's
largest reference value.

The first test pins the rounding itself: the kernels' own fp32 -> e4m3 helper
(run through the probe library) against round-to-nearest-even on the e4m3
value table, which the fp8 decode test pins to the format's definition.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as hla
from hla_inputs import BY_NAME, custom, layer_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FP8 = torch.float8_e4m3fn
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
U8 = 2.0 ** -4       # e4m3 rounding of a normal value, relative
H8 = 2.0 ** -10      # half the e4m3 subnormal spacing
NORMAL_MIN = 2.0 ** -6


def e4m3_table():
    """Values of the non-negative finite e4m3 codes 0x00 .. 0x7e, by the format's
    definition (bias 7, subnormals m/8 * 2^-6)."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


def rne_codes(x, table):
    """Round-to-nearest-even e4m3 codes of non-negative x <= 448."""
    i = np.clip(np.searchsorted(table, x), 1, len(table) - 1)
    lo, hi = i - 1, i
    dlo, dhi = x - table[lo], table[hi] - x
    even_lo = (lo % 2) == 0
    return np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(even_lo, lo, hi)))


def test_kernel_rounding_of_probabilities_is_round_to_nearest_even():
    lib = ctypes.CDLL(os.path.join(ROOT, "softmax_attention_amd", "libhla_probes.so"))
    assert len(hla.hip_runtimes_loaded()) == 1
    lib.hla_probe_cvt_fp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    table = e4m3_table()
    mids = (table[:-1] + table[1:]) / 2  # ties (exact in fp32)
    f32 = np.float32
    below = np.nextafter(mids.astype(f32), f32(0)).astype(np.float64)
    above = np.nextafter(mids.astype(f32), f32(1e9)).astype(np.float64)
    rng = np.random.default_rng(12000)
    rand = np.exp2(rng.uniform(-14, np.log2(448.0), 40000))
    x = np.concatenate([table, mids, below, above, rand, [0.0, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -10]])
    x = x.astype(f32)
    n4 = (len(x) + 3) // 4
    xin = np.zeros(4 * n4, dtype=f32)
    xin[:len(x)] = x
    xd = torch.from_numpy(xin).to(DEV)
    od = torch.zeros(n4, dtype=torch.int32, device=DEV)
    st = lib.hla_probe_cvt_fp8(ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(od.data_ptr()), n4,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    got = od.cpu().numpy().view(np.uint8)[:len(x)]
    want = rne_codes(x.astype(np.float64), table)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]
    # and torch's own cast agrees on these values
    assert np.array_equal(torch.from_numpy(x).to(FP8).view(torch.uint8).numpy(), want.astype(np.uint8))


def ref_and_bound(q, k, v, g, scale, rows):
    """fp64 reference sigma(G) O on `rows` and the per-element bound derived above."""
    qf, kf, vf, gf = (oracle.as_f64(t) for t in (q, k, v, g))
    W = oracle.softmax_probs(qf[..., rows, :], kf, scale)         # [B, H, M, N], rows sum to 1
    P = W / W.max(axis=-1, keepdims=True)                          # relative to the row maximum
    O = np.matmul(W, vf)                                           # [B, H, M, D]
    h = np.where(P >= NORMAL_MIN, U8 * P, np.minimum(P, H8))
    L = np.maximum(P.sum(-1) - h.sum(-1), (1 - U8) * np.where(P >= NORMAL_MIN, P, 0.0).sum(-1))
    assert np.all(L > 0)
    worst = np.empty_like(O)
    sigma = np.empty_like(O)
    B, H, M, _ = P.shape
    for b in range(B):
        for hh in range(H):
            for m in range(M):
                dv = np.abs(vf[b, hh] - O[b, hh, m])               # [N, D]
                worst[b, hh, m] = h[b, hh, m] @ dv
                sigma[b, hh, m] = np.sqrt((h[b, hh, m] ** 2) @ (dv ** 2) / 3)
    gate = 1 / (1 + np.exp(-gf[..., rows, :]))
    ref = gate * O
    bound = gate * np.minimum(worst, 6 * sigma) / L[..., None]
    slab = np.abs(ref).max(axis=(-1, -2), keepdims=True)
    return ref, bound + 2.0 ** -8 * np.abs(ref) + 1e-4 * slab


def run_fp8p(q, k, v, g, out_dtype=torch.bfloat16, accumulate=False, out=None):
    qd, kd, vd, gd = (t.contiguous().to(DEV) for t in (q, k, v, g))
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    hla.hla_softmax_anchor_fp8p_fwd(qd, kd, vd, gd, out=out, accumulate=accumulate)
    torch.cuda.synchronize()
    return out


def check(got, q, k, v, g, rows, tag, base=None):
    D = q.shape[-1]
    ref, bound = ref_and_bound(q, k, v, g, D ** -0.5, rows)
    gotr = oracle.as_f64(got.float().cpu())[..., rows, :]
    if base is not None:
        gotr = gotr - oracle.as_f64(base)[..., rows, :]
    err = np.abs(gotr - ref)
    ratio = float((err / bound).max())
    rel = oracle.max_rel_error(gotr, ref)
    print(f"[fp8p {tag}] max err/bound {ratio:.3f}, max rel err {rel:.3e}", flush=True)
    assert np.all(np.isfinite(gotr))
    assert np.all(err <= bound), (ratio, np.unravel_index(int(np.argmax(err / bound)), err.shape))
    return rel


def block_edge_rows(N):
    r = [0, N - 1]
    for qb in range(0, N, 256):
        r += [qb, min(N - 1, qb + 255)]
    return np.unique(np.array(r))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 257, 1000])
def test_fp8p_tails(N, D, out_dtype):
    q, k, v, g = custom((1, 2, N, D), 12100 + N + D, FP8, n=4)
    got = run_fp8p(q, k, v, g, out_dtype=out_dtype)
    assert got.dtype == out_dtype
    check(got, q, k, v, g, np.arange(N), f"N={N} D={D} {out_dtype}")


def test_fp8p_split_and_accumulate():
    # few query blocks: the last batch is split along the keys and combined
    B, H, N, D = 1, 3, 2000, 128
    q, k, v, g = custom((B, H, N, D), 12200, FP8, n=4)
    rows = np.unique(np.r_[np.arange(0, N, 5), block_edge_rows(N)])
    check(run_fp8p(q, k, v, g), q, k, v, g, rows, "split")
    base = custom((B, H, N, D), 12300, torch.float32, n=1)[0]
    acc = base.to(DEV)
    run_fp8p(q, k, v, g, accumulate=True, out=acc)
    check(acc, q, k, v, g, rows, "split, += fp32", base=base)


@pytest.mark.parametrize("shape,out_dtype", [((4, 16, 2000, 64), torch.bfloat16),
                                             ((1, 16, 4096, 128), torch.float32),
                                             ((1, 16, 4090, 128), torch.bfloat16)])
def test_fp8p_unsplit_workgroups(shape, out_dtype):
    # at least one query block per CU: whole workgroups over many key tiles
    B, H, N, D = shape
    if B * H * -(-N // 256) < torch.cuda.get_device_properties(0).multi_processor_count:
        pytest.skip("fewer query blocks than CUs on this device")
    q, k, v, g = custom(shape, 12400 + N + D, FP8, n=4)
    got = run_fp8p(q, k, v, g, out_dtype=out_dtype)
    rows = block_edge_rows(N)
    sl = (slice(0, 1), slice(H - 1, H))  # one head of the last batch entry, sampled rows
    check(got[sl], q[sl], k[sl], v[sl], g[sl], rows, f"unsplit {shape}")


def test_fp8p_peaky_logits():
    # scores four times larger: probabilities span many octaves, many fall
    # below the e4m3 normal range
    q, k, v, g = custom((1, 2, 700, 128), 12500, torch.float32, n=4)
    q8, k8, v8, g8 = ((q * 4).to(FP8), k.to(FP8), v.to(FP8), g.to(FP8))
    check(run_fp8p(q8, k8, v8, g8), q8, k8, v8, g8, np.arange(700), "peaky")


def test_fp8p_720p_sampled():
    # the 720p workload at full size in the benchmark's configuration, checked on
    # sampled rows of the first and last head
    w = BY_NAME["720p_81f"]
    q, k, v, g = layer_inputs(w, 0, dtype=FP8)
    got = run_fp8p(q, k, v, g)
    rows = np.unique(np.r_[np.linspace(0, w.N - 1, 40).astype(int), block_edge_rows(w.N)[-4:]])
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rel = check(got[sl], q[sl], k[sl], v[sl], g[sl], rows, f"720p b={b} h={h}")
        assert rel <= 5e-2


def test_fp8p_same_as_bf16_probabilities_up_to_their_rounding():
    # the same fp8 inputs through the bf16-probability anchor: both within their
    # own bounds of the oracle, and the fp8-probability call's error is the larger
    q, k, v, g = custom((2, 2, 1500, 128), 12600, FP8, n=4)
    a = run_fp8p(q, k, v, g, out_dtype=torch.float32)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    b = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    hla.hla_softmax_anchor_fwd(qd, kd, vd, gd, out=b)
    torch.cuda.synchronize()
    rows = np.arange(0, 1500, 7)
    ea = check(a, q, k, v, g, rows, "vs bf16 P")
    ref = oracle.gated_softmax(q, k, v, g, 128 ** -0.5, rows=rows)
    eb = oracle.max_rel_error(b.cpu()[..., rows, :], ref)
    print(f"[fp8p vs bf16 P] rel err fp8 P {ea:.3e}, bf16 P {eb:.3e}", flush=True)
    assert eb <= 2e-2 and eb < ea


def test_fp8p_rejects_bf16_inputs():
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        hla.hla_softmax_anchor_fp8p_fwd(q, q, q, q)
