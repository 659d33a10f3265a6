"""GPU parity: the HIP path against the fp64 oracle, element by element (MI355X).

Tolerances (metric: max |gpu - ref| / max |ref| per [b, h] slab, worst slab):
  bf16 inputs, fp32 accumulation : 2e-2
  fp8 inputs (converted exactly to bf16 in the kernels): 2e-2, against the
                                   oracle on the same fp8 values
  fp32 path                      : 1e-4
Any NaN/Inf fails. Small shapes span several tiles and ragged tails; the full
workload sizes run in the same launch configuration the benchmark times, with
the softmax anchor checked on sampled query rows that the oracle computes one
by one (the linear layer is checked in full: its oracle is O(N)).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as hla
from hla_inputs import WORKLOADS, BY_NAME, layer_inputs, residual_x0, custom

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
DEV = "cuda"
FP8 = torch.float8_e4m3fn


def out_dtype_for(dtype):
    return torch.bfloat16 if dtype == FP8 else dtype


def rel_err(got, ref):
    return oracle.max_rel_error(got.float().cpu(), ref)


def make(shape, seed, dtype):
    return custom(shape, seed, dtype, n=4)


def run_linear(q, k, v, g, eps=1e-6, out_dtype=None, accumulate=False, out=None):
    qd, kd, vd, gd = (t.contiguous().to(DEV) for t in (q, k, v, g))
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or out_dtype_for(q.dtype), device=DEV)
    hla.hla_linear_fwd(qd, kd, vd, gd, out=out, accumulate=accumulate, eps=eps)
    torch.cuda.synchronize()
    return out


def run_softmax(q, k, v, g, scale=None, out_dtype=None, accumulate=False, out=None):
    qd, kd, vd, gd = (t.contiguous().to(DEV) for t in (q, k, v, g))
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or out_dtype_for(q.dtype), device=DEV)
    hla.hla_softmax_anchor_fwd(qd, kd, vd, gd, out=out, accumulate=accumulate, scale=scale)
    torch.cuda.synchronize()
    return out


# ----------------------------------------------------------------------------
# small shapes: tiles and ragged tails
# ----------------------------------------------------------------------------

TAIL_N = [1, 2, 3, 63, 64, 65, 127, 128, 129, 255, 257, 1000]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("N", TAIL_N)
def test_linear_bf16_tails(N, D):
    q, k, v, g = make((1, 2, N, D), 1000 + N + D, torch.bfloat16)
    got = run_linear(q, k, v, g)
    ref = oracle.gated_linear(q, k, v, g, 1e-6)
    assert rel_err(got, ref) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("N", TAIL_N)
def test_softmax_bf16_tails(N, D):
    q, k, v, g = make((1, 2, N, D), 2000 + N + D, torch.bfloat16)
    got = run_softmax(q, k, v, g)
    ref = oracle.gated_softmax(q, k, v, g, D ** -0.5)
    assert rel_err(got, ref) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("N", [1, 33, 256, 1000])
def test_fp32_paths(N, D):
    q, k, v, g = make((2, 1, N, D), 3000 + N + D, torch.float32)
    lin = run_linear(q, k, v, g)
    assert rel_err(lin, oracle.gated_linear(q, k, v, g, 1e-6)) <= TOL[torch.float32]
    sm = run_softmax(q, k, v, g)
    assert rel_err(sm, oracle.gated_softmax(q, k, v, g, D ** -0.5)) <= TOL[torch.float32]


def test_tiny_workload_fp32():
    w = BY_NAME["tiny_f32"]
    q, k, v, g = layer_inputs(w, 0)
    assert rel_err(run_linear(q, k, v, g, w.eps), oracle.gated_linear(q, k, v, g, w.eps)) <= 1e-4
    assert rel_err(run_softmax(q, k, v, g, w.scale), oracle.gated_softmax(q, k, v, g, w.scale)) <= 1e-4


@pytest.mark.parametrize("op", ["linear", "softmax"])
def test_bf16_accumulate_into_fp32_and_bf16(op):
    N, D = 300, 128
    q, k, v, g = make((1, 3, N, D), 4000, torch.bfloat16)
    x0 = custom((1, 3, N, D), 4100, torch.float32, n=1)[0]
    ref = (oracle.gated_linear(q, k, v, g, 1e-6) if op == "linear"
           else oracle.gated_softmax(q, k, v, g, D ** -0.5))
    run = run_linear if op == "linear" else run_softmax
    x = x0.to(DEV)
    run(q, k, v, g, accumulate=True, out=x)
    # the residual update is checked on delta = x - x0 (x0 is far larger than O)
    assert rel_err(x.cpu() - x0, ref) <= 2e-2
    xb = x0.to(torch.bfloat16)
    y = xb.to(DEV)
    run(q, k, v, g, accumulate=True, out=y)
    assert rel_err(y.float(), oracle.as_f64(xb) + ref) <= 2e-2


# ----------------------------------------------------------------------------
# special values and invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("op", ["linear", "softmax"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gate_extremes(op, dtype):
    N, D = 200, 64
    q, k, v, g = make((1, 2, N, D), 5000, dtype)
    run = run_linear if op == "linear" else run_softmax
    closed = run(q, k, v, torch.full_like(g, -float("inf")))
    assert torch.all(closed == 0)
    assert torch.all(run(q, k, v, torch.full_like(g, -1e4)) == 0)
    full = run(q, k, v, torch.full_like(g, float("inf")))
    half = run(q, k, v, torch.zeros_like(g))
    assert torch.equal(half.float() * 2, full.float())


def test_linear_zero_feature_rows_give_zero():
    N, D = 130, 128
    q, k, v, g = make((1, 2, N, D), 5100, torch.bfloat16)
    q[:, :, ::7, :] = -q[:, :, ::7, :].abs()   # phi(Q_n) = 0 on every 7th token
    got = run_linear(q, k, v, g)
    assert torch.all(got[:, :, ::7, :] == 0)
    assert rel_err(got, oracle.gated_linear(q, k, v, g, 1e-6)) <= 2e-2


def test_linear_all_negative_keys():
    # phi(K) = 0: S = 0, z = 0, every output is 0 / eps = 0
    N, D = 100, 128
    q, k, v, g = make((1, 1, N, D), 5200, torch.bfloat16)
    got = run_linear(q, -k.abs(), v, g)
    assert torch.all(got == 0)


def test_softmax_constant_v_and_single_key():
    N, D = 333, 128
    q, k, v, g = make((1, 2, N, D), 5300, torch.bfloat16)
    c = v[:, :, :1, :].expand(-1, -1, N, -1).contiguous()
    got = run_softmax(q, k, c, g)
    ref = oracle.sigmoid(oracle.as_f64(g)) * oracle.as_f64(c)
    assert rel_err(got, ref) <= 2e-2
    one = run_softmax(q[:, :, :1], k[:, :, :1], v[:, :, :1], g[:, :, :1])
    ref1 = oracle.sigmoid(oracle.as_f64(g[:, :, :1])) * oracle.as_f64(v[:, :, :1])
    assert rel_err(one, ref1) <= 1e-2


def test_softmax_peaky_logits():
    # Q scaled x4: sharply peaked rows exercise the running-max updates
    N, D = 700, 128
    q, k, v, g = make((1, 2, N, D), 5400, torch.float32)
    q = (q * 4).to(torch.bfloat16)
    k, v, g = (t.to(torch.bfloat16) for t in (k, v, g))
    got = run_softmax(q, k, v, g)
    assert rel_err(got, oracle.gated_softmax(q, k, v, g, D ** -0.5)) <= 2e-2


@pytest.mark.parametrize("op", ["linear", "softmax"])
def test_deterministic_and_in_bounds(op):
    N, D = 517, 128
    q, k, v, g = (t.to(DEV) for t in make((2, 2, N, D), 5500, torch.bfloat16))
    n = q.numel()
    guard = 4096
    outs = []
    for _ in range(2):
        buf = torch.full((n + 2 * guard,), 7.0, dtype=torch.bfloat16, device=DEV)
        out = buf[guard:guard + n].view(q.shape)
        if op == "linear":
            hla.hla_linear_fwd(q, k, v, g, out=out)
        else:
            hla.hla_softmax_anchor_fwd(q, k, v, g, out=out)
        torch.cuda.synchronize()
        assert torch.all(buf[:guard] == 7.0) and torch.all(buf[guard + n:] == 7.0)
        outs.append(out.clone())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("dtype", [torch.bfloat16, FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 15, 17, 517])
def test_linear_output_rows_stay_in_bounds(N, D, dtype):
    """The output pass stores O in whole 1 KB runs of its 16-token groups; the
    rows of a partial last group past N are computed but never stored. Guard
    regions around `out` (NaN-filled) stay untouched, every element of `out` is
    written, and the result matches the oracle, for bf16 and fp32 outputs and
    for an fp32 stream the output is added into."""
    B, H = 1, 3
    q, k, v, g = make((B, H, N, D), 5600 + N + D, dtype)
    ref = oracle.gated_linear(q, k, v, g, 1e-6)
    n, guard = B * H * N * D, 4096
    for od in (torch.bfloat16, torch.float32):
        buf = torch.full((n + 2 * guard,), float("nan"), dtype=od, device=DEV)
        out = buf[guard:guard + n].view(B, H, N, D)
        run_linear(q, k, v, g, out=out)
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()
        assert not torch.isnan(out).any()
        assert rel_err(out, ref) <= TOL[torch.bfloat16]
    # accumulating into an fp32 stream: the previous values are read at the same
    # runs, so the guards stay NaN and every element is x0 + O
    x0 = custom((B, H, N, D), 5650 + N, torch.float32, n=1)[0]
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
    x = buf[guard:guard + n].view(B, H, N, D)
    x.copy_(x0.to(DEV))
    run_linear(q, k, v, g, out=x, accumulate=True)
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()
    assert rel_err(x.cpu() - x0, ref) <= TOL[torch.bfloat16]


def test_empty_sequence_is_a_no_op():
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    hla.hla_linear_fwd(q, q, q, q, out=torch.empty_like(q))
    hla.hla_softmax_anchor_fwd(q, q, q, q, out=torch.empty_like(q))
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# full workload sizes, in the benchmark's launch configuration
# ----------------------------------------------------------------------------

def sample_rows(N, count=40, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(N, count), replace=False).tolist())
    rows |= {0, N - 1, N - 2, (N // 128) * 128, max(0, (N // 128) * 128 - 1)}
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.parametrize("name", ["480p_81f", "720p_81f", "long_720p_193f"])
def test_full_workload(name):
    w = BY_NAME[name]
    q, k, v, g = layer_inputs(w, 0)
    print(f"[{name}] B={w.B} H={w.H} N={w.N} D={w.D}", flush=True)
    lin = run_linear(q, k, v, g, w.eps)
    ref = oracle.gated_linear(q, k, v, g, w.eps)
    e_lin = rel_err(lin, ref)
    del ref
    rows = sample_rows(w.N, seed=w.index)
    sm = run_softmax(q, k, v, g, w.scale)
    ref_s = oracle.gated_softmax(q, k, v, g, w.scale, rows=rows)
    e_sm = rel_err(sm[..., rows, :], ref_s)
    print(f"[{name}] linear err {e_lin:.3e}  softmax err {e_sm:.3e} on {len(rows)} rows", flush=True)
    assert e_lin <= 2e-2
    assert e_sm <= 2e-2


def test_hybrid_stack_small_full():
    # an 8-layer 3:1 stack at a size the oracle finishes quickly, checked in full
    B, H, N, D = 1, 4, 777, 128
    kinds = oracle.hybrid_kinds(8)
    layers = [make((B, H, N, D), 6000 + 10 * l, torch.bfloat16) for l in range(8)]
    x0 = custom((B, H, N, D), 6100, torch.float32, n=1)[0]
    x = x0.to(DEV)
    hla.hla_hybrid_stack_fwd(x, [tuple(t.to(DEV) for t in L) for L in layers], kinds)
    torch.cuda.synchronize()
    ref = oracle.hybrid_stack(x0, layers, kinds, 1e-6, D ** -0.5)
    assert rel_err(x.cpu() - x0, ref - oracle.as_f64(x0)) <= 2e-2


def test_hybrid_stack_workload_sampled():
    # the 8-layer 720p x 121-frame stack; delta = x8 - x0 on sampled rows
    w = BY_NAME["stack_720p_121f"]
    kinds = list(w.kinds)
    layers_cpu = [layer_inputs(w, l) for l in range(8)]
    x0 = residual_x0(w)
    x = x0.to(DEV)
    layers = [tuple(t.to(DEV) for t in L) for L in layers_cpu]
    hla.hla_hybrid_stack_fwd(x, layers, kinds, eps=w.eps, scale=w.scale)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, seed=4)
    delta = (x.cpu() - x0)[..., rows, :]
    ref = np.zeros(delta.shape)
    for kind, (q, k, v, g) in zip(kinds, layers_cpu):
        if kind == oracle.LINEAR:
            ref += oracle.gated_linear(q, k, v, g, w.eps)[..., rows, :]
        else:
            ref += oracle.gated_softmax(q, k, v, g, w.scale, rows=rows)
    e = rel_err(delta, ref)
    print(f"[stack] delta err {e:.3e}", flush=True)
    assert e <= 2e-2


def test_softmax_split_last_round_full():
    # 24 query blocks of 256 rows leave the last batch of workgroups incomplete,
    # so every block is split along the keys and merged by the combine kernel;
    # checked in full, plain and accumulating into fp32
    B, H, N, D = 1, 3, 2000, 128
    q, k, v, g = make((B, H, N, D), 7100, torch.bfloat16)
    ref = oracle.gated_softmax(q, k, v, g, D ** -0.5)
    got = run_softmax(q, k, v, g)
    assert rel_err(got, ref) <= TOL[torch.bfloat16]
    base = custom((B, H, N, D), 7200, torch.float32, n=1)[0]
    acc = base.to(DEV)
    run_softmax(q, k, v, g, accumulate=True, out=acc)
    assert rel_err(acc.cpu() - base, ref) <= TOL[torch.bfloat16]


def test_softmax_large_tail_split_sampled():
    # 720p x 81 frames with B = 1: 1216 query blocks leave a last batch of 192 on
    # 256 CUs, which is split four ways (768 pieces, three quarter-length
    # batches); sampled rows against the oracle, plain and accumulating
    from hla_inputs import duration_workload
    w = duration_workload(81, B=1, H=16)
    q, k, v, g = layer_inputs(w, 0)
    rows = sample_rows(w.N, count=24, seed=810)
    ref = oracle.gated_softmax(q, k, v, g, w.scale, rows=rows)
    sm = run_softmax(q, k, v, g, w.scale)
    e = rel_err(sm[..., rows, :], ref)
    base = custom((w.B, w.H, w.N, w.D), 8100, torch.float32, n=1)[0]
    acc = base.to(DEV)
    run_softmax(q, k, v, g, w.scale, accumulate=True, out=acc)
    e_acc = rel_err((acc.cpu() - base)[..., rows, :], ref)
    print(f"[{w.name} B=1] softmax err {e:.3e}, accumulated {e_acc:.3e}", flush=True)
    assert e <= TOL[torch.bfloat16] and e_acc <= TOL[torch.bfloat16]


def test_duration_sweep_longest_sampled():
    # 720p x 961 frames (60 s at 16 fps): N = 221,720 tokens, two heads; the
    # linear layer in full, the softmax anchor on sampled query rows
    from hla_inputs import duration_workload
    w = duration_workload(961, B=1, H=2)
    q, k, v, g = layer_inputs(w, 0)
    print(f"[{w.name}] B={w.B} H={w.H} N={w.N}", flush=True)
    lin = run_linear(q, k, v, g, w.eps)
    e_lin = rel_err(lin, oracle.gated_linear(q, k, v, g, w.eps))
    rows = sample_rows(w.N, count=24, seed=961)
    sm = run_softmax(q, k, v, g, w.scale)
    e_sm = rel_err(sm[..., rows, :], oracle.gated_softmax(q, k, v, g, w.scale, rows=rows))
    print(f"[{w.name}] linear err {e_lin:.3e}  softmax err {e_sm:.3e} on {len(rows)} rows", flush=True)
    assert e_lin <= TOL[torch.bfloat16]
    assert e_sm <= TOL[torch.bfloat16]


@pytest.mark.parametrize("D", [32, 128])
def test_hybrid_stack_fp32(D):
    # the stack on the fp32 path (VALU kernels): delta = x4 - x0 to the fp32 bar
    B, H, N = 1, 2, 300
    kinds = oracle.hybrid_kinds(4)
    layers = [make((B, H, N, D), 7500 + 10 * l + D, torch.float32) for l in range(4)]
    x0 = custom((B, H, N, D), 7599 + D, torch.float32, n=1)[0]
    x = x0.to(DEV)
    hla.hla_hybrid_stack_fwd(x, [tuple(t.to(DEV) for t in L) for L in layers], kinds)
    torch.cuda.synchronize()
    ref = oracle.hybrid_stack(x0, layers, kinds, 1e-6, D ** -0.5) - oracle.as_f64(x0)
    assert rel_err(x.cpu() - x0, ref) <= TOL[torch.float32]


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits); the smallest normal
    spacing at 0."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def test_hybrid_stack_bf16_residual():
    # the stack with a bf16 residual stream: each layer adds its output to x in
    # fp32 and stores x rounded to bf16. Reference: the same steps with the
    # oracle's fp64 layer outputs, x rounded to bf16 after every layer; per
    # element, each layer may add at most the operator's bar (2e-2 of its own
    # peak) plus one bf16 step of x
    B, H, N, D = 1, 2, 700, 128
    kinds = oracle.hybrid_kinds(4)
    layers = [make((B, H, N, D), 7300 + 10 * l, torch.bfloat16) for l in range(4)]
    x0 = custom((B, H, N, D), 7399, torch.float32, n=1)[0].to(torch.bfloat16)
    x = x0.to(DEV)
    hla.hla_hybrid_stack_fwd(x, [tuple(t.to(DEV) for t in L) for L in layers], kinds)
    torch.cuda.synchronize()
    xr = oracle.as_f64(x0)
    bound = np.zeros(xr.shape)
    for kind, (q, k, v, g) in zip(kinds, layers):
        o = (oracle.gated_linear(q, k, v, g, 1e-6) if kind == oracle.LINEAR
             else oracle.gated_softmax(q, k, v, g, D ** -0.5))
        xr = torch.from_numpy(xr + o).float().to(torch.bfloat16).double().numpy()
        bound += 2e-2 * np.abs(o).max() + bf16_ulp(xr)
    got = x.cpu().double().numpy()
    diff = np.abs(got - xr)
    print(f"[stack bf16 x] max diff {diff.max():.3e}, max diff/bound {(diff / bound).max():.3f}, "
          f"equal {(diff == 0).mean():.3f}", flush=True)
    assert (diff <= bound).all()
    # most elements round to the same bf16 value as the reference
    assert (diff == 0).mean() >= 0.9


def test_hybrid_stack_d64():
    # the stack at head dim 64 (fp32 residual): delta = x_L - x_0 against the
    # per-layer oracle sum
    kinds = oracle.hybrid_kinds(4)
    B, H, N, D = 2, 2, 333, 64
    layers = [make((B, H, N, D), 7400 + 10 * l, torch.bfloat16) for l in range(4)]
    x0 = custom((B, H, N, D), 7499, torch.float32, n=1)[0]
    x = x0.to(DEV)
    hla.hla_hybrid_stack_fwd(x, [tuple(t.to(DEV) for t in L) for L in layers], kinds)
    torch.cuda.synchronize()
    ref = oracle.hybrid_stack(x0, layers, kinds, 1e-6, D ** -0.5) - oracle.as_f64(x0)
    assert rel_err(x.cpu() - x0, ref) <= TOL[torch.bfloat16]


# ----------------------------------------------------------------------------
# the anchor's unsplit workgroups over many key tiles
# ----------------------------------------------------------------------------
# A call whose query blocks (256 rows each, B*H*ceil(N/256) of them) fill whole
# batches of one workgroup per compute unit is not split along the keys: every
# workgroup runs its block over all key tiles and writes the output itself
# (the main epilogue, not the combine kernel). These cases make each workgroup
# run 32 to 64 key tiles, through the unrolled steady loop.

def block_edge_rows(N, seed):
    rows = set(sample_rows(N, count=24, seed=seed).tolist())
    for r0 in range(0, N, 256):
        rows |= {r0, min(N - 1, r0 + 255)}
    return np.array(sorted(rows))


UNSPLIT_CASES = [
    # B, H, N, D, input dtype, output dtype, accumulate
    (4, 16, 2000, 64, torch.bfloat16, torch.bfloat16, False),
    (4, 16, 2000, 64, torch.bfloat16, torch.float32, True),
    (4, 16, 2000, 64, FP8, torch.bfloat16, False),
    (4, 16, 2000, 64, FP8, torch.float32, False),
    (4, 16, 2000, 64, FP8, torch.float32, True),
    (1, 16, 4096, 128, torch.bfloat16, torch.float32, False),
    (1, 16, 4090, 128, torch.bfloat16, torch.bfloat16, True),
    (1, 16, 4090, 128, FP8, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", UNSPLIT_CASES, ids=lambda c: f"B{c[0]}H{c[1]}N{c[2]}D{c[3]}-"
                         f"{str(c[4]).split('.')[-1]}-{str(c[5]).split('.')[-1]}-acc{int(c[6])}")
def test_softmax_unsplit_workgroups_many_tiles(case):
    B, H, N, D, dt, out_dt, acc = case
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = B * H * ((N + 255) // 256)
    if blocks % cus:
        pytest.skip(f"{blocks} query blocks do not fill whole batches of {cus} compute units")
    q, k, v, g = make((B, H, N, D), 9800 + N + D, dt)
    rows = block_edge_rows(N, seed=N + D)
    ref = oracle.gated_softmax(q, k, v, g, D ** -0.5, rows=rows)
    # accumulate into a stream of the output's own magnitude, so the check
    # still sees the layer's output after the rounding of the sum
    x0 = (custom((B, H, N, D), 9900 + N, torch.float32, n=1)[0] * 0.02).to(out_dt)
    out = x0.to(DEV) if acc else torch.empty((B, H, N, D), dtype=out_dt, device=DEV)
    run_softmax(q, k, v, g, out=out, accumulate=acc)
    got = out.float().cpu()[..., rows, :]
    if acc:
        got = got - x0.float()[..., rows, :]
    e = rel_err(got, ref)
    print(f"[unsplit {case}] err {e:.3e} on {len(rows)} rows x {B * H} heads", flush=True)
    assert e <= TOL[torch.bfloat16]


# ----------------------------------------------------------------------------
# write-gated linear attention
# ----------------------------------------------------------------------------

def run_linear_w(q, k, v, g, w, eps=1e-6, out_dtype=None, accumulate=False, out=None):
    qd, kd, vd, gd, wd = (t.contiguous().to(DEV) for t in (q, k, v, g, w))
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or out_dtype_for(q.dtype), device=DEV)
    hla.hla_linear_write_gated_fwd(qd, kd, vd, gd, wd, out=out, accumulate=accumulate, eps=eps)
    torch.cuda.synchronize()
    return out


def wlogits(shape, seed, dtype):
    return (custom(shape, seed, torch.float32, n=1)[0] * 2.0).to(dtype)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 257, 1000])
def test_write_gated_bf16_tails(N, D):
    q, k, v, g = make((2, 3, N, D), 8000 + N, torch.bfloat16)
    w = wlogits((2, 3, N), 8100 + N, torch.bfloat16)
    got = run_linear_w(q, k, v, g, w)
    assert rel_err(got, oracle.gated_linear_write(q, k, v, g, w, 1e-6)) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("D", [32, 128])
def test_write_gated_fp32(D):
    q, k, v, g = make((1, 2, 300, D), 8200 + D, torch.float32)
    w = wlogits((1, 2, 300), 8300 + D, torch.float32)
    got = run_linear_w(q, k, v, g, w)
    assert rel_err(got, oracle.gated_linear_write(q, k, v, g, w, 1e-6)) <= TOL[torch.float32]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_write_gate_open_equals_plain_and_closed_removes(dtype):
    # W = +inf: bitwise the plain operator; W = -inf on every other token: the
    # plain operator on the remaining keys and values
    q, k, v, g = make((1, 2, 500, 128), 8400, dtype)
    plain = run_linear(q, k, v, g)
    opened = run_linear_w(q, k, v, g, torch.full((1, 2, 500), float("inf"), dtype=dtype))
    assert torch.equal(plain, opened)
    keep = torch.arange(500) % 2 == 0
    w = torch.where(keep, float("inf"), float("-inf")).to(dtype)[None, None].expand(1, 2, 500).contiguous()
    got = run_linear_w(q, k, v, g, w)
    ref = oracle.gated_linear_write(q, k, v, g, w, 1e-6)
    assert rel_err(got, ref) <= TOL[dtype]


def test_write_gated_accumulate_fp32():
    q, k, v, g = make((1, 2, 700, 128), 8500, torch.bfloat16)
    w = wlogits((1, 2, 700), 8600, torch.bfloat16)
    base = custom((1, 2, 700, 128), 8700, torch.float32, n=1)[0]
    acc = base.to(DEV)
    run_linear_w(q, k, v, g, w, accumulate=True, out=acc)
    assert rel_err(acc.cpu() - base, oracle.gated_linear_write(q, k, v, g, w, 1e-6)) <= TOL[torch.bfloat16]


def test_write_gated_full_720p():
    w_ = BY_NAME["720p_81f"]
    q, k, v, g = layer_inputs(w_, 0)
    w = wlogits((w_.B, w_.H, w_.N), 8800, torch.bfloat16)
    got = run_linear_w(q, k, v, g, w, w_.eps)
    e = rel_err(got, oracle.gated_linear_write(q, k, v, g, w, w_.eps))
    print(f"[720p_81f write-gated] err {e:.3e}", flush=True)
    assert e <= TOL[torch.bfloat16]


def test_graph_capture_replays_match_eager():
    # the calls enqueue kernels only (no allocation, no memset), so they can be
    # captured in a HIP graph; every replay must reproduce the eager result
    # (linear, anchor, write-gated linear, the block-summary routing and the
    # e4m3-probability anchor on fp8 copies of the inputs)
    B, H, N, D = 1, 4, 1500, 128
    q, k, v, g = (t.to(DEV) for t in make((B, H, N, D), 9000, torch.bfloat16))
    w = wlogits((B, H, N), 9100, torch.bfloat16).to(DEV)
    x, s0, s1 = (t.to(DEV) for t in custom((B, H, N, D), 9200, torch.float32, n=3))
    router = (custom((D, D), 9300, torch.float32, n=1)[0] * (2.0 / D ** 0.5)).to(torch.bfloat16).to(DEV)
    ws_l, ws_a = hla.linear_workspace(q), hla.anchor_workspace(q)
    out_l, out_a, out_w, out_8 = (torch.empty_like(q) for _ in range(4))
    out_r = torch.empty_like(x)
    q8, k8, v8, g8 = (t.to(FP8) for t in (q, k, v, g))

    def calls():
        hla.hla_linear_fwd(q, k, v, g, out=out_l, workspace=ws_l)
        hla.hla_softmax_anchor_fwd(q, k, v, g, out=out_a, workspace=ws_a)
        hla.hla_linear_write_gated_fwd(q, k, v, g, w, out=out_w, workspace=ws_l)
        hla.hla_attnres_route_fwd(x, [s0, s1], router, out=out_r)
        hla.hla_softmax_anchor_fp8p_fwd(q8, k8, v8, g8, out=out_8, workspace=ws_a)

    outs = (out_l, out_a, out_w, out_r, out_8)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outs, eager):
            assert torch.equal(got, ref), rep


# ----------------------------------------------------------------------------
# fp8 (OCP e4m3) inputs
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("N", [1, 63, 65, 257, 1000])
def test_linear_fp8_tails(N, D, out_dtype):
    q, k, v, g = make((2, 2, N, D), 10000 + N + D, FP8)
    got = run_linear(q, k, v, g, out_dtype=out_dtype)
    assert got.dtype == out_dtype
    assert rel_err(got, oracle.gated_linear(q, k, v, g, 1e-6)) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("gated", [False, True])
def test_linear_fp8_matches_bf16_path_on_same_values(gated):
    # every e4m3 value is a bf16 value and the kernels convert exactly, so the
    # fp8 call computes what the bf16 call computes on the upcast tensors up to
    # the order of fp32 sums: the fp8 output pass takes the k-steps of phi(Q) S
    # in another order, and the plain fp8 state pass adds 64 products per matrix
    # instruction where the bf16 one adds 16. The write-gated layer rounds
    # beta * phi(K) to bf16 and runs the bf16 state pass, so only the output
    # pass's order differs there; on these N(0,1) values those sums are exact
    # and the two agree bit for bit. In the plain layer the fp8 instruction's own
    # summation of its 64 products moves some fp32 partial states by more than
    # an fp32 rounding, so a partial's bf16 rounding lands on the other side now
    # and then: a few percent of the outputs move by about one bf16 step of
    # their slab's largest value (measured: 2 % of them, 3.6e-3), and both calls
    # stay equally close to the fp64 oracle
    q, k, v, g = make((2, 3, 1500, 128), 10100, FP8)
    w = wlogits((2, 3, 1500), 10200, FP8)
    up = [t.to(torch.bfloat16) for t in (q, k, v, g, w)]
    if gated:
        a, b = run_linear_w(q, k, v, g, w), run_linear_w(*up)
    else:
        a, b = run_linear(q, k, v, g), run_linear(*up[:4])
    assert a.dtype == b.dtype == torch.bfloat16
    if gated:
        assert torch.equal(a, b)
        return
    a, b = a.float().cpu(), b.float().cpu()
    ref = oracle.gated_linear(q, k, v, g, 1e-6)
    differ = float((a != b).float().mean())
    print(f"[fp8 vs bf16 path] differ {differ:.2e}, rel {rel_err(a, b):.2e}, "
          f"oracle {rel_err(a, ref):.2e} / {rel_err(b, ref):.2e}", flush=True)
    assert rel_err(a, ref) <= TOL[torch.bfloat16]
    assert rel_err(b, ref) <= TOL[torch.bfloat16]
    assert differ <= 0.05
    assert rel_err(a, b) <= 2.0 ** -7
    assert abs(rel_err(a, ref) - rel_err(b, ref)) <= 2.0 ** -8


def test_linear_fp8_every_code_matches_bf16_path():
    # every finite e4m3 code (254 of them: zeros, subnormals, normals up to
    # +-448) in every input, so each conversion the kernels make meets every
    # value. Magnitudes from 2^-9 to 448 make the fp32 sums round; the fp8
    # state pass sums on the fp8 matrix instruction and the fp8 output pass
    # adds the k-steps in another order than the bf16 one, so some outputs
    # differ (measured: 5.7 % of them, by up to 5.2e-3 of their slab's largest
    # value; relative to a cancelling near-zero output the step can be large).
    # Both calls stay within the tolerance of the fp64 oracle
    codes = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    shape = (1, 2, 508, 128)
    gen = torch.Generator().manual_seed(10150)
    ts = []
    for _ in range(4):
        idx = torch.randint(0, codes.numel(), shape, generator=gen)
        t = codes[idx]
        t.view(-1)[: codes.numel()] = codes  # each code at least once
        ts.append(t.view(FP8))
    q, k, v, g = ts
    a = run_linear(q, k, v, g).float().cpu()
    b = run_linear(*[t.to(torch.bfloat16) for t in ts]).float().cpu()
    assert torch.isfinite(a).all()
    ref = oracle.gated_linear(q, k, v, g, 1e-6)
    assert rel_err(a, ref) <= TOL[torch.bfloat16]
    assert rel_err(b, ref) <= TOL[torch.bfloat16]
    differ = (a != b)
    print(f"[every e4m3 code] differ {int(differ.sum())} of {a.numel()}, "
          f"max step {float(((a - b).abs() / b.abs().clamp_min(1e-30)).max()):.2e}, "
          f"rel {rel_err(a, b):.2e}", flush=True)
    assert int(differ.sum()) <= a.numel() // 10
    assert rel_err(a, b) <= 2.0 ** -6


@pytest.mark.parametrize("D", [64, 128])
def test_linear_fp8_many_tiles_per_chunk(D):
    # few heads, so each token chunk spans many state-pass tiles (256 tokens per
    # tile at D = 64, 128 at D = 128) and a ragged last tile; bf16 and fp32 out
    q, k, v, g = make((1, 2, 20011, D), 10400 + D, FP8)
    ref = oracle.gated_linear(q, k, v, g, 1e-6)
    for od in (torch.bfloat16, torch.float32):
        got = run_linear(q, k, v, g, out_dtype=od)
        e = rel_err(got, ref)
        print(f"[fp8 linear N=20011 D={D} {od}] err {e:.3e}", flush=True)
        assert e <= TOL[torch.bfloat16]


def test_linear_fp8_binding_defaults_to_bf16_output():
    q, k, v, g = (t.to(DEV) for t in make((1, 2, 300, 64), 10300, FP8))
    out = hla.hla_linear_fwd(q, k, v, g)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    assert rel_err(out, oracle.gated_linear(q.cpu(), k.cpu(), v.cpu(), g.cpu(), 1e-6)) <= 2e-2


@pytest.mark.parametrize("N", [65, 1000])
def test_write_gated_fp8(N):
    q, k, v, g = make((2, 2, N, 128), 10400 + N, FP8)
    w = wlogits((2, 2, N), 10500 + N, FP8)
    got = run_linear_w(q, k, v, g, w, out_dtype=torch.float32)
    assert rel_err(got, oracle.gated_linear_write(q, k, v, g, w, 1e-6)) <= TOL[torch.bfloat16]


def test_linear_fp8_accumulate_and_stack():
    # accumulate into an fp32 stream, directly and through a linear-only stack
    B, H, N, D = 1, 2, 900, 128
    layers = [make((B, H, N, D), 10600 + 10 * l, FP8) for l in range(3)]
    x0 = custom((B, H, N, D), 10700, torch.float32, n=1)[0]
    x = x0.to(DEV)
    hla.hla_hybrid_stack_fwd(x, [tuple(t.to(DEV) for t in L) for L in layers], [0, 0, 0])
    torch.cuda.synchronize()
    ref = sum(oracle.gated_linear(*L, 1e-6) for L in layers)
    assert rel_err(x.cpu() - x0, ref) <= 2e-2
    acc = x0.to(DEV)
    run_linear(*layers[0], accumulate=True, out=acc)
    assert rel_err(acc.cpu() - x0, oracle.gated_linear(*layers[0], 1e-6)) <= 2e-2


def test_linear_fp8_full_720p():
    w = BY_NAME["720p_81f"]
    q, k, v, g = layer_inputs(w, 0, dtype=FP8)
    got = run_linear(q, k, v, g, w.eps)
    e = rel_err(got, oracle.gated_linear(q, k, v, g, w.eps))
    print(f"[720p_81f fp8] linear err {e:.3e}", flush=True)
    assert e <= 2e-2


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("N", [1, 63, 65, 257, 1000])
def test_softmax_fp8_tails(N, D, out_dtype):
    # Q K^T on the fp8 matrix cores, P V in bf16
    q, k, v, g = make((1, 2, N, D), 11000 + N + D, FP8)
    got = run_softmax(q, k, v, g, out_dtype=out_dtype)
    assert got.dtype == out_dtype
    assert rel_err(got, oracle.gated_softmax(q, k, v, g, D ** -0.5)) <= TOL[torch.bfloat16]


def test_softmax_fp8_close_to_bf16_path_on_same_values():
    # both paths see the same values; only the fp32 summation order of Q K^T
    # differs, so the outputs agree far inside the bf16 bar
    q, k, v, g = make((2, 2, 1500, 128), 11100, FP8)
    a = run_softmax(q, k, v, g, out_dtype=torch.float32)
    b = run_softmax(*[t.to(torch.bfloat16) for t in (q, k, v, g)], out_dtype=torch.float32)
    assert rel_err(a, oracle.as_f64(b.cpu())) <= 2e-3


def test_softmax_fp8_split_and_accumulate():
    # the key-split last batch with the combine kernel, plain and into fp32
    B, H, N, D = 1, 3, 2000, 128
    q, k, v, g = make((B, H, N, D), 11200, FP8)
    ref = oracle.gated_softmax(q, k, v, g, D ** -0.5)
    assert rel_err(run_softmax(q, k, v, g), ref) <= TOL[torch.bfloat16]
    base = custom((B, H, N, D), 11300, torch.float32, n=1)[0]
    acc = base.to(DEV)
    run_softmax(q, k, v, g, accumulate=True, out=acc)
    assert rel_err(acc.cpu() - base, ref) <= TOL[torch.bfloat16]


def test_softmax_fp8_peaky_logits():
    # large scores: one key dominates most rows, probabilities span many octaves
    q, k, v, g = make((1, 2, 700, 128), 11400, torch.float32)
    q8, k8, v8, g8 = ((q * 4).to(FP8), k.to(FP8), v.to(FP8), g.to(FP8))
    got = run_softmax(q8, k8, v8, g8)
    assert rel_err(got, oracle.gated_softmax(q8, k8, v8, g8, 128 ** -0.5)) <= TOL[torch.bfloat16]


def test_hybrid_stack_fp8_small_full():
    B, H, N, D = 1, 2, 777, 128
    kinds = oracle.hybrid_kinds(4)
    layers = [make((B, H, N, D), 11500 + 10 * l, FP8) for l in range(4)]
    x0 = custom((B, H, N, D), 11600, torch.float32, n=1)[0]
    x = x0.to(DEV)
    hla.hla_hybrid_stack_fwd(x, [tuple(t.to(DEV) for t in L) for L in layers], kinds)
    torch.cuda.synchronize()
    ref = oracle.hybrid_stack(x0, layers, kinds, 1e-6, D ** -0.5)
    assert rel_err(x.cpu() - x0, ref - oracle.as_f64(x0)) <= 2e-2


def test_softmax_fp8_full_720p_sampled():
    w = BY_NAME["720p_81f"]
    q, k, v, g = layer_inputs(w, 0, dtype=FP8)
    rows = sample_rows(w.N, seed=81)
    sm = run_softmax(q, k, v, g, w.scale)
    e = rel_err(sm[..., rows, :], oracle.gated_softmax(q, k, v, g, w.scale, rows=rows))
    print(f"[720p_81f fp8] softmax err {e:.3e} on {len(rows)} rows", flush=True)
    assert e <= TOL[torch.bfloat16]


def test_linear_beyond_2gib_per_tensor():
    # one head whose bf16 tensors exceed 2^31 bytes (N*D*2 = 2.15 GB): every byte
    # offset past the 32-bit signed range must still land right. Reference: the
    # state summed over token chunks in fp64, read out on sampled rows.
    from hla_inputs import randn
    N, D = 8_400_001, 128
    shape = (1, 1, N, D)
    print(f"[max-size linear] N={N} D={D} ({N * D * 2 / 2**30:.2f} GiB per tensor)", flush=True)
    q, k, v, g = (randn(shape, 12000 + i, torch.bfloat16) for i in range(4))
    out = run_linear(q, k, v, g)
    S = np.zeros((1, 1, D, D))
    z = np.zeros((1, 1, D))
    step = 1 << 20
    for a in range(0, N, step):
        Sc, zc = oracle.linear_state(k[..., a:a + step, :], v[..., a:a + step, :])
        S += Sc
        z += zc
    rows = sample_rows(N, count=64, seed=12)
    rows = np.unique(np.concatenate([rows, [N // 2, (1 << 23) - 1, 1 << 23, N - 3]]))  # 2^23 rows = 2^31 bytes
    rows = rows[rows < N]
    ref = oracle.linear_readout(q[..., rows, :], g[..., rows, :], S, z, 1e-6)
    e = rel_err(out[..., rows, :], ref)
    print(f"[max-size linear] err {e:.3e} on {len(rows)} rows", flush=True)
    assert e <= TOL[torch.bfloat16]


def test_concurrent_calls_on_two_streams():
    # calls on different streams with their own workspaces may run at the same
    # time: each must give exactly its sequential result
    B, H, N, D = 1, 4, 3000, 128
    q, k, v, g = (t.to(DEV) for t in make((B, H, N, D), 9400, torch.bfloat16))
    q2, k2, v2, g2 = (t.to(DEV) for t in make((B, H, N, D), 9500, torch.bfloat16))
    ref_l = hla.hla_linear_fwd(q, k, v, g)
    ref_a = hla.hla_softmax_anchor_fwd(q2, k2, v2, g2)
    ref_l2 = hla.hla_linear_fwd(q2, k2, v2, g2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        out_l, out_a, out_l2 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws1, ws2 = hla.linear_workspace(q), hla.anchor_workspace(q)
        ws3 = hla.linear_workspace(q)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            hla.hla_softmax_anchor_fwd(q2, k2, v2, g2, out=out_a, workspace=ws2)
        with torch.cuda.stream(s2):
            hla.hla_linear_fwd(q, k, v, g, out=out_l, workspace=ws1)
            hla.hla_linear_fwd(q2, k2, v2, g2, out=out_l2, workspace=ws3)
        torch.cuda.synchronize()
        outs.append((out_l, out_a, out_l2))
    for out_l, out_a, out_l2 in outs:
        assert torch.equal(out_l, ref_l)
        assert torch.equal(out_a, ref_a)
        assert torch.equal(out_l2, ref_l2)


def test_explicit_stream_argument_with_default_workspace():
    # stream= passed explicitly, no workspace and no out: the binding allocates both
    # for that stream, so a block freed after the call is not handed to other work
    # while the kernels may still use it; results equal the current-stream call's
    B, H, N, D = 2, 4, 2500, 128
    q, k, v, g = (t.to(DEV) for t in make((B, H, N, D), 9600, torch.bfloat16))
    x0 = custom((B, H, N, D), 9601, torch.float32, n=1)[0].to(DEV)
    ref_l = hla.hla_linear_fwd(q, k, v, g)
    ref_a = hla.hla_softmax_anchor_fwd(q, k, v, g)
    ref_x = hla.hla_hybrid_stack_fwd(x0.clone(), [(q, k, v, g)] * 4, [0, 0, 0, 1])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for rep in range(3):
        # the current stream keeps allocating and writing meanwhile
        junk = [torch.full((B, H, N, D), float(rep + 1), device=DEV) for _ in range(3)]
        got_l = hla.hla_linear_fwd(q, k, v, g, stream=s)
        got_a = hla.hla_softmax_anchor_fwd(q, k, v, g, stream=s)
        x = x0.clone()
        torch.cuda.current_stream().synchronize()
        hla.hla_hybrid_stack_fwd(x, [(q, k, v, g)] * 4, [0, 0, 0, 1], stream=s)
        junk += [torch.full((B, H, N, D), -1.0, device=DEV) for _ in range(3)]
        s.synchronize()
        assert torch.equal(got_l, ref_l)
        assert torch.equal(got_a, ref_a)
        assert torch.equal(x, ref_x)
        del junk


def test_binding_refuses_mixed_dtypes_on_the_gpu():
    # q's dtype fixes the element size the kernels read k, v and g with: a
    # mismatch is refused before any launch and the output stays untouched
    q, k, v, g = (t.to(DEV) for t in make((1, 2, 200, 128), 9700, torch.bfloat16))
    out = torch.full(q.shape, 7.0, dtype=torch.bfloat16, device=DEV)
    for args in [(q.float(), k, v, g), (q, k.float(), v, g), (q, k, v.to(FP8), g),
                 (q, k, v, g.float())]:
        for call in (hla.hla_linear_fwd, hla.hla_softmax_anchor_fwd):
            with pytest.raises(ValueError):
                call(*args, out=out)
    x = torch.zeros(q.shape, device=DEV)
    with pytest.raises(ValueError):
        hla.hla_hybrid_stack_fwd(x, [(q, k, v, g), (q.float(), k.float(), v.float(), g.float())],
                                 [0, 1])
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((x == 0).all())
