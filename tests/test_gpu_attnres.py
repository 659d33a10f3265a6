"""GPU parity of the block-attention-residual routing (hla_attnres_route_fwd) against
the fp64 oracle (MI355X).

Metric: the routed update out - x against the oracle's, max |gpu - ref| / max |ref|
per [b, h] slab. The bar is the bf16 one, 2e-2: the router query q = x W is formed
on the matrix cores from x split into a bf16 hi + lo pair (W is bf16 already);
scores, softmax and the mix are fp32. Shapes span several 16-token groups, ragged tails, D in {64, 128}
and 1 to 16 blocks; the 720p x 121-frame stack shape (B=1, H=16, N=28,520) is
checked in full.
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as hla
from hla_inputs import BY_NAME, Workload, attnres_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-2


def small(D, index=7):
    # a workload record only to seed the draws; shapes are passed explicitly
    return Workload(index, f"attnres_d{D}", 1, 2, 1000, D, "f32", (1, 1, 1000))


def run(x, S, w, inplace=False):
    xd = x.to(DEV)
    Sd = [s.to(DEV) for s in S]
    out = hla.hla_attnres_route_fwd(xd, Sd, w.to(DEV), out=xd if inplace else None)
    torch.cuda.synchronize()
    return out.cpu()


def update_err(got, x, S, w):
    ref = oracle.attnres_route(x, S, w) - oracle.as_f64(x)
    return oracle.max_rel_error(oracle.as_f64(got) - oracle.as_f64(x), ref)


@pytest.mark.parametrize("M", [1, 2, 3, 5])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("N", [1, 15, 16, 17, 100, 1000])
def test_route_tails(N, D, M):
    x, S, w = attnres_inputs(small(D), M, B=1, H=2, N=N)
    assert update_err(run(x, S, w), x, S, w) <= TOL


def test_route_sixteen_blocks_and_in_place():
    x, S, w = attnres_inputs(small(128, 8), 16, B=2, H=2, N=333)
    got = run(x, S, w, inplace=True)
    assert update_err(got, x, S, w) <= TOL


def test_one_block_adds_it_exactly():
    # a lone block has weight exactly 1 (exp2(0) / 1), so out = x + s in fp32
    x, S, w = attnres_inputs(small(128, 9), 1, B=1, H=3, N=500)
    assert torch.equal(run(x, S, w), x + S[0])


def test_no_block_copies_or_leaves_the_stream():
    x, _, w = attnres_inputs(small(64, 10), 0, B=1, H=2, N=77)
    assert torch.equal(run(x, [], w), x)
    xd = x.to(DEV)
    hla.hla_attnres_route_fwd(xd, [], w.to(DEV), out=xd)
    torch.cuda.synchronize()
    assert torch.equal(xd.cpu(), x)


def test_zero_router_averages_and_sharp_router_selects():
    x, S, w = attnres_inputs(small(128, 11), 3, B=1, H=2, N=400)
    zero = torch.zeros_like(w)
    got = run(x, S, zero)
    assert update_err(got, x, S, zero) <= 1e-5      # no bf16 rounding reaches the weights
    sharp = (w.float() * 24.0).to(torch.bfloat16)  # scores spread over tens of units
    assert update_err(run(x, S, sharp), x, S, sharp) <= TOL


def test_deterministic_and_in_bounds():
    x, S, w = attnres_inputs(small(128, 12), 3, B=1, H=2, N=1001)
    n = x.numel()
    guard = 4096
    buf = torch.full((n + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
    out = buf[guard:guard + n].view(x.shape)
    xd, Sd, wd = x.to(DEV), [s.to(DEV) for s in S], w.to(DEV)
    hla.hla_attnres_route_fwd(xd, Sd, wd, out=out)
    first = out.clone()
    hla.hla_attnres_route_fwd(xd, Sd, wd, out=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool((buf[:guard] == 7.0).all()) and bool((buf[guard + n:] == 7.0).all())


def test_route_stack_workload_full():
    # the 8-layer stack's shape (720p x 121 frames), two completed blocks
    w_ = BY_NAME["stack_720p_121f"]
    x, S, w = attnres_inputs(w_, 2)
    print(f"[{w_.name}] B={w_.B} H={w_.H} N={w_.N} D={w_.D} blocks=2", flush=True)
    e = update_err(run(x, S, w), x, S, w)
    print(f"[{w_.name}] routed update err {e:.3e}", flush=True)
    assert e <= TOL
