"""The allocation-free linear entry point (hla_linear_fwd_noalloc) against the
workspace entry point (hla_linear_fwd), through the C ABI on the GPU.

Two calls in a row, the second with a smaller input, so the second reuses the
scratch array the first filled: each must equal the workspace call's output on
the same inputs (same kernels and work split, so bit for bit) and so meet the
2e-2 (bf16) or 1e-4 (fp32) bar against the oracle that call is held to.
"""
import pytest
import torch

import oracle
import softmax_attention_amd as hla
from hla_inputs import custom

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_pair(shape, seed, dt, out_dt, accumulate):
    q, k, v, g = custom(shape, seed, dt, n=4)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    x0 = custom(shape, seed + 10, torch.float32, n=1)[0].to(out_dt).to(DEV)
    ref_out = x0.clone() if accumulate else torch.empty(shape, dtype=out_dt, device=DEV)
    got_out = x0.clone() if accumulate else torch.full(shape, float("nan"), dtype=out_dt, device=DEV)
    hla.hla_linear_fwd(qd, kd, vd, gd, out=ref_out, accumulate=accumulate)
    hla.hla_linear_fwd_noalloc(qd, kd, vd, gd, out=got_out, accumulate=accumulate)
    torch.cuda.synchronize()
    assert torch.equal(got_out, ref_out)
    if not accumulate:
        bar = 1e-4 if dt == torch.float32 else 2e-2
        assert oracle.max_rel_error(got_out.float().cpu(), oracle.gated_linear(q, k, v, g, 1e-6)) <= bar


@pytest.mark.parametrize("dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                       (torch.float32, torch.float32),
                                       (torch.float8_e4m3fn, torch.bfloat16)])
def test_noalloc_equals_workspace_call_twice(dt, out_dt):
    # the 720p layer shape first (17 MiB of scratch), then a smaller ragged one
    run_pair((2, 16, 19320, 128) if dt != torch.float32 else (1, 16, 3000, 128), 31, dt, out_dt, False)
    run_pair((1, 3, 777, 64), 41, dt, out_dt, False)
    run_pair((1, 3, 777, 64), 51, dt, out_dt, True)


def test_noalloc_refuses_oversize_and_leaves_out_untouched():
    shape = (1, 4000, 64, 128)  # a workspace of about 268 MiB, above the 64 MiB scratch
    q = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    out = torch.full(shape, 3.0, dtype=torch.bfloat16, device=DEV)
    d = hla.dims_of(q)
    assert hla.hla_linear_workspace_bytes(d) > hla.NOALLOC_SCRATCH_BYTES
    with pytest.raises(hla.HLAError) as e:
        hla.hla_linear_fwd_noalloc(q, q, q, q, out=out)
    assert e.value.status == 6  # HLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
