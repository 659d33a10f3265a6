"""C-ABI checks that need no GPU: the library loads, exports what include/hla.h
declares, and rejects every invalid argument on the host with its status code.

Every call here carries at least one invalid argument (or an empty tensor), so
validation returns before any HIP call: nothing is launched, which also keeps
these tests safe to run on a machine that has a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

import softmax_attention_amd as hla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hla.h")

OK, NULLP, SHAPE, UNSUP, BADARG, ALIGN, WS, HIP = range(8)
F32, BF16, FP8 = hla.HLA_F32, hla.HLA_BF16, hla.HLA_FP8_E4M3
FAKE = 0x10000  # a 16-byte-aligned address that is never dereferenced
ODD = 0x10008   # 8-byte aligned only


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hla_[a-z0-9_]+)\s*\(", src)))


def dims(B=2, H=3, N=100, D=128, i=BF16, o=BF16):
    return hla.hla_dims(B, H, N, D, i, o)


def lin(d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, out=FAKE, acc=0, eps=1e-6, ws=FAKE, wsb=1 << 40):
    return hla.lib.hla_linear_fwd(ctypes.byref(d) if d is not None else None, q, k, v, g, out, acc,
                                  eps, ws, wsb, None)


def lin_w(d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, w=FAKE, out=FAKE, acc=0, eps=1e-6, ws=FAKE,
          wsb=1 << 40):
    return hla.lib.hla_linear_write_gated_fwd(ctypes.byref(d) if d is not None else None, q, k, v,
                                              g, w, out, acc, eps, ws, wsb, None)


def sm(d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, out=FAKE, acc=0, scale=0.1, ws=FAKE, wsb=1 << 40):
    return hla.lib.hla_softmax_anchor_fwd(ctypes.byref(d) if d is not None else None, q, k, v, g,
                                          out, acc, scale, ws, wsb, None)


def sm8p(d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, out=FAKE, acc=0, scale=0.1, ws=FAKE, wsb=1 << 40):
    return hla.lib.hla_softmax_anchor_fp8p_fwd(ctypes.byref(d) if d is not None else None, q, k, v,
                                               g, out, acc, scale, ws, wsb, None)


def stack(d, n=2, kinds=(0, 1), ptrs=None, x=FAKE, eps=1e-6, scale=0.1, ws=FAKE, wsb=1 << 40):
    arr = ctypes.c_void_p * max(n, 1)
    p = ptrs if ptrs is not None else [FAKE] * max(n, 1)
    q = arr(*p)
    kd = (ctypes.c_int32 * max(len(kinds), 1))(*kinds) if kinds is not None else None
    return hla.lib.hla_hybrid_stack_fwd(ctypes.byref(d) if d is not None else None, n, kd, q, q, q,
                                        q, x, eps, scale, ws, wsb, None)


def route(d, n=2, ptrs=None, x=FAKE, w=FAKE, out=FAKE):
    arr = ctypes.c_void_p * max(n, 1)
    p = ptrs if ptrs is not None else [FAKE] * max(n, 1)
    return hla.lib.hla_attnres_route_fwd(ctypes.byref(d) if d is not None else None, n, arr(*p), x, w,
                                         out, None)


def test_header_declares_the_abi():
    fns = declared_functions()
    assert fns == sorted(hla.EXPORTS)


def test_library_exports_every_declared_symbol():
    for fn in declared_functions():
        assert hasattr(hla.lib, fn), fn
    out = subprocess.run(["nm", "-D", "--defined-only", hla.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (hla_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_header_is_plain_c_and_cpp(tmp_path):
    # every declaration compiles as strict C99 and as C++17, with no HIP or torch header
    calls = "\n".join(f"  (void)&{fn};" for fn in declared_functions())
    for lang, std, cc in (("c", "-std=c99", "gcc"), ("c++", "-std=c++17", "g++")):
        src = tmp_path / f"use.{'c' if lang == 'c' else 'cpp'}"
        src.write_text(f'#include "hla.h"\nint main(void) {{\n{calls}\n  return HLA_ABI_VERSION == 0;\n}}\n')
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                            "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_c_client_source_compiles():
    # the plain C client that a GPU test runs (C99, warnings as errors)
    src = os.path.join(ROOT, "tests", "c_client", "hla_c_client.c")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                        "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"), src], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_version_and_status_strings():
    assert hla.hla_abi_version() == 5
    for code, name in hla.STATUS.items():
        assert hla.hla_status_str(code) == name
    assert hla.hla_status_str(99) == "HLA_UNKNOWN"
    assert hla.hla_status_str(-1) == "HLA_UNKNOWN"


def test_workspace_bytes_pure_and_sized():
    d = dims(2, 16, 19320, 128)
    a = hla.hla_linear_workspace_bytes(d)
    assert a == hla.hla_linear_workspace_bytes(dims(2, 16, 19320, 128)) and a > 0
    # at least the partial states plus the reduced state of every head
    assert a >= 2 * 16 * (128 * 128 + 128) * 4
    assert a % 256 == 0
    assert hla.hla_linear_workspace_bytes(dims(1, 2, 256, 32, F32, F32)) > 0
    assert hla.hla_linear_workspace_bytes(dims(0, 2, 256, 32, F32, F32)) == 0      # empty
    assert hla.hla_linear_workspace_bytes(dims(1, 2, 256, 48, F32, F32)) == 0      # unsupported D
    assert hla.hla_linear_workspace_bytes(dims(1, 2, 256, 32, BF16, BF16)) == 0    # bf16 D=32 not built
    assert hla.lib.hla_linear_workspace_bytes(None) == 0


@pytest.mark.parametrize("call", ["lin", "lin_w", "sm"])
def test_shape_and_dtype_errors(call):
    f = {"lin": lin, "lin_w": lin_w, "sm": sm}[call]
    assert f(None) == NULLP
    assert f(dims(B=-1)) == SHAPE
    assert f(dims(N=-5)) == SHAPE
    assert f(dims(D=0)) == SHAPE
    assert f(dims(D=-128)) == SHAPE
    assert f(dims(D=96)) == UNSUP
    assert f(dims(D=32)) == UNSUP                  # bf16 path built for D in {64, 128}
    assert f(dims(i=F32, o=BF16, D=32)) == UNSUP   # fp32 in -> bf16 out not built
    assert f(dims(i=7)) == UNSUP
    assert f(dims(o=FP8)) == UNSUP                 # fp8 outputs are not built
    assert f(dims(i=FP8, o=FP8)) == UNSUP
    assert f(dims(i=FP8, D=32)) == UNSUP
    assert f(dims(N=1 << 31)) == SHAPE             # N*D overflows 32-bit offsets
    assert f(dims(B=1 << 40)) == SHAPE


def test_linear_argument_errors():
    d = dims()
    for p in ("q", "k", "v", "g", "out"):
        assert lin(d, **{p: None}) == NULLP, p
        assert lin(d, **{p: ODD}) == ALIGN, p
    assert lin(d, ws=None) == NULLP
    assert lin(d, ws=ODD) == ALIGN
    need = hla.hla_linear_workspace_bytes(d)
    assert lin(d, wsb=need - 1) == WS
    assert lin(d, wsb=0) == WS
    for eps in (float("nan"), float("inf"), -1e-6):
        assert lin(d, eps=eps) == BADARG
    assert lin(d, acc=2) == BADARG
    assert lin(d, acc=-1) == BADARG


def test_write_gated_argument_errors():
    d = dims()
    for p in ("q", "k", "v", "g", "w", "out"):
        assert lin_w(d, **{p: None}) == NULLP, p
        assert lin_w(d, **{p: ODD}) == ALIGN, p
    assert lin_w(d, ws=None) == NULLP
    assert lin_w(d, wsb=hla.hla_linear_workspace_bytes(d) - 1) == WS
    assert lin_w(d, eps=float("nan")) == BADARG
    assert lin_w(d, acc=5) == BADARG
    # empty: no-op, pointers may be NULL
    assert lin_w(dims(N=0), q=None, k=None, v=None, g=None, w=None, out=None, ws=None, wsb=0) == OK


def test_fp8_inputs():
    # fp8 inputs take the bf16 paths' workspaces (the same values, converted
    # on load)
    for o in (BF16, F32):
        for D in (64, 128):
            assert hla.hla_linear_workspace_bytes(dims(D=D, i=FP8, o=o)) == \
                hla.hla_linear_workspace_bytes(dims(D=D, i=BF16, o=o))
    d = dims(i=FP8, o=BF16)
    assert lin(d, q=ODD) == ALIGN
    assert lin_w(d, w=None) == NULLP
    assert lin(d, wsb=hla.hla_linear_workspace_bytes(d) - 1) == WS
    assert stack(dims(i=FP8, o=F32), kinds=(0, 0), ws=None) == NULLP
    # the anchor repacks V into bf16 V^T for fp8 inputs too: same workspace
    for (N, D) in [(19320, 128), (1000, 64)]:
        assert hla.hla_softmax_anchor_workspace_bytes(dims(N=N, D=D, i=FP8)) == \
            hla.hla_softmax_anchor_workspace_bytes(dims(N=N, D=D, i=BF16))
    assert sm(d, ws=None) == NULLP
    assert sm(d, wsb=hla.hla_softmax_anchor_workspace_bytes(d) - 1) == WS


def test_fp8p_anchor_errors():
    # the fp8-probability anchor takes fp8 inputs only, and otherwise checks its
    # arguments as the anchor does; its workspace is the anchor's
    assert sm8p(None) == NULLP
    assert sm8p(dims(i=BF16)) == UNSUP
    assert sm8p(dims(i=F32, o=F32, D=32)) == UNSUP
    assert sm8p(dims(B=-1, i=FP8)) == SHAPE
    assert sm8p(dims(i=FP8, D=96)) == UNSUP
    assert sm8p(dims(i=FP8, o=FP8)) == UNSUP
    d = dims(i=FP8)
    for p in ("q", "k", "v", "g", "out"):
        assert sm8p(d, **{p: None}) == NULLP, p
        assert sm8p(d, **{p: ODD}) == ALIGN, p
    for s_ in (0.0, -0.1, float("nan"), float("inf")):
        assert sm8p(d, scale=s_) == BADARG
    assert sm8p(d, acc=3) == BADARG
    assert sm8p(d, ws=None) == NULLP
    assert sm8p(d, ws=ODD) == ALIGN
    assert sm8p(d, wsb=hla.hla_softmax_anchor_workspace_bytes(d) - 1) == WS
    assert sm8p(dims(N=0, i=FP8), q=None, k=None, v=None, g=None, out=None, ws=None, wsb=0) == OK


def test_softmax_argument_errors():
    d = dims()
    for p in ("q", "k", "v", "g", "out"):
        assert sm(d, **{p: None}) == NULLP, p
        assert sm(d, **{p: ODD}) == ALIGN, p
    for s in (0.0, -0.1, float("nan"), float("inf")):
        assert sm(d, scale=s) == BADARG
    assert sm(d, acc=3) == BADARG
    assert sm(d, ws=None) == NULLP
    assert sm(d, ws=ODD) == ALIGN
    need = hla.hla_softmax_anchor_workspace_bytes(d)
    assert sm(d, wsb=need - 1) == WS
    # the fp32 path needs no workspace: validation then rejects nothing about it,
    # so only check the size query here (a valid fp32 call would launch)
    assert hla.hla_softmax_anchor_workspace_bytes(dims(i=F32, o=F32, D=32)) == 0


def test_softmax_workspace_size():
    # repacked V^T (B*H*D*ceil(N/64)*64 bf16), then room for the partial results
    # of up to P = min(1024, query blocks * key tiles) key-range pieces of 256
    # query rows: D fp32 values plus (max, sum) each; every part rounded up to
    # 256 bytes
    up = lambda x: -(-x // 256) * 256
    for (B, H, N, D) in [(2, 16, 19320, 128), (1, 2, 1, 64), (1, 1, 64, 128), (1, 1, 65, 128),
                         (1, 2, 1000, 128)]:
        n_pad = -(-N // 64) * 64
        pieces = min(1024, B * H * -(-N // 256) * (n_pad // 64))
        want = up(B * H * D * n_pad * 2) + up(pieces * 256 * D * 4) + up(pieces * 256 * 2 * 4)
        assert hla.hla_softmax_anchor_workspace_bytes(dims(B, H, N, D)) == want
    assert hla.hla_softmax_anchor_workspace_bytes(dims(N=0)) == 0
    assert hla.lib.hla_softmax_anchor_workspace_bytes(None) == 0


def test_stack_argument_errors():
    d = dims(o=F32)
    assert stack(None) == NULLP
    assert stack(d, n=0, kinds=(0,)) == BADARG
    assert stack(d, n=-3, kinds=(0,)) == BADARG
    assert stack(d, kinds=None) == NULLP
    assert stack(d, kinds=(0, 2)) == BADARG
    assert stack(d, kinds=(-1, 1)) == BADARG
    assert stack(d, eps=float("nan")) == BADARG
    assert stack(d, scale=0.0) == BADARG
    assert stack(d, ptrs=[FAKE, None]) == NULLP
    assert stack(d, ptrs=[FAKE, ODD]) == ALIGN
    assert stack(d, x=None) == NULLP
    assert stack(d, x=ODD) == ALIGN
    assert stack(d, ws=None) == NULLP                           # has a linear layer
    need = max(hla.hla_linear_workspace_bytes(d), hla.hla_softmax_anchor_workspace_bytes(d))
    assert stack(d, wsb=need - 16) == WS
    assert stack(d, kinds=(1, 1), wsb=hla.hla_softmax_anchor_workspace_bytes(d) - 16) == WS
    assert stack(dims(D=40, o=F32)) == UNSUP
    assert stack(dims(N=-1, o=F32)) == SHAPE


def test_attnres_argument_errors():
    d = dims(i=F32, o=F32)
    assert route(None) == NULLP
    assert route(dims(i=BF16, o=BF16)) == UNSUP        # the residual stream is fp32
    assert route(dims(i=BF16, o=F32)) == UNSUP
    assert route(dims(i=FP8, o=F32)) == UNSUP
    assert route(dims(i=F32, o=F32, D=32)) == UNSUP     # D in {64, 128}
    assert route(dims(i=F32, o=F32, D=96)) == UNSUP
    assert route(dims(i=F32, o=F32, N=-1)) == SHAPE
    assert route(d, n=-1) == BADARG
    assert route(d, n=17, ptrs=[FAKE] * 17) == BADARG
    assert hla.lib.hla_attnres_route_fwd(ctypes.byref(d), 2, None, FAKE, FAKE, FAKE, None) == NULLP
    for p in ("x", "w", "out"):
        assert route(d, **{p: None}) == NULLP, p
        assert route(d, **{p: ODD}) == ALIGN, p
    assert route(d, ptrs=[FAKE, None]) == NULLP
    assert route(d, ptrs=[FAKE, ODD]) == ALIGN
    # empty tensors: valid, nothing to do, pointers may be NULL
    assert route(dims(i=F32, o=F32, N=0), x=None, w=None, out=None) == OK
    # no completed block, in place: the stream passes unchanged, W is not needed
    assert route(d, n=0, ptrs=[], w=None) == OK


def test_empty_tensors_are_a_no_op():
    # B*H*N == 0: valid, nothing to do, pointers may be NULL
    for d in (dims(N=0), dims(B=0), dims(H=0, i=F32, o=F32, D=32)):
        assert lin(d, q=None, k=None, v=None, g=None, out=None, ws=None, wsb=0) == OK
        assert sm(d, q=None, k=None, v=None, g=None, out=None, ws=None, wsb=0) == OK
        assert stack(d, ptrs=[None, None], x=None, ws=None, wsb=0) == OK
    # but the other arguments are still checked
    assert lin(dims(N=0), eps=-1.0) == BADARG
    assert sm(dims(N=0), scale=-1.0) == BADARG


def test_binding_rejects_cpu_tensors():
    import torch
    t = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hla.hla_linear_fwd(t, t, t, t)
    with pytest.raises(ValueError):
        hla.hla_softmax_anchor_fwd(t, t, t, t)


def test_binding_dims():
    import torch
    t = torch.zeros(2, 3, 5, 64, dtype=torch.bfloat16)
    d = hla.dims_of(t, torch.float32)
    assert (d.B, d.H, d.N, d.D, d.in_dtype, d.out_dtype) == (2, 3, 5, 64, BF16, F32)
    d = hla.dims_of(t)
    assert d.out_dtype == BF16
    assert hla.dims_of(t.float(), t.float()).in_dtype == F32
    d = hla.dims_of(t.to(torch.float8_e4m3fn), torch.bfloat16)
    assert (d.in_dtype, d.out_dtype) == (FP8, BF16)
    # fp8 inputs default to bf16 output (as the calls do), so workspace sizes are not 0
    d = hla.dims_of(t.to(torch.float8_e4m3fn))
    assert (d.in_dtype, d.out_dtype) == (FP8, BF16)
    assert hla.hla_linear_workspace_bytes(d) > 0 and hla.hla_softmax_anchor_workspace_bytes(d) > 0
    with pytest.raises(TypeError):
        hla.dims_of(t.half())


def test_one_hip_runtime_whatever_the_import_order():
    # libhla must bind to torch's HIP runtime even when imported before torch
    import sys
    code = ("import softmax_attention_amd as h, torch; "
            "r = h.hip_runtimes_loaded(); print(len(r)); assert len(r) == 1, r")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip().endswith("1")


class _FakeGpuTensor:
    """Stands in for a device tensor in the binding's argument checks (no GPU here).

    Only the attributes the checks read are present; a call that got past the
    checks would fail on data_ptr(), which this object does not have."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True):
        import torch
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contiguous = contiguous

    def is_contiguous(self):
        return self._contiguous


def test_binding_rejects_mixed_dtypes_and_devices_before_any_launch(monkeypatch):
    import torch
    called = []
    for fn in ("hla_linear_fwd", "hla_softmax_anchor_fwd", "hla_hybrid_stack_fwd",
               "hla_linear_write_gated_fwd"):
        monkeypatch.setattr(hla.lib, fn, lambda *a, _fn=fn: called.append(_fn) or 0)
    shape = (1, 2, 64, 128)
    bf = lambda **kw: _FakeGpuTensor(shape, torch.bfloat16, **kw)
    f32 = _FakeGpuTensor(shape, torch.float32)
    f8 = _FakeGpuTensor(shape, torch.float8_e4m3fn)
    other_dev = bf(device="cuda:1")
    # q's dtype fixes the element size the kernels read k, v and g with
    for args in [(f32, bf(), bf(), bf()), (bf(), f32, bf(), bf()), (bf(), bf(), f8, bf()),
                 (bf(), bf(), bf(), f32), (bf(), other_dev, bf(), bf()),
                 (bf(), bf(), bf(contiguous=False), bf())]:
        for call in (hla.hla_linear_fwd, hla.hla_softmax_anchor_fwd):
            with pytest.raises(ValueError):
                call(*args, out=bf())
    with pytest.raises(ValueError):
        hla.hla_linear_write_gated_fwd(bf(), bf(), bf(), bf(),
                                       _FakeGpuTensor(shape[:-1], torch.float32), out=bf())
    # the output: q's device, shape and contiguity
    for out in (bf(device="cuda:1"), _FakeGpuTensor((1, 2, 63, 128), torch.bfloat16),
                bf(contiguous=False)):
        with pytest.raises(ValueError):
            hla.hla_softmax_anchor_fwd(bf(), bf(), bf(), bf(), out=out)
    # every layer of a stack shares layer 0's dtype, shape and device
    good = (bf(), bf(), bf(), bf())
    x = _FakeGpuTensor(shape, torch.float32)
    for bad in [(f32, f32, f32, f32), (bf(), bf(), f8, bf()), (bf(), bf(), bf(), other_dev)]:
        with pytest.raises(ValueError):
            hla.hla_hybrid_stack_fwd(x, [good, bad], [0, 1])
    with pytest.raises(ValueError):
        hla.hla_hybrid_stack_fwd(x, [], [])
    assert called == []


def test_noalloc_argument_errors():
    # validated on the host before any HIP call, like the other entry points
    def call(d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, out=FAKE, acc=0, eps=1e-6):
        return hla.lib.hla_linear_fwd_noalloc(ctypes.byref(d) if d is not None else None,
                                              q, k, v, g, out, acc, eps, None)
    assert call(None) == NULLP
    assert call(dims(D=96)) == UNSUP
    assert call(dims(N=-1)) == SHAPE
    assert call(dims(), eps=-1.0) == BADARG
    assert call(dims(), acc=2) == BADARG
    assert call(dims(), q=None) == NULLP
    assert call(dims(), out=ODD) == ALIGN
    assert call(dims(N=0), q=None, k=None, v=None, g=None, out=None) == OK
    # more than the scratch array holds: refused before any GPU work
    big = dims(B=1, H=4000, N=4096, D=128)
    assert hla.hla_linear_workspace_bytes(big) > hla.NOALLOC_SCRATCH_BYTES
    assert call(big) == WS
    fits = dims(B=2, H=16, N=19320, D=128)
    assert hla.hla_linear_workspace_bytes(fits) <= hla.NOALLOC_SCRATCH_BYTES
