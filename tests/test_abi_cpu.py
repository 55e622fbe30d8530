"""The C-ABI library on the host, without a GPU: it loads, exports every symbol the
header declares, and its host-only logic (codebook builder, per-step scalars,
argument checks) agrees with the oracle and with the header's contract.  No call
here reaches a kernel launch: every device entry point is exercised only on its
argument-checking paths and with n == 0.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitopt.h")


@pytest.fixture(scope="module")
def B():
    from bit_optimizers_block_amd import bitopt
    if not os.path.exists(bitopt.LIB_PATH):
        from bit_optimizers_block_amd import build
        build.build()
    bitopt.lib()
    return bitopt


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"BITOPT_API\s+[\w\s\*]+?\b(bitopt_\w+)\s*\(", src)


def test_exports_every_declared_symbol(B):
    names = declared_functions()
    assert len(names) >= 10
    L = ctypes.CDLL(B.LIB_PATH)
    for name in names:
        assert hasattr(L, name), f"{name} declared in bitopt.h but not exported"
    assert B.abi_version() == 1


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "bitopt.h"\nint main(void){bitopt_hparams h; (void)h; return BITOPT_OK;}\n')
    import subprocess
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", "-c", str(src),
                    "-o", str(tmp_path / "use.o")], check=True)


@pytest.mark.parametrize("signed", [True, False])
def test_codebook_equals_oracle(B, oref, signed):
    mine = B.create_dynamic_map(signed).numpy()
    np.testing.assert_array_equal(mine.view(np.uint32), oref.dynamic_map(signed).view(np.uint32))


HP_CASES = [
    dict(optimizer="adam", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    dict(optimizer="adam", lr=3e-4, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1),
    dict(optimizer="ademamix", lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, t_alpha=100, t_beta3=100),
    dict(optimizer="ademamix", lr=1e-3, beta3=0.999, alpha=8.0),
    dict(optimizer="momentum", lr=0.01, beta1=0.9, weight_decay=0.01),
    dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01),
    dict(optimizer="rmsprop", lr=0.01, beta1=0.9, eps=1e-8, weight_decay=0.01),
    dict(optimizer="adagrad", lr=0.01, eps=1e-10, weight_decay=0.01),
]


@pytest.mark.parametrize("hp", HP_CASES)
def test_step_scalars_equal_oracle(B, oref, hp):
    for t in (1, 2, 7, 50, 99, 100, 101, 1000, 100000):
        mine = B.step_scalars(hp, t)
        ref = oref.step_scalars(hp, t)
        for k, v in ref.items():
            assert np.float32(mine[k]) == np.float32(v), (k, t, mine[k], v)


def _call2(B, hp=None, step=1, n=16, dtype=0, ptr=16, nulls=()):
    h = B.make_hparams(hp or dict(optimizer="adam"))
    P = [ctypes.c_void_p(None if i in nulls else ptr) for i in range(8)]
    return B.lib().bitopt_step_8bit_blockwise_2state(ctypes.byref(h), step, P[0], P[1], dtype, n, P[2], P[3],
                                                     P[4], P[5], P[6], P[7], None)


def test_argument_errors(B):
    E = B.ERR_INVALID_ARG
    assert _call2(B, n=0) == B.OK                                      # empty: no-op
    assert _call2(B, n=-1) == E
    assert _call2(B, step=0) == E and "step" in B.last_error()
    assert _call2(B, dtype=7) == E and "dtype" in B.last_error()
    assert _call2(B, nulls=(3,)) == E and "NULL" in B.last_error()
    assert _call2(B, hp=dict(optimizer="adam", blocksize=512)) == E and "blocksize" in B.last_error()
    assert _call2(B, hp=dict(optimizer="adam", beta1=1.0)) == E
    assert _call2(B, hp=dict(optimizer="adam", beta2=-0.1)) == E
    assert _call2(B, hp=dict(optimizer="adam", eps=-1.0)) == E
    assert _call2(B, hp=dict(optimizer="adam", max_unorm=-1.0)) == E
    assert _call2(B, hp=dict(optimizer="momentum")) == E and "2-state" in B.last_error()
    h = B.make_hparams(dict(optimizer="adam"))
    h.optimizer = 9
    rc = B.lib().bitopt_step_8bit_blockwise_2state(ctypes.byref(h), 1, *([ctypes.c_void_p(16)] * 2), 0, 16,
                                                   *([ctypes.c_void_p(16)] * 6), None)
    assert rc == E and "optimizer" in B.last_error()
    # 1-state entry points refuse 2-state optimizers and vice versa
    h = B.make_hparams(dict(optimizer="adam"))
    P = ctypes.c_void_p(16)
    assert B.lib().bitopt_step_8bit_blockwise_1state(ctypes.byref(h), 1, P, P, 0, 16, P, P, P, None) == E
    assert B.lib().bitopt_step_32bit_1state(ctypes.byref(h), 1, P, P, 0, 16, P, None) == E
    h = B.make_hparams(dict(optimizer="lion"))
    assert B.lib().bitopt_step_32bit_2state(ctypes.byref(h), 1, P, P, 0, 16, P, P, None) == E
    assert B.lib().bitopt_step_8bit_blockwise_1state(ctypes.byref(h), 1, P, P, 0, 0, P, P, P, None) == B.OK
    # codec
    L = B.lib()
    assert L.bitopt_quantize_blockwise(P, 0, 0, P, 256, P, P, None) == B.OK
    assert L.bitopt_quantize_blockwise(P, 0, 10, P, 100, P, P, None) == E
    assert L.bitopt_quantize_blockwise(P, 3, 10, P, 256, P, P, None) == E
    assert L.bitopt_quantize_blockwise(None, 0, 10, P, 256, P, P, None) == E
    assert L.bitopt_dequantize_blockwise(P, P, P, -5, 256, P, 0, None) == E
    assert L.bitopt_dequantize_blockwise(P, P, None, 5, 256, P, 0, None) == E
    assert L.bitopt_create_dynamic_map(1, None) == E
    assert L.bitopt_step_scalars(None, 1, P) == E
    # a successful call clears the message
    assert L.bitopt_create_dynamic_map(1, (ctypes.c_float * 256)()) == B.OK and B.last_error() == ""


def test_binding_refuses_host_tensors(B):
    import torch
    p = torch.zeros(16)
    with pytest.raises(ValueError):
        B.step_8bit_blockwise_1state(dict(optimizer="lion"), 1, p, p, torch.zeros(16, dtype=torch.uint8),
                                     torch.zeros(1), torch.zeros(256))


def test_multi_argument_errors(B):
    L = B.lib()
    E = B.ERR_INVALID_ARG
    h = B.make_hparams(dict(optimizer="adam"))
    P = ctypes.c_void_p(16)
    assert L.bitopt_multi_workspace_bytes(146) == 146 * 80
    assert L.bitopt_multi_workspace_bytes(-1) < 0
    arr = (B.Tensor * 2)()
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 0, P, P, P, 0, None) == B.OK        # empty
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, -1, P, P, P, 0, None) == E
    assert L.bitopt_step_multi(ctypes.byref(h), 1, None, 2, P, P, P, 1000, None) == E
    arr[0] = B.Tensor(16, 16, 16, 16, 16, 16, 100, 0, 1)
    arr[1] = B.Tensor(16, 16, 16, None, 16, 16, 100, 0, 1)                                  # no state2
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 2, P, P, P, 1000, None) == E and "tensor 1" in B.last_error()
    arr[1] = B.Tensor(16, 16, 16, 16, 16, None, 100, 0, 1)                                  # no absmax2
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 2, P, P, P, 1000, None) == E
    arr[1] = B.Tensor(16, 16, 16, 16, None, None, 100, 0, 0)                                # 32-bit: fine
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 2, P, P, P, 10, None) == E and "workspace" in B.last_error()
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 2, P, P, ctypes.c_void_p(24), 1000, None) == E  # misaligned
    arr[1] = B.Tensor(16, 16, 16, 16, None, None, 100, 5, 0)                                # bad dtype
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 2, P, P, P, 1000, None) == E and "dtype" in B.last_error()
    arr[1] = B.Tensor(16, 16, 16, 16, None, None, -3, 0, 0)
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 2, P, P, P, 1000, None) == E
    arr[0] = B.Tensor(16, 16, 16, 16, 16, 16, 0, 0, 1)                                      # n == 0 entries skipped
    arr[1] = B.Tensor(None, None, None, None, None, None, 0, 0, 1)
    assert L.bitopt_step_multi(ctypes.byref(h), 1, arr, 2, None, None, P, 1000, None) == B.OK


def test_tensorwise_argument_errors(B):
    L = B.lib()
    E = B.ERR_INVALID_ARG
    P = ctypes.c_void_p(16)
    assert L.bitopt_tensorwise_workspace_bytes() >= 28
    h = B.make_hparams(dict(optimizer="adam", blocksize=0))
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(h), 1, P, P, 0, 0, P, P, P, P, P, P, P, None) == B.OK
    hb = B.make_hparams(dict(optimizer="adam", blocksize=256))
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(hb), 1, P, P, 0, 16, P, P, P, P, P, P, P, None) == E
    assert "blocksize" in B.last_error()
    hu = B.make_hparams(dict(optimizer="adam", blocksize=0, max_unorm=1.0))             # tensor-wide cap: accepted
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(hu), 1, P, P, 0, 0, P, P, P, P, P, P, P, None) == B.OK
    hn = B.make_hparams(dict(optimizer="adam", blocksize=0, max_unorm=-1.0))
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(hn), 1, P, P, 0, 16, P, P, P, P, P, P, P, None) == E
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(h), 1, P, P, 0, 16, P, P, P, P, P, P, None, None) == E
    assert "NULL" in B.last_error()
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(h), 1, P, P, 0, 16, P, None, P, P, P, P, P, None) == E
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(h), 1, P, P, 0, 16, P, P, P, P, P, P,
                                         ctypes.c_void_p(18), None) == E                      # misaligned
    h1 = B.make_hparams(dict(optimizer="rmsprop", blocksize=0))                               # 1-state: no state2
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(h1), 1, P, P, 0, 0, P, None, P, None, P, None, P, None) == B.OK
    assert L.bitopt_step_8bit_tensorwise(ctypes.byref(h), 0, P, P, 0, 16, P, P, P, P, P, P, P, None) == E


def test_host_state_argument_errors(B):
    L = B.lib()
    out = ctypes.c_void_p()
    assert L.bitopt_host_state_alloc(0, ctypes.byref(out)) == B.ERR_INVALID_ARG
    assert L.bitopt_host_state_alloc(16, None) == B.ERR_INVALID_ARG
    assert L.bitopt_host_state_free(None) == B.OK


def test_multi_plan_argument_errors(B):
    """The plan calls on their argument-checking paths (no device work): every check of
    the per-tensor descriptors, the workspace, and a planned step with a different
    optimizer or blocksize than its plan."""
    L = B.lib()
    E = B.ERR_INVALID_ARG
    h = B.make_hparams(dict(optimizer="adam"))
    P = ctypes.c_void_p(16)
    plan = B.MultiPlanC()
    arr = (B.Tensor * 2)()
    assert L.bitopt_multi_plan_build(ctypes.byref(h), arr, 0, P, 0, ctypes.byref(plan), None) == B.OK
    assert plan.nlaunch == 0 and plan.count == 0
    assert L.bitopt_multi_plan_build(ctypes.byref(h), arr, 0, P, 0, None, None) == E
    assert L.bitopt_multi_plan_build(ctypes.byref(h), arr, -1, P, 0, ctypes.byref(plan), None) == E
    arr[0] = B.Tensor(16, 16, 16, None, 16, 16, 100, 0, 1)                   # no state2
    assert L.bitopt_multi_plan_build(ctypes.byref(h), arr, 1, P, 1000, ctypes.byref(plan), None) == E
    arr[0] = B.Tensor(16, 16, 16, 16, 16, 16, 100, 0, 1)
    assert L.bitopt_multi_plan_build(ctypes.byref(h), arr, 1, P, 40, ctypes.byref(plan), None) == E
    assert "workspace" in B.last_error()
    # an empty plan steps as a no-op; a plan of another optimizer / blocksize is refused
    empty = B.MultiPlanC()
    assert L.bitopt_multi_plan_build(ctypes.byref(h), arr, 0, P, 0, ctypes.byref(empty), None) == B.OK
    assert L.bitopt_step_multi_planned(ctypes.byref(empty), ctypes.byref(h), 1, None, None, None) == B.OK
    h2 = B.make_hparams(dict(optimizer="momentum"))
    assert L.bitopt_step_multi_planned(ctypes.byref(empty), ctypes.byref(h2), 1, None, None, None) == E
    h3 = B.make_hparams(dict(optimizer="adam", blocksize=2048))
    assert L.bitopt_step_multi_planned(ctypes.byref(empty), ctypes.byref(h3), 1, None, None, None) == E
    assert L.bitopt_step_multi_planned(ctypes.byref(empty), ctypes.byref(h), 0, None, None, None) == E   # step 0
    assert L.bitopt_step_multi_planned(None, ctypes.byref(h), 1, None, None, None) == E


def test_page_pool_argument_errors(B):
    """The page-pool calls on their argument-checking paths (no pool is made: every
    refusal here comes before the first device call)."""
    L = B.lib()
    E = B.ERR_INVALID_ARG
    h = B.make_hparams(dict(optimizer="adam", blocksize=256))
    fb = L.bitopt_page_pool_frame_bytes(ctypes.byref(h), 4096)
    assert fb >= 2 * 4096 + 2 * 4 * 16                               # two code arrays and two absmax arrays
    assert fb % 256 == 0
    assert L.bitopt_page_pool_frame_bytes(ctypes.byref(h), 4000) < 0      # not a multiple of 4096
    assert L.bitopt_page_pool_frame_bytes(ctypes.byref(h), 0) < 0
    assert L.bitopt_page_pool_frame_bytes(None, 4096) < 0
    hm = B.make_hparams(dict(optimizer="momentum", blocksize=2048))
    assert 4096 <= L.bitopt_page_pool_frame_bytes(ctypes.byref(hm), 4096) < fb   # one state
    pool = ctypes.c_void_p()
    F = ctypes.c_void_p(1 << 20)
    assert L.bitopt_page_pool_create(ctypes.byref(h), 4096, F, 2 * fb, None) == E
    assert L.bitopt_page_pool_create(ctypes.byref(h), 4000, F, 2 * fb, ctypes.byref(pool)) == E
    assert "multiple" in B.last_error() and not pool.value
    assert L.bitopt_page_pool_create(ctypes.byref(h), 4096, None, 2 * fb, ctypes.byref(pool)) == E
    assert L.bitopt_page_pool_create(ctypes.byref(h), 4096, ctypes.c_void_p((1 << 20) + 64), 2 * fb,
                                     ctypes.byref(pool)) == E
    assert L.bitopt_page_pool_create(ctypes.byref(h), 4096, F, 2 * fb - 1, ctypes.byref(pool)) == E
    assert "at least 2" in B.last_error()
    P = ctypes.c_void_p(16)
    assert L.bitopt_step_8bit_pooled(None, ctypes.byref(h), 1, P, P, 0, 16, P, P, P, P, P, P, None) == E
    assert L.bitopt_page_pool_flush(None, 0, None) == E
    assert L.bitopt_page_pool_stats(None, (ctypes.c_int64 * 4)()) == E
    assert L.bitopt_page_pool_destroy(None) == B.OK


def test_device_scalars_layout_and_errors(B):
    """The device-form scalars hold the 14 host scalars first, in the order
    bitopt_step_scalars gives them (the kernels' struct); argument checks of the
    device-scalar planned step (no launch)."""
    L = B.lib()
    E = B.ERR_INVALID_ARG
    nbytes = L.bitopt_device_scalars_bytes()
    assert 14 * 4 <= nbytes <= 64
    for hp in (dict(optimizer="adam", lr=1e-3, weight_decay=0.01), dict(optimizer="ademamix", t_alpha=5, t_beta3=5,
                                                                       alpha=5.0)):
        h = B.make_hparams(hp)
        for t in (1, 3, 1000):
            out = (ctypes.c_uint8 * nbytes)()
            assert L.bitopt_device_scalars_write(ctypes.byref(h), t, out, nbytes) == B.OK
            host = (ctypes.c_float * 14)()
            assert L.bitopt_step_scalars(ctypes.byref(h), t, host) == B.OK
            got = np.frombuffer(bytes(out), np.float32)[:14]
            np.testing.assert_array_equal(got.view(np.uint32), np.frombuffer(bytes(host), np.uint32))
    h = B.make_hparams(dict(optimizer="adam"))
    out = (ctypes.c_uint8 * nbytes)()
    assert L.bitopt_device_scalars_write(ctypes.byref(h), 1, out, nbytes - 1) == E
    assert L.bitopt_device_scalars_write(ctypes.byref(h), 0, out, nbytes) == E
    assert L.bitopt_device_scalars_write(ctypes.byref(h), 1, None, nbytes) == E
    empty = B.MultiPlanC()
    arr = (B.Tensor * 1)()
    P = ctypes.c_void_p(16)
    assert L.bitopt_multi_plan_build(ctypes.byref(h), arr, 0, P, 0, ctypes.byref(empty), None) == B.OK
    S = ctypes.c_void_p(256)
    assert L.bitopt_step_multi_planned_dscalars(ctypes.byref(empty), ctypes.byref(h), S, None, None, None) == B.OK
    assert L.bitopt_step_multi_planned_dscalars(ctypes.byref(empty), ctypes.byref(h), None, None, None, None) == E
    assert L.bitopt_step_multi_planned_dscalars(ctypes.byref(empty), ctypes.byref(h), ctypes.c_void_p(260), None,
                                                None, None) == E
    h2 = B.make_hparams(dict(optimizer="momentum"))
    assert L.bitopt_step_multi_planned_dscalars(ctypes.byref(empty), ctypes.byref(h2), S, None, None, None) == E
    assert L.bitopt_step_multi_planned_dscalars(None, ctypes.byref(h), S, None, None, None) == E
