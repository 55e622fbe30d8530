"""ctypes wrapper of the plain C oracle (oracle/bitopt_oracle.c).

TEST INFRASTRUCTURE ONLY.  The oracle is the slow, obviously-correct CPU statement
of the 8-bit block-wise optimizer step and its codec.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the product
library (bit_optimizers_block_amd) never does.

Arrays are numpy.  Parameter/gradient dtypes: "f32" (float32), "f16" (float16) and
"bf16" (uint16 arrays holding bfloat16 bit patterns).
"""
import ctypes
import os

import numpy as np

from . import build as _build

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
OPTIMIZERS = {"adam": 0, "adamw": 0, "ademamix": 1, "momentum": 2, "lion": 3, "rmsprop": 4, "adagrad": 5}
NUM_STATES = {"adam": 2, "adamw": 2, "ademamix": 3, "momentum": 1, "lion": 1, "rmsprop": 1, "adagrad": 1}
# optimizers whose single state is non-negative (encoded with the unsigned map)
UNSIGNED_STATE1 = ("rmsprop", "adagrad")


class _HParams(ctypes.Structure):
    _fields_ = [
        ("optimizer", ctypes.c_int32),
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("beta3", ctypes.c_float), ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
        ("alpha", ctypes.c_float),
        ("t_alpha", ctypes.c_int32), ("t_beta3", ctypes.c_int32),
        ("max_unorm", ctypes.c_float),
        ("skip_zeros", ctypes.c_int32),
        ("blocksize", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # BITOPT_ORACLE_LIB: a separately built oracle (the mutation test of the pins
        # loads deliberately broken builds this way, each in its own process)
        path = os.environ.get("BITOPT_ORACLE_LIB") or _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.oref_dynamic_map.argtypes = [ctypes.c_int, P]
        L.oref_nearest.argtypes = [P, P, i64, P]
        L.oref_quantize_blockwise.argtypes = [P, ctypes.c_int, i64, P, i32, P, P]
        L.oref_dequantize_blockwise.argtypes = [P, P, P, i64, i32, P, ctypes.c_int]
        L.oref_round_to_dtype.argtypes = [P, i64, ctypes.c_int, P]
        L.oref_widen_from_dtype.argtypes = [P, i64, ctypes.c_int, P]
        L.oref_beta3_schedule.argtypes = [ctypes.c_double, ctypes.c_double, i32, i32]
        L.oref_beta3_schedule.restype = ctypes.c_double
        L.oref_alpha_schedule.argtypes = [ctypes.c_double, i32, i32]
        L.oref_alpha_schedule.restype = ctypes.c_double
        L.oref_step_scalars.argtypes = [P, i32, P]
        L.oref_step_8bit.argtypes = [P, i32, P, P, ctypes.c_int, i64, P, P, P, P, P, P, P, i64]
        L.oref_step_32bit.argtypes = [P, i32, P, P, ctypes.c_int, i64, P, P, P, i64]
        L.oref_set_threads.argtypes = [ctypes.c_int]
        L.oref_get_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, name):
    if a is None:
        return
    if not (isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"] and a.dtype == dtype):
        raise TypeError(f"{name}: expected C-contiguous {np.dtype(dtype)} ndarray, got "
                        f"{getattr(a, 'dtype', type(a))}")


def _param_np_dtype(dtype):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def hparams(hp: dict) -> _HParams:
    """Fill the oracle's hyper-parameter struct from a plain dict."""
    h = _HParams()
    h.optimizer = OPTIMIZERS[hp["optimizer"]]
    h.lr = hp.get("lr", 1e-3)
    h.beta1 = hp.get("beta1", 0.9)
    h.beta2 = hp.get("beta2", 0.999)
    h.beta3 = hp.get("beta3", 0.9999)
    h.eps = hp.get("eps", 1e-8)
    h.weight_decay = hp.get("weight_decay", 0.0)
    h.alpha = hp.get("alpha", 0.0)
    h.t_alpha = hp.get("t_alpha") or 0
    h.t_beta3 = hp.get("t_beta3") or 0
    h.max_unorm = hp.get("max_unorm", 0.0)
    h.skip_zeros = 1 if hp.get("skip_zeros", False) else 0
    h.blocksize = hp.get("blocksize", 256)
    return h


def set_threads(n: int) -> None:
    lib().oref_set_threads(int(n))


def get_threads() -> int:
    return lib().oref_get_threads()


def dynamic_map(signed: bool) -> np.ndarray:
    out = np.empty(256, np.float32)
    lib().oref_dynamic_map(1 if signed else 0, _ptr(out))
    return out


def nearest(qmap: np.ndarray, x: np.ndarray) -> np.ndarray:
    _check(qmap, np.float32, "qmap")
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oref_nearest(_ptr(qmap), _ptr(x), x.size, _ptr(out))
    return out


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, _param_np_dtype(dtype))
    lib().oref_round_to_dtype(_ptr(x), x.size, DTYPES[dtype], _ptr(out))
    return out


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    _check(x, _param_np_dtype(dtype), "x")
    out = np.empty(x.shape, np.float32)
    lib().oref_widen_from_dtype(_ptr(x), x.size, DTYPES[dtype], _ptr(out))
    return out


def quantize_blockwise(x: np.ndarray, dtype: str, qmap: np.ndarray, blocksize: int):
    _check(x, _param_np_dtype(dtype), "x")
    _check(qmap, np.float32, "qmap")
    n = x.size
    nb = (n + blocksize - 1) // blocksize
    codes = np.zeros(n, np.uint8)
    absmax = np.zeros(nb, np.float32)
    rc = lib().oref_quantize_blockwise(_ptr(x), DTYPES[dtype], n, _ptr(qmap), blocksize,
                                       _ptr(codes), _ptr(absmax))
    if rc:
        raise ValueError("oref_quantize_blockwise: invalid arguments")
    return codes, absmax


def dequantize_blockwise(codes, absmax, qmap, blocksize: int, dtype: str = "f32"):
    _check(codes, np.uint8, "codes")
    _check(absmax, np.float32, "absmax")
    out = np.empty(codes.size, _param_np_dtype(dtype))
    rc = lib().oref_dequantize_blockwise(_ptr(codes), _ptr(absmax), _ptr(qmap), codes.size,
                                         blocksize, _ptr(out), DTYPES[dtype])
    if rc:
        raise ValueError("oref_dequantize_blockwise: invalid arguments")
    return out


def beta3_schedule(beta1, beta3, t, T):
    return lib().oref_beta3_schedule(float(beta1), float(beta3), int(t), int(T or 0))


def alpha_schedule(alpha, t, T):
    return lib().oref_alpha_schedule(float(alpha), int(t), int(T or 0))


def step_scalars(hp: dict, t: int) -> dict:
    h = hparams(hp)
    out = np.empty(13, np.float32)
    lib().oref_step_scalars(ctypes.byref(h), int(t), _ptr(out))
    names = ["lr", "b1", "b2", "eps", "wd", "omb1", "omb2", "ic1", "rs2", "decay",
             "b3t", "omb3", "alpha_t"]
    return dict(zip(names, out.tolist()))


def _blocks_arg(blocks):
    if blocks is None:
        return None, 0
    b = np.ascontiguousarray(blocks, np.int64)
    return b, b.size


def step_8bit(hp, step, p, g, dtype, state1, absmax1, qmap1,
              state2=None, absmax2=None, qmap2=None, blocks=None):
    """One 8-bit block-wise step, in place on p / states / absmax."""
    pt = _param_np_dtype(dtype)
    _check(p, pt, "p"); _check(g, pt, "g")
    _check(state1, np.uint8, "state1"); _check(state2, np.uint8, "state2")
    _check(absmax1, np.float32, "absmax1"); _check(absmax2, np.float32, "absmax2")
    _check(qmap1, np.float32, "qmap1"); _check(qmap2, np.float32, "qmap2")
    if p.size != g.size:
        raise ValueError("p and g sizes differ")
    h = hparams(hp)
    b, nbl = _blocks_arg(blocks)
    rc = lib().oref_step_8bit(ctypes.byref(h), int(step), _ptr(p), _ptr(g), DTYPES[dtype], p.size,
                              _ptr(state1), _ptr(state2), _ptr(absmax1), _ptr(absmax2),
                              _ptr(qmap1), _ptr(qmap2), _ptr(b), nbl)
    if rc:
        raise ValueError("oref_step_8bit: invalid arguments")


def step_32bit(hp, step, p, g, dtype, state1, state2=None, blocks=None):
    """One 32-bit step (fp32 states, no codec), in place."""
    pt = _param_np_dtype(dtype)
    _check(p, pt, "p"); _check(g, pt, "g")
    _check(state1, np.float32, "state1"); _check(state2, np.float32, "state2")
    h = hparams(hp)
    b, nbl = _blocks_arg(blocks)
    rc = lib().oref_step_32bit(ctypes.byref(h), int(step), _ptr(p), _ptr(g), DTYPES[dtype], p.size,
                               _ptr(state1), _ptr(state2), _ptr(b), nbl)
    if rc:
        raise ValueError("oref_step_32bit: invalid arguments")
