"""ctypes binding of libbitopt.so (include/bitopt.h), argument marshalling only.

Every function takes torch tensors (device tensors for device entry points),
checks shapes/dtypes/devices, passes raw pointers and the current HIP stream to
the C ABI, and raises BitoptError on a non-zero status.  All arithmetic of the
step runs in the library's HIP kernels; if the library is not built, loading
fails with an error instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbitopt.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_DEVICE = 0, -1, -2, -3
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
OPTIMIZERS = {"adam": 0, "adamw": 0, "ademamix": 1, "momentum": 2, "lion": 3, "rmsprop": 4, "adagrad": 5}
TWO_STATE = ("adam", "adamw", "ademamix")
SCALAR_NAMES = ["lr", "b1", "b2", "eps", "wd", "omb1", "omb2", "ic1", "rs2", "decay",
                "b3t", "omb3", "alpha_t", "max_unorm"]


class BitoptError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class HParams(ctypes.Structure):
    """Mirror of bitopt_hparams."""
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


def make_hparams(hp: dict) -> HParams:
    """bitopt_hparams from a dict; missing keys take the Optimizer2State defaults."""
    if isinstance(hp, HParams):
        return hp
    h = HParams()
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


class Tensor(ctypes.Structure):
    """Mirror of bitopt_tensor."""
    _fields_ = [
        ("p", ctypes.c_void_p), ("g", ctypes.c_void_p),
        ("state1", ctypes.c_void_p), ("state2", ctypes.c_void_p),
        ("absmax1", ctypes.c_void_p), ("absmax2", ctypes.c_void_p),
        ("n", ctypes.c_int64), ("dtype", ctypes.c_int32), ("is_8bit", ctypes.c_int32),
    ]


class MultiLaunch(ctypes.Structure):
    """Mirror of bitopt_multi_launch."""
    _fields_ = [("kind8", ctypes.c_int32), ("dtype", ctypes.c_int32), ("first", ctypes.c_int32),
                ("count", ctypes.c_int32), ("tiles", ctypes.c_int64)]


MULTI_MAX_LAUNCHES = 64


class MultiPlanC(ctypes.Structure):
    """Mirror of bitopt_multi_plan."""
    _fields_ = [("optimizer", ctypes.c_int32), ("blocksize", ctypes.c_int32), ("count", ctypes.c_int32),
                ("nlaunch", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("launch", MultiLaunch * MULTI_MAX_LAUNCHES)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "or python bit_optimizers_block_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        HP = ctypes.POINTER(HParams)
        sigs = {
            "bitopt_last_error": ([], ctypes.c_char_p),
            "bitopt_abi_version": ([], i32),
            "bitopt_create_dynamic_map": ([ctypes.c_int, P], ctypes.c_int),
            "bitopt_step_scalars": ([HP, i32, P], ctypes.c_int),
            "bitopt_quantize_blockwise": ([P, i32, i64, P, i32, P, P, P], ctypes.c_int),
            "bitopt_dequantize_blockwise": ([P, P, P, i64, i32, P, i32, P], ctypes.c_int),
            "bitopt_step_8bit_blockwise_2state": ([HP, i32, P, P, i32, i64, P, P, P, P, P, P, P], ctypes.c_int),
            "bitopt_step_8bit_blockwise_1state": ([HP, i32, P, P, i32, i64, P, P, P, P], ctypes.c_int),
            "bitopt_step_32bit_2state": ([HP, i32, P, P, i32, i64, P, P, P], ctypes.c_int),
            "bitopt_step_32bit_1state": ([HP, i32, P, P, i32, i64, P, P], ctypes.c_int),
            "bitopt_multi_workspace_bytes": ([i32], i64),
            "bitopt_tensorwise_workspace_bytes": ([], i64),
            "bitopt_host_state_alloc": ([i64, ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
            "bitopt_host_state_free": ([P], ctypes.c_int),
            "bitopt_step_8bit_tensorwise": ([HP, i32, P, P, i32, i64, P, P, P, P, P, P, P, P], ctypes.c_int),
            "bitopt_step_8bit_tensorwise_noalloc": ([HP, i32, P, P, i32, i64, P, P, P, P, P, P, P], ctypes.c_int),
            "bitopt_tensorwise_scratch_bytes": ([], i64),
            "bitopt_paged_staging_bytes": ([HP, i64], i64),
            "bitopt_step_8bit_paged": ([HP, i32, P, P, i32, i64, P, P, P, P, P, P, P, i64, P, P, P], ctypes.c_int),
            "bitopt_page_pool_frame_bytes": ([HP, i64], i64),
            "bitopt_page_pool_create": ([HP, i64, P, i64, ctypes.POINTER(P)], ctypes.c_int),
            "bitopt_page_pool_destroy": ([P], ctypes.c_int),
            "bitopt_step_8bit_pooled": ([P, HP, i32, P, P, i32, i64, P, P, P, P, P, P, P], ctypes.c_int),
            "bitopt_page_pool_flush": ([P, i32, P], ctypes.c_int),
            "bitopt_page_pool_stats": ([P, ctypes.POINTER(i64)], ctypes.c_int),
            "bitopt_step_multi": ([HP, i32, ctypes.POINTER(Tensor), i32, P, P, P, i64, P], ctypes.c_int),
            "bitopt_multi_plan_build": ([HP, ctypes.POINTER(Tensor), i32, P, i64, ctypes.POINTER(MultiPlanC), P],
                                        ctypes.c_int),
            "bitopt_step_multi_planned": ([ctypes.POINTER(MultiPlanC), HP, i32, P, P, P], ctypes.c_int),
            "bitopt_device_scalars_bytes": ([], i64),
            "bitopt_device_scalars_write": ([HP, i32, P, i64], ctypes.c_int),
            "bitopt_step_multi_planned_dscalars": ([ctypes.POINTER(MultiPlanC), HP, P, P, P, P], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def last_error() -> str:
    return lib().bitopt_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise BitoptError(rc, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# --------------------------------------------------------------- state outside HBM

_host_states = {}     # address -> bytes of live bitopt_host_state_alloc buffers


def _free_host_state(ptr):
    _host_states.pop(ptr, None)
    lib().bitopt_host_state_free(ctypes.c_void_p(ptr))


def host_state(numel: int, dtype=torch.uint8) -> torch.Tensor:
    """A CPU tensor over pinned host memory mapped into the GPU address space
    (bitopt_host_state_alloc): optimizer state kept outside HBM, which every step
    accepts in place of device state.  The memory is freed when the tensor is
    garbage-collected; synchronize the streams that use it before dropping it."""
    import weakref
    import numpy as np
    nbytes = int(numel) * torch.empty(0, dtype=dtype).element_size()
    ptr = ctypes.c_void_p()
    _check(lib().bitopt_host_state_alloc(max(nbytes, 1), ctypes.byref(ptr)))
    buf = (ctypes.c_uint8 * max(nbytes, 1)).from_address(ptr.value)
    arr = np.frombuffer(buf, dtype=np.uint8)[:nbytes]
    _host_states[ptr.value] = max(nbytes, 1)
    weakref.finalize(buf, _free_host_state, ptr.value)
    return torch.from_numpy(arr).view(dtype)


def _is_host_state(t) -> bool:
    a = t.data_ptr()
    return any(p <= a and a + t.numel() * t.element_size() <= p + n for p, n in _host_states.items())


def _need(t, name, dtype=None, numel=None, device=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device == "state":
        if not (t.is_cuda or _is_host_state(t)):
            raise ValueError(f"{name} must be a device tensor or a host_state() tensor")
    elif device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")


def _dt(t):
    if t.dtype not in DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return DTYPES[t.dtype]


def abi_version() -> int:
    return lib().bitopt_abi_version()


def create_dynamic_map(signed: bool = True) -> torch.Tensor:
    """The 256-entry dynamic-exponent codebook (host fp32 tensor)."""
    out = torch.empty(256, dtype=torch.float32)
    _check(lib().bitopt_create_dynamic_map(1 if signed else 0, _ptr(out)))
    return out


def step_scalars(hp, step: int) -> dict:
    h = make_hparams(hp)
    out = torch.empty(14, dtype=torch.float32)
    _check(lib().bitopt_step_scalars(ctypes.byref(h), int(step), _ptr(out)))
    return dict(zip(SCALAR_NAMES, out.tolist()))


def nblocks(n: int, blocksize: int) -> int:
    return (n + blocksize - 1) // blocksize


def quantize_blockwise(x, qmap, blocksize: int = 256, codes=None, absmax=None, stream=None):
    n = x.numel()
    _need(x, "x"); _need(qmap, "qmap", torch.float32, 256)
    if codes is None:
        codes = torch.empty(n, dtype=torch.uint8, device=x.device)
    if absmax is None:
        absmax = torch.empty(nblocks(n, blocksize), dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8, n); _need(absmax, "absmax", torch.float32, nblocks(n, blocksize))
    _check(lib().bitopt_quantize_blockwise(_ptr(x), _dt(x), n, _ptr(qmap), blocksize, _ptr(codes),
                                           _ptr(absmax), _stream(stream)))
    return codes, absmax


def dequantize_blockwise(codes, absmax, qmap, blocksize: int = 256, out=None, dtype=torch.float32, stream=None):
    n = codes.numel()
    _need(codes, "codes", torch.uint8); _need(qmap, "qmap", torch.float32, 256)
    _need(absmax, "absmax", torch.float32, nblocks(n, blocksize))
    if out is None:
        out = torch.empty(n, dtype=dtype, device=codes.device)
    _need(out, "out", numel=n)
    _check(lib().bitopt_dequantize_blockwise(_ptr(codes), _ptr(absmax), _ptr(qmap), n, blocksize,
                                             _ptr(out), _dt(out), _stream(stream)))
    return out


def step_8bit_blockwise_2state(hp, step, p, g, state1, state2, absmax1, absmax2, qmap1, qmap2, stream=None):
    h = make_hparams(hp)
    n = p.numel()
    k = 2 if h.optimizer == OPTIMIZERS["ademamix"] else 1
    nb = nblocks(n, h.blocksize)
    _need(p, "p"); _need(g, "g", p.dtype, n)
    _need(state1, "state1", torch.uint8, k * n, device="state"); _need(state2, "state2", torch.uint8, n, device="state")
    _need(absmax1, "absmax1", torch.float32, k * nb, device="state"); _need(absmax2, "absmax2", torch.float32, nb, device="state")
    _need(qmap1, "qmap1", torch.float32, 256); _need(qmap2, "qmap2", torch.float32, 256)
    _check(lib().bitopt_step_8bit_blockwise_2state(ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n,
                                                   _ptr(state1), _ptr(state2), _ptr(absmax1), _ptr(absmax2),
                                                   _ptr(qmap1), _ptr(qmap2), _stream(stream)))


def step_8bit_blockwise_1state(hp, step, p, g, state1, absmax1, qmap1, stream=None):
    h = make_hparams(hp)
    n = p.numel()
    _need(p, "p"); _need(g, "g", p.dtype, n)
    _need(state1, "state1", torch.uint8, n, device="state"); _need(absmax1, "absmax1", torch.float32, nblocks(n, h.blocksize), device="state")
    _need(qmap1, "qmap1", torch.float32, 256)
    _check(lib().bitopt_step_8bit_blockwise_1state(ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n,
                                                   _ptr(state1), _ptr(absmax1), _ptr(qmap1), _stream(stream)))


def step_32bit_2state(hp, step, p, g, state1, state2, stream=None):
    h = make_hparams(hp)
    n = p.numel()
    k = 2 if h.optimizer == OPTIMIZERS["ademamix"] else 1
    _need(p, "p"); _need(g, "g", p.dtype, n)
    _need(state1, "state1", torch.float32, k * n, device="state"); _need(state2, "state2", torch.float32, n, device="state")
    _check(lib().bitopt_step_32bit_2state(ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n,
                                          _ptr(state1), _ptr(state2), _stream(stream)))


def step_32bit_1state(hp, step, p, g, state1, stream=None):
    h = make_hparams(hp)
    n = p.numel()
    _need(p, "p"); _need(g, "g", p.dtype, n); _need(state1, "state1", torch.float32, n, device="state")
    _check(lib().bitopt_step_32bit_1state(ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n,
                                          _ptr(state1), _stream(stream)))


def tensorwise_workspace_bytes() -> int:
    return lib().bitopt_tensorwise_workspace_bytes()


def step_8bit_tensorwise(hp, step, p, g, state1, absmax1, qmap1, state2=None, absmax2=None, qmap2=None,
                         workspace=None, stream=None):
    """Non-block-wise 8-bit step (hp blocksize 0): one absmax per state for the whole
    tensor.  Returns the workspace tensor used (pass it back to reuse it)."""
    h = make_hparams(hp)
    n = p.numel()
    k = 2 if h.optimizer == OPTIMIZERS["ademamix"] else 1
    two = h.optimizer in (OPTIMIZERS["adam"], OPTIMIZERS["ademamix"])
    _need(p, "p"); _need(g, "g", p.dtype, n)
    _need(state1, "state1", torch.uint8, k * n, device="state"); _need(absmax1, "absmax1", torch.float32, k, device="state")
    _need(qmap1, "qmap1", torch.float32, 256)
    if two:
        _need(state2, "state2", torch.uint8, n, device="state"); _need(absmax2, "absmax2", torch.float32, 1, device="state")
        _need(qmap2, "qmap2", torch.float32, 256)
    if workspace is None:
        workspace = torch.empty(tensorwise_workspace_bytes(), dtype=torch.uint8, device=p.device)
    _check(lib().bitopt_step_8bit_tensorwise(ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n,
                                             _ptr(state1), _ptr(state2), _ptr(absmax1), _ptr(absmax2),
                                             _ptr(qmap1), _ptr(qmap2), _ptr(workspace), _stream(stream)))
    return workspace


def step_8bit_tensorwise_noalloc(hp, step, p, g, state1, absmax1, qmap1, state2=None, absmax2=None, qmap2=None,
                                 stream=None):
    """The tensor-wide step with the library's own scratch array as its workspace
    (no device allocation by the call; calls that overlap on one GPU race)."""
    h = make_hparams(hp)
    n = p.numel()
    k = 2 if h.optimizer == OPTIMIZERS["ademamix"] else 1
    two = h.optimizer in (OPTIMIZERS["adam"], OPTIMIZERS["ademamix"])
    _need(p, "p"); _need(g, "g", p.dtype, n)
    _need(state1, "state1", torch.uint8, k * n, device="state"); _need(absmax1, "absmax1", torch.float32, k, device="state")
    _need(qmap1, "qmap1", torch.float32, 256)
    if two:
        _need(state2, "state2", torch.uint8, n, device="state"); _need(absmax2, "absmax2", torch.float32, 1, device="state")
        _need(qmap2, "qmap2", torch.float32, 256)
    _check(lib().bitopt_step_8bit_tensorwise_noalloc(ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n,
                                                     _ptr(state1), _ptr(state2), _ptr(absmax1), _ptr(absmax2),
                                                     _ptr(qmap1), _ptr(qmap2), _stream(stream)))


def paged_staging_bytes(hp, chunk_elems: int) -> int:
    return lib().bitopt_paged_staging_bytes(ctypes.byref(make_hparams(hp)), int(chunk_elems))


def step_8bit_paged(hp, step, p, g, state1, absmax1, qmap1, state2=None, absmax2=None, qmap2=None,
                    staging=None, h2d_stream=None, d2h_stream=None, stream=None):
    """8-bit step with the state in host memory (host_state() tensors), paged through
    a device staging buffer chunk by chunk (bitopt_step_8bit_paged).  h2d_stream and
    d2h_stream: torch streams distinct from the step stream.  Returns the staging
    tensor used (pass it back to reuse it)."""
    h = make_hparams(hp)
    n = p.numel()
    k = 2 if h.optimizer == OPTIMIZERS["ademamix"] else 1
    two = h.optimizer in (OPTIMIZERS["adam"], OPTIMIZERS["ademamix"])
    nb = nblocks(n, h.blocksize)
    _need(p, "p"); _need(g, "g", p.dtype, n)
    for t, name, dt, cnt in ((state1, "state1", torch.uint8, k * n), (absmax1, "absmax1", torch.float32, k * nb)) + (
            ((state2, "state2", torch.uint8, n), (absmax2, "absmax2", torch.float32, nb)) if two else ()):
        _need(t, name, dt, cnt, device=False)
        if t.is_cuda:
            raise ValueError(f"{name} must be host memory (host_state())")
    if staging is None:
        staging = torch.empty(paged_staging_bytes(hp, min(n, 1 << 22)), dtype=torch.uint8, device=p.device)
    if h2d_stream is None or d2h_stream is None:
        raise ValueError("step_8bit_paged needs two copy streams")
    _check(lib().bitopt_step_8bit_paged(ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n, _ptr(state1),
                                        _ptr(state2), _ptr(absmax1), _ptr(absmax2), _ptr(qmap1), _ptr(qmap2),
                                        _ptr(staging), staging.numel(), _stream(h2d_stream), _stream(d2h_stream),
                                        _stream(stream)))
    return staging


def page_pool_frame_bytes(hp, page_elems: int) -> int:
    return lib().bitopt_page_pool_frame_bytes(ctypes.byref(make_hparams(hp)), int(page_elems))


class PagePool:
    """An HBM page pool in front of host-resident 8-bit state (bitopt_page_pool_*):
    pages stay in its frames while they fit and are written back and replaced, least
    recently used first, when they do not.  `frames` is a device uint8 tensor (made
    for `nframes` frames when not given); the pool keeps it alive."""

    def __init__(self, hp, page_elems: int, nframes: int = None, frames=None, device="cuda"):
        self.hp = dict(hp)
        fb = page_pool_frame_bytes(hp, page_elems)
        if fb < 0:
            raise ValueError(f"invalid page pool arguments (page_elems={page_elems})")
        if frames is None:
            frames = torch.empty(fb * int(nframes), dtype=torch.uint8, device=device)
        self.frames = frames
        self.page_elems = int(page_elems)
        self.frame_bytes = fb
        h = ctypes.c_void_p()
        _check(lib().bitopt_page_pool_create(ctypes.byref(make_hparams(hp)), self.page_elems, _ptr(frames),
                                             frames.numel() * frames.element_size(), ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("the page pool is closed")
        return self._h

    def step(self, hp, step, p, g, state1, absmax1, qmap1, state2=None, absmax2=None, qmap2=None, stream=None):
        """One 8-bit step on host_state() buffers through the pool."""
        h = make_hparams(hp)
        n = p.numel()
        k = 2 if h.optimizer == OPTIMIZERS["ademamix"] else 1
        two = h.optimizer in (OPTIMIZERS["adam"], OPTIMIZERS["ademamix"])
        nb = nblocks(n, h.blocksize)
        _need(p, "p"); _need(g, "g", p.dtype, n)
        for t, name, dt, cnt in ((state1, "state1", torch.uint8, k * n),
                                 (absmax1, "absmax1", torch.float32, k * nb)) + (
                ((state2, "state2", torch.uint8, n), (absmax2, "absmax2", torch.float32, nb)) if two else ()):
            _need(t, name, dt, cnt, device=False)
            if t.is_cuda:
                raise ValueError(f"{name} must be host memory (host_state())")
        _check(lib().bitopt_step_8bit_pooled(self.handle, ctypes.byref(h), int(step), _ptr(p), _ptr(g), _dt(p), n,
                                             _ptr(state1), _ptr(state2), _ptr(absmax1), _ptr(absmax2), _ptr(qmap1),
                                             _ptr(qmap2), _stream(stream)))

    def flush(self, evict: bool = False, stream=None):
        _check(lib().bitopt_page_pool_flush(self.handle, 1 if evict else 0, _stream(stream)))

    def stats(self) -> dict:
        out = (ctypes.c_int64 * 4)()
        _check(lib().bitopt_page_pool_stats(self.handle, out))
        return dict(resident=out[0], page_ins=out[1], write_backs=out[2], hits=out[3])

    def close(self):
        if self._h is not None:
            h, self._h = self._h, None
            _check(lib().bitopt_page_pool_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def multi_workspace_bytes(count: int) -> int:
    return lib().bitopt_multi_workspace_bytes(int(count))


def _tensor_array(h, tensors):
    """bitopt_tensor descriptors of a list of dicts (keys p, g, state1, state2,
    absmax1, absmax2, is_8bit), with their shapes and dtypes checked."""
    two = h.optimizer in (OPTIMIZERS["adam"], OPTIMIZERS["ademamix"])
    k = 2 if h.optimizer == OPTIMIZERS["ademamix"] else 1
    arr = (Tensor * max(1, len(tensors)))()
    dev = None
    for i, t in enumerate(tensors):
        p, g = t["p"], t["g"]
        n = p.numel()
        nb = nblocks(n, h.blocksize)
        eight = bool(t.get("is_8bit", True))
        _need(p, "p"); _need(g, "g", p.dtype, n)
        sdt = torch.uint8 if eight else torch.float32
        _need(t["state1"], "state1", sdt, k * n, device="state")
        if two:
            _need(t["state2"], "state2", sdt, n, device="state")
        if eight:
            _need(t["absmax1"], "absmax1", torch.float32, k * nb, device="state")
            if two:
                _need(t["absmax2"], "absmax2", torch.float32, nb, device="state")
        arr[i] = Tensor(p.data_ptr(), g.data_ptr(), t["state1"].data_ptr(),
                        t["state2"].data_ptr() if two else None,
                        t["absmax1"].data_ptr() if eight else None,
                        t["absmax2"].data_ptr() if (eight and two) else None,
                        n, _dt(p), 1 if eight else 0)
        dev = p.device
    return arr, dev


class MultiPlan:
    """A built multi-tensor plan (bitopt_multi_plan_build): the host struct, its device
    workspace, and references to the tensors it names (kept alive with it)."""

    def __init__(self, hp, tensors, workspace=None, stream=None):
        h = make_hparams(hp)
        arr, dev = _tensor_array(h, tensors)
        need = multi_workspace_bytes(len(tensors))
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.c = MultiPlanC()
        self.workspace = workspace
        self.tensors = list(tensors)
        _check(lib().bitopt_multi_plan_build(ctypes.byref(h), arr, len(tensors), _ptr(workspace),
                                             workspace.numel(), ctypes.byref(self.c), _stream(stream)))

    def step(self, hp, step, qmap1=None, qmap2=None, stream=None):
        h = make_hparams(hp)
        _check(lib().bitopt_step_multi_planned(ctypes.byref(self.c), ctypes.byref(h), int(step), _ptr(qmap1),
                                               _ptr(qmap2), _stream(stream)))

    def step_dscalars(self, hp, scalars, qmap1=None, qmap2=None, stream=None):
        """The planned step with its per-step scalars read from `scalars` (a device
        uint8 tensor of device_scalars_bytes() bytes, see device_scalars) when the
        kernels run: a captured graph of this call steps with the buffer's contents
        at each replay."""
        h = make_hparams(hp)
        _need(scalars, "scalars", torch.uint8)
        if scalars.numel() < device_scalars_bytes():
            raise ValueError("scalars is too small")
        _check(lib().bitopt_step_multi_planned_dscalars(ctypes.byref(self.c), ctypes.byref(h), _ptr(scalars),
                                                        _ptr(qmap1), _ptr(qmap2), _stream(stream)))


def device_scalars_bytes() -> int:
    return int(lib().bitopt_device_scalars_bytes())


def device_scalars(hp, step) -> torch.Tensor:
    """The per-step scalars of (hp, step) in the kernels' device layout, as a CPU uint8
    tensor (copy it into the device buffer that step_dscalars reads)."""
    out = torch.empty(device_scalars_bytes(), dtype=torch.uint8)
    _check(lib().bitopt_device_scalars_write(ctypes.byref(make_hparams(hp)), int(step), _ptr(out), out.numel()))
    return out


def step_multi(hp, step, tensors, qmap1=None, qmap2=None, workspace=None, stream=None):
    """One step over many tensors (plan and step in one call; it waits for the
    descriptor copy -- a training loop builds a MultiPlan once instead).  `tensors`:
    list of dicts with keys p, g, state1, state2, absmax1, absmax2 (torch tensors or
    None) and is_8bit (bool).  Returns the workspace tensor used (pass it back to
    reuse it)."""
    h = make_hparams(hp)
    arr, dev = _tensor_array(h, tensors)
    need = multi_workspace_bytes(len(tensors))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib().bitopt_step_multi(ctypes.byref(h), int(step), arr, len(tensors), _ptr(qmap1), _ptr(qmap2),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace
