"""Seeded synthetic workloads: shapes, hyper-parameters and input generators.

This module holds no arithmetic of the optimizer method.  It draws the inputs
(parameters, gradients, zero-row masks) that the HIP path and the CPU oracle
both consume, so the two always see identical bytes.

Generator.  Element i of a stream belongs to chunk i // CHUNK; chunk c is drawn as
fp32 standard normals from numpy's PCG64 seeded with SeedSequence(words + [c]),
then multiplied by the scale in fp32.  Any element range can therefore be
regenerated on its own (the oracle only needs the blocks it checks), and the
values do not depend on how many threads fill the chunks.  fp16/bf16 inputs are
the fp32 samples rounded to nearest-even.

"N(0, s)" in the workload descriptions is read as mean 0, standard deviation s, as
the pages' test script scales torch.randn by 0.1 (parameters) and by its
gradient_scale of 0.01 (gradients).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 20
_THREADS = max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))))


def _chunk_values(words, c, lo, hi, scale):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words) + [c])))
    v = rng.standard_normal(hi, dtype=np.float32)[lo:hi]
    if scale != 1.0:
        v *= np.float32(scale)
    return v


def normal_f32(words, n: int, scale: float, start: int = 0, stop: int | None = None) -> np.ndarray:
    """Elements [start, stop) of the stream `words` (a list of ints) of length n."""
    stop = n if stop is None else stop
    assert 0 <= start <= stop <= n
    out = np.empty(stop - start, np.float32)
    if stop == start:
        return out
    c0, c1 = start // CHUNK, (stop - 1) // CHUNK

    def fill(c):
        base = c * CHUNK
        lo = max(start, base) - base
        hi = min(stop, base + CHUNK, n) - base
        out[base + lo - start: base + hi - start] = _chunk_values(words, c, lo, hi, scale)

    chunks = range(c0, c1 + 1)
    if len(chunks) == 1 or _THREADS == 1:
        for c in chunks:
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, chunks))
    return out


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 samples to the parameter dtype (RNE).  bf16 comes back as uint16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(x, np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def zero_row_mask(words, rows: int, frac: float) -> np.ndarray:
    """Boolean mask of rows whose gradient is exactly zero (Bernoulli(frac) per row)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words) + [0x5eed])))
    return rng.random(rows) < frac


@dataclass
class Tensor:
    name: str
    shape: tuple
    dtype: str            # "f32" | "f16" | "bf16"
    eightbit: bool        # False: kept in 32-bit states (below min_8bit_size)

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


@dataclass
class Workload:
    name: str
    cid: int                          # seed base is 1234 + cid
    hp: dict
    tensors: list
    steps: int
    p_scale: float
    g_scale: float
    zero_row_frac: float = 0.0        # fraction of gradient rows that are exactly zero
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 1234 + self.cid

    def param(self, ti: int, start=0, stop=None, dtype=None) -> np.ndarray:
        t = self.tensors[ti]
        v = normal_f32([self.seed, 1, ti], t.numel, self.p_scale, start, stop)
        return to_dtype(v, dtype or t.dtype)

    def grad(self, ti: int, step: int, start=0, stop=None, dtype=None) -> np.ndarray:
        t = self.tensors[ti]
        stop = t.numel if stop is None else stop
        v = normal_f32([self.seed, 2, ti, step], t.numel, self.g_scale, start, stop)
        if self.zero_row_frac > 0.0:
            rows = t.shape[0]
            cols = t.numel // rows
            mask = zero_row_mask([self.seed, 3, ti, step], rows, self.zero_row_frac)
            idx = np.arange(start, stop, dtype=np.int64) // cols
            v[mask[idx]] = 0.0
        return to_dtype(v, dtype or t.dtype)


def _adam_hp(**kw):
    hp = dict(optimizer="adam", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
              blocksize=256, skip_zeros=False, max_unorm=0.0)
    hp.update(kw)
    return hp


def c1_adam_256() -> Workload:
    return Workload("adam8bit_256x256_fp32_b256", 1, _adam_hp(),
                    [Tensor("w", (256, 256), "f32", True)], steps=10, p_scale=0.02, g_scale=1e-2)


def c2_adamw_4096(dtype: str = "f32", blocksize: int = 256, weight_decay: float = 0.01) -> Workload:
    return Workload(f"adamw8bit_4096x4096_{dtype}_b{blocksize}", 2,
                    _adam_hp(blocksize=blocksize, weight_decay=weight_decay),
                    [Tensor("w", (4096, 4096), dtype, True)], steps=20, p_scale=0.02, g_scale=1e-2)


def c3_ademamix_4096() -> Workload:
    hp = dict(optimizer="ademamix", lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0,
              t_alpha=100, t_beta3=100, eps=1e-8, weight_decay=0.0, blocksize=256,
              skip_zeros=False, max_unorm=0.0)
    return Workload("ademamix8bit_4096x4096_bf16_b256", 3, hp,
                    [Tensor("w", (4096, 4096), "bf16", True)], steps=200, p_scale=0.02, g_scale=1e-2)


def c4_embedding(optimizer: str = "momentum", skip_zeros: bool = True) -> Workload:
    if optimizer == "momentum":
        hp = dict(optimizer="momentum", lr=0.01, beta1=0.9, beta2=0.0, eps=1e-8)
    else:
        hp = dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, eps=1e-8)
    hp.update(weight_decay=0.01, blocksize=256, skip_zeros=skip_zeros, max_unorm=0.0)
    return Workload(f"{optimizer}8bit_50257x1024_fp16_b256_skip{int(skip_zeros)}", 4, hp,
                    [Tensor("wte", (50257, 1024), "f16", True)], steps=10, p_scale=0.02,
                    g_scale=1e-3, zero_row_frac=0.7)


def f2_one_state_4096(optimizer: str, dtype: str = "f32") -> Workload:
    """RMSprop / Adagrad 8-bit on the 4096x4096 shape: RMSprop with the optimizer
    table's RMSprop8bit(p, 0.01, 0.9); Adagrad with lr 0.01, eps 1e-10."""
    if optimizer == "rmsprop":
        hp = dict(optimizer="rmsprop", lr=0.01, beta1=0.9, eps=1e-8)
    else:
        hp = dict(optimizer="adagrad", lr=0.01, eps=1e-10)
    hp.update(weight_decay=0.0, blocksize=256, skip_zeros=False, max_unorm=0.0)
    return Workload(f"{optimizer}8bit_4096x4096_{dtype}_b256", 6, hp,
                    [Tensor("w", (4096, 4096), dtype, True)], steps=20, p_scale=0.02, g_scale=1e-2)


def f3_tensorwise_4096(dtype: str = "f32") -> Workload:
    """AdamW 8-bit on the 4096x4096 shape with one absmax per state for the whole
    tensor (blocksize 0): the non-block-wise form, same hyper-parameters as the
    block-wise AdamW workload."""
    return Workload(f"adamw8bit_4096x4096_{dtype}_tensorwise", 2, _adam_hp(blocksize=0, weight_decay=0.01),
                    [Tensor("w", (4096, 4096), dtype, True)], steps=20, p_scale=0.02, g_scale=1e-2)


def f4_paged_4096(dtype: str = "f32") -> Workload:
    """The block-wise AdamW workload with the optimizer state (codes, absmax) kept in
    pinned host memory instead of HBM ("paged" state)."""
    w = c2_adamw_4096(dtype, 256)
    w.name = f"adamw8bit_4096x4096_{dtype}_b256_paged"
    w.extra = {"paged": True}
    return w


def f4_staged_4096(dtype: str = "f32") -> Workload:
    """The block-wise AdamW workload with the state in pinned host memory, paged through
    HBM staging buffers chunk by chunk around each step (copy-in, step, write-back
    overlapped on three streams)."""
    w = c2_adamw_4096(dtype, 256)
    w.name = f"adamw8bit_4096x4096_{dtype}_b256_staged"
    w.extra = {"paged": "staged", "chunk": 1 << 23}
    return w


def f4_pooled_4096(dtype: str = "f32", page: int = 1 << 23, frames: int = 2) -> Workload:
    """The block-wise AdamW workload with the state in pinned host memory behind an HBM
    page pool of `frames` frames of `page` elements: with room for every page the state
    stays resident after the first step; with fewer frames every step pages it through."""
    w = c2_adamw_4096(dtype, 256)
    pages = -(-w.tensors[0].numel // page)
    w.name = f"adamw8bit_4096x4096_{dtype}_b256_pooled_{'resident' if frames >= pages else f'{frames}of{pages}'}"
    w.extra = {"paged": "pooled", "page": page, "frames": frames}
    return w


def codec_4096(kind: str = "quantize", dtype: str = "f32", blocksize: int = 256) -> Workload:
    """The block-wise codec pair on its own: quantize (values -> codes + absmax) or
    dequantize (codes + absmax -> values) of one 4096x4096 tensor of N(0, 1e-2) values."""
    return Workload(f"{kind}_blockwise_4096x4096_{dtype}_b{blocksize}", 8,
                    dict(optimizer="codec", blocksize=blocksize),
                    [Tensor("x", (4096, 4096), dtype, True)], steps=20, p_scale=0.02, g_scale=1e-2,
                    extra={"codec": kind})


def adam_small_1024x9() -> Workload:
    """The pages' small benchmark shape (1024 x 9 fp32, Adam 8-bit), where the step
    is launch-bound rather than bandwidth-bound."""
    return Workload("adam8bit_1024x9_fp32_b256", 7, _adam_hp(),
                    [Tensor("w", (1024, 9), "f32", True)], steps=10, p_scale=0.02, g_scale=1e-2)


def adamw_32bit_4096(dtype: str = "f32") -> Workload:
    """The 32-bit comparator of the block-wise AdamW workload: the same tensor and
    hyper-parameters with fp32 states (no codec)."""
    return Workload(f"adamw32bit_4096x4096_{dtype}", 2, _adam_hp(weight_decay=0.01),
                    [Tensor("w", (4096, 4096), dtype, False)], steps=20, p_scale=0.02, g_scale=1e-2)


MIN_8BIT_SIZE = 4096


def gpt_tensors(vocab=50257, d=2048, layers=24, ffn=8192, ctx=2048) -> list:
    """GPT-2-style parameter list; tensors under MIN_8BIT_SIZE elements stay fp32 32-bit."""
    shapes = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(layers):
        shapes += [
            (f"h{i}.ln1.w", (d,)), (f"h{i}.ln1.b", (d,)),
            (f"h{i}.attn.qkv.w", (d, 3 * d)), (f"h{i}.attn.qkv.b", (3 * d,)),
            (f"h{i}.attn.proj.w", (d, d)), (f"h{i}.attn.proj.b", (d,)),
            (f"h{i}.ln2.w", (d,)), (f"h{i}.ln2.b", (d,)),
            (f"h{i}.mlp.fc.w", (d, ffn)), (f"h{i}.mlp.fc.b", (ffn,)),
            (f"h{i}.mlp.fc2.w", (ffn, d)), (f"h{i}.mlp.fc2.b", (d,)),
        ]
    shapes += [("ln_f.w", (d,)), ("ln_f.b", (d,))]
    out = []
    for name, shp in shapes:
        n = int(np.prod(shp))
        big = n >= MIN_8BIT_SIZE
        out.append(Tensor(name, shp, "bf16" if big else "f32", big))
    return out


def c5_gpt_1p3b(**kw) -> Workload:
    return Workload("gpt_1p3b_bf16_adam8bit_b256", 5, _adam_hp(),
                    gpt_tensors(**kw), steps=1, p_scale=0.02, g_scale=1e-3)


def bytes_per_element(dtype: str, n_states: int, blocksize: int) -> float:
    """Algorithmic HBM bytes per element of one 8-bit step: read+write p, read g,
    read+write one code per state, read+write one fp32 absmax per block per state."""
    ps = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
    return 2 * ps + ps + n_states * (2 + 8.0 / blocksize)
