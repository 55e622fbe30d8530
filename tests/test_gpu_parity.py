"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case starts both sides from the same seeded inputs; the oracle runs its own
trajectory (it never takes data produced by the HIP path) and the two are
compared after every step to the bar in tests/parity.py.  Sizes span several
tiles and a ragged tail; both block sizes, all three parameter dtypes and all six
optimizers (Adam, AdEMAMix, Momentum, Lion, RMSprop, Adagrad) are covered, with
skip_zeros, max_unorm, custom and swapped maps, the 32-bit mode, the codec,
unaligned buffers and empty inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import Compare, Quant8, as_f32, param_rtol, to_dev, to_host

pytestmark = pytest.mark.gpu

OPTS = {
    "adam": dict(optimizer="adam", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    "ademamix": dict(optimizer="ademamix", lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0,
                     t_alpha=3, t_beta3=3, eps=1e-8, weight_decay=0.01),
    "momentum": dict(optimizer="momentum", lr=0.01, beta1=0.9, weight_decay=0.01),
    "lion": dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01),
    "rmsprop": dict(optimizer="rmsprop", lr=0.01, beta1=0.9, eps=1e-8, weight_decay=0.01),
    "adagrad": dict(optimizer="adagrad", lr=0.01, eps=1e-10, weight_decay=0.01),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()          # a missing library is an error where a GPU is present, not a skip


def _grad(seed, t, n, dtype, zero_frac=0.0, B=256):
    g = W.normal_f32([seed, 2, t], n, 0.01)
    if zero_frac:
        rng = np.random.default_rng([seed, t])
        g[rng.random(n) < zero_frac] = 0.0
        nb = (n + B - 1) // B
        for b in rng.choice(nb, max(1, nb // 3), replace=False):
            g[b * B:(b + 1) * B] = 0.0
    return W.to_dtype(g, dtype)


def _run(hp, n, dtype, steps, seed, zero_frac=0.0, maps=None):
    print(f"\n[case] {hp['optimizer']} {dtype} B={hp['blocksize']} n={n} steps={steps} "
          f"skip={hp.get('skip_zeros', False)} max_unorm={hp.get('max_unorm', 0.0)} "
          f"maps={'custom' if maps is not None else 'standard'}", flush=True)
    p0 = W.to_dtype(W.normal_f32([seed, 1], n, 0.02), dtype)
    q = Quant8(hp, p0, dtype, maps)
    cmp = Compare()
    for t in range(1, steps + 1):
        g = _grad(seed, t, n, dtype, zero_frac, hp["blocksize"])
        q.step_gpu(t, to_dev(g, dtype))
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")
    print("  " + cmp.summary(), flush=True)
    return cmp


RAGGED = {256: 5 * 1024 + 300 + 5, 2048: 5 * 2048 + 1500 + 3}


@pytest.mark.parametrize("bs", [256, 2048])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("name", list(OPTS))
def test_step_8bit(name, dtype, bs):
    _run(dict(OPTS[name], blocksize=bs), RAGGED[bs], dtype, 4, 100 + bs)


@pytest.mark.parametrize("bs", [256, 2048])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("name", list(OPTS))
def test_step_8bit_skip_zeros(name, dtype, bs):
    _run(dict(OPTS[name], blocksize=bs, skip_zeros=True), RAGGED[bs], dtype, 4, 200 + bs, zero_frac=0.3)


@pytest.mark.parametrize("name", list(OPTS))
def test_step_8bit_max_unorm(name):
    _run(dict(OPTS[name], blocksize=256, max_unorm=0.002), RAGGED[256], "f32", 3, 300)


def test_step_8bit_tiny_second_moments():
    """Gradients so small that v = (1 - beta2) g^2 lands in (0, 2^-96) in some blocks:
    those quads take the general square root, the rest the unscaled one."""
    for name, dtype in (("adam", "f32"), ("ademamix", "bf16")):
        n, B = RAGGED[256], 256
        hp = dict(OPTS[name], blocksize=B)
        p0 = W.to_dtype(W.normal_f32([970, 1], n, 0.02), dtype)
        q = Quant8(hp, p0, dtype)
        cmp = Compare()
        for t in range(1, 4):
            g = W.normal_f32([970, 2, t], n, 0.01)
            scale = np.ones(n, np.float32)
            for b in range(0, (n + B - 1) // B, 3):
                scale[b * B:(b + 1) * B] = 1e-18          # g^2 ~ 1e-40, v ~ 1e-43
            scale[5 * B + 7:5 * B + 40] = 1e-25             # tiny elements inside an ordinary block
            g = W.to_dtype(g * scale, dtype)
            q.step_gpu(t, to_dev(g, dtype))
            q.step_oracle(t, g)
            q.compare(cmp, f"{name} step {t}")
        print(f"\n[tiny v {name} {dtype}] " + cmp.summary())


def test_step_8bit_huge_states():
    """Gradient blocks scaled so far up that the new state's block absmax exceeds 2^30:
    the table encoder's scaled reciprocal would leave the normal range there, so those
    blocks take the binary search, next to ordinary blocks, in full and ragged tiles."""
    for name, dtype, big in (("adam", "f32", 1e12), ("momentum", "f32", 1e12), ("lion", "bf16", 1e14)):
        n, B = RAGGED[256], 256
        hp = dict(OPTS[name], blocksize=B)
        p0 = W.to_dtype(W.normal_f32([975, 1], n, 0.02), dtype)
        q = Quant8(hp, p0, dtype)
        cmp = Compare()
        nb = (n + B - 1) // B
        for t in range(1, 4):
            g = W.normal_f32([975, 2, t], n, 0.01)
            scale = np.ones(n, np.float32)
            for b in list(range(1, nb, 4)) + [nb - 1]:      # includes the ragged last block
                scale[b * B:(b + 1) * B] = big
            g = W.to_dtype(g * scale, dtype)
            q.step_gpu(t, to_dev(g, dtype))
            q.step_oracle(t, g)
            q.compare(cmp, f"{name} step {t}")
        assert np.any(q.o["a1"] > 2.0 ** 30), "no block reached an absmax above 2^30"
        print(f"\n[huge states {name} {dtype}] " + cmp.summary())
        assert cmp.bit_exact, cmp.summary()


@pytest.mark.parametrize("bs", [256, 2048])
def test_codec_absmax_around_2_pow_30(bs):
    """Block absmax just below, at and above 2^30 (the table encoder's limit) and up to
    the top of the fp32 range, next to ordinary and all-zero blocks."""
    n = RAGGED[bs]
    nb = (n + bs - 1) // bs
    x = W.normal_f32([915, bs], n, 1.0)
    targets = [2.0 ** 29, 2.0 ** 30, 2.0 ** 30 * (1 + 2.0 ** -23), 2.0 ** 31, 1e20, 2.0 ** 126, 3.0e38, 0.0]
    for b in range(nb):
        blk = x[b * bs:(b + 1) * bs]
        tgt = targets[(b * (3 if bs == 2048 else 1)) % len(targets)]
        blk *= np.float32(tgt / float(np.abs(blk).max())) if tgt > 0 else np.float32(0.0)
        if tgt > 0:
            blk[int(np.argmax(np.abs(blk)))] = np.float32(tgt)          # the exact absmax
    for signed in (True, False):
        xs = x if signed else np.abs(x)
        qmap = oracle.dynamic_map(signed)
        codes_ref, absmax_ref = oracle.quantize_blockwise(xs, "f32", qmap, bs)
        codes, absmax = bitopt.quantize_blockwise(to_dev(xs, "f32"), bitopt.create_dynamic_map(signed).cuda(), bs)
        cmp = Compare()
        cmp.codes(to_host(codes), codes_ref, "codes")
        cmp.values(to_host(absmax), absmax_ref, 1e-6, "absmax", kind="a")
        assert cmp.bit_exact, cmp.summary()


def _jittered_map(signed, seed):
    """A sorted 256-entry map close to a standard one but equal to neither standard
    map, so the kernels take the binary-search encoder."""
    q = oracle.dynamic_map(signed).astype(np.float64)
    rng = np.random.default_rng(seed)
    inner = (q != 0) & (np.abs(q) != 1)
    q[inner] *= 1 + 2e-3 * rng.uniform(-1, 1, int(inner.sum()))
    q = np.sort(q).astype(np.float32)
    assert np.all(np.diff(q) > 0)
    return q


@pytest.mark.parametrize("bs", [256, 2048])
@pytest.mark.parametrize("name", list(OPTS))
def test_step_8bit_custom_maps(name, bs):
    """Maps that are not the standard ones: binary-search encoder, full and ragged tiles."""
    dtype = "bf16" if name == "ademamix" else "f32"
    maps = (_jittered_map(True, 11), _jittered_map(False, 12))
    _run(dict(OPTS[name], blocksize=bs), RAGGED[bs], dtype, 3, 900 + bs, maps=maps)


def test_step_8bit_custom_maps_skip_unorm():
    maps = (_jittered_map(True, 13), _jittered_map(False, 14))
    _run(dict(OPTS["adam"], blocksize=256, skip_zeros=True, max_unorm=0.002), RAGGED[256], "f16", 3, 960,
         zero_frac=0.3, maps=maps)


def test_step_8bit_standard_maps_other_assignment():
    """Standard maps passed in other slots than (signed, unsigned): the kernels stage
    the matching search tables again and keep the table encoder."""
    s, u = oracle.dynamic_map(True), oracle.dynamic_map(False)
    _run(dict(OPTS["adam"], blocksize=256), RAGGED[256], "f32", 3, 950, maps=(s, s))
    _run(dict(OPTS["adam"], blocksize=2048), RAGGED[2048], "f32", 3, 951, maps=(u, s))
    _run(dict(OPTS["momentum"], blocksize=256), RAGGED[256], "f16", 3, 952, maps=(u, None))


@pytest.mark.parametrize("n", [1, 3, 255, 256, 257, 1023, 1025, 2047, 2049])
def test_small_and_ragged_sizes(n):
    for bs in (256, 2048):
        _run(dict(OPTS["adam"], blocksize=bs), n, "f32", 2, 400 + n)
        _run(dict(OPTS["ademamix"], blocksize=bs), n, "bf16", 2, 500 + n)


def test_empty_is_noop():
    for name in OPTS:
        hp = dict(OPTS[name], blocksize=256)
        q = Quant8(hp, np.zeros(0, np.float32), "f32")
        g = torch.zeros(0, device="cuda")
        q.step_gpu(1, g)
    torch.cuda.synchronize()


def test_unaligned_buffers():
    """Buffers that start one element / one byte off a 16-byte boundary take the
    element-wise path and still match."""
    n, bs = RAGGED[256], 256
    for name, dtype in (("adam", "f32"), ("ademamix", "f16"), ("lion", "bf16")):
        hp = dict(OPTS[name], blocksize=bs)
        p0 = W.to_dtype(W.normal_f32([600, 1], n, 0.02), dtype)
        q = Quant8(hp, p0, dtype)
        for key in ("p", "s1", "s2"):
            if key in q.d:
                t = q.d[key]
                big = torch.zeros(t.numel() + 1, dtype=t.dtype, device="cuda")
                big[1:].copy_(t)
                q.d[key] = big[1:]
                assert q.d[key].data_ptr() % 4 != 0 or t.element_size() == 4
        cmp = Compare()
        for t in range(1, 4):
            g = _grad(600, t, n, dtype)
            gd = torch.zeros(n + 1, dtype=q.d["p"].dtype, device="cuda")
            gd[1:].copy_(to_dev(g, dtype))
            q.step_gpu(t, gd[1:])
            q.step_oracle(t, g)
            q.compare(cmp, f"{name} step {t}")
        print(f"\n[unaligned {name} {dtype}] " + cmp.summary())


def test_deterministic():
    n, hp = 4 * 4096 + 77, dict(OPTS["ademamix"], blocksize=256)
    p0 = W.to_dtype(W.normal_f32([700, 1], n, 0.02), "bf16")
    outs = []
    for _ in range(2):
        q = Quant8(hp, p0, "bf16")
        for t in range(1, 4):
            q.step_gpu(t, to_dev(_grad(700, t, n, "bf16"), "bf16"))
        torch.cuda.synchronize()
        outs.append({k: to_host(v) for k, v in q.d.items()})
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k])


# ------------------------------------------------------------------ 32-bit mode

@pytest.mark.parametrize("unorm", [0.0, 0.002])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("name", list(OPTS))
def test_step_32bit(name, dtype, unorm):
    n = RAGGED[256]
    hp = dict(OPTS[name], blocksize=256, skip_zeros=(name == "lion"), max_unorm=unorm)
    print(f"\n[case] 32-bit {name} {dtype} max_unorm={unorm}", flush=True)
    two = oracle.NUM_STATES[name] >= 2
    k1 = 2 if name == "ademamix" else 1
    p0 = W.to_dtype(W.normal_f32([800, 1], n, 0.02), dtype)
    op, os1, os2 = p0.copy(), np.zeros(k1 * n, np.float32), np.zeros(n, np.float32) if two else None
    dp, ds1 = to_dev(p0, dtype), torch.zeros(k1 * n, device="cuda")
    ds2 = torch.zeros(n, device="cuda") if two else None
    cmp = Compare()
    for t in range(1, 5):
        g = _grad(800, t, n, dtype, zero_frac=0.2 if hp["skip_zeros"] else 0.0)
        if two:
            bitopt.step_32bit_2state(hp, t, dp, to_dev(g, dtype), ds1, ds2)
        else:
            bitopt.step_32bit_1state(hp, t, dp, to_dev(g, dtype), ds1)
        oracle.step_32bit(hp, t, op, g, dtype, os1, os2)
        torch.cuda.synchronize()
        cmp.values(as_f32(to_host(dp, dtype), dtype), as_f32(op, dtype), param_rtol(dtype), "p")
        cmp.values(to_host(ds1), os1, 1e-6, "state1", kind="a")
        if two:
            cmp.values(to_host(ds2), os2, 1e-6, "state2", kind="a")
    print(f"\n[32bit {name} {dtype}] " + cmp.summary())


# ------------------------------------------------------------------ codec

@pytest.mark.parametrize("bs", [256, 2048])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_codec(dtype, bs):
    for signed in (True, False):
        n = RAGGED[bs]
        x = W.normal_f32([900, bs], n, 0.01)
        if not signed:
            x = np.abs(x)
        x[: bs] = 0.0                                  # an all-zero block
        x = W.to_dtype(x, dtype)
        qmap = oracle.dynamic_map(signed)
        codes_ref, absmax_ref = oracle.quantize_blockwise(x, dtype, qmap, bs)
        qd = bitopt.create_dynamic_map(signed).cuda()
        codes, absmax = bitopt.quantize_blockwise(to_dev(x, dtype), qd, bs)
        cmp = Compare()
        cmp.codes(to_host(codes), codes_ref, "codes")
        cmp.values(to_host(absmax), absmax_ref, 1e-6, "absmax", kind="a")
        assert cmp.bit_exact, cmp.summary()
        out = bitopt.dequantize_blockwise(to_dev(codes_ref), to_dev(absmax_ref), qd, bs,
                                          dtype={"f32": torch.float32, "f16": torch.float16,
                                                 "bf16": torch.bfloat16}[dtype])
        ref = oracle.dequantize_blockwise(codes_ref, absmax_ref, qmap, bs, dtype)
        np.testing.assert_array_equal(to_host(out, dtype), ref)


@pytest.mark.parametrize("bs", [256, 2048])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_codec_custom_maps(dtype, bs):
    """Maps that are not the standard ones: the codec's binary-search encoder, on full
    tiles, a ragged tail and an all-zero block, signed and unsigned."""
    for signed, seed in ((True, 41), (False, 42)):
        n = RAGGED[bs]
        print(f"\n[case] codec custom map signed={signed} {dtype} B={bs} n={n}", flush=True)
        x = W.normal_f32([905, bs, int(signed)], n, 0.01)
        if not signed:
            x = np.abs(x)
        x[bs: 2 * bs] = 0.0
        x = W.to_dtype(x, dtype)
        qmap = _jittered_map(signed, seed)
        codes_ref, absmax_ref = oracle.quantize_blockwise(x, dtype, qmap, bs)
        qd = torch.from_numpy(qmap).cuda()
        codes, absmax = bitopt.quantize_blockwise(to_dev(x, dtype), qd, bs)
        cmp = Compare()
        cmp.codes(to_host(codes), codes_ref, "codes")
        cmp.values(to_host(absmax), absmax_ref, 1e-6, "absmax", kind="a")
        assert cmp.bit_exact, cmp.summary()
        out = bitopt.dequantize_blockwise(to_dev(codes_ref), to_dev(absmax_ref), qd, bs,
                                          dtype={"f32": torch.float32, "bf16": torch.bfloat16}[dtype])
        np.testing.assert_array_equal(to_host(out, dtype), oracle.dequantize_blockwise(codes_ref, absmax_ref, qmap,
                                                                                       bs, dtype))


@pytest.mark.parametrize("bs", [256, 2048])
def test_codec_custom_map_unaligned(bs):
    """The binary-search encoder's element-wise path: input and codes one element off
    their vector alignment, a ragged tail."""
    n = 2 * bs + 301
    print(f"\n[case] codec custom map unaligned B={bs} n={n}", flush=True)
    x = W.normal_f32([906, bs], n + 1, 0.01)
    qmap = _jittered_map(True, 43)
    codes_ref, absmax_ref = oracle.quantize_blockwise(x[1:], "f32", qmap, bs)
    qd = torch.from_numpy(qmap).cuda()
    cbuf = torch.zeros(n + 1, dtype=torch.uint8, device="cuda")
    codes, absmax = bitopt.quantize_blockwise(to_dev(x)[1:], qd, bs, codes=cbuf[1:])
    np.testing.assert_array_equal(to_host(codes), codes_ref)
    np.testing.assert_array_equal(to_host(absmax), absmax_ref)


# ------------------------------------------------------------------ non-finite inputs
# Reading (the pages are silent): a block's absmax ignores NaN values; a NaN normalized
# value (a NaN state, or an infinite state in a block whose absmax is then infinite)
# encodes as +0.  Both sides follow it; these cases assert the documented result.

def _nonfinite_grad(seed, t, n, dtype, B=256):
    g = W.normal_f32([seed, 2, t], n, 0.01)
    if t <= 2:
        nb = (n + B - 1) // B
        g[3] = np.nan                                   # first block
        g[B + 17] = -np.nan
        g[2 * B + 5] = np.inf                           # an infinite gradient element
        g[3 * B + 200] = -np.inf
        g[(nb - 1) * B + 1] = np.nan                    # the ragged last block
        g[4 * B: 4 * B + 40] = np.nan                   # a run of NaN inside a block
    return W.to_dtype(g, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", list(OPTS))
def test_step_8bit_nonfinite_gradients(name, dtype):
    n, B = RAGGED[256], 256
    for extra in (dict(), dict(skip_zeros=True, max_unorm=0.002)):
        hp = dict(OPTS[name], blocksize=B, **extra)
        print(f"\n[case] non-finite gradients {name} {dtype} {extra}", flush=True)
        p0 = W.to_dtype(W.normal_f32([990, 1], n, 0.02), dtype)
        q = Quant8(hp, p0, dtype)
        cmp = Compare()
        for t in range(1, 5):
            g = _nonfinite_grad(990, t, n, dtype, B)
            q.step_gpu(t, to_dev(g, dtype))
            q.step_oracle(t, g)
            q.compare(cmp, f"step {t}")
        # the rule's visible results: a NaN state never becomes a block absmax; the step
        # of a NaN gradient is NaN (Lion takes sign(NaN) = 0 and keeps its parameters finite)
        assert not np.any(np.isnan(to_host(q.d["a1"]))), "a NaN state became a block absmax"
        assert np.any(np.isnan(as_f32(to_host(q.d["p"], dtype), dtype))) == (name != "lion")
        print("  " + cmp.summary(), flush=True)


@pytest.mark.parametrize("bs", [256, 2048])
def test_codec_nonfinite_inputs(bs):
    n = RAGGED[bs]
    x = W.normal_f32([995, bs], n, 0.01)
    x[[1, bs + 3, n - 1]] = np.nan
    x[2 * bs + 7] = np.inf
    x[3 * bs + 9] = -np.inf
    for signed in (True, False):
        xs = x if signed else np.abs(x)
        qmap = oracle.dynamic_map(signed)
        codes_ref, absmax_ref = oracle.quantize_blockwise(xs, "f32", qmap, bs)
        codes, absmax = bitopt.quantize_blockwise(to_dev(xs, "f32"), bitopt.create_dynamic_map(signed).cuda(), bs)
        cmp = Compare()
        cmp.codes(to_host(codes), codes_ref, "codes")
        cmp.values(to_host(absmax), absmax_ref, 1e-6, "absmax", kind="a")
        assert cmp.bit_exact, cmp.summary()
        assert not np.any(np.isnan(to_host(absmax)))


@pytest.mark.parametrize("bs", [256, 2048])
def test_codec_subnormal_blocks(bs):
    """Blocks whose absmax is subnormal (plain reciprocal beyond fp32 range) next to
    ordinary ones: the prescaled normalization on both sides."""
    for signed in (True, False):
        n = RAGGED[bs]
        x = W.normal_f32([910, bs], n, 0.01)
        if not signed:
            x = np.abs(x)
        nb = (n + bs - 1) // bs
        for b in range(0, nb, 2):
            x[b * bs:(b + 1) * bs] *= np.float32(2.0 ** -128)
        qmap = oracle.dynamic_map(signed)
        codes_ref, absmax_ref = oracle.quantize_blockwise(x, "f32", qmap, bs)
        assert np.any((absmax_ref > 0) & (absmax_ref < 2.0 ** -126))
        codes, absmax = bitopt.quantize_blockwise(to_dev(x, "f32"), bitopt.create_dynamic_map(signed).cuda(), bs)
        cmp = Compare()
        cmp.codes(to_host(codes), codes_ref, "codes")
        cmp.values(to_host(absmax), absmax_ref, 1e-6, "absmax", kind="a")
        assert cmp.bit_exact, cmp.summary()


def test_codec_unaligned_and_empty():
    n, bs = 3000, 256
    x = W.normal_f32([901, 1], n, 0.01)
    qmap = oracle.dynamic_map(True)
    codes_ref, absmax_ref = oracle.quantize_blockwise(x[1:], "f32", qmap, bs)
    xd = to_dev(x)[1:]
    qd = bitopt.create_dynamic_map(True).cuda()
    cbuf = torch.zeros(n, dtype=torch.uint8, device="cuda")
    codes, absmax = bitopt.quantize_blockwise(xd, qd, bs, codes=cbuf[1:])
    np.testing.assert_array_equal(to_host(codes), codes_ref)
    np.testing.assert_array_equal(to_host(absmax), absmax_ref)
    obuf = torch.zeros(n + 1, device="cuda")           # codes and output both off their vector alignment
    out = bitopt.dequantize_blockwise(codes, absmax, qd, bs, out=obuf[1:n])
    np.testing.assert_array_equal(to_host(out), oracle.dequantize_blockwise(codes_ref, absmax_ref, qmap, bs, "f32"))
    e = torch.zeros(0, device="cuda")
    bitopt.quantize_blockwise(e, qd, bs)
    bitopt.dequantize_blockwise(torch.zeros(0, dtype=torch.uint8, device="cuda"),
                                torch.zeros(0, device="cuda"), qd, bs)
    torch.cuda.synchronize()
