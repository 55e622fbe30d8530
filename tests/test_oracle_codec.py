"""Pins of the oracle's block-wise codec and number-format rounding.

Pages: "8-bit Optimizers via Block-wise Quantization" (abstract: a tensor is split
into blocks quantized independently, one scale per block); "[XPU] Implemented 8bit
optimizers in triton #1692" (test body: dequantize_blockwise(code, absmax, A,
blocksize) multiplies the codebook entry by its block's absmax).

Nearest code: the oracle scans all 256 entries (the definition).  It is pinned
here against numpy.searchsorted plus one neighbour comparison, a different route
to the same answer, on every codebook value and bin boundary (and thousands of
fp32 ulps around each) and on random inputs.
"""
import numpy as np
import pytest
import torch


def _nearest_by_search(q, x):
    x = np.asarray(x, np.float32)
    i = np.searchsorted(q, x, side="right") - 1
    i = np.clip(i, 0, 254)
    lo, hi = q[i], q[i + 1]
    up = (hi - x) < (x - lo)  # fp32 distances; a tie goes to the lower index
    return (i + up).astype(np.uint8)


def _ulp_neighbourhood(centers, k):
    c = np.asarray(centers, np.float32)
    bits = c.view(np.int32).astype(np.int64)
    out = []
    for d in range(-k, k + 1):
        b = bits + d
        # step through fp32 values in value order on either side of zero
        v = np.where(c >= 0, b, bits - d).astype(np.int32).view(np.float32)
        out.append(v)
    v = np.concatenate(out)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("signed", [True, False])
def test_nearest_matches_search_around_boundaries(oref, signed):
    q = oref.dynamic_map(signed)
    mids = ((q[:-1].astype(np.float64) + q[1:]) / 2).astype(np.float32)
    x = np.concatenate([_ulp_neighbourhood(q, 512), _ulp_neighbourhood(mids, 512),
                        np.float32([0.0, -0.0, 1.0, -1.0, 1.5, -1.5, 1e-30, -1e-30])])
    got = oref.nearest(q, x)
    np.testing.assert_array_equal(got, _nearest_by_search(q, x))


@pytest.mark.parametrize("signed", [True, False])
def test_nearest_matches_search_random(oref, signed):
    q = oref.dynamic_map(signed)
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-1.05, 1.05, 400_000),
                        np.sign(rng.standard_normal(100_000)) * 10.0 ** rng.uniform(-9, 0, 100_000)])
    x = x.astype(np.float32)
    np.testing.assert_array_equal(oref.nearest(q, x), _nearest_by_search(q, x))


def test_nearest_exact_entries(oref):
    for signed in (True, False):
        q = oref.dynamic_map(signed)
        np.testing.assert_array_equal(oref.nearest(q, q), np.arange(256, dtype=np.uint8))


@pytest.mark.parametrize("blocksize", [256, 2048])
def test_quantize_recovers_codes_of_scaled_codebook(oref, blocksize):
    """x = A_b * Q[k] with one k = 255 (value A_b) per block encodes back to k."""
    q = oref.dynamic_map(True)
    rng = np.random.default_rng(3)
    nb = 9
    n = nb * blocksize - 17
    k = rng.integers(0, 256, n).astype(np.uint8)
    A = (10.0 ** rng.uniform(-6, 1, nb)).astype(np.float32)
    k[np.arange(nb) * blocksize] = 255
    x = (q[k] * A[np.arange(n) // blocksize]).astype(np.float32)
    codes, absmax = oref.quantize_blockwise(x, "f32", q, blocksize)
    np.testing.assert_array_equal(absmax, A)
    np.testing.assert_array_equal(codes, k)


@pytest.mark.parametrize("n,blocksize", [(1, 256), (255, 256), (256, 256), (257, 256),
                                         (2047, 2048), (2049, 2048), (100, 2048), (5000, 256)])
def test_quantize_tail_and_error_bound(oref, n, blocksize):
    qs = oref.dynamic_map(True)
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 0.01).astype(np.float32)
    codes, absmax = oref.quantize_blockwise(x, "f32", qs, blocksize)
    nb = (n + blocksize - 1) // blocksize
    assert absmax.shape == (nb,)
    for b in range(nb):
        blk = x[b * blocksize:(b + 1) * blocksize]
        assert absmax[b] == np.abs(blk).max()          # exact, valid elements only
    # dequantize is the codebook entry times the block scale
    deq = oref.dequantize_blockwise(codes, absmax, qs, blocksize)
    blk_a = absmax[np.arange(n) // blocksize]
    np.testing.assert_array_equal(deq, (qs[codes] * blk_a).astype(np.float32))
    # round-trip error: half the local codebook gap times the scale, plus rounding
    qd = qs.astype(np.float64)
    gaps = np.maximum(np.diff(qd, prepend=qd[0]), np.diff(qd, append=qd[-1]))
    bound = blk_a.astype(np.float64) * (gaps[codes] / 2) * (1 + 1e-6) + np.abs(x) * 1e-6
    assert np.all(np.abs(deq.astype(np.float64) - x) <= bound)
    # a second pass over the decoded values changes nothing in blocks whose largest
    # magnitude is positive (+1.0 is in the map, -1.0 is not)
    codes2, absmax2 = oref.quantize_blockwise(deq, "f32", qs, blocksize)
    assert np.all(absmax2 <= absmax)
    for b in range(nb):
        sl = slice(b * blocksize, min(n, (b + 1) * blocksize))
        if x[sl][np.argmax(np.abs(x[sl]))] > 0:
            assert absmax2[b] == absmax[b]
            np.testing.assert_array_equal(codes2[sl], codes[sl])


def test_quantize_zero_block(oref):
    for signed, zero_code in ((True, 127), (False, 0)):
        q = oref.dynamic_map(signed)
        x = np.zeros(300, np.float32)
        x[256:] = 0.5
        codes, absmax = oref.quantize_blockwise(x, "f32", q, 256)
        assert absmax[0] == 0.0 and np.all(codes[:256] == zero_code)
        assert absmax[1] == 0.5 and np.all(codes[256:] == 255)


@pytest.mark.parametrize("signed", [True, False])
def test_quantize_invariant_under_power_of_two_scaling(oref, signed):
    """Scaling a block by a power of two (exactly, no bits lost) scales its absmax by
    the same power and leaves its codes unchanged -- down into the subnormal range,
    where the plain reciprocal of the absmax would overflow."""
    q = oref.dynamic_map(signed)
    rng = np.random.default_rng(5)
    n = 4 * 256
    ints = rng.integers(-1024 if signed else 0, 1025, n).astype(np.float32)
    ints[::97] = 0.0
    x = ints / np.float32(1024.0)                      # 11 significant bits, |x| <= 1
    codes, absmax = oref.quantize_blockwise(x, "f32", q, 256)
    for k in (10, 60, 100, 126, 127, 128, 130, 134, 138):
        xs = (x.astype(np.float64) * 2.0 ** -k).astype(np.float32)
        assert np.array_equal(xs.astype(np.float64) * 2.0 ** k, x.astype(np.float64))   # exact
        c2, a2 = oref.quantize_blockwise(xs, "f32", q, 256)
        np.testing.assert_array_equal(a2.astype(np.float64), absmax.astype(np.float64) * 2.0 ** -k)
        np.testing.assert_array_equal(c2, codes, err_msg=f"2^-{k}")


def test_fp16_rounding_matches_numpy(oref):
    rng = np.random.default_rng(11)
    specials = np.float32([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e6, -1e6, 6.0e-8, 2.98e-8,
                           2.9802322e-08, 5.9604645e-08, 6.1035156e-05, 6.103515e-05, np.inf, -np.inf,
                           1.0009765625, 1.00048828125, 1.000732421875, 2049.0, 2051.0])
    x = np.concatenate([specials, (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-9, 5, 200_000))
                        .astype(np.float32), rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64)
                        .astype(np.uint32).view(np.float32)])
    x = x[~np.isnan(x)]
    got = oref.round_to_dtype(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16))
    np.testing.assert_array_equal(oref.widen(got, "f16"), got.astype(np.float32))


def test_bf16_rounding_matches_torch(oref):
    rng = np.random.default_rng(12)
    x = np.concatenate([np.float32([0.0, -0.0, 1.00390625, 1.01171875, 3.3895314e38, np.inf]),
                        rng.integers(0, 2 ** 32, 300_000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    x = x[~np.isnan(x)]
    got = oref.round_to_dtype(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(oref.widen(got, "bf16"),
                                  torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy())


# ------------------------------------------------------------------ non-finite values
# The pages say nothing about NaN or infinite data.  Reading (used by the oracle and the
# kernels alike): the block absmax is the largest magnitude among the values that are
# not NaN (0 if there is none), and a NaN normalized value -- from a NaN state, or from
# an infinite state whose block absmax is infinite (reciprocal 0, and inf * 0 = NaN) --
# is encoded as +0 is.  The pins below restate that rule with numpy (nanmax, a brute
# force argmin over the map) on blocks with NaN and +-inf next to ordinary values.

def _brute_codes(q, x):
    x = np.asarray(x, np.float32)
    xx = np.where(np.isnan(x), np.float32(0.0), x)
    d = np.abs(xx[:, None] - q[None, :])               # fp32 distances
    return np.argmin(d, axis=1).astype(np.uint8)       # argmin: first (lowest) index on ties


@pytest.mark.parametrize("signed", [True, False])
def test_quantize_nan_values_ignored_by_absmax_and_encode_as_zero(oref, signed):
    q = oref.dynamic_map(signed)
    rng = np.random.default_rng(31)
    B = 256
    x = rng.standard_normal(3 * B + 17).astype(np.float32) * np.float32(0.01)
    if not signed:
        x = np.abs(x)
    x[[3, 100, B + 5, 2 * B + 1]] = np.nan
    x[B + 6] = -np.nan
    x[2 * B + 2: 3 * B] = np.nan                        # a block that is almost all NaN
    x[3 * B:] = np.nan                                  # a ragged tail that is all NaN
    codes, absmax = oref.quantize_blockwise(x, "f32", q, B)
    for b in range(4):
        blk = x[b * B:(b + 1) * B]
        fin = blk[~np.isnan(blk)]
        A = np.float32(np.abs(fin).max()) if fin.size else np.float32(0.0)
        assert absmax[b] == A, b
        r = np.float32(1.0) / A if A > 0 else np.float32(0.0)
        want = _brute_codes(q, (blk * r).astype(np.float32))
        np.testing.assert_array_equal(codes[b * B:(b + 1) * B], want, err_msg=f"block {b}")
    zero_code = int(np.flatnonzero(q == 0.0)[0])
    assert np.all(codes[np.isnan(x)] == zero_code)


def test_quantize_infinite_value_makes_a_zero_block(oref):
    q = oref.dynamic_map(True)
    x = np.linspace(-0.5, 0.5, 512).astype(np.float32)
    x[7] = np.inf
    x[300] = -np.inf
    codes, absmax = oref.quantize_blockwise(x, "f32", q, 256)
    assert np.isinf(absmax[0]) and np.isinf(absmax[1])
    zero_code = int(np.flatnonzero(q == 0.0)[0])
    np.testing.assert_array_equal(codes, np.full(512, zero_code, np.uint8))
    # decoding such a block gives 0 * inf = NaN everywhere: the state is poisoned
    out = oref.dequantize_blockwise(codes, absmax, q, 256)
    assert np.all(np.isnan(out))


def test_step_with_nan_gradient_poisons_only_its_parameter(oref):
    """An 8-bit Adam step with a NaN gradient element: that parameter becomes NaN, its
    states encode as zero, the block absmax stays finite, and every other parameter is
    bit-identical to the step on the same data with that element's gradient set to 0
    and skip_zeros on (which leaves the element out of the update entirely) -- except
    through the block's new absmax, which the NaN element does not enter either way."""
    n, B = 2 * 256, 256
    rng = np.random.default_rng(5)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 0.01).astype(np.float32)
    qs, qu = oref.dynamic_map(True), oref.dynamic_map(False)
    hp = dict(optimizer="adam", lr=1e-3, weight_decay=0.0, blocksize=B)
    st = lambda: (np.zeros(n, np.uint8), np.zeros(2, np.float32), np.zeros(n, np.uint8), np.zeros(2, np.float32))
    gn = g.copy()
    gn[40] = np.nan
    p1 = p0.copy()
    s1, a1, s2, a2 = st()
    oref.step_8bit(hp, 1, p1, gn, "f32", s1, a1, qs, s2, a2, qu)
    assert np.isnan(p1[40])
    assert np.all(np.isfinite(a1)) and np.all(np.isfinite(a2))
    assert s1[40] == int(np.flatnonzero(qs == 0.0)[0]) and s2[40] == int(np.flatnonzero(qu == 0.0)[0])
    gz = g.copy()
    gz[40] = 0.0
    p2 = p0.copy()
    t1, b1, t2, b2 = st()
    oref.step_8bit(dict(hp, skip_zeros=True), 1, p2, gz, "f32", t1, b1, qs, t2, b2, qu)
    keep = np.arange(n) != 40
    np.testing.assert_array_equal(p1[keep], p2[keep])
    np.testing.assert_array_equal(a1, b1)
    np.testing.assert_array_equal(a2, b2)
    np.testing.assert_array_equal(s1[keep], t1[keep])
    np.testing.assert_array_equal(s2[keep], t2[keep])
