"""GPU parity with optimizer state kept outside HBM: the codes and absmax (8-bit)
or the fp32 states (32-bit) live in pinned host memory mapped into the GPU address
space (bitopt_host_state_alloc, the library's reading of paged optimizer state);
the same step kernels read and write them over the host link.  Parameters and
gradients stay in device memory.  Bar as for the device-resident step."""
import numpy as np
import pytest
import torch

import oracle
from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W
from parity import Compare, Quant8, as_f32, param_rtol, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bitopt.lib()


def _page_out(q):
    """Move q's state arrays into host_state() memory (same contents)."""
    for key in ("s1", "s2", "a1", "a2"):
        t = q.d.get(key)
        if t is None:
            continue
        h = bitopt.host_state(t.numel(), t.dtype)
        h.copy_(t.cpu())
        q.d[key] = h


CASES = [
    ("adam", "f32", 256, dict(optimizer="adam", lr=1e-3, weight_decay=0.01)),
    ("ademamix", "bf16", 256, dict(optimizer="ademamix", lr=1e-3, beta3=0.9999, alpha=5.0, t_alpha=3, t_beta3=3)),
    ("momentum", "f16", 2048, dict(optimizer="momentum", lr=0.01, beta1=0.9, weight_decay=0.01)),
    ("rmsprop", "f32", 256, dict(optimizer="rmsprop", lr=0.01, beta1=0.9, eps=1e-8)),
]


@pytest.mark.parametrize("name,dtype,bs,hp", CASES, ids=[c[0] for c in CASES])
def test_paged_state_8bit(name, dtype, bs, hp):
    n = 7 * 1024 + 300 + 4 if name != "ademamix" else 7 * 1024 + 304
    hp = dict(hp, blocksize=bs)
    p0 = W.to_dtype(W.normal_f32([1700, 1], n, 0.02), dtype)
    q = Quant8(hp, p0, dtype)
    _page_out(q)
    assert not q.d["s1"].is_cuda
    cmp = Compare()
    for t in range(1, 4):
        g = W.to_dtype(W.normal_f32([1700, 2, t], n, 0.01), dtype)
        q.step_gpu(t, to_dev(g, dtype))
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")
    print(f"\n[paged {name} {dtype} B{bs}] " + cmp.summary())


def test_paged_state_32bit():
    n = 5000
    hp = dict(optimizer="adam", lr=1e-3, weight_decay=0.01, blocksize=256)
    p0 = W.normal_f32([1710, 1], n, 0.02)
    op, os1, os2 = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    dp = to_dev(p0, "f32")
    ds1, ds2 = bitopt.host_state(n, torch.float32), bitopt.host_state(n, torch.float32)
    ds1.zero_(); ds2.zero_()
    for t in range(1, 4):
        g = W.normal_f32([1710, 2, t], n, 0.01)
        bitopt.step_32bit_2state(hp, t, dp, to_dev(g, "f32"), ds1, ds2)
        oracle.step_32bit(hp, t, op, g, "f32", os1, os2)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(dp), op)
        np.testing.assert_array_equal(ds1.numpy(), os1)
        np.testing.assert_array_equal(ds2.numpy(), os2)


def test_paged_state_tensorwise_and_paging_back():
    """Tensor-wide step on host state, then the state paged back into HBM (a copy)
    and stepped there: the trajectory is the one of the oracle throughout."""
    n = 6000
    hp = dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01, blocksize=0)
    p0 = W.normal_f32([1720, 1], n, 0.02)
    q1 = oracle.dynamic_map(True)
    o = dict(p=p0.copy(), s1=np.zeros(n, np.uint8), a1=np.zeros(1, np.float32))
    dp = to_dev(p0, "f32")
    hs1, ha1 = bitopt.host_state(n), bitopt.host_state(1, torch.float32)
    hs1.zero_(); ha1.zero_()
    dq = torch.from_numpy(q1).cuda()
    ws = None
    for t in range(1, 5):
        g = W.normal_f32([1720, 2, t], n, 0.01)
        if t == 3:                                     # page the state back into device memory
            torch.cuda.synchronize()
            hs1, ha1 = hs1.cuda(), ha1.cuda()
        ws = bitopt.step_8bit_tensorwise(hp, t, dp, to_dev(g, "f32"), hs1, ha1, dq, workspace=ws)
        oracle.step_8bit(hp, t, o["p"], g, "f32", o["s1"], o["a1"], q1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(dp), o["p"])
        np.testing.assert_array_equal(hs1.cpu().numpy(), o["s1"])
        np.testing.assert_array_equal(ha1.cpu().numpy(), o["a1"])


# ------------------------------------------------------------------ staged paging
# bitopt_step_8bit_paged: the state lives in host memory and is paged chunk by chunk
# through two HBM staging buffers (copy-in on one stream, the step on the launch
# stream, write-back on another).

STAGED = [
    ("adam", "f32", 256, dict(optimizer="adam", lr=1e-3, weight_decay=0.01)),
    ("ademamix", "bf16", 256, dict(optimizer="ademamix", lr=1e-3, beta3=0.9999, alpha=5.0, t_alpha=3, t_beta3=3)),
    ("momentum", "f16", 2048, dict(optimizer="momentum", lr=0.01, beta1=0.9, weight_decay=0.01, skip_zeros=True)),
    ("lion", "bf16", 256, dict(optimizer="lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01)),
]


def _staged_step(q, t, g_dev, staging, streams):
    d = q.d
    bitopt.step_8bit_paged(q.hp, t, d["p"], g_dev, d["s1"], d["a1"], d["q1"], d.get("s2"), d.get("a2"),
                           d["q2"] if q.two else None, staging=staging, h2d_stream=streams[0],
                           d2h_stream=streams[1])


@pytest.mark.parametrize("name,dtype,bs,hp", STAGED, ids=[c[0] for c in STAGED])
def test_staged_paged_step_matches_oracle(name, dtype, bs, hp):
    """Chunks of 4096 elements (the smallest staging), several chunks and a ragged last
    one, three steps against the oracle's own trajectory."""
    n = 3 * 4096 + 1232 + (0 if name == "ademamix" else 5)
    hp = dict(hp, blocksize=bs)
    print(f"\n[case] staged paging {name} {dtype} B{bs} n={n}", flush=True)
    p0 = W.to_dtype(W.normal_f32([1750, 1], n, 0.02), dtype)
    q = Quant8(hp, p0, dtype)
    _page_out(q)
    staging = torch.empty(bitopt.paged_staging_bytes(hp, 4096), dtype=torch.uint8, device="cuda")
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    cmp = Compare()
    for t in range(1, 4):
        g = W.normal_f32([1750, 2, t], n, 0.01)
        if hp.get("skip_zeros"):
            g[2048 * 2: 2048 * 5] = 0.0
        g = W.to_dtype(g, dtype)
        _staged_step(q, t, to_dev(g, dtype), staging, streams)
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")
    print("  " + cmp.summary())


@pytest.mark.parametrize("name,dtype,bs,hp", STAGED, ids=[c[0] for c in STAGED])
def test_staged_paged_step_equals_device_resident(name, dtype, bs, hp):
    """A larger tensor (several 1 Mi-element chunks, ragged tail): the staged step is
    bit-identical to the device-resident step over four steps, including when the
    host state is read back between steps."""
    n = 5 * (1 << 20) + 3 * 4096 + 48
    hp = dict(hp, blocksize=bs)
    print(f"\n[case] staged vs resident {name} {dtype} B{bs} n={n}", flush=True)
    p0 = W.to_dtype(W.normal_f32([1760, 1], n, 0.02), dtype)
    A = Quant8(hp, p0, dtype)          # paged
    B = Quant8(hp, p0, dtype)          # device-resident
    _page_out(A)
    staging = torch.empty(bitopt.paged_staging_bytes(hp, 1 << 20), dtype=torch.uint8, device="cuda")
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    for t in range(1, 5):
        g = W.normal_f32([1760, 2, t], n, 0.01)
        if hp.get("skip_zeros"):
            g[: n // 4] = 0.0
        gd = to_dev(W.to_dtype(g, dtype), dtype)
        _staged_step(A, t, gd, staging, streams)
        B.step_gpu(t, gd)
        torch.cuda.synchronize()
        for key in ("p", "s1", "s2", "a1", "a2"):
            if key in A.d and A.d[key] is not None:
                np.testing.assert_array_equal(to_host(A.d[key]) if A.d[key].is_cuda else A.d[key].numpy(),
                                              to_host(B.d[key]), err_msg=f"step {t} {key}")


def test_staged_paged_argument_errors():
    hp = dict(optimizer="adam", blocksize=256)
    n = 8192
    p = torch.zeros(n, device="cuda")
    s1, s2 = bitopt.host_state(n), bitopt.host_state(n)
    a1, a2 = bitopt.host_state(n // 256, torch.float32), bitopt.host_state(n // 256, torch.float32)
    q = bitopt.create_dynamic_map(True).cuda()
    st = (torch.cuda.Stream(), torch.cuda.Stream())
    small = torch.empty(bitopt.paged_staging_bytes(hp, 4096) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(bitopt.BitoptError, match="staging"):
        bitopt.step_8bit_paged(hp, 1, p, p, s1, a1, q, s2, a2, q, staging=small, h2d_stream=st[0], d2h_stream=st[1])
    ok = torch.empty(bitopt.paged_staging_bytes(hp, 4096), dtype=torch.uint8, device="cuda")
    with pytest.raises(bitopt.BitoptError, match="distinct"):
        bitopt.step_8bit_paged(hp, 1, p, p, s1, a1, q, s2, a2, q, staging=ok, h2d_stream=st[0], d2h_stream=st[0])
    torch.cuda.synchronize()


# ------------------------------------------------------------------ paged state in an HBM page pool
# bitopt_step_8bit_pooled: host-resident state cached page by page in HBM frames;
# resident pages are stepped in place, missing ones are copied in after the least
# recently used frame is written back.  Host buffers are current after a flush.

def _pooled_step(pool, q, t, g_dev, stream=None):
    d = q.d
    pool.step(q.hp, t, d["p"], g_dev, d["s1"], d["a1"], d["q1"], d.get("s2"), d.get("a2"),
              d["q2"] if q.two else None, stream=stream)


@pytest.mark.parametrize("name,dtype,bs,hp", STAGED, ids=[c[0] for c in STAGED])
def test_pooled_step_resident_matches_oracle(name, dtype, bs, hp):
    """Every page fits: the first step copies each page in once, later steps hit; the
    host buffers, flushed after each step, follow the oracle's trajectory."""
    n = 3 * 4096 + 1232 + (0 if name == "ademamix" else 5)
    hp = dict(hp, blocksize=bs)
    print(f"\n[case] pooled resident {name} {dtype} B{bs} n={n}", flush=True)
    p0 = W.to_dtype(W.normal_f32([1770, 1], n, 0.02), dtype)
    q = Quant8(hp, p0, dtype)
    _page_out(q)
    pool = bitopt.PagePool(hp, 4096, nframes=6)
    cmp = Compare()
    for t in range(1, 4):
        g = W.normal_f32([1770, 2, t], n, 0.01)
        if hp.get("skip_zeros"):
            g[2048 * 2: 2048 * 5] = 0.0
        g = W.to_dtype(g, dtype)
        _pooled_step(pool, q, t, to_dev(g, dtype))
        pool.flush()
        q.step_oracle(t, g)
        q.compare(cmp, f"step {t}")
    st = pool.stats()
    assert st == dict(resident=4, page_ins=4, write_backs=12, hits=8), st
    pool.close()
    print("  " + cmp.summary())


@pytest.mark.parametrize("name,dtype,bs,hp", STAGED, ids=[c[0] for c in STAGED])
def test_pooled_step_oversubscribed_equals_device_resident(name, dtype, bs, hp):
    """Two tensors of six pages each through three frames (every step evicts and
    writes back), one of them stepped on a second stream for a while, and an evicting
    flush midway: bit-identical to the device-resident step over four steps."""
    n = 5 * 4096 + 48
    hp = dict(hp, blocksize=bs)
    print(f"\n[case] pooled oversubscribed {name} {dtype} B{bs} n={n}", flush=True)
    pool = bitopt.PagePool(hp, 4096, nframes=3)
    side = torch.cuda.Stream()
    pairs = []
    for j in range(2):
        p0 = W.to_dtype(W.normal_f32([1780, 1, j], n, 0.02), dtype)
        A, B = Quant8(hp, p0, dtype), Quant8(hp, p0, dtype)
        _page_out(A)
        pairs.append((A, B))
    for t in range(1, 5):
        for j, (A, B) in enumerate(pairs):
            g = W.normal_f32([1780, 2, t, j], n, 0.01)
            if hp.get("skip_zeros"):
                g[: n // 3] = 0.0
            gd = to_dev(W.to_dtype(g, dtype), dtype)
            if j == 1 and t in (2, 3):                     # the second tensor on another stream
                side.wait_stream(torch.cuda.current_stream())
                _pooled_step(pool, A, t, gd, stream=side)
                torch.cuda.current_stream().wait_stream(side)
            else:
                _pooled_step(pool, A, t, gd)
            B.step_gpu(t, gd)
        pool.flush(evict=(t == 2))
        torch.cuda.synchronize()
        for j, (A, B) in enumerate(pairs):
            for key in ("p", "s1", "s2", "a1", "a2"):
                if A.d.get(key) is not None:
                    np.testing.assert_array_equal(to_host(A.d[key]) if A.d[key].is_cuda else A.d[key].numpy(),
                                                  to_host(B.d[key]), err_msg=f"step {t} tensor {j} {key}")
    st = pool.stats()
    assert st["page_ins"] == 4 * 2 * 6 and st["hits"] == 0, st
    pool.close()


def test_pooled_step_large_pages_and_refusals():
    """Adam fp32 over 1 Mi-element pages, first with room for half the pages, then in a
    pool that holds them all (no copies after the first step); the companion-buffer
    and hyper-parameter checks of a pooled step."""
    hp = dict(optimizer="adam", lr=1e-3, weight_decay=0.01, blocksize=256)
    n = 5 * (1 << 20) + 3 * 4096 + 48
    print(f"\n[case] pooled large adam f32 n={n}", flush=True)
    p0 = W.normal_f32([1790, 1], n, 0.02)
    A, B = Quant8(hp, p0, "f32"), Quant8(hp, p0, "f32")
    _page_out(A)
    small = bitopt.PagePool(hp, 1 << 20, nframes=3)
    big = bitopt.PagePool(hp, 1 << 20, nframes=6)
    for t in range(1, 6):
        gd = to_dev(W.normal_f32([1790, 2, t], n, 0.01), "f32")
        if t == 3:                                         # move the state from one pool to the other
            small.flush(evict=True)
        _pooled_step(small if t < 3 else big, A, t, gd)
        B.step_gpu(t, gd)
    big.flush()
    torch.cuda.synchronize()
    for key in ("p", "s1", "s2", "a1", "a2"):
        np.testing.assert_array_equal(to_host(A.d[key]) if A.d[key].is_cuda else A.d[key].numpy(),
                                      to_host(B.d[key]), err_msg=key)
    assert big.stats()["page_ins"] == 6 and big.stats()["hits"] == 12, big.stats()
    d = A.d
    other = bitopt.host_state(A.nb, torch.float32)
    with pytest.raises(bitopt.BitoptError, match="companion"):
        big.step(hp, 6, d["p"], d["p"], d["s1"], other, d["q1"], d["s2"], d["a2"], d["q2"])
    with pytest.raises(bitopt.BitoptError, match="blocksize"):
        nb = -(-n // 2048)
        big.step(dict(hp, blocksize=2048), 6, d["p"], d["p"], d["s1"], d["a1"][:nb], d["q1"], d["s2"], d["a2"][:nb],
                 d["q2"])
    small.close()
    big.close()
    torch.cuda.synchronize()
