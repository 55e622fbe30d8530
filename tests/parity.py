"""Shared helpers of the GPU parity tests: run the HIP path (through the C ABI) and
the CPU oracle from the same seeded inputs and compare them to the acceptance bar.

Bar: uint8 codes bit-exact except at code-boundary ties, where at most 1e-4 of
the elements may differ and each by one index; parameters and absmax within 1e-6
relative (fp32 parameters) or 1e-3 (fp16/bf16 parameters).  Inputs never come from
the HIP path: the oracle starts from the same generated inputs and runs its own
trajectory.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from bit_optimizers_block_amd import bitopt
from bit_optimizers_block_amd import workloads as W

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CODE_MISMATCH_FRAC = 1e-4


def param_rtol(dtype):
    return 1e-6 if dtype == "f32" else 1e-3


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy -> device tensor; bf16 arrays are uint16 bit patterns."""
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor, dtype=None) -> np.ndarray:
    if dtype == "bf16" or t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return oracle.widen(a, dtype) if dtype != "f32" else a.astype(np.float32)


def n_states(opt):
    return oracle.NUM_STATES[opt]


class Compare:
    """Accumulates the comparison statistics of one test."""

    def __init__(self):
        self.code_elems = 0
        self.code_mismatch = 0
        self.max_code_diff = 0
        self.max_p_rel = 0.0
        self.max_a_rel = 0.0
        self.bit_exact = True

    def codes(self, gpu: np.ndarray, ref: np.ndarray, what=""):
        assert gpu.shape == ref.shape, what
        d = np.abs(gpu.astype(np.int32) - ref.astype(np.int32))
        self.code_elems += d.size
        self.code_mismatch += int((d != 0).sum())
        self.max_code_diff = max(self.max_code_diff, int(d.max(initial=0)))
        if d.any():
            self.bit_exact = False
        assert self.max_code_diff <= 1, f"{what}: a code differs by {self.max_code_diff} indices"
        assert self.code_mismatch <= CODE_MISMATCH_FRAC * self.code_elems, \
            f"{what}: {self.code_mismatch} of {self.code_elems} codes differ"

    def values(self, gpu: np.ndarray, ref: np.ndarray, rtol: float, what="", kind="p"):
        assert gpu.shape == ref.shape, what
        g = gpu.astype(np.float64)
        r = ref.astype(np.float64)
        same = (g == r) | (np.isnan(g) & np.isnan(r))
        if not same.all():
            self.bit_exact = False
        err = np.abs(g - r)
        scale = np.abs(r)
        rel = np.where(same, 0.0, err / np.maximum(scale, 1e-30))
        worst = float(rel.max(initial=0.0))
        if kind == "p":
            self.max_p_rel = max(self.max_p_rel, worst)
        else:
            self.max_a_rel = max(self.max_a_rel, worst)
        bad = ~same & (err > rtol * scale)
        assert not bad.any(), f"{what}: {int(bad.sum())} values beyond rtol {rtol}; worst rel {worst:.3e}"

    def summary(self):
        return (f"bit_exact={self.bit_exact} code_mismatch={self.code_mismatch}/{self.code_elems} "
                f"max_p_rel={self.max_p_rel:.2e} max_absmax_rel={self.max_a_rel:.2e}")


class Quant8:
    """One tensor's 8-bit optimizer state on the device and in the oracle."""

    def __init__(self, hp: dict, p0: np.ndarray, dtype: str, maps=None):
        """maps: optional (qmap1, qmap2) float32 arrays used on both sides in place of
        the standard signed/unsigned maps."""
        self.hp = dict(hp)
        self.dtype = dtype
        self.n = n = p0.size
        B = hp.get("blocksize", 256)
        self.nb = nb = (n + B - 1) // B
        opt = hp["optimizer"]
        self.k1 = 2 if opt == "ademamix" else 1
        self.two = n_states(opt) >= 2
        q1, q2 = oracle.dynamic_map(opt not in oracle.UNSIGNED_STATE1), oracle.dynamic_map(False)
        if maps is not None:
            q1 = maps[0] if maps[0] is not None else q1
            q2 = maps[1] if maps[1] is not None else q2
        # oracle side
        self.o = dict(p=p0.copy(), s1=np.zeros(self.k1 * n, np.uint8), a1=np.zeros(self.k1 * nb, np.float32),
                      s2=np.zeros(n, np.uint8) if self.two else None,
                      a2=np.zeros(nb, np.float32) if self.two else None, q1=q1, q2=q2)
        # device side (codebooks from the library's own builder)
        self.d = dict(p=to_dev(p0, dtype), s1=torch.zeros(self.k1 * n, dtype=torch.uint8, device="cuda"),
                      a1=torch.zeros(self.k1 * nb, dtype=torch.float32, device="cuda"),
                      q1=bitopt.create_dynamic_map(opt not in oracle.UNSIGNED_STATE1).cuda(),
                      q2=bitopt.create_dynamic_map(False).cuda())
        if maps is not None:
            self.d["q1"] = torch.from_numpy(np.ascontiguousarray(q1, np.float32)).cuda()
            self.d["q2"] = torch.from_numpy(np.ascontiguousarray(q2, np.float32)).cuda()
        if self.two:
            self.d["s2"] = torch.zeros(n, dtype=torch.uint8, device="cuda")
            self.d["a2"] = torch.zeros(nb, dtype=torch.float32, device="cuda")

    def step_gpu(self, t: int, g_dev: torch.Tensor):
        d = self.d
        if self.two:
            bitopt.step_8bit_blockwise_2state(self.hp, t, d["p"], g_dev, d["s1"], d["s2"], d["a1"], d["a2"],
                                              d["q1"], d["q2"])
        else:
            bitopt.step_8bit_blockwise_1state(self.hp, t, d["p"], g_dev, d["s1"], d["a1"], d["q1"])

    def step_oracle(self, t: int, g: np.ndarray):
        o = self.o
        oracle.step_8bit(self.hp, t, o["p"], g, self.dtype, o["s1"], o["a1"], o["q1"],
                         o["s2"], o["a2"], o["q2"] if self.two else None)

    def compare(self, cmp: Compare, what=""):
        torch.cuda.synchronize()
        d, o = self.d, self.o
        cmp.codes(to_host(d["s1"]), o["s1"], what + " state1")
        cmp.values(to_host(d["a1"]), o["a1"], param_rtol(self.dtype), what + " absmax1", kind="a")
        if self.two:
            cmp.codes(to_host(d["s2"]), o["s2"], what + " state2")
            cmp.values(to_host(d["a2"]), o["a2"], param_rtol(self.dtype), what + " absmax2", kind="a")
        cmp.values(as_f32(to_host(d["p"], self.dtype), self.dtype), as_f32(o["p"], self.dtype),
                   param_rtol(self.dtype), what + " p")


class SampledTensor:
    """Full-size 8-bit (or 32-bit) state of one tensor on the device; the oracle
    follows a sample of its blocks, each block as a one-block tensor of its own
    (blocks are independent, so this is the same computation)."""

    def __init__(self, hp: dict, n: int, dtype: str, blocks, p0_full: np.ndarray, eight: bool = True):
        self.hp = dict(hp)
        self.n, self.dtype, self.eight = n, dtype, eight
        B = hp["blocksize"]
        self.B = B
        self.nb = nb = (n + B - 1) // B
        opt = hp["optimizer"]
        self.k1 = 2 if opt == "ademamix" else 1
        self.two = n_states(opt) >= 2
        self.blocks = np.array(sorted(set(int(b) for b in blocks if 0 <= b < nb)), dtype=np.int64)
        sd = torch.uint8 if eight else torch.float32
        self.d = dict(p=to_dev(p0_full, dtype),
                      s1=torch.zeros(self.k1 * n, dtype=sd, device="cuda"),
                      s2=torch.zeros(n, dtype=sd, device="cuda") if self.two else None,
                      a1=torch.zeros(self.k1 * nb, device="cuda") if eight else None,
                      a2=torch.zeros(nb, device="cuda") if (eight and self.two) else None)
        self.unsigned1 = opt in oracle.UNSIGNED_STATE1
        self.q = (oracle.dynamic_map(not self.unsigned1), oracle.dynamic_map(False))
        self.o = []
        for b in self.blocks:
            lo, hi = b * B, min(n, (b + 1) * B)
            L = hi - lo
            if eight:
                st = dict(s1=np.zeros(self.k1 * L, np.uint8), a1=np.zeros(self.k1, np.float32),
                          s2=np.zeros(L, np.uint8) if self.two else None,
                          a2=np.zeros(1, np.float32) if self.two else None)
            else:
                st = dict(s1=np.zeros(self.k1 * L, np.float32), s2=np.zeros(L, np.float32) if self.two else None)
            st["p"] = p0_full[lo:hi].copy()
            st["lo"], st["hi"] = lo, hi
            self.o.append(st)
        idx = np.concatenate([np.arange(o["lo"], o["hi"]) for o in self.o]) if self.o else np.zeros(0, np.int64)
        self.idx = torch.from_numpy(idx).cuda()
        self.bidx = torch.from_numpy(self.blocks).cuda()

    def desc(self, g_dev):
        """This tensor as a multi-tensor descriptor."""
        return dict(p=self.d["p"], g=g_dev, state1=self.d["s1"], state2=self.d["s2"],
                    absmax1=self.d["a1"], absmax2=self.d["a2"], is_8bit=self.eight)

    def step_gpu(self, t, g_dev):
        d = self.d
        if self.eight and self.two:
            bitopt.step_8bit_blockwise_2state(self.hp, t, d["p"], g_dev, d["s1"], d["s2"], d["a1"], d["a2"],
                                              *self.qdev())
        elif self.eight:
            bitopt.step_8bit_blockwise_1state(self.hp, t, d["p"], g_dev, d["s1"], d["a1"],
                                              self.qdev()[1 if self.unsigned1 else 0])
        elif self.two:
            bitopt.step_32bit_2state(self.hp, t, d["p"], g_dev, d["s1"], d["s2"])
        else:
            bitopt.step_32bit_1state(self.hp, t, d["p"], g_dev, d["s1"])

    _qd = None

    @classmethod
    def qdev(cls):
        if cls._qd is None:
            cls._qd = (bitopt.create_dynamic_map(True).cuda(), bitopt.create_dynamic_map(False).cuda())
        return cls._qd

    def step_oracle(self, t, g_full: np.ndarray):
        q1, q2 = self.q
        for st in self.o:
            g = np.ascontiguousarray(g_full[st["lo"]:st["hi"]])
            if self.eight:
                oracle.step_8bit(self.hp, t, st["p"], g, self.dtype, st["s1"], st["a1"], q1,
                                 st["s2"], st["a2"], q2 if self.two else None)
            else:
                oracle.step_32bit(self.hp, t, st["p"], g, self.dtype, st["s1"], st["s2"])

    def compare(self, cmp: Compare, what=""):
        torch.cuda.synchronize()
        if not self.o:
            return
        d = self.d
        n, nb = self.n, self.nb
        p_g = to_host(d["p"][self.idx], self.dtype)
        p_o = np.concatenate([st["p"] for st in self.o])
        cmp.values(as_f32(p_g, self.dtype), as_f32(p_o, self.dtype), param_rtol(self.dtype), what + " p")
        for k in range(self.k1):
            s_g = to_host(d["s1"][self.idx + k * n])
            s_o = np.concatenate([st["s1"][k * (st["hi"] - st["lo"]):(k + 1) * (st["hi"] - st["lo"])]
                                  for st in self.o])
            if self.eight:
                cmp.codes(s_g, s_o, what + f" state1[{k}]")
                a_g = to_host(d["a1"][self.bidx + k * nb])
                a_o = np.array([st["a1"][k] for st in self.o], np.float32)
                cmp.values(a_g, a_o, param_rtol(self.dtype), what + f" absmax1[{k}]", kind="a")
            else:
                cmp.values(s_g, s_o, 1e-6, what + " state1", kind="a")
        if self.two:
            s_g = to_host(d["s2"][self.idx])
            s_o = np.concatenate([st["s2"] for st in self.o])
            if self.eight:
                cmp.codes(s_g, s_o, what + " state2")
                a_g = to_host(d["a2"][self.bidx])
                a_o = np.array([st["a2"][0] for st in self.o], np.float32)
                cmp.values(a_g, a_o, param_rtol(self.dtype), what + " absmax2", kind="a")
            else:
                cmp.values(s_g, s_o, 1e-6, what + " state2", kind="a")


def sample_blocks(nb: int, k: int, seed: int, extra=()):
    rng = np.random.default_rng(seed)
    pick = rng.choice(nb, size=min(k, nb), replace=False)
    return np.unique(np.concatenate([pick, [0, nb - 1], np.asarray(extra, np.int64)]))
