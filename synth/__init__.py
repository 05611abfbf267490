"""Seeded synthetic teacher/student attention inputs.

This module only draws random numbers and casts them; it holds none of the
attention-KL arithmetic.  Both the HIP path (tests, bench) and the oracle read
the tensors it produces.

Workloads follow the shapes the StreamKL pages evaluate: context lengths
4K-512K, causal and non-causal masking, and a short-query / long-key case for
the split-K variant (StreamKL: arXiv 2606.20005, gist.science "Resultados
Experimentales" and "Optimizaciones de Kernel de GPU").  The pages publish no
dataset; Gaussian queries/keys stand in for real teacher/student projections.

Seeding is per (config, batch, head, tensor) so any single head can be drawn on
its own: seed = 1_000_003*cfg_id + 1009*(b*H + h) + tensor_id, tensor_id
Q1=0, K1=1, Q2-noise (or Q2)=2, K2-noise (or K2)=3.  Normals are drawn in fp32
and the student is formed in fp32; bf16 workloads then cast with
round-to-nearest-even, and everything downstream reads the cast values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "get", "make_head", "make_inputs", "upstream_grad",
           "PackedBatch", "PACKED", "make_packed", "packed_grad"]


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    B: int
    H: int
    NQ: int
    NK: int
    D: int
    dtype: str            # "fp32" or "bf16"
    causal: bool
    teacher_std: float = 1.0
    student: str = "noise"    # "noise": Q2=Q1+s*N, K2=K1+s*N ; "independent": Q2,K2 ~ N(0,1)
    noise: float = 0.1
    splits: int = 1           # split-K chunk count used for this workload (1 = unsplit)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask keeps, over all batch*heads."""
        if not self.causal:
            per_head = self.NQ * self.NK
        else:
            # bottom-right alignment: row i sees keys 0..i+(NK-NQ), i.e. i+NK-NQ+1 keys
            off = self.NK - self.NQ
            per_head = self.NQ * (off + 1) + self.NQ * (self.NQ - 1) // 2
        return self.B * self.H * per_head

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload(0, "tiny_fp32", 1, 2, 256, 256, 64, "fp32", False, noise=0.3),
        Workload(1, "causal_4k", 2, 32, 4096, 4096, 128, "bf16", True, noise=0.1),
        Workload(2, "noncausal_16k", 1, 32, 16384, 16384, 128, "bf16", False,
                 teacher_std=1.5, student="independent"),
        Workload(3, "causal_64k", 1, 32, 65536, 65536, 128, "bf16", True, noise=0.1),
        Workload(4, "splitk_512k", 1, 32, 1024, 524288, 128, "bf16", False, noise=0.2, splits=64),
        Workload(5, "splitk_bwd_128k", 1, 32, 1024, 131072, 128, "bf16", False, noise=0.2, splits=16),
        # Decode step: 16 new queries per sequence against a 128K-key cache, split-K forward.
        Workload(6, "decode_128k", 4, 32, 16, 131072, 128, "bf16", True, noise=0.2, splits=64),
        # The D = 64 kernels at long context: 64 heads of 16K, causal.
        Workload(7, "causal_16k_d64", 1, 64, 16384, 16384, 64, "bf16", True, noise=0.1),
        # Few queries against a long key range, backward: 2 query tiles per head,
        # so the query-gradient pass splits its keys.
        Workload(9, "shortq_bwd_64k", 1, 32, 256, 65536, 128, "bf16", False, noise=0.2, splits=32),
        # fp32 inputs (the 1e-5 path) at a moderate causal context.
        Workload(8, "causal_4k_fp32", 2, 16, 4096, 4096, 128, "fp32", True, noise=0.3),
        # Short query ranges against 64K keys: 16 and 128 queries per head (the
        # fused single-visit backward with one and four query blocks).
        Workload(10, "shortq16_bwd_64k", 1, 32, 16, 65536, 128, "bf16", False, noise=0.2, splits=32),
        Workload(11, "shortq128_bwd_64k", 1, 32, 128, 65536, 128, "bf16", False, noise=0.2, splits=32),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _seed(w: Workload, b: int, h: int, tensor_id: int) -> int:
    return 1_000_003 * w.cfg_id + 1009 * (b * w.H + h) + tensor_id


def _normal(shape, seed: int, device: str) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device)


def make_head(w: Workload, b: int, h: int, device: str = "cpu"):
    """Return (q1, k1, q2, k2) for one (batch, head): [NQ,D] and [NK,D] in w's dtype."""
    q1 = _normal((w.NQ, w.D), _seed(w, b, h, 0), device) * w.teacher_std
    k1 = _normal((w.NK, w.D), _seed(w, b, h, 1), device) * w.teacher_std
    if w.student == "noise":
        q2 = q1 + w.noise * _normal((w.NQ, w.D), _seed(w, b, h, 2), device)
        k2 = k1 + w.noise * _normal((w.NK, w.D), _seed(w, b, h, 3), device)
    elif w.student == "independent":
        q2 = _normal((w.NQ, w.D), _seed(w, b, h, 2), device)
        k2 = _normal((w.NK, w.D), _seed(w, b, h, 3), device)
    else:
        raise ValueError(w.student)
    dt = w.torch_dtype
    return q1.to(dt), k1.to(dt), q2.to(dt), k2.to(dt)


def make_inputs(w: Workload, device: str = "cpu", heads: Optional[Iterable] = None):
    """Full [B,H,N,D] tensors (contiguous) drawn head by head on `device`.

    `heads`, if given, is an iterable of (b, h) pairs to fill; other heads stay
    zero (used to keep host-side work bounded)."""
    dt = w.torch_dtype
    q1 = torch.empty((w.B, w.H, w.NQ, w.D), dtype=dt, device=device)
    k1 = torch.empty((w.B, w.H, w.NK, w.D), dtype=dt, device=device)
    q2 = torch.empty_like(q1)
    k2 = torch.empty_like(k1)
    todo = list(heads) if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    if heads is not None:
        for t in (q1, k1, q2, k2):
            t.zero_()
    for b, h in todo:
        a, bb, c, d = make_head(w, b, h, device)
        q1[b, h].copy_(a)
        k1[b, h].copy_(bb)
        q2[b, h].copy_(c)
        k2[b, h].copy_(d)
    return q1, k1, q2, k2


def to_fp8(t: torch.Tensor) -> torch.Tensor:
    """`t` rounded to fp8 e4m3 (torch.float8_e4m3fn), on t's device: inputs for
    the fp8 forward, whose values the oracle then takes exactly."""
    return t.to(torch.float8_e4m3fn)


def upstream_grad(w: Workload, device: str = "cpu") -> torch.Tensor:
    """Per-row upstream gradient g of a mean-reduced loss: 1/(B*H*NQ) everywhere."""
    return torch.full((w.B, w.H, w.NQ), 1.0 / (w.B * w.H * w.NQ), dtype=torch.float32, device=device)


@dataclasses.dataclass(frozen=True)
class PackedBatch:
    """Variable-length sequences packed per head: sequence b has lens_q[b] query
    rows and lens_k[b] key rows; tensors are [H, sum(lens), D] (head-major)."""
    cfg_id: int
    name: str
    H: int
    lens_q: tuple
    lens_k: tuple
    D: int
    dtype: str
    causal: bool
    noise: float = 0.1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @staticmethod
    def _cu(lens):
        out = [0]
        for n in lens:
            out.append(out[-1] + n)
        return out

    @property
    def cu_q(self):
        return self._cu(self.lens_q)

    @property
    def cu_k(self):
        return self._cu(self.lens_k)

    def sequence(self, b: int) -> Workload:
        """Sequence b as a one-sequence workload (its seeds depend on b)."""
        return Workload(self.cfg_id, f"{self.name}[{b}]", len(self.lens_q), self.H, self.lens_q[b],
                        self.lens_k[b], self.D, self.dtype, self.causal, noise=self.noise)

    def visible_pairs(self) -> int:
        return sum(self.sequence(b).visible_pairs() // len(self.lens_q) for b in range(len(self.lens_q)))


def _mixed_lengths(n: int, lo: int, hi: int, seed: int) -> tuple:
    gen = torch.Generator()
    gen.manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen))


_MIX = _mixed_lengths(16, 1024, 7168, 77)
_SHORT = _mixed_lengths(256, 64, 1024, 78)

PACKED: Dict[str, PackedBatch] = {
    pb.name: pb for pb in [
        # 16 causal sequences of 1K-7K tokens (seeded uniform lengths), 32 heads: a
        # packed long-context batch without padding.
        PackedBatch(20, "varlen_mix", 32, _MIX, _MIX, 128, "bf16", True),
        # 256 causal sequences of 64-1024 tokens, 16 heads: many short sequences,
        # each far too small to fill the GPU on its own.
        PackedBatch(21, "varlen_short", 16, _SHORT, _SHORT, 128, "bf16", True),
    ]
}


def make_packed(pb: PackedBatch, device: str = "cpu"):
    """(q1, k1, q2, k2): [H, TQ, D] and [H, TK, D]; sequence b of head h is
    make_head(pb.sequence(b), b, h)."""
    dt = pb.torch_dtype
    cq, ck = pb.cu_q, pb.cu_k
    q1 = torch.empty((pb.H, cq[-1], pb.D), dtype=dt, device=device)
    k1 = torch.empty((pb.H, ck[-1], pb.D), dtype=dt, device=device)
    q2 = torch.empty_like(q1)
    k2 = torch.empty_like(k1)
    for b in range(len(pb.lens_q)):
        w = pb.sequence(b)
        for h in range(pb.H):
            a, bb, c, d = make_head(w, b, h, device)
            q1[h, cq[b]:cq[b + 1]].copy_(a)
            q2[h, cq[b]:cq[b + 1]].copy_(c)
            k1[h, ck[b]:ck[b + 1]].copy_(bb)
            k2[h, ck[b]:ck[b + 1]].copy_(d)
    return q1, k1, q2, k2


def packed_grad(pb: PackedBatch, device: str = "cpu") -> torch.Tensor:
    """Upstream gradient of a mean over all packed rows: 1/(H*TQ) everywhere, [H, TQ]."""
    tq = pb.cu_q[-1]
    return torch.full((pb.H, tq), 1.0 / (pb.H * tq), dtype=torch.float32, device=device)
