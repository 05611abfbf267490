"""GPU: the allocation-free split-K forward against the workspace one.

streamkl_fwd_splitk_noalloc runs the same kernels as streamkl_fwd_splitk with
the partial row states in the library's own per-GPU device array, so its
results must equal the workspace entry point's bit for bit; both are also held
to the oracle.  Two calls in a row, the second on a smaller problem, check
that a call does not depend on what the previous one left in the array; the
second call must not raise the device's memory use.  A third, smaller call
takes e4m3 inputs (the fp8 path through the same scratch).
"""
import math

import pytest
import torch

import synth
from attention_kl_divergence_online_amd import StreamKLError, streamkl_fwd_splitk, streamkl_fwd_splitk_noalloc
from attention_kl_divergence_online_amd import _lib
from parity_util import TOL, assert_within, compare_forward

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rand(B, H, NQ, NK, D, seed, dtype, noise=0.2):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q1 = torch.randn(B, H, NQ, D, generator=g)
    k1 = torch.randn(B, H, NK, D, generator=g)
    q2 = q1 + noise * torch.randn(B, H, NQ, D, generator=g)
    k2 = k1 + noise * torch.randn(B, H, NK, D, generator=g)
    cast = synth.to_fp8 if dtype == "fp8" else (lambda t: t.to(torch.bfloat16))
    return [cast(t).to(DEV).contiguous() for t in (q1, k1, q2, k2)]


# Larger first, then smaller: the second call finds the first call's states in
# the scratch beyond its own range and must neither read nor need them.
CASES = [
    # B, H, NQ, NK, D, causal, splits, inputs
    (2, 4, 300, 5000, 128, True, 16, "bf16"),
    (1, 2, 40, 900, 64, False, 5, "bf16"),
]
if hasattr(torch, "float8_e4m3fn"):
    CASES.append((1, 1, 33, 700, 128, True, 3, "fp8"))


def test_noalloc_splitk_equals_workspace_entry_point():
    for i, (B, H, NQ, NK, D, causal, splits, dt) in enumerate(CASES):
        print(f"noalloc split-K call {i}: B={B} H={H} NQ={NQ} NK={NK} D={D} causal={causal} splits={splits} {dt}",
              flush=True)
        q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, seed=31 + i, dtype=dt)
        scale = 1.0 / math.sqrt(D)
        ref = streamkl_fwd_splitk(q1, k1, q2, k2, splits, scale, causal)
        got = tuple(torch.full((B, H, NQ), float("nan"), device=DEV) for _ in range(3))
        torch.cuda.synchronize()
        held = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        free_before = torch.cuda.mem_get_info()[0]
        streamkl_fwd_splitk_noalloc(q1, k1, q2, k2, splits, scale, causal, out=got)
        torch.cuda.synchronize()
        if i > 0:  # after the first call has set the array up on this GPU
            assert torch.cuda.max_memory_allocated() == held
            assert torch.cuda.mem_get_info()[0] >= free_before
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        heads = [(b, h) for b in range(B) for h in range(H)]
        assert_within(compare_forward(q1, k1, q2, k2, scale, causal, *got, heads), TOL["bf16"],
                      f"noalloc split-K call {i}")


def test_noalloc_rejects_problems_past_the_scratch():
    # 128 splits of 1024 queries x 32 heads need 80 MiB of partial states.
    B, H, NQ, NK, D = 1, 32, 1024, 8192, 64
    q1, k1, q2, k2 = (torch.zeros(B, H, n, D, dtype=torch.bfloat16, device=DEV) for n in (NQ, NK, NQ, NK))
    with pytest.raises(StreamKLError) as e:
        streamkl_fwd_splitk_noalloc(q1, k1, q2, k2, 128, None, False)
    assert e.value.status == _lib.STREAMKL_ERR_WORKSPACE
    kl, _, _ = streamkl_fwd_splitk_noalloc(q1, k1, q2, k2, 64, None, False)  # 40 MiB: fits
    torch.cuda.synchronize()
    assert torch.equal(kl, torch.zeros_like(kl))  # identical (zero) teacher and student
