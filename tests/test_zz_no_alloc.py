"""ssd_forward_noalloc (the forward on the library's static device scratch) against ssd_forward
(the same forward with a caller-owned workspace), through the C ABI.

Both calls launch the same kernels at the same chunk, so their outputs must be
identical bit for bit.  Two calls in a row, the second on a smaller problem,
show that what an earlier call leaves in the shared scratch does not leak into
a later result.
"""

from __future__ import annotations

import math

import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs(b, L, H, P, N, G, seed):
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(seed)
    f32 = dict(device=dev, dtype=torch.float32, generator=gen)
    x = torch.randn((b, L, H, P), **f32).to(torch.bfloat16)
    dt = torch.exp(torch.empty((b, L, H), device=dev, dtype=torch.float32)
                   .uniform_(math.log(1e-3), math.log(0.1), generator=gen)).to(torch.bfloat16)
    A = -torch.exp(torch.empty(H, device=dev, dtype=torch.float32).uniform_(0.0, math.log(16.0), generator=gen))
    Bm = (torch.randn((b, L, G, N), **f32) / math.sqrt(N)).to(torch.bfloat16)
    Cm = (torch.randn((b, L, G, N), **f32) / math.sqrt(N)).to(torch.bfloat16)
    D = torch.randn(H, **f32)
    h0 = 0.1 * torch.randn((b, H, P, N), **f32)
    return x, dt, A, Bm, Cm, D, h0


@pytest.mark.parametrize("shape", [
    # (b, L, H, P, N, G): the 2.7B-shaped forward at 64K tokens (about 108 MB of scratch), then a
    # smaller ragged problem on the same scratch
    [(1, 65536, 80, 64, 128, 1), (2, 3000, 24, 64, 128, 1)],
    [(1, 20000, 32, 64, 64, 1), (1, 777, 4, 64, 64, 2)],
], ids=["2p7b_64k_then_ragged", "n64_then_ragged_groups"])
def test_noalloc_matches_forward_twice(gpu_ssd, shape):
    for i, (b, L, H, P, N, G) in enumerate(shape):
        print(f"ssd_forward_noalloc call {i + 1}: b={b} L={L} H={H} P={P} N={N} G={G}", flush=True)
        x, dt, A, Bm, Cm, D, h0 = _inputs(b, L, H, P, N, G, seed=100 + i)
        y_ref, f_ref = gpu_ssd.forward(x, dt, A, Bm, Cm, D, h0)
        y = torch.empty_like(x)
        fin = torch.empty_like(f_ref)
        gpu_ssd.forward_noalloc(x, dt, A, Bm, Cm, D, h0, y=y, final_state=fin)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {i + 1}: y differs from ssd_forward"
        assert torch.equal(fin, f_ref), f"call {i + 1}: final state differs from ssd_forward"


def test_noalloc_rejects_oversize_shape(gpu_ssd):
    """A shape whose forward needs more than the 128 MiB scratch is refused before any launch."""
    # the 2.7B shape at 256K tokens: its per-position decay arrays alone take 168 MB
    b, L, H, P, N, G = 1, 262144, 80, 64, 128, 1
    x = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda:0")
    dt = torch.empty((b, L, H), dtype=torch.bfloat16, device="cuda:0")
    A = torch.empty(H, dtype=torch.float32, device="cuda:0")
    Bm = torch.empty((b, L, G, N), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError, match="workspace too small.*static scratch"):
        gpu_ssd.forward_noalloc(x, dt, A, Bm, Bm.clone())
