"""Entry points that take a stream, called with a non-default stream (queued
behind other work on it), give bit-for-bit the default-stream result."""
import numpy as np
import pytest
import torch

import fa_inputs as fi
from _gpu_util import bf16_to_dev

pytestmark = pytest.mark.gpu


def test_fwd_ex_and_decode_ex_use_the_given_stream(gpu_lib):
    fa = gpu_lib
    B, H, N, d = 1, 4, 1024, 128
    q, k, v = (bf16_to_dev(fi.bf16_tensor(9300, t, B, H, N, d)) for t in range(3))
    ref_o = torch.empty_like(q)
    ref_l = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, ref_o, ref_l, B, H, N, d, d ** -0.5, True)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    o = torch.zeros_like(q)
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    big = torch.randn(4096, 4096, device="cuda")
    with torch.cuda.stream(side):
        for _ in range(8):
            big = big @ big.T / 4096.0      # keep the side stream busy
    fa.fa_fwd_ex(q, k, v, o, lse, B, H, N, d, d ** -0.5, True, stream=side)
    side.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse, ref_l)

    # decode and grouped decode on the side stream, against the default stream
    Lkv, S = 4096, 16
    qd = bf16_to_dev(fi.bf16_tensor(9301, 0, 2, 8, 1, d))
    kc, vc = (bf16_to_dev(fi.bf16_tensor(9301, t, 2, 8, Lkv, d)) for t in (1, 2))
    nb = fa.fa_decode_workspace_bytes(2, 8, d, S)
    ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    od0, od1 = torch.empty_like(qd), torch.empty_like(qd)
    ld0, ld1 = (torch.empty((2, 8), dtype=torch.float32, device="cuda") for _ in range(2))
    fa.fa_decode_splitkv_ex(qd, kc, vc, od0, ld0, 2, 8, Lkv, d, S, d ** -0.5, ws, nb)
    torch.cuda.synchronize()
    ws2 = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    fa.fa_decode_splitkv_ex(qd, kc, vc, od1, ld1, 2, 8, Lkv, d, S, d ** -0.5, ws2, nb, stream=side)
    side.synchronize()
    assert torch.equal(od0.view(torch.int16), od1.view(torch.int16)) and torch.equal(ld0, ld1)
    og0, og1 = torch.empty_like(qd), torch.empty_like(qd)
    fa.fa_decode_splitkv_gqa(qd, kc[:, :2].contiguous(), vc[:, :2].contiguous(), og0, ld0, 2, 8, 2,
                             Lkv, d, S, d ** -0.5, ws, nb)
    torch.cuda.synchronize()
    fa.fa_decode_splitkv_gqa(qd, kc[:, :2].contiguous(), vc[:, :2].contiguous(), og1, ld1, 2, 8, 2,
                             Lkv, d, S, d ** -0.5, ws2, nb, stream=side)
    side.synchronize()
    assert torch.equal(og0.view(torch.int16), og1.view(torch.int16)) and torch.equal(ld0, ld1)


def test_bwd_uses_the_given_stream(gpu_lib):
    fa = gpu_lib
    B, H, N, d = 1, 2, 512, 128
    q, k, v, do = (bf16_to_dev(fi.bf16_tensor(9310, t, B, H, N, d)) for t in (0, 1, 2, fi.DO_ID))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, B, H, N, d, d ** -0.5, True)
    g0 = [torch.empty_like(q) for _ in range(3)]
    fa.fa_bwd(q, k, v, o, do, lse, *g0, B, H, N, d, d ** -0.5, True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g1 = [torch.zeros_like(q) for _ in range(3)]
    nb = fa.fa_bwd_workspace_bytes(B, H, N)
    ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    fa.fa_bwd(q, k, v, o, do, lse, *g1, B, H, N, d, d ** -0.5, True, ws, nb, stream=side)
    side.synchronize()
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
