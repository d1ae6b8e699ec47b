"""GPU parity of the backward pass on IEEE fp16 tensors against the fp64 oracle.

The usage notes of the Flash Attention note ("使用注意事项") describe mixed
precision training with an fp16 forward pass and fp32 softmax statistics in
the backward pass.  The forward pass runs through the library on fp16
inputs (fp16 O, fp32 LSE); the backward pass gets the same fp16 tensors.
The oracle differentiates the definition on the exact values of the fp16
inputs.  Gates as for bf16 (relative to each gradient's size).
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import dev_to_f64, f16_to_dev, say
from test_gpu_bwd import check

pytestmark = pytest.mark.gpu


def gen16(wid, B, H, N, d):
    return [fi.f16_tensor(wid, t, B, H, N, d) for t in (fi.Q_ID, fi.K_ID, fi.V_ID, fi.DO_ID)]


def run16(fa, q, k, v, do, B, H, N, d, scale, causal):
    o = torch.empty((B, H, N, d), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, in_dtype=fa.FA_FP16,
                 out_dtype=fa.FA_FP16)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    nb = fa.fa_bwd_workspace_bytes(B, H, N)
    ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    fa.fa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal, fa.FA_FP16, ws, nb)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float16
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 128, 129, 257, 500])
def test_bwd_fp16_edge_shapes(gpu_lib, N, causal, d):
    fa = gpu_lib
    B, H = 1, 2
    wid = 7500 + 4 * N + 2 * causal + (d == 128)
    say(f"bwd fp16 B={B} H={H} N={N} d={d} causal={causal} seed-id={wid}")
    qh, kh, vh, doh = gen16(wid, B, H, N, d)
    scale = d ** -0.5
    got = run16(fa, *map(f16_to_dev, (qh, kh, vh, doh)), B, H, N, d, scale, causal)
    ref = oracle.attention_backward(*map(oracle.decode_f16, (qh, kh, vh, doh)), scale, causal)
    check(got, ref, f"fp16 N={N} d={d} causal={causal}")


def test_bwd_fp16_llama_layer(gpu_lib):
    """B=2 H=32 N=2048 d=128 causal on fp16 tensors: three sampled heads, every element."""
    fa = gpu_lib
    w = fi.WORKLOADS[2]
    say(f"bwd fp16 {w.name} causal: full size, 3 sampled heads")
    qh, kh, vh, doh = gen16(w.wid, w.B, w.H, w.N, w.d)
    dq, dk, dv = run16(fa, *map(f16_to_dev, (qh, kh, vh, doh)), w.B, w.H, w.N, w.d, w.scale, True)
    g = [dev_to_f64(x) for x in (dq, dk, dv)]
    for b, h in [(0, 0), (1, 17), (1, 31)]:
        ref = oracle.attention_backward(*(oracle.decode_f16(x[b, h]) for x in (qh, kh, vh, doh)),
                                        w.scale, True)
        check([x[b, h] for x in g], ref, f"fp16 (b={b},h={h})")


def test_bwd_fp16_matches_bf16_on_common_values(gpu_lib):
    """Tensors exactly representable in both formats give gradients that agree
    within the two formats' roundings of P, dS and the outputs."""
    fa = gpu_lib
    B, H, N, d = 1, 2, 300, 128
    say("bwd fp16 vs bf16 on shared values")
    x = [np.clip(np.round(fi.normals(7990, t, 0, 0, B * H * N, d).reshape(B, H, N, d) * 8) / 8, -4, 4)
         .astype(np.float32) for t in range(4)]
    h16 = [f16_to_dev(fi.f32_to_f16_bits(a)) for a in x]
    b16 = [torch.from_numpy(a).to(torch.bfloat16).cuda() for a in x]
    g16 = run16(fa, *h16, B, H, N, d, d ** -0.5, True)
    ob = torch.empty_like(b16[0]); lb = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(*b16[:3], ob, lb, B, H, N, d, d ** -0.5, True)
    gb = [torch.empty_like(b16[0]) for _ in range(3)]
    fa.fa_bwd_ex(*b16[:3], ob, b16[3], lb, *gb, B, H, N, d, d ** -0.5, True, fa.FA_BF16)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), g16, gb):
        diff = (a.float() - b.float()).abs().max().item()
        ref = b.float().abs().max().item()
        print(f"  {name}: max |fp16 - bf16| = {diff:.3e} (|bf16| max {ref:.3e})", flush=True)
        assert diff <= 3e-2 * ref, name
