"""GPU parity of the forward pass on IEEE fp16 inputs against the fp64 oracle.

The usage notes of the Flash Attention note ("使用注意事项") list FP16 among
the supported input types.  The inputs are the bf16 tests' normals rounded to
fp16 instead; the oracle evaluates the definition on the exact values of
those fp16 bits.  The gates are the bf16 ones (the kernel rounds P and O to
fp16, eight times finer than bf16).
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import check_bf16_gates, dev_to_f64, f16_to_dev, say

pytestmark = pytest.mark.gpu


def run_fwd16(fa, q, k, v, B, H, N, d, scale, causal, out_f32=False):
    o = torch.empty((B, H, N, d), dtype=torch.float32 if out_f32 else torch.float16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, in_dtype=fa.FA_FP16,
                 out_dtype=fa.FA_FP32 if out_f32 else fa.FA_FP16)
    torch.cuda.synchronize()
    return o, lse


def gen16(wid, B, H, N, d):
    return [fi.f16_tensor(wid, t, B, H, N, d) for t in (fi.Q_ID, fi.K_ID, fi.V_ID)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 128, 129, 257, 1000])
def test_fp16_edge_shapes(gpu_lib, N, causal, d):
    fa = gpu_lib
    B, H = 2, 3
    wid = 5000 + N * 4 + 2 * causal + (d == 128)
    say(f"fwd fp16 B={B} H={H} N={N} d={d} causal={causal} seed-id={wid}")
    qb, kb, vb = gen16(wid, B, H, N, d)
    scale = d ** -0.5
    o, lse = run_fwd16(fa, *map(f16_to_dev, (qb, kb, vb)), B, H, N, d, scale, causal)
    assert o.dtype == torch.float16
    O, L = oracle.attention(*map(oracle.decode_f16, (qb, kb, vb)), scale, causal)
    check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, f"fp16 N={N} d={d} causal={causal}")


def test_fp16_fp32_out(gpu_lib):
    fa = gpu_lib
    B, H, N, d = 1, 4, 700, 128
    say("fwd fp16 in, fp32 out, causal")
    qb, kb, vb = gen16(5900, B, H, N, d)
    o, lse = run_fwd16(fa, *map(f16_to_dev, (qb, kb, vb)), B, H, N, d, d ** -0.5, True, out_f32=True)
    O, L = oracle.attention(*map(oracle.decode_f16, (qb, kb, vb)), d ** -0.5, True)
    mx, mean, _ = check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, "fp16 -> fp32 out")
    # with an fp32 output the only roundings left are P to fp16 and fp32 accumulation
    assert mean <= 2e-4, mean


def test_fp16_llama7b_layer_full_size(gpu_lib):
    """B=2 H=32 N=2048 d=128 causal on fp16 inputs; six heads compared on every row."""
    fa = gpu_lib
    w = fi.WORKLOADS[2]
    say(f"fwd fp16 {w.name} causal: full size, 6 sampled heads")
    qb, kb, vb = gen16(w.wid, w.B, w.H, w.N, w.d)
    o, lse = run_fwd16(fa, *map(f16_to_dev, (qb, kb, vb)), w.B, w.H, w.N, w.d, w.scale, True)
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    for b, h in [(0, 0), (0, 31), (1, 8), (1, 31)]:
        q, k, v = (oracle.decode_f16(x[b, h]) for x in (qb, kb, vb))
        O, L = oracle.attention(q, k, v, w.scale, True)
        check_bf16_gates(og[b, h], O, lg[b, h], L, f"fp16 (b={b},h={h})")


def test_fp16_and_bf16_agree_on_common_values(gpu_lib):
    """Inputs exactly representable in both formats (multiples of 1/8 in
    [-4, 4]) give outputs that agree within the two output roundings."""
    fa = gpu_lib
    B, H, N, d = 1, 2, 300, 64
    say("fwd fp16 vs bf16 on shared values")
    x = [np.round(fi.normals(5950, t, 0, 0, B * H * N, d).reshape(B, H, N, d) * 8) / 8 for t in range(3)]
    x = [np.clip(a, -4, 4).astype(np.float32) for a in x]
    h16 = [f16_to_dev(fi.f32_to_f16_bits(a)) for a in x]
    b16 = [torch.from_numpy(a).to(torch.bfloat16).cuda() for a in x]
    assert all(torch.equal(a.float(), b.float()) for a, b in zip(h16, b16))
    o16, l16 = run_fwd16(fa, *h16, B, H, N, d, d ** -0.5, True)
    ob = torch.empty_like(b16[0]); lb = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(*b16, ob, lb, B, H, N, d, d ** -0.5, True)
    torch.cuda.synchronize()
    assert (o16.float() - ob.float()).abs().max().item() <= 2e-2
    assert (l16 - lb).abs().max().item() <= 1e-4


@pytest.mark.parametrize("ramp", ["up", "down"])
def test_fp16_growing_and_shrinking_scores(gpu_lib, ramp):
    """fp16 inputs whose key norms double (or halve) every 256 keys: the lazy
    rescale is taken in many key tiles, P is rounded to fp16 at values up to
    2^8, and along "down" later probabilities fall below fp16's range in P*V
    while still counting in the fp32 row sum."""
    fa = gpu_lib
    B, H, N, d = 1, 2, 1024, 128
    say(f"fwd fp16 ramped key norms ({ramp}) causal N={N}")
    x = [np.stack([fi.normals(5200 + (ramp == "down"), t, 0, h, N, d) for h in range(H)])[None]
         for t in range(3)]
    f = (2.0 ** (np.arange(N) / 256.0)).astype(np.float32)
    if ramp == "down":
        f = f[::-1].copy()
    x[1] = x[1] * f[None, None, :, None]
    qb, kb, vb = (fi.f32_to_f16_bits(a.astype(np.float32)) for a in x)
    for causal in (False, True):
        o, lse = run_fwd16(fa, *map(f16_to_dev, (qb, kb, vb)), B, H, N, d, d ** -0.5, causal)
        O, L = oracle.attention(*map(oracle.decode_f16, (qb, kb, vb)), d ** -0.5, causal)
        check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, f"fp16 ramp {ramp} causal={causal}",
                         beyond_floor=True, mant_bits=11)
