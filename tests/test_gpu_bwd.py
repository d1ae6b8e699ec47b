"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 oracle.

The forward pass runs through the library first (its bf16 O and fp32 LSE are
the backward pass's inputs, as in training); the oracle differentiates the
definition on the same bf16 inputs.  Gates, per gradient tensor G with
reference R (bf16 inputs, P and dS rounded to bf16 for the matrix cores,
fp32 accumulation, bf16 output):
    max |G - R| <= 2e-2 * max |R| + 1e-5  and  mean |G - R| <= 1e-2 * mean |R| + 1e-5.
The absolute 1e-5 covers gradients that vanish exactly (one visible key:
dS = dP - D cancels), where fp32 rounding of dP and D leaves ~1e-8.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import bf16_to_dev, dev_to_f64, say

pytestmark = pytest.mark.gpu

REL_MAX = 2e-2
REL_MEAN = 1e-2
ABS = 1e-5


def gen(wid, B, H, N, d):
    return [fi.bf16_tensor(wid, t, B, H, N, d) for t in (fi.Q_ID, fi.K_ID, fi.V_ID, fi.DO_ID)]


def run(fa, q, k, v, do, B, H, N, d, scale, causal, own_ws=False):
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    if own_ws:
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal)
    else:
        nb = fa.fa_bwd_workspace_bytes(B, H, N)
        ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal, ws, nb)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(got, ref, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = dev_to_f64(g) if isinstance(g, torch.Tensor) else g
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        err = np.abs(g - r)
        amax, amean = float(np.abs(r).max()), float(np.abs(r).mean())
        rmax = float(err.max()) / max(amax, 1e-30)
        rmean = float(err.mean()) / max(amean, 1e-30)
        print(f"  {what} {name}: max_abs={err.max():.3e} (rel {rmax:.2e}) "
              f"mean_abs={err.mean():.3e} (rel {rmean:.2e}) |ref|max={amax:.3e}", flush=True)
        assert err.max() <= REL_MAX * amax + ABS, f"{what} {name}: max rel {rmax}"
        assert err.mean() <= REL_MEAN * amean + ABS, f"{what} {name}: mean rel {rmean}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 64, 100, 127, 128, 129, 200, 255, 256, 257, 500])
def test_bwd_edge_shapes(gpu_lib, N, causal, d):
    fa = gpu_lib
    B, H = 1, 2
    wid = 7000 + 4 * N + 2 * causal + (d == 128)
    say(f"bwd edge B={B} H={H} N={N} d={d} causal={causal} seed-id={wid}")
    qb, kb, vb, dob = gen(wid, B, H, N, d)
    scale = d ** -0.5
    got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), B, H, N, d, scale, causal)
    ref = oracle.attention_backward(*map(oracle.decode_bf16, (qb, kb, vb, dob)), scale, causal)
    check(got, ref, f"N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_llama_layer(gpu_lib, causal):
    """B=2 H=32 N=2048 d=128 (the LLaMA-7B-shaped layer): every element of
    three sampled (b, h) heads against the oracle."""
    fa = gpu_lib
    w = fi.WORKLOADS[2]
    say(f"bwd {w.name} causal={causal}: generating")
    qb, kb, vb, dob = gen(w.wid, w.B, w.H, w.N, w.d)
    got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), w.B, w.H, w.N, w.d, w.scale, causal)
    got = [dev_to_f64(x) for x in got]
    for b, h in [(0, 0), (1, 17), (1, 31)]:
        ref = oracle.attention_backward(*(oracle.decode_bf16(x[b, h]) for x in (qb, kb, vb, dob)),
                                        w.scale, causal)
        check([x[b, h] for x in got], ref, f"(b={b},h={h})")


def test_bwd_long_causal(gpu_lib):
    """B=1 H=16 N=16384 d=128 causal: every element of one sampled head."""
    fa = gpu_lib
    w = fi.WORKLOADS[3]
    say(f"bwd {w.name}: generating")
    qb, kb, vb, dob = gen(w.wid, w.B, w.H, w.N, w.d)
    got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), w.B, w.H, w.N, w.d, w.scale, True)
    h = 11
    got = [dev_to_f64(x[0, h]) for x in got]
    say("bwd long causal: oracle for head 11")
    ref = oracle.attention_backward(*(oracle.decode_bf16(x[0, h]) for x in (qb, kb, vb, dob)),
                                    w.scale, True)
    check(got, ref, f"(b=0,h={h})")


def test_bwd_library_workspace(gpu_lib):
    fa = gpu_lib
    B, H, N, d = 2, 2, 300, 128
    say("bwd with the library-owned workspace")
    qb, kb, vb, dob = gen(7900, B, H, N, d)
    got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), B, H, N, d, d ** -0.5, True, own_ws=True)
    ref = oracle.attention_backward(*map(oracle.decode_bf16, (qb, kb, vb, dob)), d ** -0.5, True)
    check(got, ref, "library workspace")


def test_bwd_deterministic_and_in_bounds(gpu_lib):
    """Two runs give identical bits; guard bands around dq, dk, dv and the
    workspace stay untouched."""
    fa = gpu_lib
    B, H, N, d = 2, 3, 777, 128
    say("bwd determinism + guard bands")
    qb, kb, vb, dob = gen(7950, B, H, N, d)
    q, k, v, do = map(bf16_to_dev, (qb, kb, vb, dob))
    scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, True)
    G = 4096
    nel = B * H * N * d
    bufs = [torch.full((nel + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    need = fa.fa_bwd_workspace_bytes(B, H, N)
    wbuf = torch.full((need // 4 + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        fa.fa_bwd(q, k, v, o, do, lse, *(b[G:G + nel] for b in bufs), B, H, N, d, scale, True,
                  wbuf[G:G + need // 4], need)
        torch.cuda.synchronize()
        outs.append([b[G:G + nel].clone() for b in bufs])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for b in bufs:
        assert torch.all(b[:G] == 7.0) and torch.all(b[G + nel:] == 7.0)
    assert torch.all(wbuf[:G] == 7.0) and torch.all(wbuf[G + need // 4:] == 7.0)


@pytest.mark.parametrize("ramp", ["up", "down"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_growing_and_shrinking_scores(gpu_lib, ramp, causal):
    """Key norms that double (or halve) every 256 keys: the forward's lazy
    rescale moves the reference max in many key tiles, and the backward
    recomputes P from that pass's LSE over rows that are nearly one-hot."""
    fa = gpu_lib
    B, H, N, d = 1, 2, 1024, 128
    say(f"bwd ramped key norms ({ramp}) causal={causal} N={N}")
    x = [np.stack([fi.normals(7300 + (ramp == "down"), t, 0, h, N, d) for h in range(H)])[None]
         for t in (fi.Q_ID, fi.K_ID, fi.V_ID, fi.DO_ID)]
    f = (2.0 ** (np.arange(N) / 256.0)).astype(np.float32)
    if ramp == "down":
        f = f[::-1].copy()
    x[1] = x[1] * f[None, None, :, None]
    qb, kb, vb, dob = (fi.f32_to_bf16_bits(a.astype(np.float32)) for a in x)
    got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), B, H, N, d, d ** -0.5, causal)
    ref = oracle.attention_backward(*map(oracle.decode_bf16, (qb, kb, vb, dob)), d ** -0.5, causal)
    check(got, ref, f"ramp {ramp} causal={causal}")


@pytest.mark.parametrize("scale", [0.05, 1.0])
def test_bwd_softmax_scale(gpu_lib, scale):
    """Scales other than 1/sqrt(d): nearly uniform and nearly one-hot rows."""
    fa = gpu_lib
    B, H, N, d = 1, 2, 300, 64
    say(f"bwd scale={scale} N={N} d={d}")
    qb, kb, vb, dob = gen(7400, B, H, N, d)
    for causal in (False, True):
        got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), B, H, N, d, scale, causal)
        ref = oracle.attention_backward(*map(oracle.decode_bf16, (qb, kb, vb, dob)), scale, causal)
        check(got, ref, f"scale={scale} causal={causal}")
