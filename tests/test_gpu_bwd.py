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
from _gpu_util import bf16_to_dev, bf16_values, dev_to_f64, say

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


def check(got, ref, what, names=("dQ", "dK", "dV")):
    """Gates per gradient tensor; returns each one's mean-abs error relative
    to its mean |ref|."""
    rel = []
    for name, g, r in zip(names, got, ref):
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
        rel.append(rmean)
    return np.array(rel)


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


def tile_edges_and_random(N, tile, n_random, seed):
    edges = np.r_[np.arange(0, N, tile), np.minimum(np.arange(tile - 1, N + tile - 1, tile), N - 1)]
    return np.unique(np.r_[edges, np.random.default_rng(seed).choice(N, n_random, replace=False)])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_llama_layer(gpu_lib, causal):
    """B=2 H=32 N=2048 d=128 (the LLaMA-7B-shaped layer): every element of
    every (b, h) against the oracle."""
    fa = gpu_lib
    w = fi.WORKLOADS[2]
    say(f"bwd {w.name} causal={causal}: generating")
    qb, kb, vb, dob = gen(w.wid, w.B, w.H, w.N, w.d)
    got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), w.B, w.H, w.N, w.d, w.scale, causal)
    got = [dev_to_f64(x) for x in got]
    worst = np.zeros(3)
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle.attention_backward(*(bf16_values(x[b, h]) for x in (qb, kb, vb, dob)),
                                            w.scale, causal)
            worst = np.maximum(worst, check([x[b, h] for x in got], ref, f"(b={b},h={h})"))
    say(f"[config backward C2 {'causal' if causal else 'non-causal'}] worst mean-abs error relative "
        f"to mean |ref| over all 64 heads: dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")


def test_bwd_long_causal(gpu_lib):
    """B=1 H=16 N=16384 d=128 causal, every head: dQ on the first and last
    row of every 128-query tile plus 512 random rows; dK and dV on the first
    and last key of every 128-key tile plus 256 random keys."""
    from concurrent.futures import ThreadPoolExecutor
    fa = gpu_lib
    w = fi.WORKLOADS[3]
    say(f"bwd {w.name}: generating")
    qb, kb, vb, dob = gen(w.wid, w.B, w.H, w.N, w.d)
    got = run(fa, *map(bf16_to_dev, (qb, kb, vb, dob)), w.B, w.H, w.N, w.d, w.scale, True)
    gq, gk, gv = (dev_to_f64(x[0]) for x in got)

    def ref_head(h):
        q, k, v, do = (bf16_values(x[0, h]) for x in (qb, kb, vb, dob))
        rows = tile_edges_and_random(w.N, 128, 512, 3700 + h)
        keys = tile_edges_and_random(w.N, 128, 256, 3800 + h)
        dq = oracle.attention_backward_rows(q[rows], rows, k, v, do[rows], w.scale, True)
        dk, dv = oracle.attention_backward_keys(q, k, v, do, keys, w.scale, True)
        return rows, keys, dq, dk, dv

    say("bwd long causal: oracle for all 16 heads (selected query and key rows)")
    worst = np.zeros(3)
    with ThreadPoolExecutor(4) as ex:
        for h, (rows, keys, dq, dk, dv) in enumerate(ex.map(ref_head, range(w.H))):
            r = check([gq[h, rows]], [dq], f"h={h} rows={len(rows)}")
            rk = check([gk[h, keys], gv[h, keys]], [dk, dv], f"h={h} keys={len(keys)}",
                       names=("dK", "dV"))
            worst = np.maximum(worst, np.r_[r, rk])
    say(f"[config backward C3 causal] worst mean-abs error relative to mean |ref| over all 16 "
        f"heads: dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")


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
