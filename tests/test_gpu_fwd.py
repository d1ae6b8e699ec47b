"""GPU parity of the bf16 forward pass against the fp64 oracle.

Small shapes are compared element by element over the whole output.  The
full-size workloads are compared on every (batch, head): the LLaMA-7B-shaped
layer (B=2, H=32, N=2048) on every row, the long causal sequence (B=1, H=16,
N=16384) on the first and last row of every 256-query tile plus 512 random
rows per head.  Each configuration prints one summary line of its max-abs,
mean-abs and LSE relative errors.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import (ErrStats, bf16_to_dev, bf16_values, check_bf16_gates, dev_to_f64, say)

pytestmark = pytest.mark.gpu


def run_fwd(fa, q, k, v, B, H, N, d, scale, causal, out_f32=False):
    o = torch.empty((B, H, N, d), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    if out_f32:
        fa.fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, out_dtype=fa.FA_FP32)
    else:
        fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal)
    torch.cuda.synchronize()
    return o, lse


def gen(wid, B, H, N, d):
    return [fi.bf16_tensor(wid, t, B, H, N, d) for t in (fi.Q_ID, fi.K_ID, fi.V_ID)]


def test_single_head_fp32_out(gpu_lib):
    fa = gpu_lib
    w = fi.WORKLOADS[1]
    say(f"fwd {w.name} fp32 out, non-causal")
    qb, kb, vb = gen(w.wid, w.B, w.H, w.N, w.d)
    o, lse = run_fwd(fa, *map(bf16_to_dev, (qb, kb, vb)), w.B, w.H, w.N, w.d, w.scale, False,
                     out_f32=True)
    O, L = oracle.attention(*map(oracle.decode_bf16, (qb, kb, vb)), w.scale, False)
    check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, w.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 64, 127, 128, 129, 200, 255, 256, 257, 511, 640, 1000])
def test_edge_shapes(gpu_lib, N, causal, d):
    fa = gpu_lib
    B, H = 2, 3
    wid = 1000 + N * 4 + 2 * causal + (d == 128)
    say(f"fwd edge B={B} H={H} N={N} d={d} causal={causal} seed-id={wid}")
    qb, kb, vb = gen(wid, B, H, N, d)
    scale = d ** -0.5
    o, lse = run_fwd(fa, *map(bf16_to_dev, (qb, kb, vb)), B, H, N, d, scale, causal)
    O, L = oracle.attention(*map(oracle.decode_bf16, (qb, kb, vb)), scale, causal)
    check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, f"N={N} d={d} causal={causal}",
                     beyond_floor=True)


def full_size_rows(N, tile, seed, n_random=512):
    """The first and last row of every ``tile``-query tile plus ``n_random``
    distinct random rows."""
    edges = np.r_[np.arange(0, N, tile), np.minimum(np.arange(tile - 1, N + tile - 1, tile), N - 1)]
    rnd = np.random.default_rng(seed).choice(N, min(n_random, N), replace=False)
    return np.unique(np.r_[edges, rnd])


@pytest.mark.parametrize("causal", [False, True])
def test_llama7b_layer_full_size(gpu_lib, causal):
    """B=2 H=32 N=2048 d=128: every (b, h), every row, against the oracle."""
    fa = gpu_lib
    w = fi.WORKLOADS[2]
    say(f"fwd {w.name} causal={causal}: full size, every head and row")
    qb, kb, vb = gen(w.wid, w.B, w.H, w.N, w.d)
    o, lse = run_fwd(fa, *map(bf16_to_dev, (qb, kb, vb)), w.B, w.H, w.N, w.d, w.scale, causal)
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    st = ErrStats(f"C2 {'causal' if causal else 'non-causal'} B=2 H=32 N=2048")
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = (bf16_values(x[b, h]) for x in (qb, kb, vb))
            O, L = oracle.attention(q, k, v, w.scale, causal)
            check_bf16_gates(og[b, h], O, lg[b, h], L, f"(b={b},h={h})")
            st.add(og[b, h], O, lg[b, h], L)
    st.report()


def test_long_causal_full_size(gpu_lib):
    """B=1 H=16 N=16384 d=128 causal: every head, on the tile-edge rows and
    512 random rows each."""
    fa = gpu_lib
    w = fi.WORKLOADS[3]
    say(f"fwd {w.name}: full size, every head at tile edges + random rows")
    qb, kb, vb = gen(w.wid, w.B, w.H, w.N, w.d)
    o, lse = run_fwd(fa, *map(bf16_to_dev, (qb, kb, vb)), w.B, w.H, w.N, w.d, w.scale, True)
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    st = ErrStats("C3 causal B=1 H=16 N=16384")
    for h in range(w.H):
        rows = full_size_rows(w.N, 256, 3300 + h)
        q, k, v = (bf16_values(x[0, h]) for x in (qb, kb, vb))
        O, L = oracle.attention_rows(q[rows], rows, k, v, w.scale, True)
        check_bf16_gates(og[0, h, rows], O, lg[0, h, rows], L, f"h={h} rows={len(rows)}")
        st.add(og[0, h, rows], O, lg[0, h, rows], L)
    st.report()


def test_deterministic_and_in_bounds(gpu_lib):
    """Two runs give identical bits; guard bands around o and lse stay untouched."""
    fa = gpu_lib
    B, H, N, d = 1, 4, 300, 128
    say("fwd determinism + guard bands")
    qb, kb, vb = gen(2000, B, H, N, d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    G = 4096
    nel = B * H * N * d
    obuf = torch.full((nel + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * N + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        fa.fa_fwd(q, k, v, obuf[G:G + nel], lbuf[G:G + B * H * N], B, H, N, d, d ** -0.5, True)
        torch.cuda.synchronize()
        outs.append((obuf[G:G + nel].clone(), lbuf[G:G + B * H * N].clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.all(obuf[:G] == 7.0) and torch.all(obuf[G + nel:] == 7.0)
    assert torch.all(lbuf[:G] == 7.0) and torch.all(lbuf[G + B * H * N:] == 7.0)


def test_large_scores_stay_finite(gpu_lib):
    """Scores of order 1e3 (q scaled by 100): no overflow, still matches."""
    fa = gpu_lib
    B, H, N, d = 1, 2, 256, 128
    say("fwd large scores")
    x = [fi.normals(3000, t, 0, h, N, d) for t in range(3) for h in range(H)]
    q = np.stack(x[0:2])[None] * 100
    k = np.stack(x[2:4])[None]
    v = np.stack(x[4:6])[None]
    qb, kb, vb = (fi.f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v))
    for causal in (False, True):
        o, lse = run_fwd(fa, *map(bf16_to_dev, (qb, kb, vb)), B, H, N, d, d ** -0.5, causal)
        O, L = oracle.attention(*map(oracle.decode_bf16, (qb, kb, vb)), d ** -0.5, causal)
        check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, f"x100 causal={causal}")


def ramped_inputs(wid, H, N, d, ramp):
    """N(0,1) q, k, v with the key rows scaled by 2^(j/256) ("up") or by its
    mirror ("down"): the scaled scores' spread doubles every 256 keys (or
    halves), so along "up" the running row max grows by more than 2^8 (in
    base-2 units) across many key tiles, and along "down" every later tile
    is dwarfed by the first."""
    x = [np.stack([fi.normals(wid, t, 0, h, N, d) for h in range(H)])[None] for t in range(3)]
    f = (2.0 ** (np.arange(N) / 256.0)).astype(np.float32)
    if ramp == "down":
        f = f[::-1].copy()
    x[1] = x[1] * f[None, None, :, None]
    return [fi.f32_to_bf16_bits(a.astype(np.float32)) for a in x]


@pytest.mark.parametrize("ramp", ["up", "down"])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_and_shrinking_scores(gpu_lib, ramp, causal):
    """The lazy rescale taken in many key tiles (keys of growing norm), and
    probabilities that underflow after the first tile (shrinking norm)."""
    fa = gpu_lib
    B, H, N, d = 1, 2, 1024, 128
    say(f"fwd ramped key norms ({ramp}) causal={causal} N={N}")
    qb, kb, vb = ramped_inputs(3100 + (ramp == "down"), H, N, d, ramp)
    o, lse = run_fwd(fa, *map(bf16_to_dev, (qb, kb, vb)), B, H, N, d, d ** -0.5, causal)
    O, L = oracle.attention(*map(oracle.decode_bf16, (qb, kb, vb)), d ** -0.5, causal)
    check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, f"ramp {ramp} causal={causal}",
                     beyond_floor=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [1e-3, 0.05, 1.0, 2.5])
def test_softmax_scale(gpu_lib, scale, d):
    """Scales other than 1/sqrt(d), from nearly uniform weights (1e-3) to
    nearly one-hot rows (2.5 with d = 128: scaled scores of spread ~28)."""
    fa = gpu_lib
    B, H, N = 1, 2, 300
    say(f"fwd scale={scale} d={d} N={N}")
    qb, kb, vb = gen(3200 + d, B, H, N, d)
    for causal in (False, True):
        o, lse = run_fwd(fa, *map(bf16_to_dev, (qb, kb, vb)), B, H, N, d, scale, causal)
        O, L = oracle.attention(*map(oracle.decode_bf16, (qb, kb, vb)), scale, causal)
        check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L, f"scale={scale} causal={causal}",
                         beyond_floor=True)
