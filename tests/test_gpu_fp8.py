"""GPU parity of the block-scaled fp8 (E4M3FN) forward pass.

The oracle runs on the dequantised inputs (code value times block scale, in
float64).  Gates, stated for a kernel that rounds the probabilities to
E4M3FN before the P*V product, and fixed independently of the kernel:
  F1  LSE relative error <= 1e-3 (denominator max(|LSE|, 1));
  F2  every output element within the oracle's elementwise bound
      ``oracle.fp8_p_error_bound`` for probabilities rounded as 256 * p
      (pre-scale sigma = 256 = 2^8 for every key);
  F3  mean-abs error <= 3e-3 over the checked outputs of the full-size
      workload (B=4, H=16, N=8192, causal, x20 outliers): every (batch,
      head), on the first and last row of every 128-query tile plus 512
      random rows per head.  For scale, the mean error of
      ``oracle.fp8_p_attention`` (exact attention with only P rounded as
      256 * p) is printed beside it; on the small edge shapes, where a mean
      over few elements is noisy, the mean is reported, not gated.
The max-abs error is printed beside them.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import dev_to_f64, lse_rel, say, u8_to_dev

pytestmark = pytest.mark.gpu

F3_MEAN_ABS = 3e-3
P_PRESCALE = 256.0
LSE_REL = 1e-3


def run_fp8(fa, codes, scales, B, H, N, d, scale, causal):
    q, k, v = (u8_to_dev(c) for c in codes)
    qs, ks, vs = (torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in scales)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, in_dtype=fa.FA_FP8_E4M3,
                 q_scale=qs, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return dev_to_f64(o), dev_to_f64(lse)


def check_head(og, lg, q, k, v, scale, causal, rows, what, model=False):
    """F1 and F2 for the rows ``rows`` of one (b, h); returns the abs errors
    and, with ``model``, those of the P-rounding yardstick."""
    O, L, Bnd = oracle.fp8_p_error_bound(q[rows], k, v, scale, causal, P_PRESCALE, qidx=rows)
    err = np.abs(og - O)
    lr = lse_rel(lg, L)
    ratio = float((err / Bnd).max())
    err_model = None
    extra = ""
    if model:
        Om = oracle.fp8_p_attention(q[rows], k, v, scale, causal, np.full(k.shape[0], P_PRESCALE),
                                    qidx=rows)
        err_model = np.abs(Om - O)
        extra = f" (P-rounding model {err_model.mean():.3e})"
    say(f"  {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}{extra} "
        f"lse_rel={lr.max():.3e} max err/bound={ratio:.3f}")
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    assert lr.max() <= LSE_REL, f"{what}: LSE relative {lr.max()}"
    assert np.all(err <= Bnd), f"{what}: error above the fp8 bound (ratio {ratio})"
    return err, err_model


def gen(wid, B, H, N, d, outlier_p=1e-3, v_pow2=True):
    """Q and K with max|x| / 448 block scales; V with power-of-two scales
    (the workload's rule), or with ``v_pow2=False`` max|x| / 448 too, whose
    mantissas differ from block to block."""
    codes, scales = [], []
    for t in (fi.Q_ID, fi.K_ID, fi.V_ID):
        c, s = fi.fp8_tensor(wid, t, B, H, N, d, outlier_p=outlier_p,
                             pow2=v_pow2 if t == fi.V_ID else False)
        codes.append(c)
        scales.append(s)
    return codes, scales


def test_fp8_code_semantics(gpu_lib):
    """One key: LSE is the single score, so code 0x7E (448) times code 0x38
    (1.0) at d = 0 must give scale * 448 exactly; O is that key's value row."""
    fa = gpu_lib
    B, H, N, d = 1, 1, 1, 128
    say("fp8 code semantics: 0x7E -> 448")
    q = np.zeros((B, H, N, d), np.uint8)
    k = np.zeros((B, H, N, d), np.uint8)
    q[0, 0, 0, 0] = 0x7E
    k[0, 0, 0, 0] = 0x38
    v = (np.arange(d, dtype=np.int64) % 120 + 1).astype(np.uint8).reshape(B, H, N, d)
    one = np.ones((B, H, 1), np.float32)
    scale = 0.125
    og, lg = run_fp8(fa, (q, k, v), (one, one, one), B, H, N, d, scale, False)
    assert abs(lg[0, 0, 0] - 448 * scale) <= 1e-5 * 448 * scale, lg[0, 0, 0]
    ref = oracle.decode_e4m3fn(v)
    assert np.array_equal(og, ref), (og[0, 0, 0, :8], ref[0, 0, 0, :8])


@pytest.mark.parametrize("v_pow2", [True, False])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 33, 64, 65, 127, 128, 200, 257, 640])
def test_fp8_edge_shapes(gpu_lib, N, causal, v_pow2):
    """V scales of one mantissa per head (powers of two) run the loop form
    without per-block multiplies, max|x| / 448 scales the other form."""
    fa = gpu_lib
    B, H, d = 2, 3, 128
    wid = 5000 + 4 * N + causal
    say(f"fp8 edge B={B} H={H} N={N} causal={causal} v_pow2={v_pow2} seed-id={wid}")
    codes, scales = gen(wid, B, H, N, d, outlier_p=1e-2, v_pow2=v_pow2)
    og, lg = run_fp8(fa, codes, scales, B, H, N, d, d ** -0.5, causal)
    deq = [oracle.dequant_fp8_rows(c, s) for c, s in zip(codes, scales)]
    errs, errs_model = [], []
    for b in range(B):
        for h in range(H):
            e, em = check_head(og[b, h], lg[b, h], deq[0][b, h], deq[1][b, h], deq[2][b, h],
                               d ** -0.5, causal, np.arange(N), f"(b={b},h={h})", model=True)
            errs.append(e)
            errs_model.append(em)
    # F3 is a gate on the long rows of the measured workload; rows of a few
    # keys carry the full 2^-4 rounding of P, so here it is only reported.
    mean = float(np.mean(np.concatenate([e.ravel() for e in errs])))
    mean_model = float(np.mean(np.concatenate([e.ravel() for e in errs_model])))
    say(f"  mean-abs {mean:.3e} (P-rounding model {mean_model:.3e})")


def full_size_rows(N, tile, seed, n_random=512):
    """The first and last row of every ``tile``-query tile plus ``n_random``
    distinct random rows."""
    edges = np.r_[np.arange(0, N, tile), np.minimum(np.arange(tile - 1, N + tile - 1, tile), N - 1)]
    rnd = np.random.default_rng(seed).choice(N, min(n_random, N), replace=False)
    return np.unique(np.r_[edges, rnd])


@pytest.mark.parametrize("v_pow2", [True, False])
def test_fp8_full_size(gpu_lib, v_pow2):
    """B=4, H=16, N=8192, d=128, causal, 0.1% x20 outliers: every (b, h) on
    the tile-edge rows and 512 random rows each; V with power-of-two block
    scales (the workload) and with max|x| / 448 scales."""
    fa = gpu_lib
    w = fi.WORKLOADS[5]
    say(f"fp8 {w.name} v_pow2={v_pow2}: generating")
    codes, scales = gen(w.wid, w.B, w.H, w.N, w.d, v_pow2=v_pow2)
    say("fp8 full size: running")
    og, lg = run_fp8(fa, codes, scales, w.B, w.H, w.N, w.d, w.scale, True)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    errs, errs_model = [], []
    for b in range(w.B):
        for h in range(w.H):
            rows = full_size_rows(w.N, 128, 5500 + w.H * b + h)
            q, k, v = (oracle.dequant_fp8_rows(c[b, h], s[b, h]) for c, s in zip(codes, scales))
            e, em = check_head(og[b, h, rows], lg[b, h, rows], q, k, v, w.scale, True, rows,
                               f"(b={b},h={h}) rows={len(rows)}", model=(h % 8 == 0))
            errs.append(e)
            if em is not None:
                errs_model.append(em)
    mean = float(np.mean(np.concatenate([e.ravel() for e in errs])))
    mean_model = float(np.mean(np.concatenate([e.ravel() for e in errs_model])))
    say(f"  mean-abs over all heads' checked rows: {mean:.3e} (F3 gate {F3_MEAN_ABS}); "
        f"P-rounding model on heads h=0,8: {mean_model:.3e}")
    assert mean <= F3_MEAN_ABS, (mean, mean_model)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_v_scale_mantissas(gpu_lib, causal):
    """Per head, V scales that share a mantissa other than 1/2 (3/4 here),
    and heads where one block's mantissa differs from the rest: both loop
    forms against the oracle on the same codes, N = 700 (11 scale blocks,
    a ragged tail)."""
    fa = gpu_lib
    B, H, N, d = 1, 4, 700, 128
    wid = 5950 + causal
    say(f"fp8 V-scale mantissas B={B} H={H} N={N} causal={causal} seed-id={wid}")
    codes, scales = gen(wid, B, H, N, d, outlier_p=1e-2)
    vs = scales[2].copy()
    vs[0, 0] *= np.float32(0.75)                 # one mantissa, 3/4
    vs[0, 1, 5] *= np.float32(0.75)              # one block differs
    vs[0, 2, -1] *= np.float32(1.5)              # the ragged last block differs
    # head 3 keeps its power-of-two scales
    scales = [scales[0], scales[1], vs]
    og, lg = run_fp8(fa, codes, scales, B, H, N, d, d ** -0.5, causal)
    deq = [oracle.dequant_fp8_rows(c, s) for c, s in zip(codes, scales)]
    for h in range(H):
        check_head(og[0, h], lg[0, h], deq[0][0, h], deq[1][0, h], deq[2][0, h], d ** -0.5,
                   causal, np.arange(N), f"h={h}")


def test_fp8_deterministic_and_in_bounds(gpu_lib):
    """Two runs give identical bits; guard bands around o and lse stay untouched."""
    fa = gpu_lib
    B, H, N, d = 1, 3, 300, 128
    say("fp8 determinism + guard bands")
    codes, scales = gen(5900, B, H, N, d)
    q, k, v = (u8_to_dev(c) for c in codes)
    qs, ks, vs = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in scales)
    G = 4096
    nel = B * H * N * d
    obuf = torch.full((nel + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * N + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        fa.fa_fwd_ex(q, k, v, obuf[G:G + nel], lbuf[G:G + B * H * N], B, H, N, d, d ** -0.5, True,
                     in_dtype=fa.FA_FP8_E4M3, q_scale=qs, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        outs.append((obuf[G:G + nel].clone(), lbuf[G:G + B * H * N].clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.all(obuf[:G] == 7.0) and torch.all(obuf[G + nel:] == 7.0)
    assert torch.all(lbuf[:G] == 7.0) and torch.all(lbuf[G + B * H * N:] == 7.0)
