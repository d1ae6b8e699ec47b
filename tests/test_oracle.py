"""Pins for the attention oracle (CPU only).

The oracle is the plain definition; these tests tie it to things other than
itself: hand-worked cases, brute force in scalar Python, torch's float64 CPU
attention (a library routine that also returns the log-sum-exp), the blocked
online recurrence of the pages, and closed-form invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from oracle import attention, attention_rows, merge_partials, split_partials

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# hand-worked cases
# ---------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked(case):
    q, k, v = (np.array(case[n], dtype=np.float64) for n in ("q", "k", "v"))
    O, L = attention(q, k, v, case["scale"], case["causal"])
    np.testing.assert_allclose(O, case["O"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, case["LSE"], rtol=0, atol=1e-12)
    if "num_splits" in case:
        Os, Ls = split_partials(q, k, v, case["scale"], case["num_splits"])
        np.testing.assert_allclose(Os, case["O_split"], atol=1e-12)
        np.testing.assert_allclose(Ls, case["LSE_split"], atol=1e-12)
        Om, Lm = merge_partials(Os, Ls)
        np.testing.assert_allclose(Om, case["O"], atol=1e-12)
        np.testing.assert_allclose(Lm, case["LSE"], atol=1e-12)


# ---------------------------------------------------------------------------
# brute force: scalar Python, no max subtraction, exact summation
# ---------------------------------------------------------------------------

def _brute(q, k, v, scale, causal):
    Nq, d = len(q), len(q[0])
    O, L = [], []
    for i in range(Nq):
        ws = []
        for j in range(len(k)):
            if causal and j > i:
                continue
            s = scale * math.fsum(q[i][c] * k[j][c] for c in range(d))
            ws.append((math.exp(s), j))
        tot = math.fsum(w for w, _ in ws)
        O.append([math.fsum(w * v[j][c] for w, j in ws) / tot for c in range(len(v[0]))])
        L.append(math.log(tot))
    return np.array(O), np.array(L)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 1), (3, 2), (5, 4), (8, 3)])
def test_brute_force(N, d, causal):
    rng = np.random.default_rng(1000 + 10 * N + d + causal)
    q, k, v = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d + 1)
    scale = 0.7
    O, L = attention(q, k, v, scale, causal)
    Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-12)


def test_brute_force_rectangular():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 3, 4), _rand(rng, 6, 4), _rand(rng, 6, 2)
    O, L = attention(q, k, v, 0.5)
    Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), 0.5, False)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# library routine: torch's float64 CPU flash attention (returns O and LSE)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 128, 64), (2, 3, 67, 128), (1, 2, 300, 16)])
def test_against_torch_cpu(shape, causal):
    rng = np.random.default_rng(sum(shape) + causal)
    q, k, v = (_rand(rng, *shape) for _ in range(3))
    scale = 1.0 / math.sqrt(shape[-1])
    O, L = attention(q, k, v, scale, causal, row_block=50)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    to, tl = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk, tv, 0.0, causal, scale=scale)[:2]
    np.testing.assert_allclose(O, to.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(L, tl.numpy(), rtol=1e-10, atol=1e-12)
    ts = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(O, ts.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_rows_matches_full():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 40, 8), _rand(rng, 40, 8), _rand(rng, 40, 8)
    O, L = attention(q, k, v, 0.3, True)
    idx = np.array([0, 1, 17, 39])
    Or, Lr = attention_rows(q[idx], idx, k, v, 0.3, True)
    np.testing.assert_allclose(Or, O[idx], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(Lr, L[idx], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# I1: the pages' blocked online recurrence reaches the two-pass result
# ---------------------------------------------------------------------------

def _online(q, k, v, scale, causal, bc):
    """Per query row, walk the keys in blocks of ``bc``: m_new = max(m_old,
    rowmax), l_new = l_old*e^(m_old-m_new) + sum_j e^(s_j-m_new),
    O_new = O_old*e^(m_old-m_new) + sum_j e^(s_j-m_new) v_j; O/l at the end."""
    Nq, Nk = q.shape[0], k.shape[0]
    O = np.zeros((Nq, v.shape[1]))
    L = np.zeros(Nq)
    for i in range(Nq):
        m, l, acc = -np.inf, 0.0, np.zeros(v.shape[1])
        hi = i + 1 if causal else Nk
        for j0 in range(0, hi, bc):
            j1 = min(j0 + bc, hi)
            s = scale * (k[j0:j1] @ q[i])
            m_new = max(m, s.max())
            f = math.exp(m - m_new) if np.isfinite(m) else 0.0
            p = np.exp(s - m_new)
            l = l * f + p.sum()
            acc = acc * f + p @ v[j0:j1]
            m = m_new
        O[i] = acc / l
        L[i] = m + math.log(l)
    return O, L


@pytest.mark.parametrize("bc", [1, 3, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_equals_two_pass(bc, causal):
    rng = np.random.default_rng(bc * 2 + causal)
    q, k, v = _rand(rng, 50, 16) * 3, _rand(rng, 50, 16) * 3, _rand(rng, 50, 16)
    O, L = attention(q, k, v, 0.25, causal)
    Oo, Lo = _online(q, k, v, 0.25, causal, bc)
    np.testing.assert_allclose(Oo, O, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Lo, L, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_weights_sum_to_one(causal):
    # I2: sum_j exp(s_ij - LSE_i) = 1 over the visible keys
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 33, 8), _rand(rng, 33, 8), _rand(rng, 33, 8)
    _, L = attention(q, k, v, 0.4, causal)
    S = 0.4 * q @ k.T
    vis = np.tril(np.ones((33, 33), bool)) if causal else np.ones((33, 33), bool)
    tot = np.where(vis, np.exp(S - L[:, None]), 0.0).sum(axis=1)
    np.testing.assert_allclose(tot, 1.0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_value_rows(causal):
    # I3: every V row equal to c  =>  every output row equals c
    rng = np.random.default_rng(12)
    q, k = _rand(rng, 20, 8) * 4, _rand(rng, 20, 8) * 4
    c = _rand(rng, 5)
    O, _ = attention(q, k, np.tile(c, (20, 1)), 0.5, causal)
    np.testing.assert_allclose(O, np.tile(c, (20, 1)), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys(causal):
    # I4: all keys equal => O_i = mean of the visible V rows, LSE_i = scale q_i.k + ln n_i
    rng = np.random.default_rng(13)
    N = 17
    q, kk, v = _rand(rng, N, 6), _rand(rng, 6), _rand(rng, N, 3)
    O, L = attention(q, np.tile(kk, (N, 1)), v, 0.9, causal)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(v, axis=0) / n[:, None] if causal else np.tile(v.mean(0), (N, 1))
    np.testing.assert_allclose(O, mean, atol=1e-13)
    np.testing.assert_allclose(L, 0.9 * q @ kk + np.log(n), atol=1e-13)


def test_causal_first_row():
    # I6: row 0 sees only key 0
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 9, 5), _rand(rng, 9, 5), _rand(rng, 9, 5)
    O, L = attention(q, k, v, 0.6, True)
    np.testing.assert_array_equal(O[0], v[0])
    assert L[0] == pytest.approx(0.6 * q[0] @ k[0], abs=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_uniform(causal):
    # I7: q = 0 => uniform weights
    rng = np.random.default_rng(15)
    N = 12
    k, v = _rand(rng, N, 4), _rand(rng, N, 4)
    O, L = attention(np.zeros((N, 4)), k, v, 1.0, causal)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(v, axis=0) / n[:, None] if causal else np.tile(v.mean(0), (N, 1))
    np.testing.assert_allclose(O, mean, atol=1e-14)
    np.testing.assert_allclose(L, np.log(n), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(causal):
    # I8: K' = K + 1 u^T leaves O unchanged and adds scale q.u to LSE
    rng = np.random.default_rng(16)
    q, k, v, u = _rand(rng, 15, 4), _rand(rng, 15, 4), _rand(rng, 15, 4), _rand(rng, 4)
    O, L = attention(q, k, v, 0.5, causal)
    O2, L2 = attention(q, k + u[None, :], v, 0.5, causal)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L + 0.5 * q @ u, atol=1e-13)


def test_permutation_and_linearity():
    # I9: non-causal output ignores a joint permutation of K/V rows; linear in V
    rng = np.random.default_rng(17)
    q, k, v, w = (_rand(rng, 21, 6) for _ in range(4))
    O, L = attention(q, k, v, 0.5)
    perm = rng.permutation(21)
    O2, L2 = attention(q, k[perm], v[perm], 0.5)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)
    Ow, _ = attention(q, k, w, 0.5)
    O3, _ = attention(q, k, 2.0 * v - 3.0 * w, 0.5)
    np.testing.assert_allclose(O3, 2.0 * O - 3.0 * Ow, atol=1e-12)


def test_large_scores_stable():
    # I10: scores of order 1e3 stay finite and pick the argmax key's value row
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 10, 8) * 100, _rand(rng, 10, 8), _rand(rng, 10, 8)
    O, L = attention(q, k, v, 1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    S = q @ k.T
    top2 = np.sort(S, axis=1)[:, -2:]
    sure = (top2[:, 1] - top2[:, 0]) > 40  # the runner-up weight is below e^-40
    assert sure.any()
    np.testing.assert_allclose(O[sure], v[S.argmax(axis=1)][sure], atol=1e-12)
    np.testing.assert_allclose(L, S.max(axis=1) + np.log(np.exp(S - S.max(1, keepdims=True)).sum(1)))


# ---------------------------------------------------------------------------
# I5: split-KV partials and their merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Lkv,S", [(64, 1), (64, 2), (100, 3), (1024, 64), (70, 64), (5, 4)])
def test_split_merge_equals_unsplit(Lkv, S):
    rng = np.random.default_rng(Lkv + S)
    q, k, v = _rand(rng, 2, 1, 32), _rand(rng, 2, Lkv, 32) * 2, _rand(rng, 2, Lkv, 32)
    O, L = oracle.decode_attention(q, k, v, 0.2)
    Os, Ls = split_partials(q, k, v, 0.2, S)
    assert Os.shape == (2, S, 1, 32) and Ls.shape == (2, S, 1)
    Om, Lm = merge_partials(Os, Ls)
    np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Lm, L, rtol=1e-12, atol=1e-13)
    # each partial is attention over its own key range alone
    for s, (lo, hi) in enumerate(oracle.split_bounds(Lkv, S)):
        if hi > lo:
            o, l = attention(q, k[:, lo:hi], v[:, lo:hi], 0.2)
            np.testing.assert_allclose(Os[:, s], o, atol=1e-14)
        else:
            assert np.all(Ls[:, s] == -np.inf) and np.all(Os[:, s] == 0)


def test_split_bounds():
    assert oracle.split_bounds(65536, 64)[0] == (0, 1024)
    assert oracle.split_bounds(65536, 64)[-1] == (64512, 65536)
    b = oracle.split_bounds(70, 64)   # chunk 2 -> 35 non-empty splits
    assert b[34] == (68, 70) and b[35] == (70, 70) and b[-1] == (70, 70)
    assert oracle.split_bounds(7, 7) == [(i, i + 1) for i in range(7)]


def test_merge_all_empty():
    Om, Lm = merge_partials(np.zeros((3, 1, 4)), np.full((3, 1), -np.inf))
    assert np.all(Om == 0) and np.all(Lm == -np.inf)


# ---------------------------------------------------------------------------
# the fp8-P error bound
# ---------------------------------------------------------------------------

def _sim_fp8_p(q, k, v, scale, causal, sigma, bc, normalise_by_rounded):
    """Blocked online softmax with the unnormalised P rounded to E4M3FN
    (times the pre-scale sigma) before the P*V product."""
    from fa_inputs import f64_to_e4m3fn_codes
    Nq, Nk = q.shape[0], k.shape[0]
    O = np.zeros((Nq, v.shape[1]))
    for i in range(Nq):
        m, l, acc = -np.inf, 0.0, np.zeros(v.shape[1])
        hi = i + 1 if causal else Nk
        for j0 in range(0, hi, bc):
            j1 = min(j0 + bc, hi)
            s = scale * (k[j0:j1] @ q[i])
            m_new = max(m, s.max())
            f = math.exp(m - m_new) if np.isfinite(m) else 0.0
            p = np.exp(s - m_new)
            ph = oracle.decode_e4m3fn(f64_to_e4m3fn_codes(p * sigma)) / sigma
            l = l * f + (ph.sum() if normalise_by_rounded else p.sum())
            acc = acc * f + ph @ v[j0:j1]
            m = m_new
        O[i] = acc / l
    return O


@pytest.mark.parametrize("rounded", [False, True])
@pytest.mark.parametrize("sigma", [1.0, 256.0])
def test_fp8_bound_holds_and_is_tight(rounded, sigma):
    rng = np.random.default_rng(19)
    N = 96
    q, k, v = _rand(rng, N, 16) * 2, _rand(rng, N, 16) * 2, _rand(rng, N, 16)
    v[rng.random(v.shape) < 0.02] *= 20
    O, L, Bnd = oracle.fp8_p_error_bound(q, k, v, 0.25, True, sigma)
    Oref, Lref = attention(q, k, v, 0.25, True)
    np.testing.assert_allclose(O, Oref, atol=1e-13)
    np.testing.assert_allclose(L, Lref, atol=1e-13)
    Osim = _sim_fp8_p(q, k, v, 0.25, True, sigma, 16, rounded)
    err = np.abs(Osim - O)
    assert np.all(err <= Bnd)
    # tight to within a small factor somewhere (the bound is not vacuous)
    assert np.max(err / Bnd) > 0.05


# ---------------------------------------------------------------------------
# E4M3FN rounding and attention with E4M3FN-rounded P
# ---------------------------------------------------------------------------

def _e4m3_grid():
    return [float(x) for x in oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))]


def test_round_e4m3fn_grid_points_and_ties():
    grid = np.array(_e4m3_grid())
    assert np.array_equal(oracle.round_to_e4m3fn(grid), grid)
    assert np.array_equal(oracle.round_to_e4m3fn(-grid[1:]), -grid[1:])
    mid = (grid[:-1] + grid[1:]) / 2
    r = oracle.round_to_e4m3fn(mid)
    even = np.where(np.arange(len(mid)) % 2 == 0, grid[:-1], grid[1:])   # the even code wins
    assert np.array_equal(r, even)
    eps = 1e-9 * np.maximum(mid, 1e-3)
    assert np.array_equal(oracle.round_to_e4m3fn(mid - eps), grid[:-1])
    assert np.array_equal(oracle.round_to_e4m3fn(mid + eps), grid[1:])
    assert oracle.round_to_e4m3fn(np.array([1000.0, -500.0, 464.0])).tolist() == [448.0, -448.0, 448.0]


def test_round_e4m3fn_agrees_with_the_input_quantiser():
    # two independently written encoders: grid search here, frexp arithmetic there
    from fa_inputs import f64_to_e4m3fn_codes
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 3, 20000),
                        rng.uniform(-448, 448, 5000)])
    a = oracle.round_to_e4m3fn(x)
    b = oracle.decode_e4m3fn(f64_to_e4m3fn_codes(x))
    assert np.array_equal(np.abs(a), np.abs(b))


def _brute_fp8_p(q, k, v, scale, causal, sig):
    grid = _e4m3_grid()

    def rnd(x):
        best = min(range(len(grid)), key=lambda i: (abs(x - grid[i]), i % 2))
        return grid[best]
    out = []
    for i in range(len(q)):
        keys = [j for j in range(len(k)) if not causal or j <= i]
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in keys}
        m = max(s.values())
        p = {j: math.exp(s[j] - m) for j in keys}
        l = math.fsum(p.values())
        out.append([math.fsum(rnd(p[j] * sig[j]) / sig[j] * v[j][c] for j in keys) / l
                    for c in range(len(v[0]))])
    return np.array(out)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_p_attention_brute_force(causal):
    rng = np.random.default_rng(23)
    N, d = 7, 3
    q, k, v = _rand(rng, N, d) * 2, _rand(rng, N, d) * 2, _rand(rng, N, d)
    sig = rng.uniform(4, 256, N)
    O = oracle.fp8_p_attention(q, k, v, 0.5, causal, sig)
    np.testing.assert_allclose(O, _brute_fp8_p(q, k, v, 0.5, causal, sig), rtol=0, atol=1e-12)


def test_fp8_p_attention_exact_when_weights_are_representable():
    # s_j = -j ln 2, so p_j = 2^-j: every weight is an E4M3FN value (down to
    # the subnormal 2^-9), and the rounded model equals exact attention
    N, d = 10, 4
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k = np.zeros((N, d))
    k[:, 0] = -np.arange(N) * math.log(2.0)
    v = np.random.default_rng(3).standard_normal((N, d))
    O = oracle.fp8_p_attention(q, k, v, 1.0, False, np.ones(N))
    Oref, _ = attention(q, k, v, 1.0, False)
    np.testing.assert_allclose(O, Oref, rtol=0, atol=1e-15)
    # weights 2^-e with a pre-scale of 2^-6: e <= 3 lands on 2^-6..2^-9 (still
    # E4M3FN values); e >= 5 lands at or below 2^-11, under half the smallest
    # subnormal, and rounds to 0 -- those keys, and only they, drop out
    e = np.array([0, 1, 2, 3, 5, 6, 7, 8])
    k2 = np.zeros((len(e), d))
    k2[:, 0] = -e * math.log(2.0)
    v2 = v[:len(e)]
    O2 = oracle.fp8_p_attention(q, k2, v2, 1.0, False, np.full(len(e), 2.0 ** -6))
    p = 2.0 ** -e
    np.testing.assert_allclose(O2[0], (p * (e <= 3)) @ v2 / p.sum(), rtol=0, atol=1e-15)


def test_fp8_p_attention_within_the_fp8_bound():
    rng = np.random.default_rng(29)
    N, d = 200, 16
    q, k, v = _rand(rng, N, d) * 2, _rand(rng, N, d) * 2, _rand(rng, N, d)
    v[rng.random(v.shape) < 0.02] *= 20
    sig = np.full(N, 37.0)
    O, _, Bnd = oracle.fp8_p_error_bound(q, k, v, 0.25, True, 37.0)
    Om = oracle.fp8_p_attention(q, k, v, 0.25, True, sig)
    assert np.all(np.abs(Om - O) <= Bnd)
    assert np.abs(Om - O).max() > 0          # the rounding is really applied


# ---------------------------------------------------------------------------
# grouped key/value heads (GQA / MQA) decode
# ---------------------------------------------------------------------------

def test_gqa_with_one_query_head_per_kv_head_is_mha():
    rng = np.random.default_rng(31)
    q, k, v = _rand(rng, 2, 4, 1, 8), _rand(rng, 2, 4, 50, 8), _rand(rng, 2, 4, 50, 8)
    O, L = oracle.decode_attention_gqa(q, k, v, 0.3)
    Om, Lm = oracle.decode_attention(q, k, v, 0.3)
    np.testing.assert_array_equal(O, Om)
    np.testing.assert_array_equal(L, Lm)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1), (8, 8)])
def test_gqa_brute_force(Hq, Hkv):
    rng = np.random.default_rng(37 + Hq + Hkv)
    B, L, d = 2, 9, 3
    q, k, v = _rand(rng, B, Hq, 1, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    O, Ls = oracle.decode_attention_gqa(q, k, v, 0.7)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            s = [0.7 * math.fsum(q[b, h, 0, c] * k[b, kh, j, c] for c in range(d)) for j in range(L)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = math.fsum(e)
            for c in range(d):
                ref = math.fsum(e[j] * v[b, kh, j, c] for j in range(L)) / tot
                assert abs(O[b, h, 0, c] - ref) <= 1e-12
            assert abs(Ls[b, h, 0] - (mx + math.log(tot))) <= 1e-12


def test_gqa_against_torch_sdpa():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, L, d = 2, 8, 2, 200, 16
    q, k, v = _rand(rng, B, Hq, 1, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    O, _ = oracle.decode_attention_gqa(q, k, v, 0.25)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.25, enable_gqa=True)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)


def test_gqa_rejects_uneven_groups():
    with pytest.raises(ValueError):
        oracle.decode_attention_gqa(np.zeros((1, 3, 1, 2)), np.zeros((1, 2, 4, 2)), np.zeros((1, 2, 4, 2)), 1.0)


# ---------------------------------------------------------------------------
# backward: gradients of the definition
# ---------------------------------------------------------------------------

def _loss(q, k, v, do, scale, causal):
    O, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(O * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    """Central differences of sum(O * dO) (the forward definition only)."""
    rng = np.random.default_rng(51 + causal)
    N, d, scale, h = 5, 3, 0.6, 1e-5
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale, causal)
    for x, g in ((q, dQ), (k, dK), (v, dV)):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = x0 - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,scale", [(37, 16, 0.25), (130, 64, 0.125), (600, 8, 0.9)])
def test_backward_against_torch_autograd(N, d, scale, causal):
    rng = np.random.default_rng(N + d)
    q, k, v, do = (_rand(rng, 2, 3, N, d) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    out.backward(torch.from_numpy(do))
    for ours, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """Row-softmax gradients sum to zero over the keys, so the key gradients
    sum to zero; each P row sums to one, so dV sums to the sum of dO; with
    causal masking row 0 sees one key and its query gradient vanishes."""
    rng = np.random.default_rng(61 + causal)
    N, d = 77, 8
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, 0.4, causal, row_block=16)
    np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dV.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)
    if causal:
        assert np.all(dQ[0] == 0.0)
        # the last key is seen by the last query only
        p_last = 1.0 / np.exp(oracle.attention(q, k, v, 0.4, True)[1][-1] - 0.4 * q[-1] @ k[-1])
        np.testing.assert_allclose(dV[-1], p_last * do[-1], rtol=1e-12, atol=1e-14)
    dQ2, dK2, dV2 = oracle.attention_backward(q, k, v, do, 0.4, causal)
    for a, b in ((dQ, dQ2), (dK, dK2), (dV, dV2)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_selected_rows_and_keys_against_torch(causal):
    """dQ of selected query rows and dK, dV of selected key rows equal those
    rows of torch's float64 autograd through SDPA, with row blocks smaller
    than the sequence so that the key-side sums cross blocks."""
    rng = np.random.default_rng(81 + causal)
    N, d, scale = 97, 16, 0.35
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    out.backward(torch.from_numpy(do))
    rows = np.array([0, 1, 31, 32, 50, 96])
    dq = oracle.attention_backward_rows(q[rows], rows, k, v, do[rows], scale, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy()[rows], rtol=0, atol=1e-12)
    keys = np.array([0, 5, 63, 64, 95, 96])
    dk, dv = oracle.attention_backward_keys(q, k, v, do, keys, scale, causal, row_block=20)
    np.testing.assert_allclose(dk, tk.grad.numpy()[keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy()[keys], rtol=0, atol=1e-12)
    # and the same rows of the full oracle gradients
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, dQ[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dK[keys], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dV[keys], rtol=0, atol=1e-13)


def test_backward_keys_last_key_closed_form():
    """With causal masking the last key is seen by the last query only:
    dV_last = P_last,last dO_last, and dK_last = scale P (dP - sum P dP) q."""
    rng = np.random.default_rng(83)
    N, d, scale = 40, 8, 0.5
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    dk, dv = oracle.attention_backward_keys(q, k, v, do, [N - 1], scale, True, row_block=7)
    s = scale * (q[-1] @ k.T)
    p = np.exp(s - s.max())
    p /= p.sum()
    dp = v @ do[-1]
    np.testing.assert_allclose(dv[0], p[-1] * do[-1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk[0], scale * p[-1] * (dp[-1] - p @ dp) * q[-1], rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------------------
# ragged batches (packed sequences, unequal query/key lengths)
# ---------------------------------------------------------------------------

def _pack(rng, lens, H, d):
    return _rand(rng, int(sum(lens)), H, d), np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_dense_attention(causal):
    rng = np.random.default_rng(71 + causal)
    lens, H, d = [5, 17, 1, 40], 3, 8
    q, cu = _pack(rng, lens, H, d)
    k, _ = _pack(rng, lens, H, d)
    v, _ = _pack(rng, lens, H, d)
    O, L = oracle.attention_varlen(q, k, v, cu, cu, 0.3, causal)
    for b, n in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        Od, Ld = oracle.attention(q[sl].transpose(1, 0, 2), k[sl].transpose(1, 0, 2),
                                  v[sl].transpose(1, 0, 2), 0.3, causal)
        np.testing.assert_allclose(O[sl], Od.transpose(1, 0, 2), rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[:, sl], Ld, rtol=0, atol=1e-13)


def test_varlen_chunked_prefill_is_tail_of_full_causal():
    """Lq new queries against Lk >= Lq keys, end-aligned: exactly the last Lq
    rows of causal attention over the whole length-Lk sequence."""
    rng = np.random.default_rng(73)
    H, d = 2, 16
    for Lk, Lq in [(50, 7), (64, 64), (33, 1), (100, 37)]:
        qf, kf, vf = (_rand(rng, H, Lk, d) for _ in range(3))
        Ofull, Lfull = oracle.attention(qf, kf, vf, 0.25, True)
        q = qf[:, Lk - Lq:].transpose(1, 0, 2)
        O, L = oracle.attention_varlen(q, kf.transpose(1, 0, 2), vf.transpose(1, 0, 2),
                                       [0, Lq], [0, Lk], 0.25, True)
        np.testing.assert_allclose(O, Ofull[:, Lk - Lq:].transpose(1, 0, 2), rtol=0, atol=1e-13)
        np.testing.assert_allclose(L, Lfull[:, Lk - Lq:], rtol=0, atol=1e-13)


def test_varlen_against_torch_masked_sdpa():
    """More queries than keys (leading rows see nothing) and more keys than
    queries, against torch float64 SDPA with the explicit boolean mask."""
    rng = np.random.default_rng(79)
    H, d = 2, 8
    lq, lk = [9, 3, 12], [4, 10, 12]
    q, cuq = _pack(rng, lq, H, d)
    k, cuk = _pack(rng, lk, H, d)
    v, _ = _pack(rng, lk, H, d)
    O, L = oracle.attention_varlen(q, k, v, cuq, cuk, 0.5, True)
    for b in range(3):
        Lq, Lk = lq[b], lk[b]
        qs = torch.from_numpy(q[cuq[b]:cuq[b + 1]].transpose(1, 0, 2).copy())
        ks = torch.from_numpy(k[cuk[b]:cuk[b + 1]].transpose(1, 0, 2).copy())
        vs = torch.from_numpy(v[cuk[b]:cuk[b + 1]].transpose(1, 0, 2).copy())
        mask = torch.from_numpy(np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq))
        seen = mask.any(dim=1).numpy()
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=0.5)
        got = O[cuq[b]:cuq[b + 1]].transpose(1, 0, 2)
        np.testing.assert_allclose(got[:, seen], ref.numpy()[:, seen], rtol=0, atol=1e-12)
        assert np.all(got[:, ~seen] == 0.0)
        assert np.all(np.isneginf(L[:, cuq[b]:cuq[b + 1]][:, ~seen]))
        scores = 0.5 * (qs @ ks.transpose(1, 2))
        lse_ref = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1).numpy()
        np.testing.assert_allclose(L[:, cuq[b]:cuq[b + 1]][:, seen], lse_ref[:, seen], rtol=0, atol=1e-12)
    # sequence 0 (9 queries, 4 keys): its first 5 queries see no key
    assert np.all(np.isneginf(L[:, :5])) and np.all(np.isfinite(L[:, 5:9]))


# ---------------------------------------------------------------------------
# backward over ragged batches
# ---------------------------------------------------------------------------

def _varlen_loss(q, k, v, do, cuq, cuk, scale, causal):
    O, _ = oracle.attention_varlen(q, k, v, cuq, cuk, scale, causal)
    return float(np.sum(O * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_finite_differences(causal):
    """Central differences of sum(O * dO) through the packed forward
    definition, with more queries than keys in one sequence (its first
    queries see no key under causal masking), more keys than queries in
    another, and an empty query range."""
    rng = np.random.default_rng(91 + causal)
    H, d, scale, h = 2, 3, 0.7, 1e-5
    lq, lk = [3, 2, 0, 4], [2, 5, 3, 4]
    q, cuq = _pack(rng, lq, H, d)
    k, cuk = _pack(rng, lk, H, d)
    v, _ = _pack(rng, lk, H, d)
    do, _ = _pack(rng, lq, H, d)
    dQ, dK, dV = oracle.attention_backward_varlen(q, k, v, do, cuq, cuk, scale, causal)
    for x, g in ((q, dQ), (k, dK), (v, dV)):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _varlen_loss(q, k, v, do, cuq, cuk, scale, causal)
            x[idx] = x0 - h
            lm = _varlen_loss(q, k, v, do, cuq, cuk, scale, causal)
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)
    # the empty query range leaves its keys without gradient
    assert np.all(dK[cuk[2]:cuk[3]] == 0.0) and np.all(dV[cuk[2]:cuk[3]] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_against_torch_autograd(causal):
    """torch float64 autograd through an explicitly masked softmax, per
    sequence; rows with no visible key produce the constant 0."""
    rng = np.random.default_rng(93 + causal)
    H, d, scale = 3, 8, 0.45
    lq, lk = [9, 3, 12, 1], [4, 10, 12, 30]
    q, cuq = _pack(rng, lq, H, d)
    k, cuk = _pack(rng, lk, H, d)
    v, _ = _pack(rng, lk, H, d)
    do, _ = _pack(rng, lq, H, d)
    dQ, dK, dV = oracle.attention_backward_varlen(q, k, v, do, cuq, cuk, scale, causal)
    for b in range(len(lq)):
        Lq, Lk = lq[b], lk[b]
        tq = torch.from_numpy(q[cuq[b]:cuq[b + 1]].transpose(1, 0, 2).copy()).requires_grad_()
        tk = torch.from_numpy(k[cuk[b]:cuk[b + 1]].transpose(1, 0, 2).copy()).requires_grad_()
        tv = torch.from_numpy(v[cuk[b]:cuk[b + 1]].transpose(1, 0, 2).copy()).requires_grad_()
        if causal:
            mask = torch.from_numpy(np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq))
        else:
            mask = torch.ones(Lq, Lk, dtype=torch.bool)
        seen = mask.any(dim=1)
        s = scale * (tq @ tk.transpose(1, 2))
        s = s.masked_fill(~mask, float("-inf")).masked_fill(~seen[:, None], 0.0)
        out = (torch.softmax(s, dim=-1) @ tv) * seen[:, None].to(torch.float64)
        out.backward(torch.from_numpy(do[cuq[b]:cuq[b + 1]].transpose(1, 0, 2).copy()))
        np.testing.assert_allclose(dQ[cuq[b]:cuq[b + 1]], tq.grad.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dK[cuk[b]:cuk[b + 1]], tk.grad.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dV[cuk[b]:cuk[b + 1]], tv.grad.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
        if causal and Lq > Lk:
            assert np.all(dQ[cuq[b]:cuq[b] + Lq - Lk] == 0.0)


def test_backward_varlen_chunk_is_tail_of_full_causal_backward():
    """Lq new queries against Lk keys, end-aligned: the gradients equal those
    of causal attention over the whole length-Lk sequence with an upstream
    gradient that is zero on its first Lk - Lq rows."""
    rng = np.random.default_rng(95)
    H, d, scale = 2, 16, 0.3
    for Lk, Lq in [(50, 7), (64, 64), (33, 1)]:
        qf, kf, vf, dof = (_rand(rng, H, Lk, d) for _ in range(4))
        dof[:, :Lk - Lq] = 0.0
        dQf, dKf, dVf = oracle.attention_backward(qf, kf, vf, dof, scale, True)
        t = (1, 0, 2)
        dQ, dK, dV = oracle.attention_backward_varlen(
            qf[:, Lk - Lq:].transpose(t), kf.transpose(t), vf.transpose(t),
            dof[:, Lk - Lq:].transpose(t), [0, Lq], [0, Lk], scale, True)
        np.testing.assert_allclose(dQ, dQf[:, Lk - Lq:].transpose(t), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dK, dKf.transpose(t), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dV, dVf.transpose(t), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_invariants(causal):
    """Per (sequence, head): the key gradients sum to zero (each row of dS
    sums to zero), dV sums to the sum of dO over the rows that see a key,
    and no sequence's gradients depend on another sequence's data."""
    rng = np.random.default_rng(97 + causal)
    H, d, scale = 2, 8, 0.5
    lq, lk = [20, 6, 13], [7, 40, 13]
    q, cuq = _pack(rng, lq, H, d)
    k, cuk = _pack(rng, lk, H, d)
    v, _ = _pack(rng, lk, H, d)
    do, _ = _pack(rng, lq, H, d)
    dQ, dK, dV = oracle.attention_backward_varlen(q, k, v, do, cuq, cuk, scale, causal)
    for b in range(3):
        Lq, Lk = lq[b], lk[b]
        sk = slice(cuk[b], cuk[b + 1])
        np.testing.assert_allclose(dK[sk].sum(axis=0), 0.0, atol=1e-12)
        first_seen = max(0, Lq - Lk) if causal else 0
        np.testing.assert_allclose(dV[sk].sum(axis=0),
                                   do[cuq[b] + first_seen:cuq[b + 1]].sum(axis=0), rtol=0, atol=1e-12)
    # change sequence 1's data: sequences 0 and 2 keep their gradients
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x, cu in ((q2, cuq), (k2, cuk), (v2, cuk), (do2, cuq)):
        x[cu[1]:cu[2]] = _rand(rng, cu[2] - cu[1], H, d)
    g2 = oracle.attention_backward_varlen(q2, k2, v2, do2, cuq, cuk, scale, causal)
    for b in (0, 2):
        for g, gg, cu in zip((dQ, dK, dV), g2, (cuq, cuk, cuk)):
            np.testing.assert_array_equal(g[cu[b]:cu[b + 1]], gg[cu[b]:cu[b + 1]])


# ---------------------------------------------------------------------------
# incoherent processing (random-sign Hadamard rotation) and block quantisation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 8, 64, 128])
def test_hadamard_matches_scipy_and_is_orthogonal(n):
    from scipy.linalg import hadamard
    H = oracle.hadamard_matrix(n)
    np.testing.assert_array_equal(H, hadamard(n))
    np.testing.assert_array_equal(H @ H.T, n * np.eye(n))


def test_rotation_preserves_scores_and_spreads_outliers():
    rng = np.random.default_rng(81)
    d = 128
    s = rng.choice([-1.0, 1.0], size=d)
    q, k = _rand(rng, 40, d), _rand(rng, 30, d)
    qr, kr = oracle.incoherent_rotation(q, s), oracle.incoherent_rotation(k, s)
    np.testing.assert_allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-11)
    np.testing.assert_allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(q, axis=1), rtol=1e-14)
    # a one-hot row becomes a row of +-1/sqrt(d)
    e = np.zeros(d)
    e[37] = 5.0
    np.testing.assert_allclose(np.abs(oracle.incoherent_rotation(e, s)), 5.0 / np.sqrt(d), rtol=1e-15)
    # the attention of rotated Q, K equals that of Q, K
    v = _rand(rng, 30, 16)
    O1, L1 = oracle.attention(qr, kr, v, 0.2, False)
    O2, L2 = oracle.attention(q, k, v, 0.2, False)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-12)


def test_pow2_block_scale_is_the_smallest_power_of_two():
    """The power-of-two scale against a search over exponents: the smallest k
    with amax <= 448 * 2^k, at random magnitudes and at the boundaries
    448 * 2^k and one ulp either side of them."""
    rng = np.random.default_rng(87)
    amaxes = list(np.exp(rng.uniform(-60, 60, 300)))
    for k in (-20, -3, 0, 1, 7):
        b = 448.0 * 2.0 ** k
        amaxes += [b, np.nextafter(b, 0), np.nextafter(b, np.inf)]
    amaxes += [2.0 ** -130, 1.0, 224.0, 448.0, 449.0, 1e30]
    for a in amaxes:
        s = oracle.smallest_pow2_scale(a)
        k = next(k for k in range(-200, 200) if a <= 448.0 * 2.0 ** k)
        assert s == 2.0 ** k, (a, s, k)
        assert 224.0 < a / s <= 448.0
        assert s == fi.pow2_scale(a)           # the generator's bit-field rule
    # the boundaries themselves
    assert oracle.smallest_pow2_scale(448.0) == 1.0
    assert oracle.smallest_pow2_scale(np.nextafter(448.0, np.inf)) == 2.0
    assert oracle.smallest_pow2_scale(224.0) == 0.5


def test_pow2_block_quantisation():
    """With power-of-two scales x / scale is exact, so the oracle and the
    generator's quantiser agree on every code; each block's largest ratio lies
    in (224, 448] and every value is within half an E4M3FN step."""
    rng = np.random.default_rng(89)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    x[rng.random(x.shape) < 1e-3] *= 20
    x[128:192] = 0.0                                   # an all-zero block
    x[192:256] *= np.float32(2.0 ** -40)               # a tiny block
    vals, scales, ratio = oracle.quantize_e4m3_blocks(x, pow2=True)
    codes, gscales = fi.quantize_e4m3_rows(x, pow2=True)
    np.testing.assert_array_equal(scales, gscales.astype(np.float64))
    assert scales[2] == 1.0
    np.testing.assert_array_equal(oracle.round_to_e4m3fn(ratio), oracle.decode_e4m3fn(codes))
    for i in (0, 1, 3, 4):
        r = np.abs(ratio[i * 64:(i + 1) * 64]).max()
        assert 224.0 < r <= 448.0
        m, _ = np.frexp(scales[i])
        assert m == 0.5
    err = np.abs(vals - x)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ratio), 2.0 ** -6))) - 3)
    assert np.all(err <= 0.5 * step * scales[np.arange(300) // 64][:, None] * (1 + 1e-12))
    # amax / 448 scales on the same data: a different rule, different scales
    _, s448, _ = oracle.quantize_e4m3_blocks(x)
    assert np.all(s448[[0, 1, 3, 4]] <= scales[[0, 1, 3, 4]])
    assert np.all(scales[[0, 1, 3, 4]] < 2 * s448[[0, 1, 3, 4]])


def test_block_quantisation_matches_the_generator_quantiser():
    """Two independent E4M3FN quantisers (grid search here, bit arithmetic in
    the input generator) agree except where x/scale is a rounding tie."""
    rng = np.random.default_rng(83)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    x[rng.random(x.shape) < 1e-3] *= 20
    vals, scales, ratio = oracle.quantize_e4m3_blocks(x)
    codes, gscales = fi.quantize_e4m3_rows(x)
    np.testing.assert_allclose(scales, gscales, rtol=1e-7)
    ours = oracle.round_to_e4m3fn(ratio)          # grid values, before scaling back
    theirs = oracle.decode_e4m3fn(codes)
    assert np.mean(ours == theirs) > 0.9999
    # any disagreement is one grid step at a near-tie of x / scale
    diff = ours != theirs
    grid_step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ours[diff]), 2 ** -6))) - 3)
    assert np.all(np.abs(ours[diff] - theirs[diff]) <= grid_step * 1.0000001)
    assert np.all(np.abs(np.abs(ratio[diff]) - (np.abs(ours[diff]) + np.abs(theirs[diff])) / 2)
                  <= 1e-6 * np.abs(ratio[diff]))
    assert np.max(np.abs(ratio)) <= 448.0 and np.all(scales > 0)
    np.testing.assert_allclose(vals, ours * scales[np.arange(200) // 64][:, None], rtol=1e-15)


def test_ragged_decode_is_varlen_attention_with_one_query():
    """Per-sequence cache lengths: the same as packed attention with one query
    per sequence (end-aligned causal lets it see every cached key), which the
    varlen oracle computes by a separate path; empty caches give O = 0 and
    LSE = -inf."""
    rng = np.random.default_rng(91)
    B, H, Lcap, d = 4, 3, 40, 8
    lens = [40, 1, 0, 17]
    q, k, v = _rand(rng, B, H, 1, d), _rand(rng, B, H, Lcap, d), _rand(rng, B, H, Lcap, d)
    O, L = oracle.decode_attention_ragged(q, k, v, lens, 0.4)
    qp = q[:, :, 0].copy()                                          # [B, H, d] = packed [total_q, H, d]
    kp = np.concatenate([k[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)])
    vp = np.concatenate([v[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)])
    Ov, Lv = oracle.attention_varlen(qp, kp, vp, np.arange(B + 1), np.concatenate([[0], np.cumsum(lens)]),
                                     0.4, causal=True)
    np.testing.assert_allclose(O[:, :, 0], Ov, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L[:, :, 0], Lv.T, rtol=0, atol=1e-13)
    assert np.all(O[2] == 0) and np.all(np.isneginf(L[2]))
    # full-length caches are plain decode
    Of, Lf = oracle.decode_attention_ragged(q, k, v, [Lcap] * B, 0.4)
    Od, Ld = oracle.decode_attention(q, k, v, 0.4)
    np.testing.assert_array_equal(Of, Od)
    np.testing.assert_array_equal(Lf, Ld)
