"""The attention oracle: the plain definition, in float64, on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed (FlashAttention note, "标准注意力的实现问题" and
"问题分析": S = Q K^T, A = softmax(S / sqrt(d)), O = A V, per (batch, head)
on (batch, heads, seq_len, head_dim) tensors; the softmax is taken along the
key axis, after subtracting the row maximum for stability, as in "递归计算
softmax").  The call's ``scale`` replaces 1/sqrt(d) (the ``softmax_scale``
argument of the flash_attn_func call shown in "框架集成").

For query row i and key j::

    s_ij  = scale * sum_c q_ic k_jc         (-inf where masked)
    m_i   = max_j s_ij
    l_i   = sum_j exp(s_ij - m_i)
    O_ic  = sum_j exp(s_ij - m_i) / l_i * v_jc
    LSE_i = m_i + ln l_i                    (natural log)

Causal masking (the ``causal=True`` flag in "使用注意事项"): query i sees key j
iff j <= i; every configuration has as many queries as keys, so no row is
ever empty.  A key range with no visible key (only possible for an empty
split) has LSE = -inf and O = 0.

This file is the definition, evaluated two-pass with the score matrix
materialised one block of query rows at a time.  It deliberately does not use
the blocked online recurrence the GPU kernels use; that recurrence appears only
in the tests, as an invariant checked against this file.
"""
from __future__ import annotations

import numpy as np

from .codecs import round_to_e4m3fn

ROW_BLOCK = 512


def _rows(q, k, v, scale, causal, qidx):
    """O and LSE for query rows ``qidx`` of one (batch, head).

    q: [r, d] the selected query rows; k, v: [Nk, d]; qidx: [r] their indices.
    """
    S = scale * (q @ k.T)                                   # [r, Nk] fp64
    if causal:
        j = np.arange(k.shape[0])
        S = np.where(j[None, :] <= qidx[:, None], S, -np.inf)
    m = S.max(axis=1)                                       # pass 1: row max
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    E = np.exp(S - m_safe[:, None])                         # pass 2: exp, sum
    l = E.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = E / l[:, None]
    P = np.where(finite[:, None], P, 0.0)
    O = P @ v
    lse = np.where(finite, m_safe + np.log(np.where(finite, l, 1.0)), -np.inf)
    return O, lse


def attention(q, k, v, scale, causal=False, row_block=ROW_BLOCK):
    """Exact attention over the last two axes.

    q: [..., Nq, d]; k, v: [..., Nk, d] (float64 or anything castable).
    Returns (O [..., Nq, d], LSE [..., Nq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    Nq, d = q.shape[-2:]
    qf = q.reshape((-1, Nq, d))
    kf = k.reshape((-1,) + k.shape[-2:])
    vf = v.reshape((-1,) + v.shape[-2:])
    O = np.empty(qf.shape[:-1] + (vf.shape[-1],), dtype=np.float64)
    L = np.empty(qf.shape[:-1], dtype=np.float64)
    for g in range(qf.shape[0]):
        for r0 in range(0, Nq, row_block):
            idx = np.arange(r0, min(r0 + row_block, Nq))
            O[g, idx], L[g, idx] = _rows(qf[g, idx], kf[g], vf[g], scale, causal, idx)
    return O.reshape(lead + (Nq, vf.shape[-1])), L.reshape(lead + (Nq,))


def attention_rows(q_rows, qidx, k, v, scale, causal=False):
    """Exact attention for selected query rows of one (batch, head).

    q_rows: [r, d] the query rows; qidx: their row indices (for the mask);
    k, v: [Nk, d].  Returns (O [r, d], LSE [r]).
    """
    return _rows(np.asarray(q_rows, np.float64), np.asarray(k, np.float64),
                 np.asarray(v, np.float64), scale, causal,
                 np.asarray(qidx, dtype=np.int64))


# ---------------------------------------------------------------------------
# Ragged batches: packed sequences of unequal lengths
# ---------------------------------------------------------------------------

def attention_varlen(q, k, v, cu_q, cu_k, scale, causal=False):
    """Exact attention over a batch of packed sequences of unequal lengths.

    q: [total_q, H, d], k, v: [total_k, H, d] (tokens of sequence b at rows
    cu_q[b]:cu_q[b+1] and cu_k[b]:cu_k[b+1]).  Causal masking is aligned at
    the end of the sequences: with Lq queries and Lk keys, query i sees key j
    iff j <= i + (Lk - Lq), so the queries are the last Lq positions of a
    length-Lk sequence (a chunk of a prefill against the keys already
    cached); for Lq == Lk this is the usual j <= i.  A query that sees no key
    gets O = 0 and LSE = -inf.  Returns (O [total_q, H, d], LSE [H, total_q]).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    total_q, H, d = q.shape
    O = np.zeros((total_q, H, v.shape[-1]))
    L = np.full((H, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0 or Lk == 0:
            continue
        for h in range(H):
            S = scale * (q[q0:q1, h] @ k[k0:k1, h].T)               # [Lq, Lk]
            if causal:
                i = np.arange(Lq)[:, None]
                j = np.arange(Lk)[None, :]
                S = np.where(j <= i + (Lk - Lq), S, -np.inf)
            m = S.max(axis=1)
            seen = np.isfinite(m)
            ms = np.where(seen, m, 0.0)
            E = np.exp(S - ms[:, None])
            l = E.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):
                P = np.where(seen[:, None], E / l[:, None], 0.0)
            O[q0:q1, h] = P @ v[k0:k1, h]
            L[h, q0:q1] = np.where(seen, ms + np.log(np.where(seen, l, 1.0)), -np.inf)
    return O, L


# ---------------------------------------------------------------------------
# Backward: gradients of the definition (dQ, dK, dV for an upstream dO)
# ---------------------------------------------------------------------------

def _backward_rows(q, k, v, do, scale, causal, qidx):
    """The chain rule through the definition for query rows ``qidx``.

    With P = softmax_j(s_ij) and O = P V, for an upstream gradient dO:
        dV   = P^T dO
        dP   = dO V^T
        dS   = P * (dP - sum_j P * dP)        (Jacobian of the row softmax)
        dQ   = scale * dS K,   dK = scale * dS^T Q
    Returns (dQ rows, this block's share of dK, of dV).
    """
    S = scale * (q @ k.T)
    if causal:
        j = np.arange(k.shape[0])
        S = np.where(j[None, :] <= qidx[:, None], S, -np.inf)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    P = E / E.sum(axis=1)[:, None]
    dV = P.T @ do
    dP = do @ v.T
    dS = P * (dP - (P * dP).sum(axis=1)[:, None])
    return scale * (dS @ k), scale * (dS.T @ q), dV


def attention_backward(q, k, v, do, scale, causal=False, row_block=ROW_BLOCK):
    """Gradients of sum(O * dO) with respect to q, k and v, in float64.

    q, do: [..., N, d]; k, v: [..., N, d] (as many keys as queries when
    causal, so no row is empty).  Recomputes P from q and k (the pages'
    recomputation in place of a stored score matrix) and sums the key-side
    gradients over blocks of query rows.  Returns (dQ, dK, dV).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    lead = q.shape[:-2]
    N, d = q.shape[-2:]
    qf, kf, vf, dof = (x.reshape((-1,) + x.shape[-2:]) for x in (q, k, v, do))
    dQ = np.empty_like(qf)
    dK = np.zeros_like(kf)
    dV = np.zeros_like(vf)
    for g in range(qf.shape[0]):
        for r0 in range(0, N, row_block):
            idx = np.arange(r0, min(r0 + row_block, N))
            dq, dk, dv = _backward_rows(qf[g, idx], kf[g], vf[g], dof[g, idx], scale, causal, idx)
            dQ[g, idx] = dq
            dK[g] += dk
            dV[g] += dv
    return (dQ.reshape(lead + (N, d)), dK.reshape(lead + kf.shape[-2:]),
            dV.reshape(lead + vf.shape[-2:]))


def attention_backward_varlen(q, k, v, do, cu_q, cu_k, scale, causal=False):
    """Gradients of sum(O * dO) for ``attention_varlen``: packed sequences of
    unequal lengths, causal masking aligned at the end of each sequence
    (query i sees key j iff j <= i + (Lk - Lq)).

    The same chain rule as ``_backward_rows`` per (sequence, head):
        dV = P^T dO,  dP = dO V^T,  dS = P * (dP - sum_j P * dP),
        dQ = scale * dS K,  dK = scale * dS^T Q,
    where a query that sees no key has P = 0 (its output is the constant 0),
    so it gets dQ = 0 and adds nothing to dK and dV; keys of a sequence with
    no queries get dK = dV = 0.

    q, do: [total_q, H, d]; k, v: [total_k, H, d]; cu_q, cu_k: the B+1
    offsets.  Returns (dQ [total_q, H, d], dK [total_k, H, d],
    dV [total_k, H, d]).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    H = q.shape[1]
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0 or Lk == 0:
            continue
        for h in range(H):
            qs, ks, vs, dos = q[q0:q1, h], k[k0:k1, h], v[k0:k1, h], do[q0:q1, h]
            S = scale * (qs @ ks.T)                                  # [Lq, Lk]
            if causal:
                i = np.arange(Lq)[:, None]
                j = np.arange(Lk)[None, :]
                S = np.where(j <= i + (Lk - Lq), S, -np.inf)
            m = S.max(axis=1)
            seen = np.isfinite(m)
            ms = np.where(seen, m, 0.0)
            E = np.exp(S - ms[:, None])
            l = E.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):
                P = np.where(seen[:, None], E / l[:, None], 0.0)
            dP = dos @ vs.T
            dS = P * (dP - (P * dP).sum(axis=1)[:, None])
            dQ[q0:q1, h] = scale * (dS @ ks)
            dK[k0:k1, h] = scale * (dS.T @ qs)
            dV[k0:k1, h] = P.T @ dos
    return dQ, dK, dV


def attention_backward_rows(q_rows, qidx, k, v, do_rows, scale, causal=False):
    """dQ for selected query rows of one (batch, head): the query-side
    gradient of a row needs only that row's scores, probabilities and dO.

    q_rows, do_rows: [r, d] (rows ``qidx``); k, v: [Nk, d].  Returns dQ [r, d].
    """
    q_rows, k, v, do_rows = (np.asarray(x, np.float64) for x in (q_rows, k, v, do_rows))
    dq, _, _ = _backward_rows(q_rows, k, v, do_rows, scale, causal, np.asarray(qidx, np.int64))
    return dq


def attention_backward_keys(q, k, v, do, kidx, scale, causal=False, row_block=ROW_BLOCK):
    """dK and dV for selected key rows ``kidx`` of one (batch, head).

    Key j's gradients sum over every query row i that sees it:
        dV_j = sum_i P_ij dO_i,   dK_j = scale * sum_i dS_ij q_i,
        dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij'),  dP_ij = dO_i . v_j,
    so each query row still needs its full scores (for its max and sum) and
    its full dP (for the row term), but only the columns ``kidx`` of P and
    dS enter the sums.  q, do: [N, d]; k, v: [Nk, d].  Returns
    (dK [len(kidx), d], dV [len(kidx), d]).
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    kidx = np.asarray(kidx, np.int64)
    dK = np.zeros((kidx.size, k.shape[1]))
    dV = np.zeros((kidx.size, v.shape[1]))
    N = q.shape[0]
    for r0 in range(0, N, row_block):
        idx = np.arange(r0, min(r0 + row_block, N))
        S = scale * (q[idx] @ k.T)
        if causal:
            j = np.arange(k.shape[0])
            S = np.where(j[None, :] <= idx[:, None], S, -np.inf)
        m = S.max(axis=1)
        E = np.exp(S - m[:, None])
        P = E / E.sum(axis=1)[:, None]
        dP = do[idx] @ v.T
        row_term = (P * dP).sum(axis=1)
        Pc = P[:, kidx]
        dSc = Pc * (dP[:, kidx] - row_term[:, None])
        dV += Pc.T @ do[idx]
        dK += scale * (dSc.T @ q[idx])
    return dK, dV


# ---------------------------------------------------------------------------
# Split-KV (Flash-Decoding): partial results per key range, then the merge
# ---------------------------------------------------------------------------

def split_bounds(Lkv: int, num_splits: int):
    """Key ranges of the splits: chunk = ceil(Lkv/S); split s covers
    [s*chunk, min((s+1)*chunk, Lkv)), possibly empty at the end."""
    chunk = -(-Lkv // num_splits)
    return [(min(s * chunk, Lkv), min((s + 1) * chunk, Lkv)) for s in range(num_splits)]


def split_partials(q, k, v, scale, num_splits):
    """Per-split normalised partial outputs and their log-sum-exps.

    The pages' split example (FlashAttention V2 overview: K and V cut in two,
    each part giving its own S, A and O, the two O then joined into the final
    result) generalised to ``num_splits`` key ranges.  Each partial is the
    exact attention of the queries over that key range alone.

    q: [..., Nq, d]; k, v: [..., Nk, d].  Returns
    (O_s [..., S, Nq, d], LSE_s [..., S, Nq]); an empty range gives O_s = 0,
    LSE_s = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    outs, lses = [], []
    for lo, hi in split_bounds(k.shape[-2], num_splits):
        if hi > lo:
            o, l = attention(q, k[..., lo:hi, :], v[..., lo:hi, :], scale, causal=False)
        else:
            o = np.zeros(q.shape[:-1] + (v.shape[-1],))
            l = np.full(q.shape[:-1], -np.inf)
        outs.append(o)
        lses.append(l)
    return np.stack(outs, axis=-3), np.stack(lses, axis=-2)


def merge_partials(O_s, LSE_s):
    """Merge split partials: M = max_s LSE_s, w_s = exp(LSE_s - M),
    O = sum_s w_s O_s / sum_s w_s, LSE = M + ln sum_s w_s.

    O_s: [..., S, Nq, d]; LSE_s: [..., S, Nq].  All -inf -> O = 0, LSE = -inf.
    """
    O_s = np.asarray(O_s, np.float64)
    LSE_s = np.asarray(LSE_s, np.float64)
    M = LSE_s.max(axis=-2)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(LSE_s), np.exp(LSE_s - Ms[..., None, :]), 0.0)
    W = w.sum(axis=-2)
    Wsafe = np.where(finite, W, 1.0)
    O = (w[..., None] * O_s).sum(axis=-3) / Wsafe[..., None]
    O = np.where(finite[..., None], O, 0.0)
    LSE = np.where(finite, Ms + np.log(Wsafe), -np.inf)
    return O, LSE


def decode_attention(q, k, v, scale):
    """Single-query decode: exact, unmasked attention of q [..., 1, d] over the
    whole cache k, v [..., Lkv, d].  Splitting the keys does not change the
    result, so the reference for the split-KV path is the unsplit definition."""
    return attention(q, k, v, scale, causal=False)


def decode_attention_gqa(q, k, v, scale):
    """Single-query decode with grouped key/value heads (GQA; MQA when there is
    one key/value head): query head h attends over key/value head h // G,
    G = Hq / Hkv, so consecutive query heads share a cached K/V head (CSDN,
    "flash attention CUDA programming, pipeline-parallel acceleration V6",
    related-post note on MQA: keys and values drop to one shared head while
    queries keep all of theirs; GQA is the plain generalisation to Hkv heads).

    q: [..., Hq, 1, d]; k, v: [..., Hkv, Lkv, d] with Hq a multiple of Hkv.
    Returns (O [..., Hq, 1, d], LSE [..., Hq, 1]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Hq, Hkv = q.shape[-3], k.shape[-3]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    kv_of = np.arange(Hq) // (Hq // Hkv)
    return attention(q, k[..., kv_of, :, :], v[..., kv_of, :, :], scale, causal=False)


def decode_attention_ragged(q, k, v, seqlens, scale):
    """Single-query decode over a padded cache with a length per sequence:
    sequence b attends over the first seqlens[b] cached keys only (grouped
    heads as in ``decode_attention_gqa``).  A sequence with no cached key
    gets O = 0 and LSE = -inf.

    q: [B, Hq, 1, d]; k, v: [B, Hkv, Lcap, d]; seqlens: [B], 0 <= seqlens[b] <= Lcap.
    Returns (O [B, Hq, 1, d], LSE [B, Hq, 1]).
    """
    q = np.asarray(q, np.float64)
    B, Hq = q.shape[:2]
    O = np.zeros(q.shape[:3] + (np.shape(v)[-1],))
    L = np.full((B, Hq, 1), -np.inf)
    for b in range(B):
        n = int(seqlens[b])
        if n > 0:
            O[b], L[b] = decode_attention_gqa(q[b], np.asarray(k[b])[:, :n], np.asarray(v[b])[:, :n],
                                              scale)
    return O, L


# ---------------------------------------------------------------------------
# fp8: the elementwise bound on an fp8-P kernel's error
# ---------------------------------------------------------------------------

def fp8_p_error_bound(q, k, v, scale, causal, p_prescale, qidx=None):
    """Elementwise bound |O_kernel - O| <= B for a kernel that rounds the
    unnormalised probabilities to E4M3FN before the P*V product.

    q, k, v are the *dequantised* inputs of one (batch, head): q [r, d] (rows
    ``qidx``), k, v [Nk, d].  With p_ij = exp(s_ij - m_i) / l_i the exact
    probabilities, a kernel storing sigma*exp(s - m') for some running max
    m' <= m_i in E4M3FN makes an error per weight of at most 2^-4 relative
    (3 mantissa bits, half an ulp) or 2^-10/sigma absolute (half the subnormal
    quantum 2^-9, undone by the pre-scale sigma).  Rescaling by
    exp(m' - m_i) <= 1 only shrinks the absolute part.  Whether the kernel
    divides by the unrounded sum or by the sum of the rounded weights, the
    output error is at most sum_j |dp_j| (|v_jc| + |O_ic|) / (l_i (1 - 2^-4)),
    hence the 16/15.  bf16 rounding of the output adds 2^-8 |O_ic|, and
    1e-4 covers float32 accumulation.

    Returns (O [r, d], LSE [r], B [r, d]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    r = q.shape[0]
    if qidx is None:
        qidx = np.arange(r)
    qidx = np.asarray(qidx, np.int64)
    S = scale * (q @ k.T)
    if causal:
        j = np.arange(k.shape[0])
        visible = j[None, :] <= qidx[:, None]
        S = np.where(visible, S, -np.inf)
    else:
        visible = np.ones(S.shape, dtype=bool)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    l = E.sum(axis=1)
    P = E / l[:, None]
    O = P @ v
    lse = m + np.log(l)
    absv = np.abs(v)
    absO = np.abs(O)
    n_vis = visible.sum(axis=1).astype(np.float64)
    # sum_j P_ij (|v_jc| + |O_ic|)   and   sum_{visible j} (|v_jc| + |O_ic|) / l_i
    rel_term = P @ absv + absO
    abs_term = (visible.astype(np.float64) @ absv + n_vis[:, None] * absO) / l[:, None]
    Bnd = (16.0 / 15.0) * (2.0 ** -4 * rel_term + 2.0 ** -10 / p_prescale * abs_term) \
        + 2.0 ** -8 * absO + 1e-4
    return O, lse, Bnd


def fp8_p_attention(q, k, v, scale, causal, p_scale, qidx=None):
    """Attention whose probability weights are rounded to E4M3FN before the
    P*V product -- the precision of the fp8 path of the FlashAttention-3
    snippets, where the second product also runs in fp8 -- with everything
    else exact.

    It states the error that rounding P alone causes, as a yardstick for the
    typical (mean) error of an fp8 kernel; the exact result is ``attention``.
    For each query row: p_ij = exp(s_ij - m_i) with the row's true max;
    key j's weight is rounded as round_e4m3(p_ij * p_scale[j]) / p_scale[j];
    O_i = sum_j rounded_ij v_j / sum_j p_ij (the unrounded row sum).

    q [r, d] (rows ``qidx``), k, v [Nk, d] of one (batch, head), float64;
    p_scale [Nk] > 0.  Returns O [r, d].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sig = np.asarray(p_scale, np.float64)
    if qidx is None:
        qidx = np.arange(q.shape[0])
    qidx = np.asarray(qidx, np.int64)
    O = np.empty((q.shape[0], v.shape[1]))
    for r0 in range(0, q.shape[0], ROW_BLOCK):
        sl = slice(r0, r0 + ROW_BLOCK)
        S = scale * (q[sl] @ k.T)
        if causal:
            j = np.arange(k.shape[0])
            S = np.where(j[None, :] <= qidx[sl, None], S, -np.inf)
        m = S.max(axis=1)
        P = np.exp(S - m[:, None])
        Ph = round_to_e4m3fn(P * sig[None, :]) / sig[None, :]
        O[sl] = (Ph @ v) / P.sum(axis=1)[:, None]
    return O
