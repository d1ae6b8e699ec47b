"""GPU parity of the forward pass over packed sequences of unequal lengths
(queries and keys may differ; causal masking aligned at the sequence end)."""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import bf16_to_dev, check_bf16_gates, dev_to_f64, say

pytestmark = pytest.mark.gpu


def packed(wid, tensor, lens, H, d):
    """uint16 bf16 bits [sum(lens), H, d]: sequence b, head h is the (b, h)
    stream of the generator, rows 0..lens[b]-1."""
    out = np.empty((int(sum(lens)), H, d), dtype=np.uint16)
    r = 0
    for b, n in enumerate(lens):
        for h in range(H):
            out[r:r + n, h] = fi.bf16_slice(wid, tensor, b, h, n, d)
        r += n
    return out


def cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def run(fa, lq, lk, H, d, causal, wid, scale=None):
    scale = scale or d ** -0.5
    qb = packed(wid, fi.Q_ID, lq, H, d)
    kb = packed(wid, fi.K_ID, lk, H, d)
    vb = packed(wid, fi.V_ID, lk, H, d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    cq, ck = (torch.from_numpy(cu(x)).cuda() for x in (lq, lk))
    o = torch.empty_like(q)
    lse = torch.empty((H, int(sum(lq))), dtype=torch.float32, device="cuda")
    fa.fa_fwd_varlen(q, k, v, o, lse, cq, ck, len(lq), H, max(lq), max(lk), int(sum(lq)),
                     int(sum(lk)), d, scale, causal)
    torch.cuda.synchronize()
    return (qb, kb, vb), o, lse, scale


CASES = [
    ([1, 31, 200, 257, 64], [1, 31, 200, 257, 64]),          # equal lengths
    ([7, 100, 256, 33], [50, 612, 256, 1000]),                 # prefill chunks against cached keys
    ([40, 300, 5], [9, 200, 1]),                               # more queries than keys
    ([1, 1, 1, 1], [1000, 3, 64, 257]),                        # one query per sequence
    # several 256-query tiles per sequence, paired in one workgroup (tiles 2 and
    # 0, then 1): in the first sequence the first query tile sees no key at all
    # while its partner sees one key tile
    ([600, 513, 40], [40, 700, 300]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_varlen_small(gpu_lib, ci, causal, d):
    fa = gpu_lib
    lq, lk = CASES[ci]
    H = 3
    wid = 8000 + 10 * ci + 2 * causal + (d == 128)
    say(f"varlen lq={lq} lk={lk} H={H} d={d} causal={causal} seed-id={wid}")
    (qb, kb, vb), o, lse, scale = run(fa, lq, lk, H, d, causal, wid)
    O, L = oracle.attention_varlen(*map(oracle.decode_bf16, (qb, kb, vb)), cu(lq), cu(lk), scale,
                                   causal)
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    empty = np.isneginf(L)
    assert np.array_equal(np.isneginf(lg), empty)
    assert np.all(og.transpose(1, 0, 2)[empty] == 0.0)
    seen = ~empty.T              # [total_q, H]
    check_bf16_gates(og[seen], O[seen], lg[~empty], L[~empty], f"case {ci}", beyond_floor=True)


def test_varlen_equal_lengths_match_dense_kernel(gpu_lib):
    """Equal lengths through the packed path and through the dense entry
    point (same bf16 inputs, transposed layout): identical bits."""
    fa = gpu_lib
    lens, H, d = [300, 300], 4, 128
    (qb, kb, vb), o, lse, scale = run(fa, lens, lens, H, d, True, 8100)
    B, N = 2, 300
    dense = [torch.from_numpy(np.ascontiguousarray(x.reshape(B, N, H, d).transpose(0, 2, 1, 3)))
             for x in (qb, kb, vb)]
    q, k, v = (bf16_to_dev(x.numpy()) for x in dense)
    od = torch.empty_like(q)
    ld = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, od, ld, B, H, N, d, scale, True)
    torch.cuda.synchronize()
    o_packed = o.view(B, N, H, d).permute(0, 2, 1, 3)
    assert torch.equal(o_packed.contiguous().view(torch.int16), od.view(torch.int16))
    assert torch.equal(lse.view(H, B, N).permute(1, 0, 2).contiguous(), ld)


def test_varlen_chunked_prefill_full_size(gpu_lib):
    """The ragged chunked-prefill workload: 8 sequences, H=32, d=128, each a
    chunk of new queries against its cached keys plus itself; sampled
    (sequence, head) pairs against the oracle."""
    fa = gpu_lib
    w = fi.VARLEN_PREFILL
    say(f"varlen {w['name']}: generating")
    (qb, kb, vb), o, lse, scale = run(fa, w["lq"], w["lk"], w["H"], w["d"], True, w["wid"])
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    cq, ck = cu(w["lq"]), cu(w["lk"])
    for b, h in [(0, 0), (3, 17), (6, 31), (7, 5)]:
        sl_q, sl_k = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        O, L = oracle.attention_varlen(*(oracle.decode_bf16(x[s, h:h + 1]) for x, s in
                                         ((qb, sl_q), (kb, sl_k), (vb, sl_k))),
                                       [0, w["lq"][b]], [0, w["lk"][b]], scale, True)
        check_bf16_gates(og[sl_q, h], O[:, 0], lg[h, sl_q], L[0], f"(seq={b},h={h})")


def test_varlen_in_bounds(gpu_lib):
    """Guard bands around o and lse stay untouched; padding rows of the
    launch (sequences shorter than max_seqlen_q) write nothing."""
    fa = gpu_lib
    lq, lk, H, d = [5, 300, 77], [5, 700, 20], 2, 128
    qb, kb, vb = (packed(8200, t, lens, H, d) for t, lens in
                  ((fi.Q_ID, lq), (fi.K_ID, lk), (fi.V_ID, lk)))
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    cq, ck = (torch.from_numpy(cu(x)).cuda() for x in (lq, lk))
    G = 4096
    nel = sum(lq) * H * d
    obuf = torch.full((nel + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((H * sum(lq) + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    fa.fa_fwd_varlen(q, k, v, obuf[G:G + nel], lbuf[G:G + H * sum(lq)], cq, ck, 3, H, 400, 700,
                     sum(lq), sum(lk), d, d ** -0.5, True)
    torch.cuda.synchronize()
    assert torch.all(obuf[:G] == 7.0) and torch.all(obuf[G + nel:] == 7.0)
    assert torch.all(lbuf[:G] == 7.0) and torch.all(lbuf[G + H * sum(lq):] == 7.0)
    assert torch.all(torch.isfinite(obuf[G:G + nel].float()))
