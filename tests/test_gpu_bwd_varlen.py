"""GPU parity of the backward pass over packed sequences of unequal lengths
(fa_bwd_varlen) against the fp64 oracle (``oracle.attention_backward_varlen``).

As for the dense backward pass, the forward pass runs through the library
first (fa_fwd_varlen's bf16 O and fp32 LSE are the backward pass's inputs)
and the oracle differentiates the definition on the same bf16 inputs.  The
gates are the dense backward's (per gradient tensor G with reference R):
    max |G - R| <= 2e-2 * max |R| + 1e-5  and  mean |G - R| <= 1e-2 * mean |R| + 1e-5,
and gradients the definition makes exactly zero (a query that sees no key,
keys of a sequence without queries) must be exactly zero.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import bf16_to_dev, dev_to_f64, say
from test_gpu_bwd import check

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


def run(fa, lq, lk, H, d, causal, wid, own_ws=False):
    scale = d ** -0.5
    bits = (packed(wid, fi.Q_ID, lq, H, d), packed(wid, fi.K_ID, lk, H, d),
            packed(wid, fi.V_ID, lk, H, d), packed(wid, fi.DO_ID, lq, H, d))
    q, k, v, do = map(bf16_to_dev, bits)
    cq, ck = (torch.from_numpy(cu(x)).cuda() for x in (lq, lk))
    B, tq, tk = len(lq), int(sum(lq)), int(sum(lk))
    mq, mk = max(max(lq), 1), max(max(lk), 1)
    o = torch.empty_like(q)
    lse = torch.empty((H, tq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_varlen(q, k, v, o, lse, cq, ck, B, H, mq, mk, tq, tk, d, scale, causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if own_ws:
        fa.fa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, cq, ck, B, H, mq, mk, tq, tk, d, scale,
                         causal)
    else:
        nb = fa.fa_bwd_workspace_bytes(1, H, tq)
        ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
        fa.fa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, cq, ck, B, H, mq, mk, tq, tk, d, scale,
                         causal, ws, nb)
    torch.cuda.synchronize()
    return bits, (dq, dk, dv), scale


def reference(bits, lq, lk, scale, causal):
    q, k, v, do = map(oracle.decode_bf16, bits)
    return oracle.attention_backward_varlen(q, k, v, do, cu(lq), cu(lk), scale, causal)


def check_zeros(got, lq, lk, causal):
    """dQ of queries that see no key, and dK, dV of keys in a sequence with
    no queries, are exactly zero."""
    dq, dk, dv = (dev_to_f64(g) for g in got)
    cq, ck = cu(lq), cu(lk)
    for b in range(len(lq)):
        Lq, Lk = lq[b], lk[b]
        blind = Lq if Lk == 0 else (max(0, Lq - Lk) if causal else 0)
        assert np.all(dq[cq[b]:cq[b] + blind] == 0.0), f"sequence {b}: dQ of blind queries"
        if Lq == 0:
            assert np.all(dk[ck[b]:ck[b + 1]] == 0.0) and np.all(dv[ck[b]:ck[b + 1]] == 0.0), \
                f"sequence {b}: dK, dV of a sequence without queries"


CASES = [
    ([1, 31, 200, 257, 64], [1, 31, 200, 257, 64]),          # equal lengths
    ([7, 100, 256, 33], [50, 612, 256, 1000]),                 # prefill chunks against cached keys
    ([40, 300, 5], [9, 200, 1]),                               # more queries than keys
    ([1, 1, 1, 1], [1000, 3, 64, 257]),                        # one query per sequence
    ([600, 513, 40], [40, 700, 300]),                          # several query and key tiles
    ([0, 50, 129, 10], [70, 60, 129, 0]),                      # no queries; no keys
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_bwd_varlen_small(gpu_lib, ci, causal, d):
    fa = gpu_lib
    lq, lk = CASES[ci]
    H = 3
    wid = 9000 + 10 * ci + 2 * causal + (d == 128)
    say(f"bwd varlen lq={lq} lk={lk} H={H} d={d} causal={causal} seed-id={wid}")
    bits, got, scale = run(fa, lq, lk, H, d, causal, wid, own_ws=(ci % 2 == 1))
    ref = reference(bits, lq, lk, scale, causal)
    check(got, ref, f"case {ci} d={d} causal={causal}")
    check_zeros(got, lq, lk, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_equal_lengths_match_dense_kernel(gpu_lib, causal):
    """Equal lengths through the packed entry point and through fa_bwd on the
    same bf16 inputs in the dense layout: identical bits."""
    fa = gpu_lib
    B, H, N, d = 3, 4, 300, 128
    wid = 9100 + causal
    say(f"bwd varlen vs dense B={B} H={H} N={N} causal={causal} seed-id={wid}")
    bits, got, scale = run(fa, [N] * B, [N] * B, H, d, causal, wid)
    dense = [bf16_to_dev(np.ascontiguousarray(b.reshape(B, N, H, d).transpose(0, 2, 1, 3)))
             for b in bits]
    q, k, v, do = dense
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal)
    torch.cuda.synchronize()
    for name, g, r in zip(("dQ", "dK", "dV"), got, (dq, dk, dv)):
        r_packed = r.view(torch.int16).permute(0, 2, 1, 3).reshape(B * N, H, d)
        assert torch.equal(g.view(torch.int16), r_packed), f"{name} differs from the dense kernel"


def test_bwd_varlen_ragged_prefill_workload(gpu_lib):
    """The ragged chunked-prefill batch (8 sequences, H=32, d=128, causal),
    every sequence on heads 0 and 31 against the oracle."""
    fa = gpu_lib
    wv = fi.VARLEN_PREFILL
    lq, lk, H, d = wv["lq"], wv["lk"], wv["H"], wv["d"]
    say(f"bwd varlen {wv['name']}: running")
    bits, got, scale = run(fa, lq, lk, H, d, True, wv["wid"])
    heads = [0, H - 1]
    sub = [b[:, heads] for b in bits]
    ref = reference(sub, lq, lk, scale, True)
    got_sub = [dev_to_f64(g)[:, heads] for g in got]
    check(got_sub, ref, f"{wv['name']} heads {heads}")
    check_zeros(got, lq, lk, True)


@pytest.mark.parametrize("seed", range(8))
def test_bwd_varlen_random_length_mixes(gpu_lib, seed):
    """Seeded random batches: 1-6 sequences of 0-700 queries and 0-900 keys
    (at least one of each overall), H in {1, 2, 5}, d in {64, 128}, causal or
    not."""
    fa = gpu_lib
    rng = np.random.default_rng(9200 + seed)
    B = int(rng.integers(1, 7))
    while True:
        lq = [int(x) for x in rng.integers(0, 701, B)]
        lk = [int(x) for x in rng.integers(0, 901, B)]
        if sum(lq) > 0 and sum(lk) > 0:
            break
    H = int(rng.choice([1, 2, 5]))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    wid = 9300 + seed
    say(f"bwd varlen random lq={lq} lk={lk} H={H} d={d} causal={causal} seed-id={wid}")
    bits, got, scale = run(fa, lq, lk, H, d, causal, wid, own_ws=bool(seed % 2))
    ref = reference(bits, lq, lk, scale, causal)
    check(got, ref, f"random {seed}")
    check_zeros(got, lq, lk, causal)
