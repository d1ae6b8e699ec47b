"""GPU parity of the grouped-K/V-head (GQA / MQA) split-KV decode against the
oracle: partials per query head and the merged output."""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import bf16_to_dev, check_bf16_gates, dev_to_f64, say

pytestmark = pytest.mark.gpu


def gen(wid, B, Hq, Hkv, Lkv, d):
    q = fi.bf16_tensor(wid, fi.Q_ID, B, Hq, 1, d)
    k = fi.bf16_tensor(wid, fi.K_ID, B, Hkv, Lkv, d)
    v = fi.bf16_tensor(wid, fi.V_ID, B, Hkv, Lkv, d)
    return q, k, v


def run(fa, q, k, v, B, Hq, Hkv, Lkv, d, S, scale, own_ws=False):
    o = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    if own_ws:
        fa.fa_decode_splitkv_gqa(q, k, v, o, lse, B, Hq, Hkv, Lkv, d, S, scale)
        torch.cuda.synchronize()
        return o, lse, None, None
    nbytes = fa.fa_decode_workspace_bytes(B, Hq, d, S)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.fa_decode_splitkv_gqa(q, k, v, o, lse, B, Hq, Hkv, Lkv, d, S, scale, ws, nbytes)
    torch.cuda.synchronize()
    po = ws[:B * Hq * S * d].view(B, Hq, S, d)
    pl = ws[B * Hq * S * d:B * Hq * S * (d + 1)].view(B, Hq, S)
    return o, lse, po, pl


GROUPS = [(3, 3), (6, 3), (8, 2), (8, 1), (32, 2), (40, 2)]   # G = 1, 2, 4, 8, 16, 20


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", GROUPS)
@pytest.mark.parametrize("Lkv,S", [(1, 1), (5, 4), (100, 3), (1000, 64), (4097, 7), (333, 333)])
def test_gqa_small(gpu_lib, Lkv, S, Hq, Hkv, d):
    fa = gpu_lib
    B = 2
    wid = 6000 + 7 * Lkv + S + Hq + 3 * Hkv + d
    say(f"gqa decode B={B} Hq={Hq} Hkv={Hkv} Lkv={Lkv} d={d} splits={S} seed-id={wid}")
    qb, kb, vb = gen(wid, B, Hq, Hkv, Lkv, d)
    scale = d ** -0.5
    o, lse, po, pl = run(fa, *map(bf16_to_dev, (qb, kb, vb)), B, Hq, Hkv, Lkv, d, S, scale)
    q, k, v = map(oracle.decode_bf16, (qb, kb, vb))
    O, L = oracle.decode_attention_gqa(q, k, v, scale)
    check_bf16_gates(dev_to_f64(o)[:, :, 0], O[:, :, 0], dev_to_f64(lse), L[:, :, 0], "merged",
                     beyond_floor=Lkv < 64)
    # the partials of query head h are those of plain attention over K/V head h // G
    kv_of = np.arange(Hq) // (Hq // Hkv)
    Os, Ls = oracle.split_partials(q, k[:, kv_of], v[:, kv_of], scale, S)
    pog, plg = dev_to_f64(po), dev_to_f64(pl)
    empty = np.isneginf(Ls[:, :, :, 0])
    assert np.array_equal(np.isneginf(plg), empty)
    assert np.all(pog[empty] == 0)
    err = np.abs(pog - Os[:, :, :, 0])
    assert err.max() <= 1e-2, err.max()     # bf16 P in the second product, fp32 accumulation
    lr = np.abs(plg[~empty] - Ls[:, :, :, 0][~empty]) / np.maximum(np.abs(Ls[:, :, :, 0][~empty]), 1)
    assert lr.max() <= 1e-5, lr.max()


def test_gqa_one_head_per_group_matches_plain_decode(gpu_lib):
    """Hkv = Hq through the grouped kernel and through the plain decode
    kernel: both within the gates of the same oracle."""
    fa = gpu_lib
    B, H, Lkv, d, S = 2, 4, 3000, 128, 16
    say("gqa decode with G = 1 vs the plain decode entry point")
    qb, kb, vb = gen(6500, B, H, H, Lkv, d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    scale = d ** -0.5
    o, lse, _, _ = run(fa, q, k, v, B, H, H, Lkv, d, S, scale)
    o2 = torch.empty_like(o)
    fa.fa_decode_splitkv(q, k, v, o2, B, H, Lkv, d, S)
    torch.cuda.synchronize()
    O, L = oracle.decode_attention(*map(oracle.decode_bf16, (qb, kb, vb)), scale)
    check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L[:, :, 0], "grouped kernel")
    assert np.abs(dev_to_f64(o2) - O).max() <= 1e-2


def test_gqa_library_workspace(gpu_lib):
    fa = gpu_lib
    B, Hq, Hkv, Lkv, d, S = 2, 16, 2, 2500, 128, 12
    say("gqa decode with the library-owned workspace")
    qb, kb, vb = gen(6600, B, Hq, Hkv, Lkv, d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    o, lse, _, _ = run(fa, q, k, v, B, Hq, Hkv, Lkv, d, S, d ** -0.5, own_ws=True)
    O, L = oracle.decode_attention_gqa(*map(oracle.decode_bf16, (qb, kb, vb)), d ** -0.5)
    check_bf16_gates(dev_to_f64(o), O, dev_to_f64(lse), L[:, :, 0], "library workspace")


@pytest.mark.parametrize("wid", [6, 7])
def test_gqa_full_size(gpu_lib, wid):
    """B=8, Lkv=65536, d=128, 64 splits with 8 query heads per K/V head
    (Hq=64, Hkv=8) and with one K/V head for 32 query heads: sampled query
    heads against the oracle, every head against the single-split run."""
    fa = gpu_lib
    w = fi.WORKLOADS[wid]
    say(f"gqa decode {w.name}: generating K/V")
    qb, kb, vb = gen(w.wid, w.B, w.H, w.Hkv, w.Lkv, w.d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    say(f"gqa decode {w.name}: running")
    o, lse, _, _ = run(fa, q, k, v, w.B, w.H, w.Hkv, w.Lkv, w.d, w.num_splits, w.scale)
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    G = w.H // w.Hkv
    for b, h in [(0, 0), (3, 17), (7, w.H - 1), (5, G % w.H)]:
        Q = oracle.decode_bf16(qb[b, h])
        K, V = (oracle.decode_bf16(x[b, h // G]) for x in (kb, vb))
        O, L = oracle.decode_attention(Q, K, V, w.scale)
        check_bf16_gates(og[b, h], O, lg[b, h:h + 1], L, f"(b={b},h={h})")
    o1, lse1, _, _ = run(fa, q, k, v, w.B, w.H, w.Hkv, w.Lkv, w.d, 1, w.scale)
    assert np.abs(dev_to_f64(o1) - og).max() <= 1e-2
    assert np.abs(dev_to_f64(lse1) - lg).max() <= 1e-3


def test_gqa_deterministic_and_in_bounds(gpu_lib):
    """Two runs give identical bits; guard bands around o, lse and the
    workspace stay untouched."""
    fa = gpu_lib
    B, Hq, Hkv, Lkv, d, S = 2, 20, 1, 5000, 128, 9
    say("gqa decode determinism + guard bands")
    qb, kb, vb = gen(6700, B, Hq, Hkv, Lkv, d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    Gd = 4096
    nel = B * Hq * d
    obuf = torch.full((nel + 2 * Gd,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * Hq + 2 * Gd,), 7.0, dtype=torch.float32, device="cuda")
    need = fa.fa_decode_workspace_bytes(B, Hq, d, S)
    wbuf = torch.full((need // 4 + 2 * Gd,), 7.0, dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        fa.fa_decode_splitkv_gqa(q, k, v, obuf[Gd:Gd + nel], lbuf[Gd:Gd + B * Hq], B, Hq, Hkv,
                                 Lkv, d, S, d ** -0.5, wbuf[Gd:Gd + need // 4], need)
        torch.cuda.synchronize()
        outs.append((obuf[Gd:Gd + nel].clone(), lbuf[Gd:Gd + B * Hq].clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    for buf, n in ((obuf, nel), (lbuf, B * Hq), (wbuf, need // 4)):
        assert torch.all(buf[:Gd] == 7.0) and torch.all(buf[Gd + n:] == 7.0)


# ---------------------------------------------------------------------------
# a length per sequence in a padded cache
# ---------------------------------------------------------------------------

def run_varlen(fa, q, k, v, lens, B, Hq, Hkv, Lkv, d, S, scale):
    o = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    nbytes = fa.fa_decode_workspace_bytes(B, Hq, d, S)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    fa.fa_decode_splitkv_varlen(q, k, v, o, lse, sl, B, Hq, Hkv, Lkv, d, S, scale, ws, nbytes)
    torch.cuda.synchronize()
    po = ws[:B * Hq * S * d].view(B, Hq, S, d)
    pl = ws[B * Hq * S * d:B * Hq * S * (d + 1)].view(B, Hq, S)
    return o, lse, po, pl


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (40, 2)])
@pytest.mark.parametrize("S", [1, 7, 64])
def test_varlen_decode_small(gpu_lib, S, Hq, Hkv, d):
    fa = gpu_lib
    Lkv = 3000
    lens = [3000, 1, 0, 5, 2999, 64, 1000, 63]
    B = len(lens)
    wid = 6800 + S + Hq + Hkv + d
    say(f"varlen decode lens={lens} Hq={Hq} Hkv={Hkv} d={d} splits={S} seed-id={wid}")
    qb, kb, vb = gen(wid, B, Hq, Hkv, Lkv, d)
    # padding past each sequence's length holds garbage the kernel must not read
    for b, n in enumerate(lens):
        kb[b, :, n:] = 0x7F80   # +inf in bf16
        vb[b, :, n:] = 0x7FC0   # NaN
    scale = d ** -0.5
    o, lse, po, pl = run_varlen(fa, *map(bf16_to_dev, (qb, kb, vb)), lens, B, Hq, Hkv, Lkv, d, S,
                                scale)
    q, k, v = map(oracle.decode_bf16, (qb, kb, vb))
    O, L = oracle.decode_attention_ragged(q, k, v, lens, scale)
    og, lg = dev_to_f64(o)[:, :, 0], dev_to_f64(lse)
    empty = np.array([n == 0 for n in lens])
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty]))
    check_bf16_gates(og[~empty], O[~empty, :, 0], lg[~empty], L[~empty, :, 0], "merged",
                     beyond_floor=True)
    pog, plg = dev_to_f64(po), dev_to_f64(pl)
    kv_of = np.arange(Hq) // (Hq // Hkv)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(np.isneginf(plg[b])) and np.all(pog[b] == 0)
            continue
        Os, Ls = oracle.split_partials(q[b], k[b, kv_of, :n], v[b, kv_of, :n], scale, S)
        e = np.isneginf(Ls[:, :, 0])
        assert np.array_equal(np.isneginf(plg[b]), e)
        assert np.abs(pog[b] - Os[:, :, 0]).max() <= 1e-2


def test_varlen_decode_serving_batch(gpu_lib):
    """A serving-style batch over a 64 Ki-token padded cache: B=8, Hq=64,
    Hkv=8, d=128, 64 splits, sequence lengths from 1 to 65536; sampled heads
    against the oracle."""
    fa = gpu_lib
    lens = [65536, 1000, 30000, 7, 65535, 4096, 300, 50000]
    B, Hq, Hkv, Lkv, d, S = 8, 64, 8, 65536, 128, 64
    say("varlen decode serving batch: generating")
    qb, kb, vb = gen(6900, B, Hq, Hkv, Lkv, d)
    o, lse, _, _ = run_varlen(fa, *map(bf16_to_dev, (qb, kb, vb)), lens, B, Hq, Hkv, Lkv, d, S,
                              d ** -0.5)
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    for b, h in [(0, 0), (1, 9), (3, 63), (4, 17), (6, 40), (7, 8)]:
        n = lens[b]
        Q = oracle.decode_bf16(qb[b, h])
        K, V = (oracle.decode_bf16(x[b, h // 8, :n]) for x in (kb, vb))
        O, L = oracle.decode_attention(Q, K, V, d ** -0.5)
        check_bf16_gates(og[b, h], O, lg[b, h:h + 1], L, f"(b={b},h={h},len={n})")


@pytest.mark.parametrize("ramp", ["up", "down"])
def test_gqa_splits_of_very_different_weight(gpu_lib, ramp):
    """Grouped heads over a cache whose key norms double (or halve) every
    1024 keys, 64 splits: most splits' merge weights underflow."""
    fa = gpu_lib
    B, Hq, Hkv, Lkv, d, S = 2, 8, 2, 8192, 128, 64
    say(f"gqa decode ramped key norms ({ramp}) Hq={Hq} Hkv={Hkv} Lkv={Lkv} splits={S}")
    qb = fi.bf16_tensor(6900, fi.Q_ID, B, Hq, 1, d)
    k = np.stack([np.stack([fi.normals(6900 + (ramp == "down"), fi.K_ID, b, h, Lkv, d) for h in range(Hkv)])
                  for b in range(B)])
    f = (2.0 ** (np.arange(Lkv) / 1024.0)).astype(np.float32)
    if ramp == "down":
        f = f[::-1].copy()
    kb = fi.f32_to_bf16_bits(k * f[None, None, :, None])
    vb = fi.bf16_tensor(6900, fi.V_ID, B, Hkv, Lkv, d)
    scale = d ** -0.5
    o, lse, _, _ = run(fa, *map(bf16_to_dev, (qb, kb, vb)), B, Hq, Hkv, Lkv, d, S, scale)
    O, L = oracle.decode_attention_gqa(*map(oracle.decode_bf16, (qb, kb, vb)), scale)
    check_bf16_gates(dev_to_f64(o)[:, :, 0], O[:, :, 0], dev_to_f64(lse), L[:, :, 0], f"gqa ramp {ramp}",
                     beyond_floor=True)
