"""GPU parity of the split-KV decode (partials and merge) against the oracle."""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import ErrStats, bf16_values, bf16_to_dev, check_bf16_gates, dev_to_f64, say

pytestmark = pytest.mark.gpu


def gen(wid, B, H, Lkv, d):
    q = fi.bf16_tensor(wid, fi.Q_ID, B, H, 1, d)
    k = fi.bf16_tensor(wid, fi.K_ID, B, H, Lkv, d)
    v = fi.bf16_tensor(wid, fi.V_ID, B, H, Lkv, d)
    return q, k, v


def run_ex(fa, q, k, v, B, H, Lkv, d, S, scale):
    o = torch.empty((B, H, 1, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    nbytes = fa.fa_decode_workspace_bytes(B, H, d, S)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.fa_decode_splitkv_ex(q, k, v, o, lse, B, H, Lkv, d, S, scale, ws, nbytes)
    torch.cuda.synchronize()
    po = ws[:B * H * S * d].view(B, H, S, d)
    pl = ws[B * H * S * d:B * H * S * (d + 1)].view(B, H, S)
    return o, lse, po, pl


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lkv,S", [(1, 1), (5, 4), (70, 64), (100, 3), (1000, 64), (4097, 7),
                                   (4096, 1), (333, 333), (20000, 64)])
def test_decode_small(gpu_lib, Lkv, S, d):
    fa = gpu_lib
    B, H = 2, 3
    wid = 4000 + Lkv + S + d
    say(f"decode B={B} H={H} Lkv={Lkv} d={d} splits={S} seed-id={wid}")
    qb, kb, vb = gen(wid, B, H, Lkv, d)
    scale = d ** -0.5
    o, lse, po, pl = run_ex(fa, *map(bf16_to_dev, (qb, kb, vb)), B, H, Lkv, d, S, scale)
    q, k, v = map(oracle.decode_bf16, (qb, kb, vb))
    O, L = oracle.decode_attention(q, k, v, scale)
    check_bf16_gates(dev_to_f64(o)[:, :, 0], O[:, :, 0], dev_to_f64(lse), L[:, :, 0], "merged")
    Os, Ls = oracle.split_partials(q, k, v, scale, S)
    pog, plg = dev_to_f64(po), dev_to_f64(pl)
    empty = np.isneginf(Ls[:, :, :, 0])
    assert np.array_equal(np.isneginf(plg), empty)
    assert np.all(pog[empty] == 0)
    err = np.abs(pog - Os[:, :, :, 0])
    assert err.max() <= 2e-3, err.max()     # fp32 partials: bf16 inputs, fp32 math
    lr = np.abs(plg[~empty] - Ls[:, :, :, 0][~empty]) / np.maximum(np.abs(Ls[:, :, :, 0][~empty]), 1)
    assert lr.max() <= 1e-5, lr.max()


def test_decode_default_entry_point(gpu_lib):
    fa = gpu_lib
    B, H, Lkv, d, S = 2, 4, 3000, 128, 16
    say("decode via fa_decode_splitkv (library-owned workspace)")
    qb, kb, vb = gen(4500, B, H, Lkv, d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    o = torch.empty((B, H, 1, d), dtype=torch.bfloat16, device="cuda")
    fa.fa_decode_splitkv(q, k, v, o, B, H, Lkv, d, S)
    torch.cuda.synchronize()
    O, L = oracle.decode_attention(*map(oracle.decode_bf16, (qb, kb, vb)), d ** -0.5)
    err = np.abs(dev_to_f64(o) - O)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
    # a second, larger call grows the workspace
    o2 = torch.empty_like(o)
    fa.fa_decode_splitkv(q, k, v, o2, B, H, Lkv, d, 3000)
    torch.cuda.synchronize()
    assert np.abs(dev_to_f64(o2) - O).max() <= 1e-2


def test_decode_full_size(gpu_lib):
    """B=8, H=32, Lkv=65536, d=128, 64 splits: every (b, h) against the
    oracle.  The one-split run of the same kernels is checked too."""
    fa = gpu_lib
    w = fi.WORKLOADS[4]
    say(f"decode {w.name}: generating 8 GiB of K/V")
    qb, kb, vb = gen(w.wid, w.B, w.H, w.Lkv, w.d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    say("decode full size: running")
    o, lse, _, _ = run_ex(fa, q, k, v, w.B, w.H, w.Lkv, w.d, w.num_splits, w.scale)
    o1, lse1, _, _ = run_ex(fa, q, k, v, w.B, w.H, w.Lkv, w.d, 1, w.scale)
    og, lg = dev_to_f64(o), dev_to_f64(lse)
    og1, lg1 = dev_to_f64(o1), dev_to_f64(lse1)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    st = ErrStats("C4 decode B=8 H=32 Lkv=65536 S=64")
    st1 = ErrStats("C4 decode, one split")
    say("decode full size: oracle for all 256 (b, h)")
    for b in range(w.B):
        for h in range(w.H):
            Q, K, V = (bf16_values(x[b, h]) for x in (qb, kb, vb))
            O, L = oracle.decode_attention(Q, K, V, w.scale)
            check_bf16_gates(og[b, h], O, lg[b, h:h + 1], L, f"(b={b},h={h})")
            check_bf16_gates(og1[b, h], O, lg1[b, h:h + 1], L, f"(b={b},h={h}) one split")
            st.add(og[b, h], O, lg[b, h:h + 1], L)
            st1.add(og1[b, h], O, lg1[b, h:h + 1], L)
    st.report()
    st1.report()


def test_decode_deterministic_and_in_bounds(gpu_lib):
    """Two runs give identical bits; guard bands around o, lse and the
    workspace stay untouched (a workspace larger than needed)."""
    fa = gpu_lib
    B, H, Lkv, d, S = 2, 3, 5000, 128, 9
    say("decode determinism + guard bands")
    qb, kb, vb = gen(4700, B, H, Lkv, d)
    q, k, v = map(bf16_to_dev, (qb, kb, vb))
    G = 4096
    nel = B * H * d
    obuf = torch.full((nel + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    need = fa.fa_decode_workspace_bytes(B, H, d, S)
    wbuf = torch.full((need // 4 + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        fa.fa_decode_splitkv_ex(q, k, v, obuf[G:G + nel], lbuf[G:G + B * H], B, H, Lkv, d, S,
                                d ** -0.5, wbuf[G:G + need // 4], need)
        torch.cuda.synchronize()
        outs.append((obuf[G:G + nel].clone(), lbuf[G:G + B * H].clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    for buf, n in ((obuf, nel), (lbuf, B * H), (wbuf, need // 4)):
        assert torch.all(buf[:G] == 7.0) and torch.all(buf[G + n:] == 7.0)


def test_decode_owned_workspace_from_two_threads(gpu_lib):
    """Two host threads share the library-owned workspace on one stream while
    it grows: each call queues its split and merge launches under the
    workspace lock, so no call reads a freed buffer or another call's
    partials.  Every output meets the gates and equals the other calls of
    its size bit for bit."""
    import threading
    fa = gpu_lib
    d, Lkv, S, H = 64, 64, 64, 16
    sizes = [32, 64, 128]       # B: workspace of 8.5, 17 and 34 MB
    rounds = 3
    say(f"decode from two threads, library-owned workspace, B in {sizes}, H={H} Lkv={Lkv} d={d} splits={S}")
    data, refs = {}, {}
    for B in sizes:
        qb, kb, vb = gen(4700 + B, B, H, Lkv, d)
        data[B] = tuple(map(bf16_to_dev, (qb, kb, vb)))
        refs[B] = oracle.decode_attention(*map(oracle.decode_bf16, (qb, kb, vb)), d ** -0.5)[0]
    outs = {(t, r, B): torch.empty((B, H, 1, d), dtype=torch.bfloat16, device="cuda")
            for t in range(2) for r in range(rounds) for B in sizes}
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            order = sizes if t == 0 else sizes[::-1]
            for r in range(rounds):
                for B in order:
                    q, k, v = data[B]
                    fa.fa_decode_splitkv(q, k, v, outs[(t, r, B)], B, H, Lkv, d, S)
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for B in sizes:
        first = outs[(0, 0, B)]
        for key, o in outs.items():
            if key[2] == B:
                assert torch.equal(o, first), key
        err = np.abs(dev_to_f64(first) - refs[B])
        assert err.max() <= 1e-2 and err.mean() <= 1e-3, (B, err.max(), err.mean())


@pytest.mark.parametrize("ramp", ["up", "down"])
def test_decode_splits_of_very_different_weight(gpu_lib, ramp):
    """Key norms that double (or halve) every 1024 keys of an 8192-key cache
    cut into 64 splits: the splits' LSE differ by tens, so most merge weights
    exp(LSE_s - LSE) underflow and one end of the cache decides the output."""
    fa = gpu_lib
    B, H, Lkv, d, S = 2, 4, 8192, 128, 64
    say(f"decode ramped key norms ({ramp}) Lkv={Lkv} splits={S}")
    qb = fi.bf16_tensor(4800, fi.Q_ID, B, H, 1, d)
    k = np.stack([np.stack([fi.normals(4800 + (ramp == "down"), fi.K_ID, b, h, Lkv, d) for h in range(H)])
                  for b in range(B)])
    f = (2.0 ** (np.arange(Lkv) / 1024.0)).astype(np.float32)
    if ramp == "down":
        f = f[::-1].copy()
    kb = fi.f32_to_bf16_bits(k * f[None, None, :, None])
    vb = fi.bf16_tensor(4800, fi.V_ID, B, H, Lkv, d)
    scale = d ** -0.5
    o, lse, po, pl = run_ex(fa, *map(bf16_to_dev, (qb, kb, vb)), B, H, Lkv, d, S, scale)
    q, kk, v = map(oracle.decode_bf16, (qb, kb, vb))
    O, L = oracle.decode_attention(q, kk, v, scale)
    check_bf16_gates(dev_to_f64(o)[:, :, 0], O[:, :, 0], dev_to_f64(lse), L[:, :, 0], f"ramp {ramp}",
                     beyond_floor=True)
    Ls = oracle.split_partials(q, kk, v, scale, S)[1][:, :, :, 0]
    spread = float((Ls.max(-1) - Ls.min(-1)).min())
    say(f"  smallest spread of split LSEs over (b, h): {spread:.1f}")
    assert spread > 20.0   # the case really has splits of negligible weight
