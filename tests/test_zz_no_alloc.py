"""GPU: the decode entry point that allocates nothing.

fa_decode_splitkv_noalloc keeps the split partials in the library's fixed
scratch instead of a workspace.  Two calls in a row, the second smaller,
must each give the same bits as fa_decode_splitkv_ex with a caller
workspace (same kernels), meet the bf16 gates against the oracle, and
leave guard bands around their outputs untouched.  The second call reads
no partial left behind by the first.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import oracle
from _gpu_util import bf16_to_dev, check_bf16_gates, dev_to_f64, say

pytestmark = pytest.mark.gpu

GUARD = 4096


def guarded(n, dtype):
    buf = torch.full((n + 2 * GUARD,), 7.0, dtype=dtype, device="cuda")
    return buf, buf[GUARD:GUARD + n]


def guards_intact(buf, n):
    return bool(torch.all(buf[:GUARD] == 7.0)) and bool(torch.all(buf[GUARD + n:] == 7.0))


def test_noalloc_matches_workspace_entry(gpu_lib):
    fa = gpu_lib
    cases = [(4, 16, 20000, 128, 64, 7100), (2, 3, 5000, 64, 9, 7101)]   # second call smaller
    for B, H, Lkv, d, S, wid in cases:
        say(f"decode noalloc B={B} H={H} Lkv={Lkv} d={d} S={S} seed-id={wid}")
        assert fa.fa_decode_workspace_bytes(B, H, d, S) <= fa.FA_DECODE_SCRATCH_BYTES
        qb = fi.bf16_tensor(wid, fi.Q_ID, B, H, 1, d)
        kb = fi.bf16_tensor(wid, fi.K_ID, B, H, Lkv, d)
        vb = fi.bf16_tensor(wid, fi.V_ID, B, H, Lkv, d)
        q, k, v = map(bf16_to_dev, (qb, kb, vb))
        scale = d ** -0.5
        nel = B * H * d
        obuf, o = guarded(nel, torch.bfloat16)
        lbuf, lse = guarded(B * H, torch.float32)
        fa.fa_decode_splitkv_noalloc(q, k, v, o, lse, B, H, Lkv, d, S, scale)
        torch.cuda.synchronize()
        need = fa.fa_decode_workspace_bytes(B, H, d, S)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o_ref = torch.empty(nel, dtype=torch.bfloat16, device="cuda")
        l_ref = torch.empty(B * H, dtype=torch.float32, device="cuda")
        fa.fa_decode_splitkv_ex(q, k, v, o_ref, l_ref, B, H, Lkv, d, S, scale, ws, need)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from the workspace call"
        assert torch.equal(lse, l_ref), "LSE differs from the workspace call"
        assert guards_intact(obuf, nel) and guards_intact(lbuf, B * H)
        O, L = oracle.decode_attention(*map(oracle.decode_bf16, (qb, kb, vb)), scale)
        check_bf16_gates(dev_to_f64(o).reshape(B, H, 1, d), O, dev_to_f64(lse).reshape(B, H, 1), L,
                         f"noalloc B={B} H={H}")


def test_noalloc_rejects_oversized_partials(gpu_lib):
    """Partials beyond the fixed scratch are refused before any launch."""
    fa = gpu_lib
    B, H, Lkv, d, S = 8, 32, 512, 128, 255
    q = torch.zeros((B, H, 1, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, H, Lkv, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_splitkv_noalloc(q, kv, kv, o, None, B, H, Lkv, d, S, d ** -0.5)
    assert e.value.status == fa.FA_ERR_WORKSPACE
