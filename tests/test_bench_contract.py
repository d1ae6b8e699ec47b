"""bench.py's metric arithmetic and its one-GPU contract, checked on the CPU.

Prefill is reported as 4*B*H*N^2*d FLOPs (halved for causal) per time, and
decode as the bytes of K, V, q and o moved once per time.  The expected
counts below are written out from the shapes of each configuration (the
per-config table of the metric's definition), not recomputed by the bench's
own helpers.
"""
import json
import os
import subprocess
import sys

import bench
import fa_inputs as fi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
W = fi.WORKLOADS


def test_prefill_flops():
    assert bench.fwd_flops(W[1], False) == 4_194_304               # 4*1*1*128^2*64
    assert bench.fwd_flops(W[2], False) == 137_438_953_472         # 4*2*32*2048^2*128
    assert bench.fwd_flops(W[2], True) == 68_719_476_736
    assert bench.fwd_flops(W[3], True) == 1_099_511_627_776        # 4*1*16*16384^2*128 / 2
    assert bench.fwd_flops(W[5], True) == 1_099_511_627_776        # 4*4*16*8192^2*128 / 2


def test_prefill_bytes():
    # q, k, v read once, o written once, lse (fp32) written once
    assert bench.fwd_bytes(W[1], out_bytes=4) == 82_432
    assert bench.fwd_bytes(W[2]) == 134_742_016
    assert bench.fwd_bytes(W[3]) == 269_484_032
    # fp8: one-byte inputs; the fp32 block scales (3 * 4*16*128 * 4 B) are counted apart
    assert bench.fwd_bytes(W[5], in_bytes=1) + 98_304 == 337_739_776


def test_ragged_prefill_pairs():
    # chunk of Lq queries against Lk >= Lq keys, end-aligned causal: Lq*Lk - Lq(Lq-1)/2 pairs
    assert bench.varlen_pairs([3], [3]) == 6
    assert bench.varlen_pairs([2], [5]) == 9             # 4 + 5
    assert bench.varlen_pairs([5], [2]) == 3             # 0, 0, 0, 1, 2: the first three see no key
    # the ragged prefill batch: 2098176 + 1573376 + 2228480 + 1568896 + 1966848 + 1868160
    # + 1040448 + 2067300
    v = fi.VARLEN_PREFILL
    assert bench.varlen_pairs(v["lq"], v["lk"]) == 14_411_684


def test_decode_bytes():
    assert bench.decode_bytes(W[4]) == 8_590_065_664     # K+V 8 589 934 592 + q + o 131 072
    assert bench.decode_bytes(W[6]) == 2_147_745_792     # 8 K/V heads; q, o over 64 query heads
    assert bench.decode_bytes(W[7]) == 268_566_528       # one K/V head; q, o over 32 query heads


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_is_null_once_the_kernel_changed(monkeypatch):
    entry = dict(bench.TRAFFIC_KIB["c3"])
    entry["sha256"] = "0" * 64
    monkeypatch.setitem(bench.TRAFFIC_KIB, "c3", entry)
    assert bench.traffic_bytes("c3") is None
    assert bench.traffic_bytes("no-such-workload") is None
