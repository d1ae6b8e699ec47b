#!/usr/bin/env python
"""Throughput of the attention library on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * bf16 forward, B=2 H=32 N=2048 d=128, causal and non-causal
  * bf16 forward, B=1 H=16 N=16384 d=128, causal
  * split-KV decode, B=8 H=32 Lkv=65536 d=128, 64 splits (split + merge kernels),
    and for context the same with one split, and one sequence of it (B=1)
    with 64 splits and with one: what splitting the KV length buys on this
    GPU (with 256 (b,h) pairs every CU already has work; with 32 it does not)
  * split-KV decode with grouped K/V heads, B=8 Lkv=65536 d=128, 64 splits:
    Hq=64 over Hkv=8 (GQA), and Hq=32 over one K/V head (MQA)
  * bf16 -> block-scaled fp8 quantisation of the fp8 workload's Q and K
    (with the incoherent Hadamard rotation) and V (power-of-two scales), the
    input pass of the fp8 forward from bf16 activations (HBM-bound: 2 bytes
    read, 1 written)
  * ragged chunked prefill: 8 packed sequences of unequal lengths, H=32,
    d=128, each a chunk of new queries against its cached keys, causal
    aligned at the sequence end (FLOPs: 4*d per visible query-key pair)
  * backward (dQ, dK, dV) of the B=2 H=32 N=2048 causal and B=1 H=16 N=16384
    causal forward passes, and of the ragged chunked prefill (FLOPs counted
    as 2.5x the forward's: five matrix products against two)
  * fp8 forward, B=4 H=16 N=8192 d=128, causal (when the library has it),
    V with power-of-two block scales, and again with max|x| / 448 V scales

``value`` is the bf16 causal forward throughput over the N=2048 and N=16384
workloads (their FLOPs over their summed kernel time, 4*B*H*N^2*d/2 per
causal call); the decode bandwidth is reported beside it.  Each launch is
bracketed by HIP events on the stream it runs on.  After the timed steps,
C3, C2 causal, the ragged prefill and the three backward workloads are also timed
as 20 or more back-to-back launches under one event pair (``steady``): no
event between launches, and no decode launch letting the clock recover.  The
CPU oracle is timed on a bounded sample of the same workloads (rank 0, N=1
only).
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd TFLOPS (bf16 causal, N=2K-16K) + split-KV decode HBM GB/s, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 (and fp16) MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_FP8_TFLOPS = 5033.2      # dense fp8
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch, from rocprofv3 counter runs (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, averaged over the dispatches of
# `bench.py --only <w> --steps 2 --warmup 1 --copy-calibration`; kernels of
# several launches per workload are summed).  The same counters read a 1 GiB
# device copy as 524306 KiB fetched and 1048576 KiB written, so fetches are
# scaled by 1048576/524306 and writes by 1.  Each
# entry is tied to the SHA-256 of its kernel source plus the shared device
# header: once either changes, the figure no longer describes the kernel and
# the bench reports traffic as null.  (A digest is moved to a new source only
# when the measured kernels' instructions were compared and found identical.)  Split-KV decode entries add the
# split-merge kernel's counters to the split kernel's.
COUNTER_SCALE = {"fetch": 1048576.0 / 524306.0, "write": 1.0}
TRAFFIC_KIB = {
    "c3": {"src": ["fa_fwd_bf16.hip"], "fetch_kib": 216148.6, "write_kib": 68608.0,
           "sha256": "ecdf90041e517b2d5cd99d06309bcf1600c87e194a150bc76296d5954801fa54"},
    "c4": {"src": ["fa_decode.hip"], "fetch_kib": 4198860.0, "write_kib": 8777.7,
           "sha256": "5e97611a26ac2cfece3c36bca4885bf4a61a66ef052765835b53367d362e873e"},
    "c5": {"src": ["fa_fwd_fp8.hip"], "fetch_kib": 456066.1, "write_kib": 106499.2,
           "sha256": "f09e1f40ea42b9852f993b74cc5a4067dc42a7715519cab56e494b536cc8d1b0"},
    "c6": {"src": ["fa_decode_gqa.hip", "fa_decode.hip"], "fetch_kib": 1057863.5, "write_kib": 17699.4,
           "sha256": "5173b008bb12a55976be3113d7be1d4c27cdcd419827915ad4c16c6113ac15a9"},
    "c7": {"src": ["fa_decode_gqa.hip", "fa_decode.hip"], "fetch_kib": 135572.7, "write_kib": 8777.7,
           "sha256": "5173b008bb12a55976be3113d7be1d4c27cdcd419827915ad4c16c6113ac15a9"},
}


def traffic_bytes(workload):
    """Counter-measured HBM bytes per launch, or None if the kernel changed."""
    import hashlib
    t = TRAFFIC_KIB.get(workload)
    if t is None:
        return None
    csrc = os.path.join(ROOT, "exact_attention_116_amd", "csrc")
    blob = b""
    for name in t["src"] + ["fa_device.hpp"]:
        with open(os.path.join(csrc, name), "rb") as f:
            blob += f.read()
    digest = hashlib.sha256(blob).hexdigest()
    if digest != t["sha256"]:
        return None
    return 1024.0 * (t["fetch_kib"] * COUNTER_SCALE["fetch"] + t["write_kib"] * COUNTER_SCALE["write"])


def traffic_source(workload):
    """Where a ``traffic`` figure comes from: it is not measured by this run."""
    t = TRAFFIC_KIB.get(workload)
    if t is None:
        return None
    state = "current" if traffic_bytes(workload) is not None else "stale: kernel source changed, traffic null"
    return (f"stored rocprofv3 FETCH_SIZE/WRITE_SIZE counters of an earlier run "
            f"(profiles/hbm_traffic_counters.md), for sources {'+'.join(t['src'])} + fa_device.hpp "
            f"with sha256 {t['sha256'][:16]}...; {state}")


def fwd_flops(w, causal):
    f = 4.0 * w.B * w.H * w.N * w.N * w.d
    return f / 2 if causal else f


def varlen_pairs(lq, lk):
    """Visible (query, key) pairs of a packed causal batch: query i of a
    sequence with Lq queries and Lk keys sees min(Lk, i + 1 + Lk - Lq) keys
    (end-aligned; none when that is negative)."""
    return sum(sum(max(0, min(k, i + 1 + k - q)) for i in range(q)) for q, k in zip(lq, lk))


def fwd_bytes(w, in_bytes=2, out_bytes=2):
    n = w.B * w.H * w.N * w.d
    return 3 * n * in_bytes + n * out_bytes + w.B * w.H * w.N * 4


def decode_bytes(w):
    """K and V read once, q read and o written once (bf16)."""
    hkv = w.Hkv or w.H
    kv = 2 * w.B * hkv * w.Lkv * w.d * 2
    return kv + 2 * w.B * w.H * w.d * 2


def log(msg):
    """Progress on stderr; the JSON result is the only line on stdout."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def cpu_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, AttributeError):
        pass
    return model


def cpu_baseline(seconds):
    """Time the fp64 oracle on a bounded sample of the forward and decode workloads."""
    import numpy as np
    import fa_inputs as fi
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    w = fi.WORKLOADS[2]
    t0 = time.perf_counter()
    flops, heads = 0.0, 0
    while time.perf_counter() - t0 < seconds * 0.75 or heads == 0:
        b, h = divmod(heads % (w.B * w.H), w.H)
        q, k, v = (oracle.decode_bf16(fi.bf16_slice(w.wid, t, b, h, w.N, w.d)) for t in range(3))
        oracle.attention(q, k, v, w.scale, True)
        flops += 4.0 * w.N * w.N * w.d / 2
        heads += 1
    t_fwd = time.perf_counter() - t0
    # decode: only the oracle call is timed (generation excluded), (b,h) pairs
    # until about a quarter of the budget is spent
    wd = fi.WORKLOADS[4]
    t_dec, nbytes, pairs = 0.0, 0, 0
    while t_dec < seconds * 0.25 or pairs == 0:
        b, h = divmod(pairs % (wd.B * wd.H), wd.H)
        qb = fi.bf16_slice(wd.wid, 0, b, h, 1, wd.d)
        kb = fi.bf16_slice(wd.wid, 1, b, h, wd.Lkv, wd.d)
        vb = fi.bf16_slice(wd.wid, 2, b, h, wd.Lkv, wd.d)
        ts = time.perf_counter()
        oracle.decode_attention(*(oracle.decode_bf16(x) for x in (qb, kb, vb)), wd.scale)
        t_dec += time.perf_counter() - ts
        nbytes += kb.nbytes + vb.nbytes
        pairs += 1
    return {
        "value": flops / t_fwd / 1e12,
        "value_full_s": 2 * flops / t_fwd / 1e12,   # the oracle materialises all of S, masked or not
        "unit": "TFLOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 two-pass oracle on (b,h) heads of causal B=2 H=32 N=2048 d=128, "
                   f"cycling over the 64 heads: {heads} head evaluations in {t_fwd:.1f} s "
                   f"(input generation and bf16 decoding included); decode oracle on (b,h) "
                   f"pairs of B=8 H=32 Lkv=65536 d=128: {pairs} pairs in {t_dec:.1f} s"),
        "decode_value": nbytes / t_dec / 1e9,
        "decode_unit": "GB/s",
        "cpu_model": cpu_info(),
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", default="all",
                    help="all, or a comma list of: c2c c2n c3 c3h c4 c4s1 c5 c5a q5 c6 c7 c8 b2c b3 b8 "
                         "(profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy per step (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_116_amd as fa
    import fa_inputs as fi

    torch.cuda.set_device(0)
    fa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    jobs = []   # (name, launch-fn, flops, bytes, kind)
    want = (lambda n: args.only == "all" or n in args.only.split(","))

    w2, w3, w4, w5 = (fi.WORKLOADS[i] for i in (2, 3, 4, 5))
    if want("c2c") or want("c2n"):
        log("generating B=2 H=32 N=2048 d=128 inputs")
        q2, k2, v2 = (up_bf16(fi.bf16_tensor(w2.wid, t, w2.B, w2.H, w2.N, w2.d)) for t in range(3))
        o2 = torch.empty_like(q2)
        l2 = torch.empty((w2.B, w2.H, w2.N), dtype=torch.float32, device=dev)
        for causal, tag in ((True, "c2c"), (False, "c2n")):
            if want(tag):
                jobs.append((tag, (lambda c=causal: fa.fa_fwd_ex(
                    q2, k2, v2, o2, l2, w2.B, w2.H, w2.N, w2.d, w2.scale, c, stream=stream)),
                    fwd_flops(w2, causal), fwd_bytes(w2), "fwd_bf16"))
    if want("c3"):
        log("generating B=1 H=16 N=16384 d=128 inputs")
        q3, k3, v3 = (up_bf16(fi.bf16_tensor(w3.wid, t, w3.B, w3.H, w3.N, w3.d)) for t in range(3))
        o3 = torch.empty_like(q3)
        l3 = torch.empty((w3.B, w3.H, w3.N), dtype=torch.float32, device=dev)
        jobs.append(("c3", lambda: fa.fa_fwd_ex(q3, k3, v3, o3, l3, w3.B, w3.H, w3.N, w3.d,
                                                w3.scale, True, stream=stream),
                     fwd_flops(w3, True), fwd_bytes(w3), "fwd_bf16"))
    if want("c3h"):
        log("generating B=1 H=16 N=16384 d=128 fp16 inputs")
        q3h, k3h, v3h = (torch.from_numpy(fi.f16_tensor(w3.wid, t, w3.B, w3.H, w3.N, w3.d).view(np.int16))
                         .view(torch.float16).to(dev) for t in range(3))
        o3h = torch.empty_like(q3h)
        l3h = torch.empty((w3.B, w3.H, w3.N), dtype=torch.float32, device=dev)
        jobs.append(("c3h", lambda: fa.fa_fwd_ex(q3h, k3h, v3h, o3h, l3h, w3.B, w3.H, w3.N, w3.d,
                                                 w3.scale, True, in_dtype=fa.FA_FP16,
                                                 out_dtype=fa.FA_FP16, stream=stream),
                     fwd_flops(w3, True), fwd_bytes(w3), "fwd_fp16"))
    if want("c4") or want("c4s1"):
        log("generating decode B=8 H=32 Lkv=65536 d=128 inputs (8 GiB)")
        q4 = up_bf16(fi.bf16_tensor(w4.wid, 0, w4.B, w4.H, 1, w4.d))
        k4 = up_bf16(fi.bf16_tensor(w4.wid, 1, w4.B, w4.H, w4.Lkv, w4.d))
        v4 = up_bf16(fi.bf16_tensor(w4.wid, 2, w4.B, w4.H, w4.Lkv, w4.d))
        o4 = torch.empty_like(q4)
        l4 = torch.empty((w4.B, w4.H), dtype=torch.float32, device=dev)
        wsb = fa.fa_decode_workspace_bytes(w4.B, w4.H, w4.d, w4.num_splits)
        ws4 = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
        if want("c4"):
            jobs.append(("c4", lambda: fa.fa_decode_splitkv_ex(
                q4, k4, v4, o4, l4, w4.B, w4.H, w4.Lkv, w4.d, w4.num_splits, w4.scale, ws4, wsb,
                stream=stream), 4.0 * w4.B * w4.H * w4.Lkv * w4.d, decode_bytes(w4), "decode"))
        if args.only == "all":
            # one sequence (the first batch row, a contiguous view) with 64 splits and with 1
            q1, k1, v1, o1, l1 = q4[:1], k4[:1], v4[:1], o4[:1], l4[:1]
            for tag, S1 in (("c4b1", w4.num_splits), ("c4b1s1", 1)):
                jobs.append((tag, (lambda S1=S1: fa.fa_decode_splitkv_ex(
                    q1, k1, v1, o1, l1, 1, w4.H, w4.Lkv, w4.d, S1, w4.scale, ws4, wsb,
                    stream=stream)), 4.0 * w4.H * w4.Lkv * w4.d, decode_bytes(w4) // w4.B,
                    "decode"))
        if want("c4s1"):
            jobs.append(("c4s1", lambda: fa.fa_decode_splitkv_ex(
                q4, k4, v4, o4, l4, w4.B, w4.H, w4.Lkv, w4.d, 1, w4.scale, ws4, wsb,
                stream=stream), 4.0 * w4.B * w4.H * w4.Lkv * w4.d, decode_bytes(w4), "decode"))
    for tag, wid in (("c6", 6), ("c7", 7)):
        if not want(tag):
            continue
        wg = fi.WORKLOADS[wid]
        log(f"generating grouped decode B={wg.B} Hq={wg.H} Hkv={wg.Hkv} Lkv={wg.Lkv} inputs")
        qg = up_bf16(fi.bf16_tensor(wg.wid, 0, wg.B, wg.H, 1, wg.d))
        kg = up_bf16(fi.bf16_tensor(wg.wid, 1, wg.B, wg.Hkv, wg.Lkv, wg.d))
        vg = up_bf16(fi.bf16_tensor(wg.wid, 2, wg.B, wg.Hkv, wg.Lkv, wg.d))
        og = torch.empty_like(qg)
        lg = torch.empty((wg.B, wg.H), dtype=torch.float32, device=dev)
        wsg_b = fa.fa_decode_workspace_bytes(wg.B, wg.H, wg.d, wg.num_splits)
        wsg = torch.empty(wsg_b // 4, dtype=torch.float32, device=dev)
        jobs.append((tag, (lambda w=wg, q=qg, k=kg, v=vg, o=og, l=lg, ws=wsg, nb=wsg_b:
                           fa.fa_decode_splitkv_gqa(q, k, v, o, l, w.B, w.H, w.Hkv, w.Lkv, w.d,
                                                    w.num_splits, w.scale, ws, nb,
                                                    stream=stream)),
                     4.0 * wg.B * wg.H * wg.Lkv * wg.d, decode_bytes(wg), "decode"))

    if want("q5"):
        log("generating bf16 inputs of the fp8 workload for the quantisation pass")
        xq = [up_bf16(fi.outlier_bf16_tensor(w5.wid, t, w5.B, w5.H, w5.N, w5.d))
              for t in (fi.Q_ID, fi.K_ID, fi.V_ID)]
        sg5 = torch.from_numpy(fi.rotation_signs(w5.wid, w5.d)).to(dev)
        cq5 = [torch.empty(x.shape, dtype=torch.uint8, device=dev) for x in xq]
        sq5 = [torch.empty((w5.B, w5.H, (w5.N + 63) // 64), dtype=torch.float32, device=dev)
               for _ in xq]

        def runq5():
            for i, x in enumerate(xq):
                fa.fa_fp8_quantize(x, sg5 if i < 2 else None, cq5[i], sq5[i], w5.B, w5.H, w5.N,
                                   w5.d, stream=stream,
                                   scale_rule=fa.FA_FP8_SCALE_POW2 if i == 2 else None)
        nq = xq[0].numel()
        jobs.append(("q5", runq5, 0.0, 3 * nq * 3 + 3 * sq5[0].numel() * 4, "quant"))

    wv = fi.VARLEN_PREFILL
    Hv, dv_ = wv["H"], wv["d"]
    pairs = varlen_pairs(wv["lq"], wv["lk"])   # FLOPs: 4*d per visible pair and head

    def packed(tensor, lens):
        out = np.empty((int(sum(lens)), Hv, dv_), dtype=np.uint16)
        r = 0
        for b, n in enumerate(lens):
            for h in range(Hv):
                out[r:r + n, h] = fi.bf16_slice(wv["wid"], tensor, b, h, n, dv_)
            r += n
        return up_bf16(out)

    if want("c8"):
        log(f"generating ragged prefill inputs ({len(wv['lq'])} sequences)")
        q8 = packed(fi.Q_ID, wv["lq"])
        k8, v8 = packed(fi.K_ID, wv["lk"]), packed(fi.V_ID, wv["lk"])
        o8 = torch.empty_like(q8)
        l8 = torch.empty((Hv, q8.shape[0]), dtype=torch.float32, device=dev)
        cq8 = torch.tensor(np.concatenate([[0], np.cumsum(wv["lq"])]), dtype=torch.int32, device=dev)
        ck8 = torch.tensor(np.concatenate([[0], np.cumsum(wv["lk"])]), dtype=torch.int32, device=dev)
        jobs.append(("c8", lambda: fa.fa_fwd_varlen(
            q8, k8, v8, o8, l8, cq8, ck8, len(wv["lq"]), Hv, max(wv["lq"]), max(wv["lk"]),
            q8.shape[0], k8.shape[0], dv_, dv_ ** -0.5, True, stream=stream),
            4.0 * dv_ * Hv * pairs, (2 * q8.numel() + k8.numel() + v8.numel()) * 2 + l8.numel() * 4,
            "fwd_bf16"))

    for tag, wid in (("b2c", 2), ("b3", 3)):
        if not want(tag):
            continue
        wb = fi.WORKLOADS[wid]
        log(f"generating backward B={wb.B} H={wb.H} N={wb.N} inputs")
        qb_, kb_, vb_, dob_ = (up_bf16(fi.bf16_tensor(wb.wid, t, wb.B, wb.H, wb.N, wb.d))
                               for t in (fi.Q_ID, fi.K_ID, fi.V_ID, fi.DO_ID))
        ob_ = torch.empty_like(qb_)
        lb_ = torch.empty((wb.B, wb.H, wb.N), dtype=torch.float32, device=dev)
        fa.fa_fwd_ex(qb_, kb_, vb_, ob_, lb_, wb.B, wb.H, wb.N, wb.d, wb.scale, True, stream=stream)
        grads = [torch.empty_like(qb_) for _ in range(3)]
        wsb_b = fa.fa_bwd_workspace_bytes(wb.B, wb.H, wb.N)
        wsb_ = torch.empty(wsb_b // 4, dtype=torch.float32, device=dev)
        jobs.append((tag, (lambda w=wb, q=qb_, k=kb_, v=vb_, o=ob_, do=dob_, l=lb_, gr=grads,
                           ws=wsb_, nb=wsb_b:
                           fa.fa_bwd(q, k, v, o, do, l, gr[0], gr[1], gr[2], w.B, w.H, w.N, w.d,
                                     w.scale, True, ws, nb, stream=stream)),
                     2.5 * fwd_flops(wb, True), 8 * wb.B * wb.H * wb.N * wb.d * 2, "bwd_bf16"))

    if want("b8"):
        log("generating ragged prefill backward inputs")
        qr, dor = packed(fi.Q_ID, wv["lq"]), packed(fi.DO_ID, wv["lq"])
        kr, vr = packed(fi.K_ID, wv["lk"]), packed(fi.V_ID, wv["lk"])
        tq, tk, nseq = qr.shape[0], kr.shape[0], len(wv["lq"])
        orr = torch.empty_like(qr)
        lr = torch.empty((Hv, tq), dtype=torch.float32, device=dev)
        cqr = torch.tensor(np.concatenate([[0], np.cumsum(wv["lq"])]), dtype=torch.int32, device=dev)
        ckr = torch.tensor(np.concatenate([[0], np.cumsum(wv["lk"])]), dtype=torch.int32, device=dev)
        mq, mk = max(wv["lq"]), max(wv["lk"])
        fa.fa_fwd_varlen(qr, kr, vr, orr, lr, cqr, ckr, nseq, Hv, mq, mk, tq, tk, dv_, dv_ ** -0.5,
                         True, stream=stream)
        gr_ = [torch.empty_like(qr), torch.empty_like(kr), torch.empty_like(vr)]
        wsr_b = fa.fa_bwd_workspace_bytes(1, Hv, tq)
        wsr = torch.empty(wsr_b // 4, dtype=torch.float32, device=dev)
        jobs.append(("b8", lambda: fa.fa_bwd_varlen(
            qr, kr, vr, orr, dor, lr, gr_[0], gr_[1], gr_[2], cqr, ckr, nseq, Hv, mq, mk, tq, tk,
            dv_, dv_ ** -0.5, True, wsr, wsr_b, stream=stream),
            2.5 * 4.0 * dv_ * Hv * pairs, (4 * qr.numel() + 4 * kr.numel()) * 2 + lr.numel() * 4,
            "bwd_bf16"))

    def fp8_built():
        t = torch.zeros((1, 1, 64, 128), dtype=torch.uint8, device=dev)
        sc = torch.ones((1, 1, 1), dtype=torch.float32, device=dev)
        ob = torch.empty((1, 1, 64, 128), dtype=torch.bfloat16, device=dev)
        lb = torch.empty((1, 1, 64), dtype=torch.float32, device=dev)
        try:
            fa.fa_fwd_ex(t, t, t, ob, lb, 1, 1, 64, 128, 0.1, True, in_dtype=fa.FA_FP8_E4M3,
                         q_scale=sc, k_scale=sc, v_scale=sc, stream=stream)
            return True
        except fa.FaError as e:
            if e.status != fa.FA_ERR_UNSUPPORTED:
                raise
            return False

    if (want("c5") or want("c5a")) and fp8_built():
        if True:
            x = {}
            for n, t in (("q", 0), ("k", 1), ("v", 2)):
                c, s = fi.fp8_tensor(w5.wid, t, w5.B, w5.H, w5.N, w5.d)
                x[n] = torch.from_numpy(c).to(dev)
                x[n + "s"] = torch.from_numpy(s).to(dev)
            o5 = torch.empty((w5.B, w5.H, w5.N, w5.d), dtype=torch.bfloat16, device=dev)
            l5 = torch.empty((w5.B, w5.H, w5.N), dtype=torch.float32, device=dev)

            def run5():
                fa.fa_fwd_ex(x["q"], x["k"], x["v"], o5, l5, w5.B, w5.H, w5.N, w5.d, w5.scale,
                             True, in_dtype=fa.FA_FP8_E4M3, q_scale=x["qs"], k_scale=x["ks"],
                             v_scale=x["vs"], stream=stream)
            run5()
            torch.cuda.synchronize()
            n5 = w5.B * w5.H * w5.N
            bytes5 = 3 * n5 * w5.d + 3 * n5 // 64 * 4 + n5 * w5.d * 2 + n5 * 4
            if want("c5"):
                jobs.append(("c5", run5, fwd_flops(w5, True), bytes5, "fwd_fp8"))
            if want("c5a"):
                # the same codes of Q and K, V quantised with max|x| / 448
                # scales, whose mantissas differ between blocks
                c, s = fi.fp8_tensor(w5.wid, fi.V_ID, w5.B, w5.H, w5.N, w5.d, pow2=False)
                x["va"] = torch.from_numpy(c).to(dev)
                x["vas"] = torch.from_numpy(s).to(dev)

                def run5a():
                    fa.fa_fwd_ex(x["q"], x["k"], x["va"], o5, l5, w5.B, w5.H, w5.N, w5.d,
                                 w5.scale, True, in_dtype=fa.FA_FP8_E4M3, q_scale=x["qs"],
                                 k_scale=x["ks"], v_scale=x["vas"], stream=stream)
                jobs.append(("c5a", run5a, fwd_flops(w5, True), bytes5, "fwd_fp8"))
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        jobs.append(("copy_1GiB", lambda: dst.copy_(src), 0.0, 2 * src.numel() * 4, "copy"))

    def step(evs=None):
        for i, (_, fn, _, _, _) in enumerate(jobs):
            if evs is not None:
                evs[i][0].record(stream)
            fn()
            if evs is not None:
                evs[i][1].record(stream)

    log(f"warmup {args.warmup} steps over {[j[0] for j in jobs]}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in jobs] for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for s in range(args.steps):
        step(evs[s])
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_all0.elapsed_time(t_all1) / args.steps

    # Back to back: K launches of one workload under one event pair, with no
    # other workload between them.  Inside a step the memory-bound decode
    # launches let the clock recover between the heavy ones, and every launch
    # there is bracketed by its own events, which leaves the GPU idle for some
    # microseconds between kernels: for the short workloads a sizeable part of
    # their in-step time.  C3's figure is the roofline's `steady`; the others
    # sit beside their workloads.
    steady_of = {}
    for sname in ("c3", "c2c", "c8", "b2c", "b3", "b8"):
        job = next((j for j in jobs if j[0] == sname), None)
        if job is None:
            continue
        n_steady = max(20, args.steps)
        for _ in range(3):
            job[1]()
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record(stream)
        for _ in range(n_steady):
            job[1]()
        s1.record(stream)
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / n_steady
        a = job[2] / (ms * 1e-3) / 1e12
        steady_of[sname] = {"launches": n_steady, "ms_mean": ms, "achieved": a, "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": a / PEAK_BF16_TFLOPS}
    steady = steady_of.get("c3")

    res = {}
    for i, (name, _, flops, nbytes, kind) in enumerate(jobs):
        ts = np.array([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)])
        res[name] = {"kind": kind, "ms_mean": float(ts.mean()), "ms_median": float(np.median(ts)),
                     "ms_min": float(ts.min()), "flops": flops, "bytes": nbytes}
        if kind.startswith("fwd") or kind.startswith("bwd"):
            res[name]["tflops"] = flops / (ts.mean() * 1e-3) / 1e12
            if name in steady_of:
                res[name]["steady"] = steady_of[name]
        else:
            res[name]["gbs"] = nbytes / (ts.mean() * 1e-3) / 1e9

    causal = [n for n in ("c2c", "c3") if n in res]
    value = None
    if causal:
        value = sum(res[n]["flops"] for n in causal) / (
            sum(res[n]["ms_mean"] for n in causal) * 1e-3) / 1e12
    dom = "c3" if "c3" in res else (causal[0] if causal else next(iter(res), None))
    roof = None
    if dom and res[dom]["kind"].startswith("fwd"):
        pk = PEAK_FP8_TFLOPS if res[dom]["kind"] == "fwd_fp8" else PEAK_BF16_TFLOPS
        a = res[dom]["tflops"]
        roof = {"kernel": f"fa_fwd_bf16_kernel ({dom})", "bound": "mfma", "achieved": a,
                "peak": pk, "unit": "TFLOP/s", "frac": a / pk, "traffic": traffic_bytes(dom),
                "traffic_source": traffic_source(dom),
                "algorithmic_bytes": res[dom]["bytes"]}
        if dom == "c3" and steady is not None:
            roof["steady"] = steady
    decode = None
    if "c4" in res:
        g = res["c4"]["gbs"]
        decode = {"value": g, "unit": "GB/s", "ms": res["c4"]["ms_mean"],
                  "one_split": ({"value": res["c4s1"]["gbs"], "ms": res["c4s1"]["ms_mean"],
                                 "speedup_of_64_splits": res["c4s1"]["ms_mean"] / res["c4"]["ms_mean"]}
                                if "c4s1" in res else None),
                  "one_sequence": ({"workload": "B=1 H=32 Lkv=65536 d=128",
                                    "value_64_splits": res["c4b1"]["gbs"],
                                    "value_1_split": res["c4b1s1"]["gbs"],
                                    "speedup_of_64_splits": res["c4b1s1"]["ms_mean"] / res["c4b1"]["ms_mean"]}
                                   if "c4b1" in res else None),
                  "roofline": {"kernel": "fa_decode_split_kernel + fa_decode_combine_kernel",
                               "bound": "hbm", "achieved": g, "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": g / PEAK_HBM_GBS,
                               "traffic": traffic_bytes("c4"),
                               "traffic_source": traffic_source("c4"),
                               "algorithmic_bytes": res["c4"]["bytes"]}}
    decode_gqa = {}
    for tag in ("c6", "c7"):
        if tag in res:
            g = res[tag]["gbs"]
            wg = fi.WORKLOADS[int(tag[1])]
            decode_gqa[tag] = {"workload": wg.name, "value": g, "unit": "GB/s",
                               "ms": res[tag]["ms_mean"],
                               "roofline": {"kernel": "fa_decode_gqa_split_kernel + "
                                                      "fa_decode_combine_kernel",
                                            "bound": "hbm", "achieved": g,
                                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                            "frac": g / PEAK_HBM_GBS,
                                            "traffic": traffic_bytes(tag),
                                            "traffic_source": traffic_source(tag),
                                            "algorithmic_bytes": res[tag]["bytes"]}}
    varlen = None
    if "c8" in res:
        a = res["c8"]["tflops"]
        varlen = {"workload": fi.VARLEN_PREFILL["name"], "value": a, "unit": "TFLOPS",
                  "ms": res["c8"]["ms_mean"],
                  "roofline": {"kernel": "fa_fwd_bf16_kernel (packed)", "bound": "mfma",
                               "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": a / PEAK_BF16_TFLOPS, "traffic": None,
                               "algorithmic_bytes": res["c8"]["bytes"],
                               "steady": steady_of.get("c8")}}
    fp16 = None
    if "c3h" in res:
        a = res["c3h"]["tflops"]
        fp16 = {"workload": w3.name + " causal, fp16 inputs and output", "value": a, "unit": "TFLOPS",
                "ms": res["c3h"]["ms_mean"],
                "roofline": {"kernel": "fa_fwd_bf16_kernel (fp16 instance)", "bound": "mfma",
                             "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": a / PEAK_BF16_TFLOPS, "traffic": None,
                             "algorithmic_bytes": res["c3h"]["bytes"]}}
    quant = None
    if "q5" in res:
        g = res["q5"]["gbs"]
        quant = {"workload": w5.name + " bf16 -> fp8, Q and K rotated", "value": g, "unit": "GB/s",
                 "ms": res["q5"]["ms_mean"],
                 "roofline": {"kernel": "fa_fp8_quant_kernel (x3)", "bound": "hbm",
                              "achieved": g, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": g / PEAK_HBM_GBS, "traffic": None,
                              "algorithmic_bytes": res["q5"]["bytes"]}}
    fp8 = None
    if "c5" in res:
        a = res["c5"]["tflops"]
        fp8 = {"workload": w5.name + " causal, V block scales powers of two", "value": a,
               "unit": "TFLOPS", "ms": res["c5"]["ms_mean"],
               "amax_v_scales": ({"value": res["c5a"]["tflops"], "ms": res["c5a"]["ms_mean"]}
                                 if "c5a" in res else None),
               "roofline": {"kernel": "fa_fwd_fp8_dl_kernel", "bound": "mfma", "achieved": a,
                            "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                            "frac": a / PEAK_FP8_TFLOPS, "traffic": traffic_bytes("c5"),
                            "traffic_source": traffic_source("c5"),
                            "algorithmic_bytes": res["c5"]["bytes"]}}
    backward = {}
    for tag in ("b2c", "b3", "b8"):
        if tag in res:
            a = res[tag]["tflops"]
            wname = (fi.VARLEN_PREFILL["name"] if tag == "b8"
                     else fi.WORKLOADS[2 if tag == "b2c" else 3].name) + " causal"
            backward[tag] = {"workload": wname,
                             "value": a, "unit": "TFLOPS", "ms": res[tag]["ms_mean"],
                             "roofline": {"kernel": "fa_bwd_pre_kernel + fa_bwd_dkdv_kernel + "
                                                    "fa_bwd_dq_kernel",
                                          "bound": "mfma", "achieved": a,
                                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                          "frac": a / PEAK_BF16_TFLOPS, "traffic": None,
                                          "algorithmic_bytes": res[tag]["bytes"],
                                          "steady": steady_of.get(tag)}}
    prop = torch.cuda.get_device_properties(0)
    clock_khz = None
    try:   # hipDeviceAttributeClockRate (kHz), from the HIP runtime torch already loaded
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        attr_clock_rate = 5   # hipDeviceAttributeClockRate
        if hip.hipDeviceGetAttribute(ctypes.byref(val), attr_clock_rate, 0) == 0:
            clock_khz = val.value
    except (OSError, AttributeError):
        pass
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 causal fwd B2H32N2048d128 + B1H16N16384d128 "
                               "(value); split-KV decode B8H32Lkv65536d128 S64 (decode); "
                               "grouped decode B8 Hq64/Hkv8 and Hq32/Hkv1 Lkv65536 (decode_gqa); "
                               "causal backward of B2H32N2048d128, B1H16N16384d128 and of the "
                               "ragged chunked prefill (backward); "
                               "ragged chunked prefill of 8 packed sequences H32d128 (varlen_prefill); "
                               "bf16->fp8 quantisation of the fp8 workload (fp8_quantize); "
                               "fp16 causal fwd B1H16N16384d128 (fp16_prefill); "
                               "fp8 causal fwd B4H16N8192d128 (fp8_forward)",
                   "only": args.only},
        "roofline": roof,
        "decode": decode,
        "decode_gqa": decode_gqa or None,
        "varlen_prefill": varlen,
        "fp8_quantize": quant,
        "fp16_prefill": fp16,
        "fp8_forward": fp8,
        "backward": backward or None,
        "workloads": res,
        "device": {"name": prop.name, "cus": prop.multi_processor_count,
                   "gcn_arch": getattr(prop, "gcnArchName", ""), "clock_khz": clock_khz},
        "wall_s_timed": wall,
    }
    log(f"timed {args.steps} steps in {wall:.2f} s")
    if not args.no_cpu_baseline and args.only == "all":
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
