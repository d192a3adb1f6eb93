#!/usr/bin/env python3
"""Benchmark of the HEAL hot path on one MI355X.

One step is one pass over every step of the path, each on its synthetic
workload (inputs resident in HBM before timing starts):

  smoke    the small configuration: a 16 x 256 x 256 compensated GEMM and the INT16
           quant of 16 x 256 values, two calls (launch-bound: reported as time per call)
  split    activation split of the two prefill GEMMs (fp32 -> packed fp16 hi/lo)
  prefill  compensated GEMM, M=2048 tokens, (K,N) = (4096,14336) and (14336,4096),
           weights split once beforehand (as deployed: weights are fixed)
  prefill_w16  the same GEMMs with the weights held as binary16 and packed
           once: the two-product form (2 of the 3 MFMA products)
  prefill_1p  the same GEMMs in the one-product mode (plain FP16, no
           compensation): the cost the compensation is measured against
  prefill_bf16x3  the same GEMMs in the BF16 three-way precision mode (six
           BF16 products; operands packed in that form beforehand)
  decode   16 compensated GEMMs of a Llama-3-8B-like layer: M = 1, 8, 32, 64
           x (K,N) in {(4096,4096), (4096,1024), (4096,14336), (14336,4096)},
           fp32 weights streamed from HBM (M-outer order, so consecutive calls
           touch different weights and the 256 MB MALL cannot serve repeats)
  decode_w16  the same 16 GEMMs with the weights held as binary16 (2 bytes each;
           the paper's two-product form for 16-bit weights)
  decode_packed  the same 16 GEMMs with the fp32 weights split once beforehand
           (heal_pack_w: row-normalized fp16 hi and residual, 4 bytes each)
  decode_w16_packed  the binary16 weights packed once (2 bytes each)
  decode_kshift  the same 16 GEMMs with massive activation channels beyond
           FP16's range (0.5% of channels x 2e5), rescaled per channel by powers
           of two in the split (a_kshift) against a once-rescaled weight
  qkv_proj the fused Q/K/V projection of a 2048-token prefill chunk (K = 4096,
           32 + 8 + 8 heads of 128: N = 6144), compensated, stored as INT16
           (Q codes, K/V codes written into a KV cache by slot)
  quant    INT16 quant of a Qwen3-8B-like layer's Q/K/V: 32 x 2048 tokens,
           32 + 8 + 8 heads of 128 (one [65536, 48, 128] launch)
  dequant  INT16 -> fp32 dequant of the same codes
  attn_prefill  causal self-attention of a 2048-token prompt over INT16 Q/K/V
           (32 query / 8 KV heads, D = 128), dual-FP16 expansion on MFMA
  attn     decode attention over the INT16 KV cache: batch 16, context 8192,
           32 query / 8 KV heads, D = 128

Before each row an untimed read of a 512 MiB buffer evicts the Infinity
Cache, so no row is served or slowed by what the previous one left there.

Output: one JSON line.  `value` is the metric's first half, FP32-accurate GEMM
TFLOP/s on the prefill workload (useful flops 2MNK over the time of split +
GEMM); `quant_GBps` is its second half.  `roofline` is the prefill GEMM kernel
against the 16-bit MFMA peak (3 fp16 products per useful multiply-add).
`cpu_baseline` is the CPU oracle timed on host cores on a bounded sample;
`calibration` holds the measured MFMA and HBM ceilings; `vendor_gemm` times the
vendor's GEMM (torch.matmul) on the same shapes as context (never part of `value`).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP32-accurate GEMM TFLOP/s (% of 16-bit MFMA peak); INT16 QKV quant GB/s"
PEAK_MFMA16_TFLOPS = 2516.6      # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_prefill_kernel_traffic.json")
PREFILL_SRC = os.path.join(ROOT, "error_compensated_gemm_heal_amd", "csrc", "gemm_prefill.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def build_workload(rows_sel):
    import torch
    import error_compensated_gemm_heal_amd as heal
    import heal_workloads as WL

    dev = "cuda:0"
    W = {}
    t0 = time.time()

    if any(r in rows_sel for r in ("split", "prefill", "prefill_w16", "prefill_1p", "prefill_bf16x3")):
        pre = []
        for i, (K, N) in enumerate(WL.PREFILL_KN):
            A, Wt = WL.prefill_gemm(WL.PREFILL_M, K, N, seed=3000 + i)
            Ad = torch.from_numpy(A).to(dev)
            Wd = torch.from_numpy(Wt).to(dev)
            Wp = heal.heal_pack_w(Wd)                                  # one-time weight split
            # the same weight as binary16 (an FP16 checkpoint), packed once
            Wp16 = heal.heal_pack_w(Wd.half()) if "prefill_w16" in rows_sel else None
            Ap = heal.heal_pack_w(Ad)                                  # output buffer of the split row
            x3 = "prefill_bf16x3" in rows_sel
            Wp3 = heal.heal_pack_w(Wd, bf16x3=True) if x3 else None
            Ap3 = heal.heal_pack_w(Ad, bf16x3=True) if x3 else None
            C = torch.empty((WL.PREFILL_M, N), dtype=torch.float32, device=dev)
            pre.append(dict(M=WL.PREFILL_M, K=K, N=N, A=Ad, Ap=Ap, Wp=Wp, Wp16=Wp16, Ap3=Ap3, Wp3=Wp3, C=C))
            del A, Wt, Wd
        W["prefill"] = pre
        log(f"[bench] prefill inputs ready ({time.time() - t0:.1f}s)")

    if rows_sel & {"decode", "decode_w16", "decode_packed", "decode_w16_packed"}:
        weights = {}
        acts = {}
        for i, (K, N) in enumerate(WL.LLAMA3_8B_DECODE_KN):
            A, Wt = WL.decode_gemm(64, K, N, seed=2000 + i)
            weights[(K, N)] = torch.from_numpy(Wt).to(dev)
            acts[(K, N)] = torch.from_numpy(A).to(dev)
        calls = []
        for M in WL.DECODE_M:
            for (K, N) in WL.LLAMA3_8B_DECODE_KN:
                Wd = weights[(K, N)]
                ws_bytes = heal.heal_gemm_f32c_workspace(M, N, K, 0)
                ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
                C = torch.empty((M, N), dtype=torch.float32, device=dev)
                calls.append(dict(M=M, K=K, N=N, A=acts[(K, N)][:M], W=Wd, C=C, ws=ws))
        W["decode"] = calls
        # the same layers with 16-bit weights (the paper's two-product form):
        # the fp32 weights rounded to binary16, as an FP16 checkpoint holds them
        calls16 = []
        w16 = {kn: w.half() for kn, w in weights.items()}
        for c in calls:
            calls16.append(dict(c, W=w16[(c["K"], c["N"])]))
        W["decode_w16"] = calls16
        if "decode_packed" in rows_sel:
            wp = {kn: heal.heal_pack_w(w) for kn, w in weights.items()}
            W["decode_packed"] = [dict(c, W=wp[(c["K"], c["N"])]) for c in calls]
        if "decode_w16_packed" in rows_sel:
            wp16 = {kn: heal.heal_pack_w(w) for kn, w in w16.items()}
            W["decode_w16_packed"] = [dict(c, W=wp16[(c["K"], c["N"])]) for c in calls]
        torch.cuda.synchronize()
        log(f"[bench] decode inputs ready ({time.time() - t0:.1f}s)")

    if "decode_kshift" in rows_sel:
        callsk = []
        shifted = {}
        for i, (K, N) in enumerate(WL.LLAMA3_8B_DECODE_KN):
            A, Wt = WL.overflow_gemm(64, K, N, seed=2100 + i)
            ks = torch.from_numpy(heal.heal_kshift_from_absmax(abs(A).max(axis=0))).to(dev)
            Ws = heal.heal_scale_k(torch.from_numpy(Wt).to(dev), -ks)      # one-time weight rescaling
            shifted[(K, N)] = (torch.from_numpy(A).to(dev), Ws, ks)
        for M in WL.DECODE_M:
            for (K, N) in WL.LLAMA3_8B_DECODE_KN:
                Ad, Ws, ks = shifted[(K, N)]
                ws = torch.empty(max(heal.heal_gemm_f32c_workspace(M, N, K, 0), 1), dtype=torch.uint8, device=dev)
                C = torch.empty((M, N), dtype=torch.float32, device=dev)
                callsk.append(dict(M=M, K=K, N=N, A=Ad[:M], W=Ws, ks=ks, C=C, ws=ws))
        W["decode_kshift"] = callsk
        log(f"[bench] rescaled decode inputs ready ({time.time() - t0:.1f}s)")

    if "qkv_proj" in rows_sel:
        M, K, Hq, Hkv, D = WL.PREFILL_M, 4096, 32, 8, 128
        A, Wt = WL.prefill_gemm(M, K, (Hq + 2 * Hkv) * D, seed=3500)
        Ad = torch.from_numpy(A).to(dev)
        Wp = heal.heal_pack_w(torch.from_numpy(Wt).to(dev))
        slots = torch.arange(M, dtype=torch.int64, device=dev)
        kc = torch.empty((M, Hkv, D), dtype=torch.int16, device=dev)
        vc = torch.empty_like(kc)
        ks = torch.empty((M, Hkv), dtype=torch.float32, device=dev)
        vs = torch.empty_like(ks)
        qc = torch.empty((M, Hq, D), dtype=torch.int16, device=dev)
        qs = torch.empty((M, Hq), dtype=torch.float32, device=dev)
        ws = torch.empty(heal.heal_qkv_proj_quant_workspace(M, K, Hq, Hkv, D, heal.HEAL_W_PACKED), dtype=torch.uint8,
                         device=dev)
        W["qkv_proj"] = dict(A=Ad, Wp=Wp, slots=slots, kc=kc, vc=vc, ks=ks, vs=vs, qc=qc, qs=qs, ws=ws, M=M, K=K,
                             Hq=Hq, Hkv=Hkv, D=D)
        del A, Wt
        log(f"[bench] qkv projection inputs ready ({time.time() - t0:.1f}s)")

    if "quant" in rows_sel or "dequant" in rows_sel:
        tokens = 32 * 2048
        Q, K_, V = WL.qkv(tokens, 32, 8, 128, seed=4000)
        X = torch.empty((tokens, 48, 128), dtype=torch.float32, device=dev)
        X[:, :32] = torch.from_numpy(Q).to(dev)
        X[:, 32:40] = torch.from_numpy(K_).to(dev)
        X[:, 40:] = torch.from_numpy(V).to(dev)
        del Q, K_, V
        codes = torch.empty(X.shape, dtype=torch.int16, device=dev)
        scales = torch.empty(X.shape[:-1], dtype=torch.float32, device=dev)
        deq = torch.empty(X.shape, dtype=torch.float32, device=dev)
        heal.heal_qkv_quant_i16(X, codes, scales)
        W["quant"] = dict(X=X, codes=codes, scales=scales, deq=deq, n=X.numel(), rows=X.numel() // 128)
        log(f"[bench] quant inputs ready ({time.time() - t0:.1f}s)")

    if "attn_prefill" in rows_sel:
        B, T, Hq, Hkv, D = 1, 2048, 32, 8, 128
        qf, kf, vf = WL.attention_prefill_fp32(B, T, Hq, Hkv, D, seed=5500)
        q, qs = heal.heal_qkv_quant_i16(torch.from_numpy(qf).to(dev))
        k, ks = heal.heal_qkv_quant_i16(torch.from_numpy(kf).to(dev))
        v, vs = heal.heal_qkv_quant_i16(torch.from_numpy(vf).to(dev))
        del qf, kf, vf
        out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
        W["attn_prefill"] = dict(args=(q, qs, k, ks, v, vs), out=out, B=B, T=T, Hq=Hq, D=D)
        log(f"[bench] prefill attention inputs ready ({time.time() - t0:.1f}s)")

    if "smoke" in rows_sel:
        A, Wt = WL.smoke_gemm()
        X = WL.smoke_quant()
        W["smoke"] = dict(A=torch.from_numpy(A).to(dev), W=torch.from_numpy(Wt).to(dev),
                          C=torch.empty((A.shape[0], Wt.shape[0]), dtype=torch.float32, device=dev),
                          X=torch.from_numpy(X).to(dev),
                          codes=torch.empty(X.shape, dtype=torch.int16, device=dev),
                          scales=torch.empty(X.shape[:-1], dtype=torch.float32, device=dev))

    if "attn" in rows_sel:
        B, T, Hq, Hkv, D = 16, 8192, 32, 8, 128
        qf, kf, vf = WL.attention_fp32(B, T, Hq, Hkv, D, seed=5000)
        q, qs = heal.heal_qkv_quant_i16(torch.from_numpy(qf).to(dev))
        k, ks = heal.heal_qkv_quant_i16(torch.from_numpy(kf).to(dev))
        v, vs = heal.heal_qkv_quant_i16(torch.from_numpy(vf).to(dev))
        del qf, kf, vf
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        ws = torch.empty(heal.heal_attn_decode_workspace(B, T, Hq, Hkv, D), dtype=torch.uint8, device=dev)
        W["attn"] = dict(args=(q, qs, k, ks, v, vs), out=out, ws=ws, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D)
        log(f"[bench] attention inputs ready ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    return W


def make_rows(W):
    """(name, launch function, work, unit) for each row present in W."""
    import error_compensated_gemm_heal_amd as heal
    rows = []
    if "prefill" in W:
        pre = W["prefill"]

        def run_split():
            for p in pre:
                heal.heal_pack_w(p["A"], out=p["Ap"])

        def run_prefill():
            for p in pre:
                heal.heal_gemm_f32c(p["Ap"], p["Wp"], C=p["C"])

        split_bytes = sum(p["M"] * p["K"] * 8 for p in pre)          # 4 B in + 2 x 2 B out per element
        useful = sum(2.0 * p["M"] * p["N"] * p["K"] for p in pre)
        rows.append(("split", run_split, split_bytes, "B"))
        rows.append(("prefill", run_prefill, useful, "flop"))
        if pre[0]["Wp16"] is not None:
            def run_prefill16():
                for p in pre:
                    heal.heal_gemm_f32c(p["Ap"], p["Wp16"], C=p["C"])

            rows.append(("prefill_w16", run_prefill16, useful, "flop"))

        def run_prefill1():
            for p in pre:
                heal.heal_gemm_f32c(p["Ap"], p["Wp"], C=p["C"], one_product=True)

        rows.append(("prefill_1p", run_prefill1, useful, "flop"))
        if pre[0]["Wp3"] is not None:
            def run_prefill3():
                for p in pre:
                    heal.heal_gemm_f32c(p["Ap3"], p["Wp3"], C=p["C"], bf16x3=True)

            rows.append(("prefill_bf16x3", run_prefill3, useful, "flop"))
    if "decode" in W:
        calls = W["decode"]

        def run_decode():
            for c in calls:
                heal.heal_gemm_f32c(c["A"], c["W"], C=c["C"], workspace=c["ws"])

        dbytes = sum(4 * (c["K"] * c["N"] + c["M"] * c["K"] + c["M"] * c["N"]) for c in calls)
        rows.append(("decode", run_decode, dbytes, "B"))
    if "decode_w16" in W:
        calls16 = W["decode_w16"]

        def run_decode16():
            for c in calls16:
                heal.heal_gemm_f32c(c["A"], c["W"], C=c["C"], workspace=c["ws"])

        d16bytes = sum(2 * c["K"] * c["N"] + 4 * (c["M"] * c["K"] + c["M"] * c["N"]) for c in calls16)
        rows.append(("decode_w16", run_decode16, d16bytes, "B"))
    for name, esz in (("decode_packed", 4), ("decode_w16_packed", 2)):
        if name in W:
            pcalls = W[name]

            def run_packed(pcalls=pcalls):
                for c in pcalls:
                    heal.heal_gemm_f32c(c["A"], c["W"], C=c["C"], workspace=c["ws"])

            # algorithmic bytes: the weight's elements at esz bytes, A and C in fp32
            pbytes = sum(esz * c["K"] * c["N"] + 4 * (c["M"] * c["K"] + c["M"] * c["N"]) for c in pcalls)
            rows.append((name, run_packed, pbytes, "B"))
    if "decode_kshift" in W:
        callsk = W["decode_kshift"]

        def run_decodek():
            for c in callsk:
                heal.heal_gemm_f32c(c["A"], c["W"], C=c["C"], workspace=c["ws"], a_kshift=c["ks"])

        dkbytes = sum(4 * (c["K"] * c["N"] + c["M"] * c["K"] + c["M"] * c["N"]) + c["K"] for c in callsk)
        rows.append(("decode_kshift", run_decodek, dkbytes, "B"))
    if "qkv_proj" in W:
        p = W["qkv_proj"]

        def run_qkv():
            heal.heal_qkv_proj_quant_i16(p["A"], p["Wp"], p["Hq"], p["Hkv"], p["D"], p["slots"], p["kc"], p["ks"],
                                         p["vc"], p["vs"], q_codes=p["qc"], q_scales=p["qs"], workspace=p["ws"])

        rows.append(("qkv_proj", run_qkv, 2.0 * p["M"] * p["K"] * (p["Hq"] + 2 * p["Hkv"]) * p["D"], "flop"))
    if "quant" in W:
        q = W["quant"]
        qbytes = q["n"] * (4 + 2) + q["rows"] * 4
        rows.append(("quant", lambda: heal.heal_qkv_quant_i16(q["X"], q["codes"], q["scales"]), qbytes, "B"))
        rows.append(("dequant", lambda: heal.heal_kv_dequant_i16(q["codes"], q["scales"], "f32", out=q["deq"]),
                     qbytes, "B"))
    if "attn_prefill" in W:
        a = W["attn_prefill"]
        # useful flops: two products of D multiply-adds per (query, visible key, head)
        pairs = a["B"] * a["T"] * (a["T"] + 1) // 2
        rows.append(("attn_prefill", lambda a=a: heal.heal_attn_prefill_i16(*a["args"], out=a["out"]),
                     4.0 * a["D"] * a["Hq"] * pairs, "flop"))
    if "smoke" in W:
        sm = W["smoke"]

        def run_smoke():
            heal.heal_gemm_f32c(sm["A"], sm["W"], C=sm["C"])
            heal.heal_qkv_quant_i16(sm["X"], sm["codes"], sm["scales"])

        rows.append(("smoke", run_smoke, 2, "call"))   # two calls: latency only
    if "attn" in W:
        a = W["attn"]
        B, T, Hq, Hkv, D = a["B"], a["T"], a["Hq"], a["Hkv"], a["D"]
        abytes = 2 * B * T * Hkv * D * 2 + 2 * B * T * Hkv * 4 + B * Hq * D * 2 + B * Hq * 4 + B * Hq * D * 4
        rows.append(("attn", lambda a=a: heal.heal_attn_decode_i16(*a["args"], out=a["out"], workspace=a["ws"]),
                     abytes, "B"))
    return rows


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _gemm_rows_rate(fn, seconds, nth):
    """Rows of the two prefill shapes through an oracle GEMM (row-parallel), until
    about `seconds` of CPU work: (flops per second, sample text)."""
    import numpy as np
    import heal_workloads as WL
    flops, total, parts = 0.0, 0.0, []
    for K, N in WL.PREFILL_KN:
        left = seconds - total
        if left <= 0.25 * seconds / len(WL.PREFILL_KN):
            break
        A, Wt = WL.prefill_gemm(WL.PREFILL_M, K, N, seed=3000)
        probe = np.arange(nth, dtype=np.int64)
        t0 = time.perf_counter()
        fn(A, Wt, probe)
        dt = time.perf_counter() - t0
        # dt covers nth rows: scale the sample to its share of the time left (whole multiples of nth)
        share = left if K == WL.PREFILL_KN[-1][0] else left / 2
        nrows = int(max(nth, min(WL.PREFILL_M, round(share / max(dt, 1e-6)) * nth)))
        rows = np.arange(nrows, dtype=np.int64)
        t0 = time.perf_counter()
        fn(A, Wt, rows)
        dt = time.perf_counter() - t0
        flops += 2.0 * nrows * N * K
        total += dt
        parts.append(f"{nrows} of {WL.PREFILL_M} rows of K={K}, N={N}")
        del A, Wt
    return flops / total, "; ".join(parts) + f" ({total:.1f} s)"


def _quant_rate(seconds):
    """The oracle's INT16 quant and dequant on a token slice of the Q/K/V layer
    (48 heads of 128 per token): (quant B/s, dequant B/s, sample text); bytes
    counted as the GPU rows count them (4 in + 2 out per element + 4 per row)."""
    import heal_workloads as WL
    import oracle
    tokens = 4096
    Q, K_, V = WL.qkv(tokens, 32, 8, 128, seed=4000)
    import numpy as np
    X = np.concatenate([Q, K_, V], axis=1)
    del Q, K_, V
    n, rows = X.size, X.size // 128
    nbytes = n * 6 + rows * 4
    out = []
    for fn in (lambda: oracle.quant_i16(X), None):
        if fn is None:
            codes, scales = oracle.quant_i16(X)
            fn = (lambda c=codes, s_=scales: oracle.dequant_f32(c, s_))
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds / 2:
                break
        out.append(nbytes * reps / dt)
    return out[0], out[1], f"{tokens} tokens x 48 heads x 128 ({n / 1e6:.1f} M elements)"


def _attn_rate(seconds):
    """The oracle's binary64 decode attention on a batch slice of the decode-attention
    workload (T = 8192, 32 / 8 heads of 128): (B/s, sample text), bytes counted as the
    GPU row counts them (codes and scales of K and V, q in, o out)."""
    import heal_workloads as WL
    import oracle
    B, T, Hq, Hkv, D = 2, 8192, 32, 8, 128
    qf, kf, vf = WL.attention_fp32(B, T, Hq, Hkv, D, seed=5000)
    ins = oracle.quant_i16(qf) + oracle.quant_i16(kf) + oracle.quant_i16(vf)
    del qf, kf, vf
    nbytes = 2 * B * T * Hkv * D * 2 + 2 * B * T * Hkv * 4 + B * Hq * D * 2 + B * Hq * 4 + B * Hq * D * 4
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attn_decode_f64(*ins)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return nbytes * reps / dt, f"{B} of 16 sequences of T={T}, {Hq}/{Hkv} heads ({reps} passes, {dt:.1f} s)"


def cpu_baseline(seconds):
    """The oracle, as it stands, on bounded samples of the benchmark's workloads, on
    all host threads and on one: `value` is its FP64-accumulated GEMM on row samples
    of the two prefill shapes (the metric's first half, the GPU `value`'s unit);
    `parts` adds the naive FP32 GEMM, the INT16 quant and dequant (the metric's
    second half, GB/s), the binary64 decode attention (GB/s of the cache it
    reads), and the one-thread rates."""
    import oracle
    nth = oracle.num_threads()
    share = seconds / 7
    parts = {}
    f64, s64 = _gemm_rows_rate(oracle.gemm_f64_rows, 2 * share, nth)
    f32, s32 = _gemm_rows_rate(oracle.gemm_f32_naive_rows, share, nth)
    q, dq, sq = _quant_rate(share)
    at, sat = _attn_rate(share)
    parts["gemm_f64_TFLOPs"] = f64 / 1e12
    parts["gemm_f32_naive_TFLOPs"] = f32 / 1e12
    parts["quant_GBps"] = q / 1e9
    parts["dequant_GBps"] = dq / 1e9
    parts["attn_decode_f64_GBps"] = at / 1e9
    oracle.set_num_threads(1)
    try:
        f64_1, s64_1 = _gemm_rows_rate(oracle.gemm_f64_rows, share, 1)
        q1, dq1, _ = _quant_rate(share)
    finally:
        oracle.set_num_threads(nth)
    parts["gemm_f64_TFLOPs_1thread"] = f64_1 / 1e12
    parts["quant_GBps_1thread"] = q1 / 1e9
    parts["dequant_GBps_1thread"] = dq1 / 1e9
    return {"value": f64 / 1e12, "unit": "TFLOP/s", "cores": nth, "kind": "oracle",
            "cpu_model": _cpu_model(), "parts": parts,
            "sample": f"the oracle on {nth} threads and on 1: FP64 GEMM on {s64}; naive FP32 GEMM on {s32}; "
                      f"quant/dequant of {sq}; decode attention on {sat}; one thread: FP64 GEMM on {s64_1}"}


def calibrate(torch, heal):
    """Measured ceilings: the register-only 16-bit MFMA rate in the prefill GEMM's
    launch shape (one workgroup of 4 waves per CU), the HBM read rate of a
    streaming kernel (2 GiB, best of five grid sizes), and a device copy (1 GiB
    each way), all timed with HIP events on the current stream (best of 5 after
    a warm-up)."""
    def best(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda:0")
    iters = 20000
    _, mflop = heal.heal_calib_mfma_f16(iters, 256, out)
    t_mfma = best(lambda: heal.heal_calib_mfma_f16(iters, 256, out))
    buf = torch.ones(1 << 29, dtype=torch.float32, device="cuda:0")      # 2 GiB
    out = torch.empty(16384 * 256, dtype=torch.float32, device="cuda:0")
    reads = {wg: best(lambda wg=wg: heal.heal_calib_read(buf, wg, out)) for wg in (1024, 2048, 4096, 8192, 16384)}
    wg_read = min(reads, key=reads.get)
    t_read = reads[wg_read]
    src = buf[: 1 << 28]
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src))
    res = {"mfma_f16_TFLOPs": mflop / t_mfma / 1e12, "hbm_read_GBps": buf.numel() * 4 / t_read / 1e9,
           "copy_GBps": 2 * src.numel() * 4 / t_copy / 1e9,
           "note": "register-only v_mfma_f32_32x32x16_f16 loop, 256 workgroups x 4 waves x 16 accumulators; "
                   f"2 GiB streaming read (8 non-temporal 16-byte loads in flight per thread; the best grid, "
                   f"{wg_read} workgroups of 256); 1 GiB device copy (read + write bytes)"}
    del buf, dst
    return res


def vendor_gemms(torch, reps=20):
    """The vendor's GEMM (torch.matmul, i.e. hipBLASLt/rocBLAS) on the same shapes,
    as context beside the calibration: plain fp16 and bf16 (one 16-bit product,
    no compensation: the library's own 16-bit rate on these shapes) and plain
    FP32 (the FP32 pipeline the pages compare HEAL with; TF32-style reduced
    precision switched off) on the two prefill shapes; FP32 and fp16 on the 16
    decode calls in bench order.  C = A.W^T with W in nn.Linear's [N, K]
    layout, random normal operands; each timed with HIP events on the current
    stream after the same untimed cache flush as the rows (mean of `reps`).
    Nothing here is part of the HEAL path or of `value`."""
    import heal_workloads as WL
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.backends.cuda.matmul.allow_fp16_reduced_precision_reduction = False
    torch.backends.cuda.matmul.allow_bf16_reduced_precision_reduction = False
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    flush = torch.ones(512 << 18, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        tot = 0.0
        for _ in range(reps):
            torch.amax(flush, dim=0, out=flush_out)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1) * 1e-3
        return tot / reps

    out = {}
    flop = sum(2.0 * WL.PREFILL_M * K * N for K, N in WL.PREFILL_KN)
    for name, dt in (("fp16", torch.float16), ("bf16", torch.bfloat16), ("fp32", torch.float32)):
        ops = [(torch.randn(WL.PREFILL_M, K, device=dev, generator=gen).to(dt),
                torch.randn(N, K, device=dev, generator=gen).to(dt)) for K, N in WL.PREFILL_KN]
        t = timed(lambda ops=ops: [torch.matmul(a, w.t()) for a, w in ops])
        out[f"prefill_{name}"] = {"ms": t * 1e3, "TFLOPs": flop / t / 1e12}
        del ops
    for name, dt, esz in (("fp32", torch.float32, 4), ("fp16", torch.float16, 2)):
        ws = {(K, N): torch.randn(N, K, device=dev, generator=gen).to(dt) for K, N in WL.LLAMA3_8B_DECODE_KN}
        calls = [(torch.randn(M, K, device=dev, generator=gen).to(dt), ws[(K, N)])
                 for M in WL.DECODE_M for K, N in WL.LLAMA3_8B_DECODE_KN]
        nbytes = sum(esz * (w.numel() + a.numel() + a.shape[0] * w.shape[0]) for a, w in calls)
        t = timed(lambda calls=calls: [torch.matmul(a, w.t()) for a, w in calls])
        out[f"decode_{name}"] = {"ms": t * 1e3, "GBps": nbytes / t / 1e9}
        del ws, calls
    del flush
    out["note"] = ("torch.matmul (vendor BLAS), not HEAL: prefill = both M=2048 shapes, useful TFLOP/s; "
                   "decode = the 16 calls, GB/s of weights + activations + outputs in that dtype")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rows", default="smoke,split,prefill,prefill_w16,prefill_1p,prefill_bf16x3,decode,decode_w16,"
                                      "decode_packed,decode_w16_packed,decode_kshift,"
                                      "qkv_proj,quant,dequant,attn_prefill,attn",
                    help="comma-separated subset of rows to run (profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vendor", action="store_true", help="skip the vendor-GEMM context timings")
    ap.add_argument("--cpu-seconds", type=float, default=24.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure the MFMA and HBM ceilings (calibration kernels) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}, WORLD_SIZE {world}): the HEAL hot "
              "path here is a single-GPU library; how it would shard is described in DESIGN.md.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import error_compensated_gemm_heal_amd as heal
    heal.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}))
        return

    if args.calibrate:
        print(json.dumps(calibrate(torch, heal)))
        return

    sel = set(args.rows.split(","))
    W = build_workload(sel)
    rows = [r for r in make_rows(W) if r[0] in sel]

    # Before each row, an untimed read of a 512 MiB buffer (twice the
    # 256 MB Infinity Cache) evicts whatever the previous row left there: the
    # row's own inputs (so weights are not served from the cache) and the
    # previous row's dirty lines (so their write-back to HBM does not land in
    # this row's time).
    flush = torch.ones(512 << 18, dtype=torch.float32, device="cuda:0")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda:0")

    def step(events=None):
        for i, (name, fn, _, _) in enumerate(rows):
            torch.amax(flush, dim=0, out=flush_out)
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in rows]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / max(args.steps, 1) * 1e3

    per_row = {}
    for i, (name, _, work, unit) in enumerate(rows):
        ts = sorted(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps))
        ms = sum(ts) / max(args.steps, 1)       # mean: the rates, `value` and the roofline use it
        med = ts[len(ts) // 2] if ts else 0.0
        rate = work / (ms * 1e-3)
        if unit == "flop":
            per_row[name] = {"ms": ms, "ms_median": med, "TFLOPs": rate / 1e12}
        elif unit == "call":
            per_row[name] = {"ms": ms, "ms_median": med, "us_per_call": ms * 1e3 / work}
        else:
            per_row[name] = {"ms": ms, "ms_median": med, "GBps": rate / 1e9, "hbm_frac": rate / 1e9 / PEAK_HBM_GBPS}

    res = {"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp32 in/out; fp16 hi/lo MFMA products, fp32 accumulate; int16 codes",
           "data": "synthetic (seeded; model-shaped, see heal_workloads.py)"}
    cfg = {"workload": "HEAL hot path step: split + prefill GEMM (M=2048; K,N = 4096,14336 and 14336,4096; "
                       "fp32 weights; also fp16 weights in the two-product form, the one-product mode and the "
                       "BF16 three-way mode), "
                       "16 decode GEMMs (M=1,8,32,64 x Llama-3-8B q/o, k/v, gate/up, down; fp32 and fp16 weights, "
                       "streamed or packed once, and fp32 with per-channel rescaled massive activations), "
                       "fused Q/K/V projection to INT16 (2048 tokens, K=4096, N=6144), "
                       "INT16 quant + dequant "
                       "(32x2048 tokens, 32+8+8 heads x 128), INT16 prefill attention (T=2048, 32/8 heads), "
                       "INT16 decode attention (B=16, T=8192, 32/8 heads)",
           "rows": sorted(sel)}
    res["config"] = cfg
    if "prefill" in per_row:
        pre = W["prefill"]
        useful = sum(2.0 * p["M"] * p["N"] * p["K"] for p in pre)
        t_gemm = per_row["prefill"]["ms"] * 1e-3
        t_split = per_row["split"]["ms"] * 1e-3 if "split" in per_row else 0.0
        res["value"] = useful / (t_gemm + t_split) / 1e12
        launches = len(pre)
        mfma_flops_per_launch = 3.0 * useful / launches
        avg_launch = t_gemm / launches
        achieved = mfma_flops_per_launch / avg_launch / 1e12
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            tr = json.load(open(TRAFFIC_FILE))
            if tr.get("source_sha") == source_sha(PREFILL_SRC):
                traffic = tr.get("bytes_per_launch")
        res["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA16_TFLOPS, "unit": "TFLOP/s",
                           "frac": achieved / PEAK_MFMA16_TFLOPS, "traffic": traffic,
                           "kernel": "gemm_prefill_kernel", "per_launch_mfma_flop": mfma_flops_per_launch,
                           "avg_launch_ms": avg_launch * 1e3}
        res["prefill_gemm_only_TFLOPs"] = useful / t_gemm / 1e12
    else:
        res["value"] = None
    if "quant" in per_row:
        res["quant_GBps"] = per_row["quant"]["GBps"]
    # measured ceilings, after the timed steps: the fractions beside the spec ones
    cal = calibrate(torch, heal)
    res["calibration"] = cal
    if "roofline" in res:
        res["roofline"]["peak_measured"] = cal["mfma_f16_TFLOPs"]
        res["roofline"]["frac_measured"] = res["roofline"]["achieved"] / cal["mfma_f16_TFLOPs"]
    for name, r in per_row.items():
        if "GBps" in r:
            r["hbm_frac_measured"] = r["GBps"] / cal["hbm_read_GBps"]
    res["rows"] = per_row
    if not args.no_vendor:
        res["vendor_gemm"] = vendor_gemms(torch)

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
