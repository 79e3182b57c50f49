#!/usr/bin/env python3
"""Bench of the online KV-cache compression hot path on one MI355X.

One step = one pass of the whole path over one layer's worth of synthetic
input: quantize the K and V vectors of every kv head into the packed caches
(one tq_quantize_kv call: two equal launches of the quantize kernel), then one
decode-attention step (one query per query head) over a packed cache.
Default workload: Llama-3.1-8B-shaped layer, batch 1, 32K context, 8 kv heads,
32 query heads, d = 128, bf16 K/V, b = 4 (3 index bits + 1 sign bit).

Inputs and caches rotate through enough copies (>= 1 GiB) that neither the
step's input nor the cache the decode reads is still in the 256 MB
last-level cache: the decode reads a cache written several steps earlier.

Prints one JSON line.  value = packed-KV decode-attention GB/s (algorithmic
packed bytes read per decode / decode time); the quantize rate (token
positions per second, each position = K and V of every kv head) is reported
beside it.  Kernel durations come from HIP events on the launch stream.

Other modes: --workload 5 (d = 256, 64K tokens x 2); --search (inner-product
search over a 2^23-key packed index, tq_score_keys); --calibrate-copy and
--traffic (HBM counter calibration and the traffic table, for the profiles).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, spec
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix, spec
METRIC = "packed-KV decode-attention GB/s (% HBM peak); KV quantize tokens/s"
SEARCH_WORKLOAD = "search-d128-8m-b4"


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_online_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def packed_record_bytes(d, m, bits_mse, sketch):
    """Bytes of one packed vector in the cache layout: b' index planes of d bits,
    a sign plane of m bits when the sketch is kept, two fp16 scales."""
    return bits_mse * d // 8 + (m // 8 if sketch else 0) + 4


def traffic_for(prefixes, workload):
    """HBM bytes per call (sum over the call's kernels, each by name prefix) from
    the committed rocprofv3 counter runs, if they were taken on this source and
    this workload."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash() or workload not in t.get("workloads", {}):
        return None
    ks = t["workloads"][workload].get("kernels", {})
    total = 0.0
    for pre, n in prefixes:
        hit = [v["bytes"] for k, v in ks.items() if k.startswith(pre)]
        if not hit:
            return None
        total += n * hit[0]
    return total


def copy_calibration(nbytes=1 << 30, reps=5):
    """Plain device-to-device copies of a known size, for scaling HBM byte counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, workload):
    """profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of
    this bench and of copy_calibration (counters in KiB per dispatch).  Each
    counter is scaled by bytes / counter of the plain copy: FETCH against the
    bytes the copy reads, WRITE against the bytes it writes."""
    import csv
    import re

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") != counter:
                continue
            k = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].split("::")[-1]
            vals.setdefault(k, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sorted(v)[len(v) // 2] for k, v in vals.items()}

    cf = per_kernel(copy_fetch_csv, "FETCH_SIZE")
    cw = per_kernel(copy_write_csv, "WRITE_SIZE")
    ck = max(cf, key=cf.get)                      # the copy is the largest dispatch
    f_scale, w_scale = copy_bytes / cf[ck], copy_bytes / cw[ck]
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    kernels = {}
    for k in fetch:
        if k in write and k.startswith(("quantize", "decode")):
            kernels[k] = {"fetch_bytes": fetch[k] * f_scale, "write_bytes": write[k] * w_scale,
                          "bytes": fetch[k] * f_scale + write[k] * w_scale}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    workloads = {}
    if os.path.exists(path):   # keep the other workloads' entries taken on the same sources
        try:
            old = json.load(open(path))
            if old.get("source_hash") == source_hash():
                workloads = old.get("workloads", {})
        except (OSError, ValueError):
            pass
    workloads[workload] = {"kernels": kernels}
    out = {"source_hash": source_hash(), "copy_kernel": ck, "copy_bytes": copy_bytes,
           "fetch_scale": f_scale, "write_scale": w_scale, "workloads": workloads}
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def quality_vs_unquantized(w, Kn, Vn, Qn, out):
    """The decode output against softmax attention over the unquantized K, V and q
    (float64 on the host, scale 1/sqrt(d)): relative L2 error and cosine per query
    head.  Reported, not pass/fail."""
    import workloads as W
    G = w.n_q_heads // w.n_kv_heads
    scale = 1.0 / math.sqrt(w.d)
    rel, cos = [], []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            k = W.to_f64(Kn[b, h], w.dtype)
            v = W.to_f64(Vn[b, h], w.dtype)
            q = W.to_f64(Qn[b, h * G:(h + 1) * G], w.dtype)
            sc = (q @ k.T) * scale
            sc -= sc.max(axis=1, keepdims=True)
            pr = np.exp(sc)
            ref = (pr @ v) / pr.sum(axis=1, keepdims=True)
            got = out[b, h * G:(h + 1) * G].astype(np.float64)
            rel.extend(np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1))
            cos.extend(np.sum(got * ref, axis=1) / (np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1)))
    return {"reference": "softmax attention over the unquantized K, V, q (float64, host)",
            "query_heads": len(rel), "rel_l2_mean": float(np.mean(rel)), "rel_l2_max": float(np.max(rel)),
            "cosine_min": float(np.min(cos))}


def quality_report(w, s, rot, proj, K0, V0, Q, st_d, ln_d, max_len, cap, dst, Kn, Vn, Qn, out):
    """quality_vs_unquantized for the workload's preset and, beside it, for the
    same index bits with the residual sketch off (MSE-only): the sketch makes the
    inner products unbiased at the price of variance, which the softmax
    amplifies where the scores are spread (outlier channels)."""
    from kv_cache_online_amd.session import TQSession
    rep = {"preset": quality_vs_unquantized(w, Kn, Vn, Qn, out)}
    if w.sketch:
        s2 = TQSession(w.d, w.n_kv_heads, w.n_q_heads, rot, proj, k_bits=w.bits_mse, v_bits=w.bits_mse,
                       k_sketch=0, v_sketch=0)
        kc, vc = s2.new_caches(cap)
        s2.quantize(K0, V0, dst, kc, vc)
        out2 = s2.decode(Q, st_d, ln_d, max_len, kc, vc)
        rep[f"mse_only_{w.bits_mse}bit"] = quality_vs_unquantized(w, Kn, Vn, Qn, out2.cpu().numpy())
    return rep


def oracle_threads():
    """Threads the oracle's NumPy/BLAS calls use (the BLAS pool, else the CPUs this process may run on)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 0) for i in blas] + [1])
    except Exception:
        pass
    return cores


def cpu_baseline(w, rot, proj, seconds):
    """Time the oracle (float64 NumPy) on a bounded sample of the same workload."""
    import oracle as O
    import workloads as W
    cores = oracle_threads()
    cb = O.build_codebook(w.bits_mse, 1 / math.sqrt(w.d))
    # decode: one kv head over the full context (oracle-packed cache), G query heads
    T = w.seq_len
    K = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=T), w.dtype)
    V = W.to_f64(W.kv_chunk(w, 1, 0, 0, n_tokens=T), w.dtype)
    qk = O.quantize(K, rot, proj, cb)
    qv = O.quantize(V, rot, proj, cb)
    kp = O.pack_token_major(qk["idx"], qk["sgn"], qk["nu_bits"], qk["rho_bits"], w.bits_mse)
    vp = O.pack_block32(qv["idx"], qv["sgn"], qv["nu_bits"], qv["rho_bits"], w.bits_mse)
    q = W.to_f64(W.queries(w)[0, :w.group], w.dtype)
    f16 = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    reps, t_dec = 0, 0.0
    t_start = time.perf_counter()
    while reps < 1 or (time.perf_counter() - t_start < seconds / 2 and reps < 40):
        t0 = time.perf_counter()
        i, s, nb, rb = O.unpack_token_major(*kp, w.bits_mse)
        kh = O.dequantize(i, s, f16(nb), f16(rb), rot, proj, cb)
        i, s, nb, rb = O.unpack_block32(*vp, w.bits_mse)
        vh = O.dequantize(i, s, f16(nb), f16(rb), rot, proj, cb)
        O.attention(q, kh[None], vh[None])
        t_dec += time.perf_counter() - t0
        reps += 1
    rec = O.record_bytes(w.d, w.m, w.bits_mse, w.sketch)
    dec_gbs = reps * T * 2 * rec / t_dec / 1e9
    # quantize: token positions (K and V of every kv head) on a sample of vectors
    n_pos = 49152
    X = W.to_f64(W.kv_chunk(w, 0, 0, 1, n_tokens=n_pos * w.n_kv_heads * 2), w.dtype)
    t0 = time.perf_counter()
    qq = O.quantize(X, rot, proj, cb)
    O.pack_token_major(qq["idx"], qq["sgn"], qq["nu_bits"], qq["rho_bits"], w.bits_mse)
    tq = time.perf_counter() - t0
    return {"value": dec_gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"decode: unpack + float64 dequantize + attention over one kv head x {T} tokens "
                       f"(K and V), {w.group} query heads, {reps} reps, {t_dec:.1f} s; quantize: "
                       f"{n_pos} token positions ({n_pos * w.n_kv_heads * 2} vectors), {tq:.1f} s"),
            "quantize_tokens_per_s": n_pos / tq}


def search_cpu_baseline(w, rot, proj, Qn, n_q, seconds):
    """Time the oracle's search scores (unpack + float64 dequantize + q @ k^T) on a
    bounded sample of keys."""
    import oracle as O
    import workloads as W
    cores = oracle_threads()
    cb = O.build_codebook(w.bits_mse, 1 / math.sqrt(w.d))
    n = 65536
    K = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=n), w.dtype)
    qk = O.quantize(K, rot, proj, cb)
    kp = O.pack_token_major(qk["idx"], qk["sgn"], qk["nu_bits"], qk["rho_bits"], w.bits_mse)
    q = W.to_f64(Qn[0, :n_q], w.dtype)
    f16 = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    reps, t = 0, 0.0
    while reps < 1 or (t < seconds and reps < 40):
        t0 = time.perf_counter()
        i, sg, nb, rb = O.unpack_token_major(*kp, w.bits_mse)
        O.score_keys(q, i, sg, f16(nb), f16(rb), rot, proj, cb)
        t += time.perf_counter() - t0
        reps += 1
    rec = O.record_bytes(w.d, w.m, w.bits_mse, w.sketch)
    return {"value": reps * n * (rec + 4 * n_q) / t / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} packed keys x {n_q} queries: unpack + float64 dequantize + scores, {reps} reps, "
                      f"{t:.1f} s"}


def bench_search(args):
    """Inner-product search over packed keys (tq_score_keys): a 2^23-vector key
    index (the keys of the default workload, repeated), scored by n_q queries per
    call for each n_q of --search-nq (default 8 and 32).  Algorithmic bytes per call: the packed keys read once plus
    the fp32 scores written."""
    import torch
    import workloads as W
    from kv_cache_online_amd.session import TQSession

    w = W.WORKLOADS[2]
    rot, proj = W.rotation(w.d, w.wid), W.sketch(w.m, w.d, w.wid)
    s = TQSession(w.d, 1, 8, rot, proj, k_bits=w.bits_mse, v_bits=w.bits_mse, k_sketch=w.sketch,
                  v_sketch=w.sketch)
    Kn, Qn = W.kv_batch(w, 0), W.queries(w)
    base = w.n_kv_heads * w.seq_len                       # 2^18 key vectors
    N = 1 << 23
    K = torch.from_numpy(np.ascontiguousarray(Kn)).cuda().view(torch.bfloat16).reshape(1, 1, base, w.d)
    kc = s.new_caches(N)[0]
    for c in range(N // base):
        s.quantize(K, None, torch.tensor([c * base], dtype=torch.int64, device="cuda"), kc, None)
    del K
    stream = torch.cuda.current_stream()
    rec = packed_record_bytes(w.d, w.m, w.bits_mse, w.sketch)
    Q = torch.from_numpy(np.ascontiguousarray(Qn)).cuda().view(torch.bfloat16).reshape(-1, w.d)
    runs = []
    for n_q in args.search_nq:
        q = Q[:n_q].contiguous()
        out = torch.empty(n_q, N, dtype=torch.float32, device="cuda")
        ws = s.score_workspace(n_q, N)
        for _ in range(args.warmup):
            s.score_keys(q, kc, 0, 0, N, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            ev[i][0].record(stream)
            s.score_keys(q, kc, 0, 0, N, out=out, workspace=ws, stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
        assert torch.isfinite(out).all(), "scores not finite"
        nbytes = N * rec + n_q * N * 4 + n_q * w.d * 2
        gbs = nbytes / t / 1e9
        runs.append({"n_q": n_q, "avg_call_s": t, "bytes_per_call": nbytes, "GBps": gbs,
                     "frac": gbs / HBM_PEAK_GBS, "scores_per_s": n_q * N / t,
                     "key_GBps": N * rec / t / 1e9})
        del out
    status = int(s.status.item()) & 0xFFFFFFFF
    assert status == 0, f"device status flags {status:#x}"
    top = runs[-1]
    res = {
        "metric": "packed-key inner-product search GB/s (packed keys read + fp32 scores written)",
        "value": top["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": top["avg_call_s"] * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+i8", "data": "synthetic (keys of the default workload, repeated)",
        "config": {"workload": SEARCH_WORKLOAD, "n_keys": N, "head_dim": w.d, "bits": w.bits, "n_q": top["n_q"]},
        "roofline": {"bound": "hbm", "achieved": top["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": top["frac"],
                     "traffic": traffic_for([("decode_qprep", 1), ("decode_partial", 1)], SEARCH_WORKLOAD),
                     "kernel": "tq_score_keys call: query prep + split scoring", "bytes_per_launch": top["bytes_per_call"],
                     "avg_launch_s": top["avg_call_s"]},
        "runs": runs, "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = search_cpu_baseline(w, rot, proj, Qn, top["n_q"], args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 5])
    ap.add_argument("--copies", type=int, default=0, help="rotation copies (0: enough for 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only plain 1 GiB device copies (HBM counter calibration)")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 counter CSVs (no GPU)")
    ap.add_argument("--search", action="store_true",
                    help="measure inner-product search over a packed key index instead")
    ap.add_argument("--search-nq", type=lambda v: [int(x) for x in v.split(",")], default=[8, 32],
                    help="query counts of the search measurement (multiples of 8; the last one is the headline)")
    args = ap.parse_args()
    if args.traffic:
        import workloads as W
        write_traffic(*args.traffic, copy_bytes=1 << 30,
                      workload=SEARCH_WORKLOAD if args.search else W.WORKLOADS[args.workload].name)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this hot path runs on one GPU; multi-GPU runs are not part of this build "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from kv_cache_online_amd.session import TQSession

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        copy_calibration()
        return
    if args.search:
        bench_search(args)
        return
    w = W.WORKLOADS[args.workload]
    rot, proj = W.rotation(w.d, w.wid), W.sketch(w.m, w.d, w.wid)
    s = TQSession(w.d, w.n_kv_heads, w.n_q_heads, rot, proj, k_bits=w.bits_mse, v_bits=w.bits_mse,
                  k_sketch=w.sketch, v_sketch=w.sketch)
    B, H, T, d = w.batch, w.n_kv_heads, w.seq_len, w.d
    lens = W.seq_lengths(w)
    cap = W.capacity(lens)
    starts = W.seq_starts(lens)
    esize = 4 if w.dtype == "f32" else 2
    rec = packed_record_bytes(d, w.m, w.bits_mse, w.sketch)
    in_bytes = 2 * B * H * T * d * esize
    packed_bytes = 2 * B * H * T * rec
    footprint = in_bytes + 2 * H * cap * rec
    R = args.copies or max(3, math.ceil((1 << 30) / footprint))

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    Kn, Vn, Qn = W.kv_batch(w, 0), W.kv_batch(w, 1), W.queries(w)
    K0, V0 = dev(Kn), dev(Vn)
    Ks, Vs = [K0] + [K0.clone() for _ in range(R - 1)], [V0] + [V0.clone() for _ in range(R - 1)]
    caches = [s.new_caches(cap) for _ in range(R)]
    Q = dev(Qn)
    dst = torch.from_numpy(starts).cuda()
    st_d = torch.from_numpy(starts).cuda()
    ln_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    max_len = int(lens.max())
    ws = s.workspace(B, max_len)
    out = torch.empty(B, w.n_q_heads, d, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, evs=None):
        r = i % R
        kc, vc = caches[r]
        if evs is not None:
            evs[0].record(stream)
        s.quantize(Ks[r], Vs[r], dst, kc, vc, stream=stream)   # two launches: K, then V
        if evs is not None:
            evs[1].record(stream)
        kd, vd = caches[(r + R // 2) % R]
        s.decode(Q, st_d, ln_d, max_len, kd, vd, out=out, workspace=ws, stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(R):          # populate every cache copy
        step(i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    qt = np.array([e[0].elapsed_time(e[1]) for e in events]) * 1e-3   # K and V launches
    dt_ = np.array([e[1].elapsed_time(e[2]) for e in events]) * 1e-3
    assert torch.isfinite(out).all(), "decode produced non-finite output"
    status = int(s.status.item()) & 0xFFFFFFFF
    assert status == 0, f"device status flags {status:#x}"

    q_avg, d_avg = float(qt.mean()), float(dt_.mean())
    # one launch of the quantize kernel: the call runs two equal launches (K, V)
    # back to back, so a launch takes half the call (its short gap included)
    ql_avg = q_avg / 2
    dec_gbs = packed_bytes / d_avg / 1e9
    q_bytes = in_bytes + packed_bytes
    q_gbs = q_bytes / q_avg / 1e9
    q_tok = B * T / q_avg
    q_flops = 2 * B * H * T * 4 * d * d           # two d x d contractions per vector
    roof_dec = {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dec_gbs / HBM_PEAK_GBS,
                "traffic": traffic_for([("decode_qprep", 1), ("decode_partial", 1), ("decode_merge", 1)], w.name),
                "kernel": "tq_decode_attention call: query prep + split partials + merge",
                "bytes_per_launch": packed_bytes, "avg_launch_s": d_avg}
    # quantize: the bound at algorithmic cost is the larger of the bytes at HBM peak
    # and the two contractions at bf16 matrix peak (HBM at d = 128, MFMA at d = 256)
    pieces = 6 if d == 128 or w.bits_mse == 3 else 5
    note = (f"algorithmic 4 d^2 flops per vector; executed as {pieces} bf16 piece products per vector "
            f"({pieces - 3} for Pi x, 3 for the sketch)")
    # per launch of the quantize kernel (one tensor: half the call's bytes and flops)
    qkern = "quantize_mfma" if d == 128 else "quantize_wide"
    ql_bytes, ql_flops = q_bytes / 2, q_flops / 2
    ql_gbs, ql_tf = ql_bytes / ql_avg / 1e9, ql_flops / ql_avg / 1e12
    q_traffic = traffic_for([("quantize", 1)], w.name)
    hbm_view = {"achieved": ql_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ql_gbs / HBM_PEAK_GBS}
    mfma_view = {"achieved": ql_tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": ql_tf / BF16_MFMA_PEAK_TFLOPS, "flops_per_launch": ql_flops, "note": note}
    kdesc = f"{qkern}: one launch per tensor (K or V), {B * H * T} vectors"
    if ql_flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) > ql_bytes / (HBM_PEAK_GBS * 1e9):
        roof_q = {"bound": "mfma", **{k: v for k, v in mfma_view.items() if k != "note"}, "traffic": q_traffic,
                  "kernel": kdesc, "bytes_per_launch": ql_bytes, "avg_launch_s": ql_avg, "note": note,
                  "hbm": hbm_view}
    else:
        roof_q = {"bound": "hbm", **hbm_view, "traffic": q_traffic, "kernel": kdesc,
                  "bytes_per_launch": ql_bytes, "avg_launch_s": ql_avg, "mfma": mfma_view}
    dominant = roof_q if ql_avg >= d_avg else roof_dec
    res = {
        "metric": METRIC, "value": dec_gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": (t1 - t0) / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+i8",
        "data": "synthetic (seeded Gaussian K/V/Q with per-channel scales and outlier channels)",
        "config": {"workload": w.name, "batch": B, "kv_heads": H, "q_heads": w.n_q_heads, "seq_len": T,
                   "head_dim": d, "bits": w.bits, "input_dtype": w.dtype, "rotation_copies": R},
        "decode_pct_hbm_peak": 100 * dec_gbs / HBM_PEAK_GBS,
        "quantize_tokens_per_s": q_tok, "quantize_GBps": q_gbs,
        "compute": "quantize: bf16-piece MFMA, fp32 accumulate; decode: exact int8 MFMA, int32 "
                   "accumulate, fp32/fp64 softmax and merge",
        "roofline": dominant, "roofline_decode": roof_dec, "roofline_quantize": roof_q,
        "source_hash": source_hash(),
        "quality": quality_report(w, s, rot, proj, K0, V0, Q, st_d, ln_d, max_len, cap, dst, Kn, Vn, Qn,
                                  out.cpu().numpy()),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, rot, proj, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
