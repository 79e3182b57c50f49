"""CPU tests of the bench's host-side bookkeeping: record sizes and the HBM traffic
table built from rocprofv3 counter CSVs (no GPU, no kernel)."""
import csv
import json
import os

import pytest

import bench


def test_packed_record_bytes():
    # b' index planes of d bits + m sign bits + two fp16 scales
    assert bench.packed_record_bytes(128, 128, 2, 1) == 52
    assert bench.packed_record_bytes(128, 128, 3, 1) == 68
    assert bench.packed_record_bytes(256, 256, 1, 1) == 68
    assert bench.packed_record_bytes(128, 128, 3, 0) == 52


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, kib) in enumerate(rows):
            w.writerow([i, name, counter, kib])


@pytest.fixture
def tmp_root(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "family_hash", lambda name: "feedface" + bench.kernel_family(name))
    return tmp_path


def test_traffic_scaling_and_lookup(tmp_root, monkeypatch):
    """Counters in KiB per dispatch, scaled by what they read for a 1 GiB copy; the median
    dispatch of each kernel is kept; workloads accumulate in one file."""
    q = "void tq::(anonymous namespace)::quantize_mfma<3, false>(tq::QuantArgs)"
    d = "void tq::(anonymous namespace)::decode_partial_fast<128, 1, 3, 3, true, false>(tq::DecodeArgs)"
    copy = "__amd_rocclr_copyBuffer"
    p = {k: str(tmp_root / f"{k}.csv") for k in ("f", "w", "cf", "cw", "f2", "w2")}
    gib_kib = (1 << 30) / 1024
    _counter_csv(p["cf"], "FETCH_SIZE", [(copy, gib_kib / 2)] * 3 + [("small", 1.0)])  # reads counted at half
    _counter_csv(p["cw"], "WRITE_SIZE", [(copy, gib_kib)] * 3)
    _counter_csv(p["f"], "FETCH_SIZE", [(q, 100.0), (q, 1000.0), (q, 101.0), (d, 50.0)])
    _counter_csv(p["w"], "WRITE_SIZE", [(q, 10.0), (q, 10.0), (q, 10.0), (d, 2.0)])
    bench.write_traffic(p["f"], p["w"], p["cf"], p["cw"], copy_bytes=1 << 30, workload="wl-a")
    t = json.load(open(tmp_root / "profiles" / "traffic.json"))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    k = t["workloads"]["wl-a"]["kernels"]["quantize_mfma<3, false>"]
    assert k["fetch_bytes"] == pytest.approx(101.0 * 1024 * 2)      # median of 100, 101, 1000
    assert k["write_bytes"] == pytest.approx(10.0 * 1024)
    assert bench.traffic_for([("quantize", 2)], "wl-a") == pytest.approx(2 * (101.0 * 2048 + 10240))
    assert bench.traffic_for([("quantize", 1), ("decode_partial", 1)], "wl-a") == pytest.approx(
        101.0 * 2048 + 10240 + 50.0 * 2048 + 2048)
    assert bench.traffic_for([("decode_merge", 1)], "wl-a") is None  # kernel not counted
    assert bench.traffic_for([("quantize", 1)], "wl-b") is None      # workload not counted
    # a second workload joins the file; the first stays
    _counter_csv(p["f2"], "FETCH_SIZE", [(d, 7.0)])
    _counter_csv(p["w2"], "WRITE_SIZE", [(d, 1.0)])
    bench.write_traffic(p["f2"], p["w2"], p["cf"], p["cw"], copy_bytes=1 << 30, workload="wl-b")
    assert bench.traffic_for([("decode_partial", 1)], "wl-b") == pytest.approx(7.0 * 2048 + 1024)
    assert bench.traffic_for([("quantize", 1)], "wl-a") is not None
    # entries taken on other kernel sources are not used; each family has its own hash
    monkeypatch.setattr(bench, "family_hash", lambda name: "0ther" if name.startswith("quantize") else
                        "feedface" + bench.kernel_family(name))
    assert bench.traffic_for([("quantize", 1)], "wl-a") is None
    assert bench.traffic_for([("decode_partial", 1)], "wl-b") is not None


class _ExactScores:
    """Stand-in for a session: score_keys returns q.k over given keys (optionally
    perturbed on one token), on the CPU."""

    device = "cpu"

    def __init__(self, keys, bump=None):
        self.keys, self.bump = keys, bump

    def score_keys(self, q, kc, kv_head, start, n):
        import numpy as np
        import torch
        import workloads as W
        qf = q.float().numpy().astype(np.float64)
        s = qf @ W.to_f64(self.keys[kv_head], "bf16")[start - start:start - start + n].T
        if self.bump is not None:
            s[:, self.bump[0]] += self.bump[1]
        return torch.from_numpy(s.astype(np.float32))


def test_score_fidelity_bookkeeping():
    """Exact scores give zero error and the same top token everywhere; a bump on the
    top token of every head moves the RMS error by exactly bump / sqrt(d) / sqrt(n)."""
    import math
    import numpy as np
    import workloads as W
    w = W.small(W.WORKLOADS[2], batch=1, n_kv_heads=2, n_q_heads=8, seq_len=64)
    keys = [W.kv_chunk(w, 0, 0, h, n_tokens=64) for h in range(2)]
    Qn = W.queries(w)
    ctx = lambda b, h: (keys[h], None)
    r = bench.score_fidelity(w, _ExactScores(keys), None, Qn, ctx, [0])
    assert r["logit_err_rms"] < 1e-4 * r["logit_std_mean"] and r["top1_same_frac"] == 1.0
    assert r["query_heads"] == 8 and r["tokens"] == 64 and r["top2_gap_median"] > 0
    r2 = bench.score_fidelity(w, _ExactScores(keys, bump=(5, 3.0)), None, Qn, ctx, [0])
    assert abs(r2["logit_err_rms"] - 3.0 / math.sqrt(w.d) / math.sqrt(64)) < 1e-4
