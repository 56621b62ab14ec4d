"""Host-side arithmetic of the benchmark's figures (no GPU): the flop count
the prefill line is rated by, against a brute-force count of the (query,
attended token) pairs the causal definition gives."""

import numpy as np
import pytest

import bench


def brute_flops(ctx, nq, H, D):
    pairs = 0
    for c, n in zip(ctx, nq):
        for i in range(n):
            pos = c - n + i                  # position of chunk row i
            pairs += sum(1 for t in range(c) if t <= pos)
    return 4 * D * H * pairs                 # q.k and the weighted v sum, 2·D flops each


@pytest.mark.parametrize("ctx,nq", [([1], [1]), ([17, 100], [17, 3]), ([64, 50, 9], [0, 50, 1]),
                                    ([300], [129])])
def test_causal_prefill_flops_counts_attended_pairs(ctx, nq):
    assert bench.causal_prefill_flops(ctx, nq, 3, 64) == brute_flops(ctx, nq, 3, 64)


def test_prefill_workload_flops():
    # 16 whole prompts of 2048 tokens at 40 x 128: 4·128·40·16·(2048·2049/2).
    S, n = bench.PREFILL_SHAPE["S"], bench.PREFILL_SHAPE["n"]
    assert bench.causal_prefill_flops([n] * S, [n] * S, 40, 128) == 4 * 128 * 40 * S * n * (n + 1) // 2
    assert bench.causal_prefill_flops([n] * S, [n] * S, 40, 128) == 687_530_311_680
    # A decode is a one-row chunk: 4·D·ctx per head.
    rng = np.random.default_rng(0)
    ctx = [int(c) for c in rng.integers(1, 500, 7)]
    assert bench.causal_prefill_flops(ctx, [1] * 7, 2, 128) == 4 * 128 * 2 * sum(ctx)


def test_quantised_pool_summary(tmp_path, monkeypatch):
    """The quantised-pool profile summary classifies the three decode
    instantiations by their mangled names and rates each by its own bytes;
    the traffic lines scale the counters by the calibration copy."""
    import json
    names = {"f16": "_ZN2pa12_GLOBAL__N_113decode_kernelIDF16_DF16_Li128ELb1EvLb0ELb0ELb0EEEvNS0_6ParamsEPKiS4_PKl",
             "i8": "_ZN2pa12_GLOBAL__N_113decode_kernelIaDF16_Li128ELb1EvLb0ELb0ELb0EEEvNS0_6ParamsEPKiS4_PKl",
             "i4": "_ZN2pa12_GLOBAL__N_113decode_kernelINS0_4Int4EDF16_Li128ELb1EvLb0ELb0ELb0EEEvNS0_6ParamsEPKiS4_PKl"}
    avg_ns = {"f16": 200000.0, "i8": 100000.0, "i4": 50000.0}
    nbytes = {"f16": 1_400_000_000, "i8": 700_000_000, "i4": 350_000_000}
    pools = {k: {"decode_us": avg_ns[k] / 1e3 + 5, "bytes": nbytes[k], "gbs": 0.0} for k in names}
    rec = {"quantised_pools": pools, "decode_source_sha256": "abc"}
    (tmp_path / "prof_quant_trace").mkdir()
    (tmp_path / "prof_quant_trace.log").write_text("noise\n" + json.dumps(rec) + "\n")
    rows = ["Name,Calls,AverageNs,MinNs,MaxNs,Percentage"]
    rows += [f"{names[k]},21,{avg_ns[k]},{avg_ns[k] * 0.9},{avg_ns[k] * 1.2},10" for k in names]
    rows += ["write_kv_kernel,10,1000,900,1100,1"]
    (tmp_path / "prof_quant_trace" / "trace_kernel_stats.csv").write_text("\n".join(rows) + "\n")
    cal_kib = bench.CALIBRATION_BYTES / 1024
    for sub, counter, cal, per in (("prof_quant_fetch", "FETCH_SIZE", cal_kib / 2, 0.5),
                                   ("prof_quant_write", "WRITE_SIZE", cal_kib, 0.0)):
        (tmp_path / sub).mkdir()
        lines = ["Kernel_Name,Counter_Name,Counter_Value", f"stream_copy_kernel,{counter},{cal}"]
        # Fetch counters read half the bytes (factor 2), writes none.
        lines += [f"{names[k]},{counter},{nbytes[k] / 1024 * per}" for k in names]
        (tmp_path / sub / "x_counter_collection.csv").write_text("\n".join(lines) + "\n")
    out = tmp_path / "summary.txt"
    monkeypatch.setattr(bench, "QUANT_STATS_FILE", str(out))
    assert bench.summarize_quantised_profiles(str(tmp_path)) == 0
    text = out.read_text()
    for k in names:
        line = next(l for l in text.splitlines() if l.startswith(k + " ") and "decode_kernel" in l)
        fields = line.split()
        # ... calls, avg_us, min_us, bytes, avg_GB/s, min_GB/s, event_us
        assert float(fields[-6]) == pytest.approx(avg_ns[k] / 1e3)
        assert int(fields[-4]) == nbytes[k]
        assert float(fields[-3]) == pytest.approx(nbytes[k] / (avg_ns[k] / 1e9) / 1e9, rel=1e-3)
        traffic = next(l for l in text.splitlines() if l.startswith(k + " ") and "traffic_bytes" in l)
        assert traffic.split("=")[-1].strip() == "1.0000"
    assert "decode_source_sha256 = abc" in text
