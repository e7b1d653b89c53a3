"""Host-side checks of bench.py's profile reduction: the rocprofv3 CSVs of the
profiled runs are synthesized with known contents, reduced into a temporary
directory, and the summaries' figures are checked against what the inputs
fix (the copy calibration, the headline dispatches, the traffic ratios)."""
import csv
import json
import os

import pytest

import bench

SHA = "0123456789abcdef"
SCAN = ("void kda::(anonymous namespace)::kda_scan_kernel<16, {c}, {bf}, "
        "(kda::(anonymous namespace)::Rows){ma}, (kda::(anonymous namespace)::Rows){mb}, "
        "{table}, {dual}, {tail}>(kda::ScanArgs)")
COPY = ("kda::(anonymous namespace)::kda_copy_kernel(HIP_vector_type<float, 4u> const*, "
        "HIP_vector_type<float, 4u>*, unsigned long)")
FILL = ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, "
        "std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)")
ROUND = SCAN.format(c=4, bf="false", ma=3, mb=1, table="false", dual="false", tail=2)
ROUND_REC = SCAN.format(c=4, bf="false", ma=2, mb=1, table="false", dual="false", tail=2)
SCAN_K = SCAN.format(c=4, bf="false", ma=0, mb=1, table="false", dual="false", tail=2)
LAYER = SCAN.format(c=1, bf="false", ma=3, mb=1, table="false", dual="true", tail=0)


def test_kernel_labels():
    assert bench.kernel_label(ROUND) == "round_stash_t2"
    assert bench.kernel_label(ROUND_REC) == "round_recompute_t2"
    assert bench.kernel_label(SCAN_K) == "scan_t2"
    assert bench.kernel_label(LAYER) == "round_stash_c1_dual"
    assert bench.kernel_label(SCAN.format(c=2, bf="true", ma=0, mb=2, table="false",
                                          dual="false", tail=0)) == "replay_c2_bf16"
    assert bench.kernel_label(SCAN.format(c=4, bf="false", ma=0, mb=1, table="true",
                                          dual="false", tail=0)) == "batched"
    assert bench.kernel_label(SCAN.format(c=4, bf="false", ma=0, mb=4, table="false",
                                          dual="false", tail=0)) == "scan_columns"
    assert bench.kernel_label(SCAN.format(c=4, bf="false", ma=3, mb=1, table="false",
                                          dual="false", tail=1)) == "round_stash_t4"
    assert bench.kernel_label(SCAN.format(c=4, bf="true", ma=3, mb=1, table="false",
                                          dual="false", tail=2)) == "round_stash_t2_bf16"
    assert bench.kernel_label(COPY) == "copy"
    assert bench.kernel_label(FILL) == "fill"
    assert bench.kernel_label("void some_other_kernel(int)") is None


def _line(warmup, steps, sha=SHA, **extra):
    d = {"config": {"kernel_source_sha256_16": sha}, "warmup": warmup, "steps": steps}
    d.update(extra)
    return json.dumps(d)


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _fake_runs(d, sha_fetch=SHA):
    """Synthetic outputs of the profiled runs.  The kernel trace holds the
    headline kernel's warm-up dispatches, then its timed ones (1, 2, ..., K us
    above 80 us), each after a fill; the counter passes read FETCH_SIZE at half
    and WRITE_SIZE at the full true bytes of the copy and of the fused round."""
    W, K = 5, 20
    round_us = {"mean": 100.0, "p10": 90.0, "p50": 99.0, "p90": 110.0,
                "each": [85.0 + i for i in range(K)]}
    with open(os.path.join(d, "kt.log"), "w") as f:
        f.write("progress line\n" + _line(W, K, round_us=round_us) + "\n")
    with open(os.path.join(d, "bench.log"), "w") as f:
        f.write(_line(W, K, round_us=round_us) + "\n")
    trace, t, disp = [], 1_000_000, 0
    for i in range(W + K):
        for name, us in ((FILL, 5.0), (ROUND, 80.0 + (i - W + 1 if i >= W else 50))):
            disp += 1
            trace.append(["KERNEL_DISPATCH", disp, name, t, t + int(us * 1000)])
            t += int(us * 1000) + 4500
    for i in range(3):
        disp += 1
        trace.append(["KERNEL_DISPATCH", disp, LAYER, t, t + 11_000])
        t += 20_000
    _write_csv(os.path.join(d, "kt", "host", "kt_kernel_trace.csv"),
               ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    _write_csv(os.path.join(d, "kt", "host", "kt_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[ROUND, W + K, 95000.0, 81000.0, 130000.0], [FILL, W + K, 5000.0, 5000.0, 5000.0]])
    # counter passes: warm-up 2, 8 timed rounds of the fused kernel, then one copy
    Wc, Kc = 2, 8
    L, H, T = 34, 64, 15
    chains = L * H
    keeps = bench._headline_keeps(Wc, Kc)
    copy_bytes = chains * bench.STATE_BYTES
    for tag, counter, factor, shas in (("fetch", "FETCH_SIZE", 0.5, sha_fetch),
                                       ("write", "WRITE_SIZE", 1.0, SHA)):
        with open(os.path.join(d, f"{tag}.log"), "w") as f:
            f.write(_line(Wc, Kc, sha=shas) + "\n")
        rows, disp = [], 0
        for i in range(Wc + Kc):
            disp += 1
            # the fused round moves 1.25x its algorithmic bytes, split 60/40 read/write
            alg = chains * bench.round_bytes_per_head(keeps[i - Wc] if i >= Wc else 0, T)
            share = 0.6 if tag == "fetch" else 0.4
            rows.append([disp, ROUND, counter, 1.25 * alg * share * factor / 1024, 0, 1])
        disp += 1
        rows.append([disp, COPY, counter, copy_bytes * factor / 1024, 0, 1])
        _write_csv(os.path.join(d, tag, "host", "t_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"], rows)
    return K


def test_profile_summary_reduces_synthetic_runs(tmp_path):
    d, out = tmp_path / "prof", tmp_path / "out"
    d.mkdir()
    out.mkdir()
    K = _fake_runs(str(d))
    bench.profile_summary(str(d), str(out))
    traffic = json.load(open(out / "traffic.json"))
    assert traffic["kernel_source_sha256_16"] == SHA
    cal = traffic["copy_calibration"]
    assert cal["fetch_factor"] == pytest.approx(0.5)
    assert cal["write_factor"] == pytest.approx(1.0)
    # 60% + 40% of 1.25x the algorithmic bytes, after the calibration
    assert traffic["kernels"]["round"]["ratio_to_algorithmic"] == pytest.approx(1.25)
    md = open(out / "verify_k14_kernel_stats.md").read()
    assert f"`{SHA}`" in md
    # the timed dispatches ran 81..100 us: mean 90.5, events 85..104, 4 us above each
    assert "| kernel time (rocprofv3 trace) | 90.5 |" in md
    assert "median 4.0 us, min 4.0, max 4.0" in md
    assert f"The {K} timed rounds" in md
    assert "3 dispatches, mean 11.00 us" in md
    assert "| round_stash_t2 | 25 | 95.0 |" in md
    assert "ratio" in open(out / "verify_k14_traffic.md").read()


def test_profile_summary_refuses_mixed_sources(tmp_path):
    d, out = tmp_path / "prof", tmp_path / "out"
    d.mkdir()
    out.mkdir()
    _fake_runs(str(d), sha_fetch="fedcba9876543210")
    with pytest.raises(RuntimeError, match="do not share one recorded kernel source"):
        bench.profile_summary(str(d), str(out))
    assert not (out / "traffic.json").exists()


def test_stats_and_headline_selection():
    s = bench.stats_us([1.0, 2.0, 3.0, 4.0])
    assert s["mean"] == 2.5 and s["p50"] == 2.5
    rows = [{"Kernel_Name": ROUND, "Dispatch_Id": str(i)} for i in (9, 3, 7, 1, 5)]
    rows.append({"Kernel_Name": COPY, "Dispatch_Id": "2"})
    sel = bench._headline_rows(rows, "Dispatch_Id", 1, 3)
    assert [r["Dispatch_Id"] for r in sel] == ["3", "5", "7"]
    with pytest.raises(RuntimeError):
        bench._headline_rows(rows, "Dispatch_Id", 3, 3)
