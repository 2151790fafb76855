"""Host-side byte accounting of the benchmark against figures the pages print
(tests/golden/page_figures.json), and the launch-independent bookkeeping of
bench.py (no GPU)."""

import json
import os

import pytest

import bench

G = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                "page_figures.json")))


def test_message_sizes():
    assert bench.plane_bytes(1, 8192) == G["bytes_per_token_d8192_bf16"]["value"]
    assert bench.plane_bytes(8, 4096) == G["message_bytes_t8_d4096_bf16"]["value"]
    assert bench.plane_bytes(8, 8192) == G["message_bytes_t8_d8192_16bit"]["value"]


def test_ring_wire_bytes():
    n, s = 8, bench.plane_bytes(8, 4096)
    assert 2 * (n - 1) * s // n == G["ring_wire_bytes_n8_t8_d4096"]["value"]


def test_fused_and_unfused_per_token():
    r, w = bench.page_fused_bytes_per_token(8192)
    g = G["fused_traffic_per_token_d8192"]
    assert (r, w, r + w) == (g["reads"], g["writes"], g["total"])
    r, w = bench.page_unfused_bytes_per_token(8192)
    g = G["unfused_traffic_per_token_d8192"]
    assert (r, w, r + w) == (g["reads"], g["writes"], g["total"])
    saved = (sum(bench.page_unfused_bytes_per_token(8192)) -
             sum(bench.page_fused_bytes_per_token(8192))) * 64 * 108 // 1024
    assert saved == G["saved_per_forward_pass_kb_64tok_108layers"]["value"]


def test_oneshot_twoshot_traffic():
    n, D = 8, 2 << 20
    g = G["oneshot_vs_twoshot_traffic_n8_D2MB"]
    assert n * (n - 1) * D // (1 << 20) == g["oneshot_total_mb"]
    assert 2 * (n - 1) * D // (1 << 20) == g["twoshot_total_mb"]


def test_algorithmic_bytes_add_the_slot_reads():
    # the page's fused figure plus the N partial reads and gamma
    n, t, d = 8, 4096, 8192
    rd, wr = bench.algorithmic_bytes(n, t, d)
    pr, pw = bench.page_fused_bytes_per_token(d)
    assert rd == t * pr + n * bench.plane_bytes(t, d) + 4 * d
    assert wr == t * pw
    assert rd + wr == 738230272
    assert bench.counted_bytes(n, t, d) == 12 * 64 * (1 << 20)
    rd, wr = bench.algorithmic_bytes(4, 512, 8192, out=False, fp4=True)
    assert rd + wr == 52723712
    rd, _ = bench.algorithmic_bytes(8, 8, 8192, ll=True)
    assert rd == 8 * 2 * 131072 + 131072 + 4 * 8192


def test_algorithmic_bytes_of_the_patterns():
    """Each fusion pattern moves what it reads and writes: no residual read
    without a residual; without gamma neither gamma nor any norm output; FP8
    one byte per element; a sentinel reset writes the N slot planes again."""
    n, t, d = 8, 4096, 8192
    P = bench.plane_bytes(t, d)
    base_rd, base_wr = bench.algorithmic_bytes(n, t, d)
    assert bench.algorithmic_bytes(n, t, d, residual=False) == (base_rd - P, base_wr)
    assert bench.algorithmic_bytes(n, t, d, norm=False) == (n * P + P, P)
    assert bench.algorithmic_bytes(n, t, d, norm=False, fp4=True, fp8=True) == (n * P + P, P)
    assert bench.algorithmic_bytes(n, t, d, out=False, fp8=True) == (base_rd, P + t * d)
    assert bench.algorithmic_bytes(n, t, d, rout=False) == (base_rd, base_wr - P)
    assert bench.algorithmic_bytes(n, t, d, reset=True) == (base_rd, base_wr + n * P)
    # the per-call figures quoted for these patterns at this shape
    assert sum(bench.algorithmic_bytes(n, t, d, norm=False)) == 671088640
    assert sum(bench.algorithmic_bytes(n, t, d, out=False, fp8=True)) == 704675840
    assert sum(bench.algorithmic_bytes(n, t, d, reset=True)) == 1275101184


def test_extras_table_labels_and_modes():
    """The secondary measurements are named by their shapes and modes."""
    t = bench.extra_table()
    assert "decode_n8_t8_d8192_chain160_sentinel_fresh" in t
    assert "prefill_n8_t512_d65536" in t
    assert all(callable(f) for f in t.values())
    assert set(bench.DECODE_PROFILED) <= set(t)


@pytest.mark.parametrize("call_bytes,sets", [(738230272, 2), (92307456, 7), (1, 2 * 256 * 2 ** 20 + 1)])
def test_rotation_defeats_infinity_cache(call_bytes, sets):
    n = bench.n_sets_for(call_bytes)
    assert n == sets
    assert (n - 1) * call_bytes >= 2 * bench.INFINITY_CACHE_BYTES


def test_bench_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_bench_record_is_compact_and_complete():
    """The last stdout line of bench.py stays a few KB even with every decode
    configuration, the t = 512 figures and both CPU baselines in it (a
    collector that keeps only the tail of stdout must get all of it)."""
    dec = {}
    for label, *_ in bench.DECODE_MAP:
        dec[label] = {"floor_us": 1.604, "whole_us": 7.512, "whole_x": 4.683, "split": 8,
                      "split_floor_us": 1.655, "split_us": 4.281, "split_x": 2.587, "best_x": 2.587}
    t512 = {"C4_n8_t512_d8192": {"us": 16.94, "gbps_counted": 5943.1, "pct_counted": 74.3,
                                 "gbps_alg": 5449.0, "mix_us": 15.33, "mix_gbps": 6021.4},
            "C5_n4_t512_d8192_fp4": {"us": 12.56, "gbps_alg": 4197.3, "mix_us": 9.12,
                                     "mix_gbps": 5519.9}}
    cpu = {"value": 0.904123, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "14 full calls of n=8 t=4096 d=8192 on one host thread (median 0.891 s/call; "
                     "host AMD EPYC 9575F 64-Core Processor)"}
    line = bench.bench_record("prefill_n8_t4096_d8192", 8, 4096, 8192, 20, 5, 0.11712, 0.11698,
                              6876.2, 6303.3, 738396486, cpu,
                              {"value": 13.41, "cores": 16}, dec, t512)
    text = json.dumps(line, separators=(",", ":"))
    assert len(text) < 3072, len(text)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["config"]["workload"] == "prefill_n8_t4096_d8192"
    assert set(line["roofline"]) == {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert {"value", "unit", "cores", "kind", "sample"} <= set(line["cpu_baseline"])
    # every decode configuration of the workload definition is in the map
    names = {lbl for lbl, *_ in bench.DECODE_MAP}
    assert set(line["decode"]) == names
    for want in ("C1_", "C2_", "C3_n4", "C3_n8", "_ll", "C5_n4_t1_", "C5_n4_t8_", "C5_n4_t64_"):
        assert any(want in x for x in names), want


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summaries_from_synthetic_rocprof_outputs(tmp_path):
    """bench.py --summarize-profiles reads the CSV files the profile commands
    write and produces every summary, with the byte counters scaled by the
    copy calibration (synthetic counter values, no GPU)."""
    out, dest = str(tmp_path / "prof"), str(tmp_path / "profiles")
    stats_h = ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"]
    pmc_h = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    row8 = "void arfuse_detail::row_kernel<8, 1, false, false, 1, 0>(arfuse_detail::RowArgs)"
    mix = "void arfuse_detail::(anonymous namespace)::mix_kernel<1, false>(MixArgs)"
    fp4 = "void arfuse_detail::row_kernel<4, 1, false, false, 2, 0>(arfuse_detail::RowArgs)"
    _write_csv(os.path.join(out, "prof_trace", "prefill_kernel_stats.csv"), stats_h,
               [[row8, 55, 117000, 116000, 119000, 99.0]])
    for c, v in (("FETCH_SIZE", 295065.5), ("WRITE_SIZE", 131072.0)):
        _write_csv(os.path.join(out, "pmc_prefill_%s" % c, "pmc_counter_collection.csv"), pmc_h,
                   [[row8, c, v]] * 3)
    for c, v in (("FETCH_SIZE", 524288.0), ("WRITE_SIZE", 1048576.0)):
        _write_csv(os.path.join(out, "pmc_copy_%s" % c, "pmc_counter_collection.csv"), pmc_h,
                   [["copy_kernel(...)", c, v]])
    _write_csv(os.path.join(out, "prof_small", "small_kernel_stats.csv"), stats_h,
               [[row8, 510, 16940, 14520, 22240, 50], [fp4, 510, 11330, 9400, 16360, 30],
                [mix, 510, 16300, 15000, 18000, 20]])
    for c, v in (("FETCH_SIZE", 37000.0), ("WRITE_SIZE", 16384.0)):
        _write_csv(os.path.join(out, "pmc_small_%s" % c, "pmc_counter_collection.csv"), pmc_h,
                   [[row8, c, v], [fp4, c, v / 2], [mix, c, v]])
    kern = {lbl: "void arfuse_detail::%s(arfuse_detail::RowArgs)" % bench._counted_kernel(lbl)
            for lbl in bench.DECODE_COUNTED}
    _write_csv(os.path.join(out, "prof_counted", "decode_kernel_stats.csv"), stats_h,
               [[k, 1600, 4000, 3000, 9000, 10] for k in kern.values()]
               + [["floor_kernel(RowArgs)", 9600, 1300, 1000, 2000, 5]])
    for key, counters in bench.DECODE_COUNTER_SETS.items():
        rows = []
        for k in kern.values():
            for c in counters.split():
                rows.append([k, c, 1400.0 * 18000 if "LEVEL" in c else 18000.0])
        _write_csv(os.path.join(out, "pmc_counted_%s" % key, "pmc_counter_collection.csv"), pmc_h, rows)
    bench.summarize_profiles(out, dest)
    got = sorted(os.listdir(dest))
    for f in ("row_kernel_prefill_n8_t4096_d8192_stats.md", "row_kernel_prefill_n8_t4096_d8192_traffic.json",
              "row_kernel_prefill_t512_stats.md", "row_kernel_prefill_t512_traffic.json",
              "row_kernel_decode_counters.md", "row_kernel_decode_counters.json"):
        assert f in got, (f, got)
    tr = json.load(open(os.path.join(dest, "row_kernel_prefill_n8_t4096_d8192_traffic.json")))
    assert tr["copy_calibration"]["fetch_factor"] == 2.0
    assert abs(tr["read_bytes_per_launch"] - 295065.5 * 1024 * 2) < 1
    small = json.load(open(os.path.join(dest, "row_kernel_prefill_t512_traffic.json")))
    assert set(small["workloads"]) == set(bench.SMALL_PREFILL_KERNELS)
    dec = json.load(open(os.path.join(dest, "row_kernel_decode_counters.json")))
    assert set(dec["chains"]) == set(bench.DECODE_COUNTED)
    for rec in dec["chains"].values():
        assert abs(rec["read_latency_cycles"] - 1400.0) < 1e-9
