"""Host logic of bench.py's profiler digests, on the CPU: the short kernel
names, the kernel-trace summary and its leaf table (launches grouped by
width and split by whether the other kernels left a CU per tile), the HBM
traffic scaled by the copy calibration (and the bench's use of it only for
matching kernel sources), and the derived counter ratios; checked on small
synthetic files in rocprofv3's CSV layout with hand-worked answers."""
import csv
import json

import bench


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_ALL)
        w.writerow(header)
        w.writerows(rows)


def _table(lines, first_cell):
    """Rows of the markdown table whose header starts with `first_cell`, as
    lists of cell strings."""
    out, on = [], False
    for ln in lines:
        if ln.startswith(f"| {first_cell} |"):
            on = True
            continue
        if on:
            if not ln.startswith("|"):
                break
            if ln.startswith("|---"):
                continue
            out.append([c.strip() for c in ln.strip().strip("|").split("|")])
    return out


def test_kernel_key_shortens_demangled_names():
    k = bench._kernel_key
    assert k("void bk::k_f_tile<1>(float*, float*, float*, long, long, long, int, int, int)") == "k_f_tile<1>"
    assert k("bk::k_leaf(bk::LeafArgs)") == "k_leaf"
    assert k("void bk::(anonymous namespace)::k_x<std::array<char*, 3ul> >(int)") == "k_x<std::array<char*,3ul>>"
    assert k("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


TRACE_HEADER = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"]


def _launch(name, t0, t1, workgroups, threads):
    return ["KERNEL_DISPATCH", name, str(t0), str(t1), str(workgroups * threads), str(threads)]


LEAF = "bk::k_leaf(bk::LeafArgs)"
FAR = "bk::k_prop_rows_far(float const*, float const*, float*, long, long, int, int, int, int, int, int, unsigned int const*, unsigned int, int)"
TILE = "void bk::k_prop_cols_t(float const*, float const*, float*, long, long, int, int, int, int, int, int, unsigned int, int)"


def test_leaf_width_table_groups_and_splits(tmp_path):
    rows = [
        # a far part on 192 workgroups from t = 0 to 100 us
        _launch(FAR, 0, 100_000, 192, 512),
        # 100 tiles beside it (midpoint 25 us): 192 + 100 > 256 CUs, short
        _launch(LEAF, 0, 50_000, 100, 512),
        # 100 tiles alone: a CU each
        _launch(LEAF, 200_000, 240_000, 100, 512),
        # a 4096-workgroup launch counts as 256, so even one tile is short beside it
        _launch(TILE, 300_000, 400_000, 4096, 256),
        _launch(LEAF, 310_000, 350_000, 1, 512),
        # 64 tiles beside 192 workgroups: exactly 256, a CU each
        _launch(FAR, 500_000, 600_000, 192, 512),
        _launch(LEAF, 510_000, 546_000, 64, 512),
    ]
    _write_csv(tmp_path / "run_kernel_trace.csv", TRACE_HEADER, rows)
    t = _table(bench.leaf_width_table(str(tmp_path)), "tiles")
    got = {r[0]: r[1:] for r in t}
    # tiles: calls, avg us, calls with a CU per tile, avg us, calls short, avg us
    assert got["1"] == ["1", "40.00", "0", "", "1", "40.00"]
    assert got["33-64"] == ["1", "36.00", "1", "36.00", "0", ""]
    assert got["65-128"] == ["2", "45.00", "1", "40.00", "1", "50.00"]
    assert set(got) == {"1", "33-64", "65-128"}


def test_leaf_width_table_without_a_trace_is_empty(tmp_path):
    assert bench.leaf_width_table(str(tmp_path)) == []


def test_stats_digest_sums_and_orders_kernels(tmp_path):
    stats = tmp_path / "a"
    stats.mkdir()
    _write_csv(stats / "run_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs"],
               [[LEAF, "3", "120000"], [TILE, "10", "50000"]])
    other = tmp_path / "b"
    other.mkdir()
    # the same kernel from a second file is summed under its short name
    _write_csv(other / "run_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs"], [[LEAF, "1", "40000"]])
    log = tmp_path / "bench.err"
    log.write_text("[bench] 5 steps: 1.000 ms/step fused\n"
                   "[bench] kernels: " + json.dumps({"k_leaf": {"avg_us": 39.5}}) + "\n")
    lines = bench.stats_digest(str(tmp_path), str(log), "Title", "the command").split("\n")
    assert lines[0] == "# Title"
    assert "the command" in lines
    assert any(ln == "Bench line of the same run: `[bench] 5 steps: 1.000 ms/step fused`" for ln in lines)
    t = _table(lines, "kernel")
    assert [r[0] for r in t] == ["k_leaf", "k_prop_cols_t"]     # by total time
    assert t[0] == ["k_leaf", "4", "0.160", "40.00", "39.5"]
    assert t[1] == ["k_prop_cols_t", "10", "0.050", "5.00", ""]


COUNTER_HEADER = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counters(path, rows):
    path.mkdir()
    _write_csv(path / "run_counter_collection.csv", COUNTER_HEADER,
               [[str(i), k, c, str(v)] for i, (k, c, v) in enumerate(rows)])


def test_traffic_digest_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_digest", lambda: "sha-A")
    (tmp_path / "profiles").mkdir()
    copy = "void at::native::copy_kernel(int)"
    # a 1 GiB copy that FETCH_SIZE reports as 512 MiB (factor 2) and WRITE_SIZE as 1 GiB (factor 1)
    _counters(tmp_path / "cf", [(copy, "FETCH_SIZE", 524288.0)])
    _counters(tmp_path / "cw", [(copy, "WRITE_SIZE", 1048576.0)])
    _counters(tmp_path / "f", [(LEAF, "FETCH_SIZE", 3000.0), (LEAF, "FETCH_SIZE", 3400.0)])
    _counters(tmp_path / "w", [(LEAF, "WRITE_SIZE", 2300.0)])
    bench.traffic_digest([str(tmp_path / d) for d in ("f", "w", "cf", "cw")], "tiny", "cmd")
    t = json.loads((tmp_path / "profiles" / "traffic_tiny.json").read_text())
    assert t["sources_sha256"] == "sha-A"
    assert t["calibration"]["FETCH_SIZE"]["factor"] == 2.0 and t["calibration"]["WRITE_SIZE"]["factor"] == 1.0
    leaf = t["kernels"]["k_leaf"]
    assert leaf["dispatches"] == 2
    assert leaf["hbm_bytes_per_launch"] == 1024 * (3200 * 2 + 2300)   # KiB means, scaled, in bytes
    # the bench uses the numbers only while the kernel sources are the ones they were taken on
    assert bench.load_traffic("tiny")["kernels"]["k_leaf"]["hbm_bytes_per_launch"] == 8908800
    monkeypatch.setattr(bench, "sources_digest", lambda: "sha-B")
    assert bench.load_traffic("tiny") is None
    assert bench.load_traffic("absent") is None


def test_pmc_digest_derived_ratios(tmp_path):
    k = "void bk::k_prop_rows(float const*)"
    _counters(tmp_path / "a", [(k, "SQ_INSTS_VALU", 100.0), (k, "SQ_INSTS_VALU", 300.0),
                               (k, "SQ_WAVES", 4.0), (k, "SQ_WAVES", 4.0)])
    _counters(tmp_path / "b", [(k, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0), (k, "GRBM_GUI_ACTIVE", 8000.0),
                               (k, "TCC_HIT_sum", 30.0), (k, "TCC_MISS_sum", 10.0)])
    lines = bench.pmc_digest([str(tmp_path / "a"), str(tmp_path / "b")], "T", "").split("\n")
    mean = _table(lines, "kernel")[0]
    assert mean[:2] == ["k_prop_rows", "2"]
    derived = _table(lines[lines.index("Derived (only where the counters were collected):"):], "kernel")[0]
    names = [d[0] for d in bench.PMC_DERIVED]
    got = dict(zip(names, derived[1:]))
    assert got["valu/wave"] == "50"            # mean 200 VALU over mean 4 waves
    assert got["mfma_busy"] == "0.5"           # 512,000 busy cycles over 1,000 active cycles x 1024 SIMDs
    assert got["l2_hit"] == "0.75"
    assert got["lds/wave"] == ""               # counters not collected


def test_roofline_entry_by_bound():
    traffic = {"kernels": {"k_prop_rows": {"hbm_bytes_per_launch": 123}}}
    # MFMA: 2e11 flops in 2 ms = 100 TFLOP/s against the fp32 matrix peak
    r = bench.roofline_entry("k_prop_rows", {"launches": 4, "total_ms": 2.0, "alg_flops": 2e11, "alg_bytes": 1e9},
                             traffic)
    assert (r["bound"], r["unit"], r["peak"]) == ("mfma", "TFLOP/s", bench.PEAK_FP32_MFMA_TFLOPS)
    assert r["achieved"] == 100.0 and r["frac"] == round(100.0 / 157.3, 4)
    assert r["avg_launch_us"] == 500.0 and r["traffic"] == 123
    assert r["alg_flops_per_launch"] == 5e10
    # the leaf: fp32 vector peak of the non-packed instructions, with the packed figure in a note
    r = bench.roofline_entry("k_leaf", {"launches": 2, "total_ms": 1.0, "alg_flops": 7.86e10, "alg_bytes": 0.0}, None)
    assert (r["bound"], r["peak"], r["traffic"]) == ("alu", 78.6, None)
    assert r["achieved"] == 78.6 and r["frac"] == 1.0 and "157.3" in r["peak_note"]
    # HBM: bytes over time in GB/s against 8 TB/s
    r = bench.roofline_entry("k_copy_pad", {"launches": 1, "total_ms": 1.0, "alg_flops": 0.0, "alg_bytes": 4e9}, None)
    assert (r["bound"], r["unit"], r["achieved"], r["frac"]) == ("hbm", "GB/s", 4000.0, 0.5)


def test_kernel_bounds_cover_the_library_kernels():
    # every MFMA kernel of the recursion and propagation is priced against the matrix peak
    for k in ("k_prop_rows", "k_prop_cols_t_far", "k_f_tile<4>", "k_f_update", "k_ad_update", "k_moment<true>"):
        assert bench.kernel_bound(k) == "mfma", k
    for k in ("k_load_damped", "k_f_finish", "k_ad_quant"):
        assert bench.kernel_bound(k) == "hbm", k
    for k in ("k_leaf", "k_f_diag", "k_gptq_sweep"):
        assert bench.kernel_bound(k) == "alu", k


def test_stage_fractions():
    m, n = 64, 128
    agg = {"k_prop_rows": {"total_ms": 1.0, "alg_flops": 3e9}, "k_prop_rows_far": {"total_ms": 1.0, "alg_flops": 1e9},
           "k_prop_cols_t": {"total_ms": 0.5, "alg_flops": 1e9}, "k_leaf": {"total_ms": 9.0, "alg_flops": 1e9}}
    st = bench.stage_fractions(agg, m, n)
    s1, s2 = st["stage1"], st["stage2"]
    assert s1["kernels_ms"] == 2.0 and s1["alg_flops"] == m * n * (n + 1)   # E P_A^T, triangular
    assert s1["alg_tflops"] == round(m * n * (n + 1) / 2e-3 / 1e12, 3)
    assert s1["executed_tflops"] == 2.0                                     # 4e9 flops in 2 ms
    assert s2["kernels_ms"] == 0.5 and s2["alg_flops"] == m * (m + 1) * n   # P_B Y
    assert bench.stage_fractions({"k_leaf": {"total_ms": 1.0, "alg_flops": 1.0}}, m, n) == {}
