"""Host logic of bench.py's profiler digests, on the CPU: the short kernel
names, the kernel-trace summary and its leaf table (launches grouped by
width and split by whether the other kernels left a CU per tile), checked on
small synthetic files in rocprofv3's CSV layout with hand-worked answers."""
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
