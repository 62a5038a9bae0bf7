"""The rocprofv3 summaries under profiles/: each one states the command that
made it, and that command runs committed files only (bench.py with options
it accepts, on a workload it knows).  CPU only."""
import json
import pathlib
import re

import workloads

ROOT = pathlib.Path(__file__).resolve().parent.parent
PROFILES = ROOT / "profiles"


def _bench_options():
    src = (ROOT / "bench.py").read_text()
    return set(re.findall(r'add_argument\(\s*"(--[a-z0-9-]+)"', src))


def _bench_default_config():
    m = re.search(r'add_argument\(\s*"--config",\s*default="([^"]+)"', (ROOT / "bench.py").read_text())
    assert m, "bench.py names no default workload"
    return m.group(1)


def _command_block(text):
    m = re.search(r"^```\n(.*?)^```$", text, re.S | re.M)
    assert m, "no fenced command block"
    return m.group(1)


def _summaries():
    files = sorted(PROFILES.glob("*.md"))
    assert files, "profiles/ holds no summaries"
    return files


def test_every_summary_states_a_runnable_command():
    opts = _bench_options()
    known = {c.name for c in workloads.CONFIGS}
    for f in _summaries():
        cmd = _command_block(f.read_text())
        assert "_work/" not in cmd, f.name
        assert "bench.py" in cmd, f.name
        for tool in re.findall(r"rocprofv3 ([^\n]*)", cmd):
            assert " -- python3 " in tool, (f.name, "the profiled program follows -- directly")
        for opt in re.findall(r"(?<![\w-])(--[a-z][a-z0-9-]*)", cmd):
            if opt in ("--kernel-trace", "--stats", "--pmc"):
                continue
            assert opt in opts, (f.name, opt)
        for name in re.findall(r"--config (\S+)", cmd):
            assert name in known, (f.name, name)


def test_summary_names_match_their_workload():
    known = {c.name for c in workloads.CONFIGS}
    for f in _summaries():
        stem = f.stem
        assert any(stem.endswith("_" + w) for w in known), f.name
        cmd = _command_block(f.read_text())
        named = re.findall(r"--config (\S+)", cmd)
        workload = next(w for w in known if stem.endswith("_" + w))
        assert (named[0] if named else _bench_default_config()) == workload, f.name


def test_traffic_table_is_consistent():
    for f in sorted(PROFILES.glob("traffic_*.json")):
        d = json.loads(f.read_text())
        assert re.fullmatch(r"[0-9a-f]{64}", d["sources_sha256"]), f.name
        assert f.stem == "traffic_" + d["workload"], f.name
        assert d["kernels"], f.name
