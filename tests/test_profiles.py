"""The committed rocprofv3 summaries agree with the workloads they name: the
algorithmic bytes a traffic summary divides by are the packed bytes one decode
step reads, its traffic is the scaled counter sum, the utilisation shares lie
in range, and every quoted command runs the committed bench on a known
workload with flags the bench accepts."""

import glob
import os
import re

import pytest

from oracle.bytes import per_token_head
from synth.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _fields(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


# bench flags that resize a workload, and the field each sets
RESIZE = {"--batch": "batch", "--context": "context", "--q-heads": "hq", "--kv-heads": "hkv", "--head-dim": "head_dim"}


def _workload(path):
    """The workload a summary covers: the one its file name holds, resized by
    the flags of its quoted bench command (all its commands agree)."""
    names = [w for w in CONFIGS if f"_{w}_" in os.path.basename(path)]
    assert len(names) == 1, path
    sizes = set()
    for line in open(path):
        if line.startswith("# command") and "bench.py" in line:
            args = line.split("bench.py", 1)[1].split()
            sizes.add(tuple(sorted((RESIZE[a], int(args[i + 1])) for i, a in enumerate(args) if a in RESIZE)))
    assert len(sizes) <= 1, path
    return CONFIGS[names[0]].scaled(**dict(sizes.pop())) if sizes else CONFIGS[names[0]]


PMC = sorted(glob.glob(os.path.join(PROFILES, "*_pmc.txt")))
PMC = [p for p in PMC if not os.path.basename(p).startswith("copy_")]
UTIL = sorted(glob.glob(os.path.join(PROFILES, "*util.txt")))


def test_every_workload_has_traffic_and_utilisation_summaries():
    for w in CONFIGS:
        assert any(f"_{w}_pmc" in p for p in PMC), w
        assert any(p.endswith(f"_{w}_util.txt") for p in UTIL), w


def test_resized_summaries_are_not_read_as_the_workload_itself():
    """The bench reads profiles/*_<workload>_<kind>.txt for a workload's own
    sizes: a summary of a resized copy must carry more in its name."""
    for path in PMC + UTIL:
        base = os.path.basename(path)
        if _workload(path) not in CONFIGS.values():
            assert not any(base.endswith(f"_{w}_pmc.txt") or base.endswith(f"_{w}_util.txt") for w in CONFIGS), base


@pytest.mark.parametrize("path", PMC, ids=os.path.basename)
def test_traffic_summary_is_consistent(path):
    cfg = _workload(path)
    kv = _fields(path)
    per_tok = per_token_head(cfg.fmt, cfg.head_dim, cfg.rope_dim)
    assert int(kv["algorithmic_bytes_per_launch"]) == per_tok * cfg.hkv * cfg.batch * cfg.context
    traffic = (float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
               + float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["write_scale"]))
    assert abs(int(kv["traffic_bytes_per_launch"]) - traffic) <= 1024
    ratio = int(kv["traffic_bytes_per_launch"]) / int(kv["algorithmic_bytes_per_launch"])
    assert abs(float(kv["traffic_over_algorithmic"]) - ratio) < 1e-3
    assert os.path.isfile(os.path.join(ROOT, kv["source"]))


@pytest.mark.parametrize("path", UTIL, ids=os.path.basename)
def test_utilisation_summary_is_in_range(path):
    _workload(path)
    kv = _fields(path)
    assert kv["role"] in ("attention", "append")
    for k in ("mfma_busy", "valu_active", "lds_active", "coexec", "wait_inst_share", "wait_any_share"):
        assert 0.0 <= float(kv[k]) <= 1.0, k
    assert float(kv["coexec"]) <= float(kv["mfma_busy"]) + 1e-3
    assert float(kv["waves_per_simd"]) > 0
    assert os.path.isfile(os.path.join(ROOT, kv["source"]))


def _bench_flags():
    text = open(os.path.join(ROOT, "bench.py")).read()
    return set(re.findall(r'add_argument\("(--[\w-]+)"', text))


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(PROFILES, "*.txt"))), ids=os.path.basename)
def test_quoted_commands_run_the_committed_bench(path):
    flags = _bench_flags()
    commands = [line for line in open(path) if line.startswith("# command")]
    assert commands, path
    for line in commands:
        assert "rocprofv3" in line
        if "bench.py" not in line:
            continue
        args = line.split("bench.py", 1)[1].split()
        for a in args:
            if a.startswith("--"):
                assert a in flags, (path, a)
        assert args[args.index("--config") + 1] in CONFIGS
