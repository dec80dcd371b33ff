"""The bench script's command-line contract, on the CPU (no GPU needed).

bench.py runs on one GPU only and refuses more; its defaults time the decode step
with sub-records of the other headline workloads; a counter summary counts only
while it was taken on the current kernel code (comments and blank lines aside).
"""
import json
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "4"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for a configuration it does not run


def test_defaults():
    a = bench.parse_args([])
    assert (a.gpus, a.workload, a.sets) == (1, "decode_8b", 4)
    assert a.steps > 0 and a.warmup > 0 and not a.no_sub_records and not a.unfused and not a.alibi


def test_sub_records_name_known_workloads():
    from paged_gqa_attention_attn_amd import _lib
    for name, cfg, options in bench.SUB_RECORDS:
        assert cfg in bench.WORKLOADS.values(), name
        if options:   # a known workload run with other kernel options, under its own name
            assert all(k in _lib.OPTIONS for k in options), name
        else:
            assert bench.WORKLOADS[name] == cfg, name


def test_code_hash_ignores_comments_and_blank_lines():
    src = "int f(int x) {\n  // a note\n  return x; /* why */\n}\n"
    assert bench._code_only(src) == bench._code_only("int f(int x) {\n\n  return x;\n}\n")
    assert bench._code_only(src) != bench._code_only("int f(int x) {\n  return x + 1;\n}\n")


@pytest.mark.parametrize("f", sorted((ROOT / "profiles").glob("*_traffic.json")), ids=lambda p: p.name)
def test_counter_summaries_name_their_sources(f):
    rec = json.loads(f.read_text())
    assert rec.get("source_hash") and rec.get("hbm_bytes_per_launch", 0) > 0, f.name
