"""Host-side checks of bench.py's bookkeeping (no GPU)."""
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_drops_comments_and_blank_lines():
    src = "int a; // one\n\n/* two\n   lines */ int b;\n  // three\nint c;  \n"
    assert bench._code_only(src) == "int a;\n int b;\nint c;"


def test_source_digest_ignores_comment_edits(tmp_path, monkeypatch):
    csrc = tmp_path / bench.CSRC
    csrc.mkdir(parents=True)
    for name in bench._COMMON_SOURCES:
        (csrc / name).write_text("// header\nint h;\n")
    (csrc / "k.hip").write_text("__global__ void k() {}  // a kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.source_digest(["k.hip"])
    (csrc / "k.hip").write_text("// reworded\n__global__ void k() {}\n\n")
    assert bench.source_digest(["k.hip"]) == d0
    (csrc / "k.hip").write_text("__global__ void k() { int x; }\n")
    assert bench.source_digest(["k.hip"]) != d0


def test_traffic_entries_name_known_configs():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        data = json.load(f)
    for config, ent in data.items():
        assert config in bench.CONFIGS
        cls = bench.CONFIGS[config][0]
        assert sorted(ent["sources"]) == sorted(cls.sources)
        assert set(ent["kernels"]) == set(cls.kernel_re)
        assert ent["hbm_bytes_per_launch"] > 0


@pytest.mark.parametrize("config", sorted(bench.CONFIGS))
def test_every_config_has_a_profile_summary(config):
    names = os.listdir(os.path.join(ROOT, "profiles"))
    assert any(f"config name in bench.py: {config}\n" in open(os.path.join(ROOT, "profiles", n)).read()
               for n in names if n.endswith(".txt"))
