"""Host logic of bench.py that needs no GPU: the code hash that keys the
committed HBM counters to the kernels they were taken on."""
import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(root):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.ROOT = root
    return mod


def _tree(tmp_path, text):
    src = tmp_path / "vla_robot_policy_amd" / "csrc"
    src.mkdir(parents=True, exist_ok=True)
    (src / "k.h").write_text(text)
    return str(tmp_path)


def test_strip_comments_keeps_strings():
    b = _bench(ROOT)
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // y /* z */";\n\n'
    assert b._strip_comments(src) == 'int a = 1;\n const char* s = "x // y /* z */";'


@pytest.mark.parametrize("edit, same", [
    ("int f(int x) { return x + 1; }  // adds one\n", True),          # comment change only
    ("/* header */\nint f(int x) { return x + 1; }\n\n", True),       # comment and blank lines
    ("int f(int x) { return x + 2; }\n", False),                      # code change
])
def test_code_hash_ignores_comments_only(tmp_path, edit, same):
    base = _bench(_tree(tmp_path / "a", "int f(int x) { return x + 1; }\n")).kernel_source_sha()
    other = _bench(_tree(tmp_path / "b", edit)).kernel_source_sha()
    assert (base == other) == same


def test_committed_traffic_matches_sources_or_is_withheld():
    b = _bench(ROOT)
    t = b.measured_traffic("dit.layers", 4)
    assert t is None or t > 0
    assert b.measured_traffic("no.such.label", 4) is None
    assert b.measured_traffic("dit.layers", 99) is None          # another workload's counters


def test_phase_of_covers_every_step_label():
    b = _bench(ROOT)
    labels = ["vit.patch_embed", "vit.ln1", "mrg.fc1", "llm.stage", "llm.rope_table", "llm.qkv", "llm.final_norm",
              "proj", "dit.time_embed", "dit.adaln", "dit.cross_kv", "dit.cross_vt", "dit.clear", "dit.in_proj",
              "dit.layers", "dit.tail", "dit.sa_qkv", "dit.mlp_down"]
    ph = {lb: b.phase_of(lb) for lb in labels}
    assert "other" not in ph.values(), ph
    assert ph["dit.cross_kv"] == "dit_once" and ph["dit.layers"] == "dit_step" and ph["dit.sa_qkv"] == "dit_step"
