"""Host logic of bench.py (no GPU): the single-GPU refusal, the byte and flop
models behind the roofline fields (pinned to a hand count), and the rule that
a stored HBM-traffic figure is only used while the kernel sources it was
measured on are unchanged."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_layer_bytes_match_a_hand_count():
    # B 8, T 4096, H 8, d 128, bf16 inputs: per token-head q, k, v (3 x 128 x 2 B),
    # beta (4 B) and the fp32 output (512 B); the fp32 final state once per head.
    per_token_head = 3 * 128 * 2 + 4 + 128 * 4
    expect = 8 * 4096 * 8 * per_token_head + 8 * 8 * 128 * 128 * 4
    assert bench.walk_algorithmic_bytes(8, 4096, 8, 128, 128, 2, False) == expect
    # an initial state is read once more
    assert bench.walk_algorithmic_bytes(8, 4096, 8, 128, 128, 2, True) == expect + 8 * 8 * 128 * 128 * 4
    # with the 4-byte gate g the fused kernel's figure is the one its bench line reports
    assert expect + 4 * 8 * 4096 * 8 == 341835776


def test_full_tile_flops_hand_count():
    # per token-head: 2*64*(3*128 + 2*128) for A, W, U and the intra output, 6*128*128 for the state products
    assert bench.gdn_flops_full_tile(1, 64, 1, 128, 128) == 64 * (2 * 64 * 640 + 6 * 128 * 128)


def _copy_tree(tmp_path):
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "gated_delta_rule_34_amd", "csrc"), root / "gated_delta_rule_34_amd" / "csrc")
    shutil.copy(os.path.join(ROOT, "gated_delta_rule_34_amd", "build.py"), root / "gated_delta_rule_34_amd")
    (root / "profiles").mkdir()
    return root


def test_traffic_figure_is_used_only_for_unchanged_sources(tmp_path, monkeypatch):
    root = _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    sha = bench.source_sha("fused_kernel")
    summary = root / "profiles" / "fused_kernel_layer_bf16_traffic.txt"
    summary.write_text(f"# test\nsource_sha: {sha}\ntraffic_bytes_per_launch: 123456\n")
    assert bench.read_traffic("fused_kernel", "layer_bf16") == 123456.0
    # any change to a source of the kernel makes the stored figure stale
    src = root / "gated_delta_rule_34_amd" / "csrc" / "gdn_tile.h"
    src.write_text(src.read_text() + "\n")
    assert bench.source_sha("fused_kernel") != sha
    assert bench.read_traffic("fused_kernel", "layer_bf16") is None
    # no summary at all: no figure
    assert bench.read_traffic("fused_kernel", "long_bf16") is None

