"""Host-side checks of the benchmark's contract (no GPU): the one-GPU exit,
the algorithmic byte counts behind every GB/s and roofline figure, and the
recorded PMC traffic that bench.py reports only while the kernel sources
still hash to it.

The byte counts are fixed by the operation, not by the kernels: weights
H*128*512 (bf16) or H*128*512 + H*128*16 (E4M3 payload + E8M0 scales),
q_nope M*H*128 bf16, q_pe M*H*64 bf16, the [M,H,576] output (bf16 or E4M3)
and 4 bytes of q_scale for E4M3 output; for attention every cached row of
576 bf16 once, the queries, the live block-table entries, the lengths and
the bf16 [M,H,512] output."""

import hashlib
import subprocess
import sys
from pathlib import Path

import pytest

import bench
import workloads as wl

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("M,H,wf,od,want", [
    (1, 8, wl.WEIGHT_BF16, wl.OUT_BF16, 1_060_864),      # smallest case: H=8, M=1
    (1, 16, wl.WEIGHT_BF16, wl.OUT_BF16, 2_121_728),
    (32, 16, wl.WEIGHT_BF16, wl.OUT_BF16, 2_883_584),
    (7, 11, wl.WEIGHT_BF16, wl.OUT_BF16, 1_560_064),     # odd head count
    (32, 11, wl.WEIGHT_BF16, wl.OUT_BF16, 1_982_464),
    (1, 16, wl.WEIGHT_MXFP8, wl.OUT_BF16, 1_105_920),
    (32, 16, wl.WEIGHT_MXFP8, wl.OUT_BF16, 1_867_776),
    (32, 16, wl.WEIGHT_BF16, wl.OUT_E4M3, 2_588_676),    # decode-step layers
    (32, 16, wl.WEIGHT_MXFP8, wl.OUT_E4M3, 1_572_868),
])
def test_algorithmic_bytes_per_call(M, H, wf, od, want):
    assert wl.algorithmic_bytes(M, H, wf, od) == want


def test_decode_step_bytes():
    # 32 BF16 + 32 MXFP8 layers, H = 16, M = 32, E4M3 output.
    step = 32 * wl.algorithmic_bytes(32, 16, wl.WEIGHT_BF16, wl.OUT_E4M3) + \
        32 * wl.algorithmic_bytes(32, 16, wl.WEIGHT_MXFP8, wl.OUT_E4M3)
    assert step == 133_169_408


def test_k192_bytes():
    # The pages' GLM shape: 1.5x the weight bytes and the q_nope bytes of K = 128.
    assert wl.algorithmic_bytes(1, 8, wl.WEIGHT_BF16, wl.OUT_BF16, K=192) == \
        8 * 192 * 512 * 2 + 1 * 8 * 192 * 2 + 1 * 8 * 64 * 2 + 1 * 8 * 576 * 2


def test_attention_bytes():
    # 32 sequences x 4096 tokens, 16 heads, pages of 64.
    rows = 32 * 4096 * 576 * 2
    q = 32 * 16 * 576 * 2
    table = 32 * 64 * 4
    lens = 32 * 4
    out = 32 * 16 * 512 * 2
    assert wl.attn_algorithmic_bytes([4096] * 32, 16) == rows + q + table + lens + out == 152_117_376
    # ragged, with an empty sequence and a partial last page
    assert wl.attn_algorithmic_bytes([0, 65, 64], 2) == \
        129 * 1152 + 3 * 2 * 1152 + (0 + 2 + 1) * 4 + 3 * 4 + 3 * 2 * 1024


@pytest.mark.parametrize("name,sources,key", [
    ("fused_query_decode_step_traffic.txt", bench.KERNEL_SOURCES, "traffic_bytes_per_launch"),
    ("dense_mla_attention_traffic.txt", bench.ATTN_SOURCES, "traffic_bytes_per_call"),
])
def test_recorded_traffic_follows_the_sources(name, sources, key, tmp_path, monkeypatch):
    rec = ROOT / "profiles" / name
    assert rec.exists(), name
    text = rec.read_text()
    kv = dict(line.split(None, 1) for line in text.splitlines() if line and not line.startswith("#"))
    assert int(kv[key]) > 0
    # A copy of the tree whose record names a different source hash reports nothing.
    prof = tmp_path / "profiles"
    prof.mkdir()
    csrc = tmp_path / "mla_decode_query_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in sources:
        (csrc / f).write_bytes((ROOT / "mla_decode_query_amd" / "csrc" / f).read_bytes())
    good = hashlib.sha256(b"".join((csrc / f).read_bytes() for f in sources)).hexdigest()
    lines = [ln for ln in text.splitlines() if not ln.startswith("kernel_source_sha256")]
    (prof / name).write_text("\n".join(lines + [f"kernel_source_sha256 {good}"]) + "\n")
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench._recorded(name, sources, key) == int(kv[key])
    (csrc / sources[0]).write_bytes((csrc / sources[0]).read_bytes() + b"\n// edited\n")
    assert bench._recorded(name, sources, key) is None


def test_cpu_baseline_object_on_a_tiny_budget():
    """The cpu_baseline object the bench line carries: the oracle as it stands,
    timed on the host over the step's layers (a budget small enough for the
    CPU suite), with its thread count, and a single-thread figure beside it."""
    r = bench.cpu_baseline_leg(wl, None, 0.05)
    assert {"value", "unit", "cores", "kind", "sample", "single_thread"} <= set(r)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 16 and f"{r['cores']} threads" in r["sample"]
    one = r["single_thread"]
    assert one["cores"] == 1 and one["value"] > 0 and one["layer_calls"] >= 1
