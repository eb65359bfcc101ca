"""Host-side checks of the benchmark's contract and of its byte and flop accounting."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_match_the_stated_totals():
    per = bench.alg_bytes_per_row()
    rows = bench.rows_per_layer()
    # forward 4 V_t + 4 BHN and backward 8 V_t + 4 BHN per layer, V_t = B*H*N*d*2 bytes
    vt = bench.B * bench.H * bench.N * bench.D * 2
    bhn = bench.B * bench.H * bench.N
    assert per["step"] * rows == (4 * vt + 4 * bhn) + (8 * vt + 4 * bhn)
    assert per["step"] * rows * bench.LAYERS == 1_619_001_344
    # the two stages move exactly the step's bytes: the backward reads back o and lse
    assert (per["fwd"] + per["bwd"]) * rows == per["step"] * rows


def test_dense_flops():
    assert bench.dense_flops_per_layer() == 2 * 8 * 4 * 64 * (4096 * 4097 // 2)
    assert abs(bench.dense_flops_per_layer() / 1e9 - 34.4) < 0.1


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    # the counter readings stay keyed to the kernel code: a comment edit keeps the hash,
    # a code edit changes it
    csrc = os.path.join(ROOT, "fibonacci_offset_transformer_amd", "csrc")
    pkg = tmp_path / "fibonacci_offset_transformer_amd" / "csrc"
    pkg.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        (pkg / name).write_text(open(os.path.join(csrc, name)).read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_sha()
    f = pkg / "fsa_forward.hip"
    text = f.read_text()
    f.write_text("// an added comment line\n" + text.replace("\n", "  // trailing note\n", 1) + "\n/* block */\n")
    assert bench.kernel_source_sha() == base
    f.write_text(text.replace("kNegInf", "-kNegInf", 1))
    assert bench.kernel_source_sha() != base
