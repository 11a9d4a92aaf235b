"""Host logic of bench.py (CPU only): the algorithmic byte count behind the
roofline figure, the guard that reports measured traffic only for the
gemm.hip it was taken on, and the refusal of more than one GPU."""
import hashlib
import os
import subprocess
import sys

import bench


def test_gemm_bytes_of_the_dominant_shape():
    # FP8 A [64][7168] + FP8 B [2112][7168] + FP32 sa [56][64] + FP32 sb
    # [17][56] + BF16 D [64][2112], written out operand by operand
    M, N, K = 64, 2112, 7168
    a, b = M * K, N * K
    sa, sb = 4 * (K // 128) * M, 4 * 17 * (K // 128)
    d = 2 * M * N
    assert bench.gemm_bytes(M, N, K) == a + b + sa + sb + d == 15_886_048
    assert bench.gemm_bytes(M, N, K, out_bytes=4) == a + b + sa + sb + 2 * d


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    src = tmp_path / "gemm.hip"
    src.write_bytes(b"// kernel source\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    assert bench.measured_traffic(str(prof)) is None                      # no summary
    prof.write_text(f"source_sha256: {digest}\ntraffic_bytes_per_launch: 26420910\n")
    assert bench.measured_traffic(str(prof)) == 26420910
    src.write_bytes(b"// kernel source, edited\n")
    assert bench.measured_traffic(str(prof)) is None                      # stale summary
    prof.write_text(f"source_sha256: {hashlib.sha256(src.read_bytes()).hexdigest()}\n")
    assert bench.measured_traffic(str(prof)) is None                      # no figure
    other = tmp_path / "decode.hip"
    other.write_bytes(b"// another kernel file\n")
    prof.write_text(f"source_file: decode.hip\nsource_sha256: "
                    f"{hashlib.sha256(other.read_bytes()).hexdigest()}\n"
                    f"traffic_bytes_per_launch: 123\n")
    assert bench.measured_traffic(str(prof)) == 123                       # named source file


def test_percentile_and_quantize_bytes():
    vals = sorted(float(v) for v in range(1, 101))
    assert bench.percentile(vals, 0.5) in (50.0, 51.0) and bench.percentile(vals, 0.95) == 95.0
    assert bench.quant_bytes(64, 7168) == 64 * 7168 * 5 + 4 * 64 * 56


def test_bad_step_counts_are_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--steps", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and r.stdout == ""


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
