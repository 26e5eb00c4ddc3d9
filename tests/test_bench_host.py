"""Host checks of bench.py that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_step_bytes_are_the_algorithmic_bytes():
    sys.path.insert(0, ROOT)
    import bench
    elems = bench.M * bench.N
    # dual-axis: bf16 in, two E4M3 copies and two E8M0 scale arrays out (4.0625 B/element)
    assert round(elems * bench.DUAL_BYTES_PER_ELEM) == 1_090_519_040
    # MX9 pack of bf16 and unpack to bf16: 3.125 B/element each way
    assert round(elems * bench.PACK_BF16_BYTES_PER_ELEM) == round(elems * bench.UNPACK_BF16_BYTES_PER_ELEM) == 838_860_800
