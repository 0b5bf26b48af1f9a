"""Host-side checks of bench.py: the one-GPU guard and the op bookkeeping (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_every_op_has_kernels_and_work():
    # the step's ops and the two gradients timed on their own
    ops = ["quantize_xw", "quantize_g", "conv_fwd", "conv_backward", "conv_wgrad", "conv_dgrad"]
    for op in ops:
        assert bench.OP_KERNELS.get(op), op
    # the one-call backward runs the weight-gradient and input-gradient kernels
    assert set(bench.OP_KERNELS["conv_wgrad"]) <= set(bench.OP_KERNELS["conv_backward"])
    assert set(bench.OP_KERNELS["conv_dgrad"]) <= set(bench.OP_KERNELS["conv_backward"])


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)
