"""Host-side logic of bench.py (CPU): the single-GPU contract and the plan
name -> kernel launch mapping that matches counter rows to plans."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stream_plan_launch_names_the_kernel_and_grid():
    w = synth.WORKLOADS[1]          # M16 K8192 N8192
    name, items = bench.stream_plan_launch("stream_mt1_nt2_w4_k128_d4_wnt_s1", w)
    assert name == "stream_kernel<1, 2, 4, 128, 4, 1, true>"
    assert items == (8192 // 32) * 256      # 256 workgroups of 4 waves
    w3 = synth.WORKLOADS[2]         # M64 K8192 N28672
    name, items = bench.stream_plan_launch("stream_mt4_nt7_w4_k128_d3_s1", w3)
    assert name == "stream_kernel<4, 7, 4, 128, 3, 0, true>"
    assert items == (28672 // 112) * 256
    with pytest.raises(SystemExit):
        bench.stream_plan_launch("stream_mt1_nt1_w4_k128_d6_s4", w)      # split plans add a kernel
    with pytest.raises(SystemExit):
        bench.stream_plan_launch("gemmpp64p_256x256x64_w4x2_g4", w)


def test_counters_follow_the_kernel_sources():
    """Traffic is reported only while the sources the counters were taken on
    are unchanged: the stored hash is compared with the files' hash."""
    h = bench.kernel_sources_hash("stream_kernel")
    assert isinstance(h, str) and len(h) >= 16
    assert h == bench.kernel_sources_hash("stream_kernel")
    assert h != bench.kernel_sources_hash("gemm_kernel")
