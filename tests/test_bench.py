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


def test_plan_launch_names_the_dominant_kernel_and_grid():
    w = synth.WORKLOADS[1]          # M16 K8192 N8192
    assert bench.plan_launch("stream_mt1_nt2_w4_k128_d4_wnt_s1", w) == \
        ("stream_kernel", "stream_kernel<1, 2, 4, 128, 4, 1, true>", (8192 // 32) * 256)
    w3 = synth.WORKLOADS[2]         # M64 K8192 N28672
    assert bench.plan_launch("stream_mt4_nt7_w4_k128_d3_s1", w3) == \
        ("stream_kernel", "stream_kernel<4, 7, 4, 128, 3, 0, true>", (28672 // 112) * 256)
    w0 = synth.WORKLOADS[0]         # M16 K8192 N1024: split plans, the streaming kernel dominates
    assert bench.plan_launch("stream_mt1_nt1_w4_k128_d6_s4_atomic", w0) == \
        ("stream_kernel", "stream_kernel<1, 1, 4, 128, 6, 0, true>", 64 * 4 * 256)
    assert bench.plan_launch("stream_mt1_nt1_w4_k128_d6_s4", w0)[2] == 64 * 4 * 256
    # the K-walk stride (_r1) is a runtime argument of the same kernel
    assert bench.plan_launch("stream_mt1_nt1_w4_k128_d6_s4_atomic_r1", w0) == \
        bench.plan_launch("stream_mt1_nt1_w4_k128_d6_s4_atomic", w0)
    assert bench.plan_launch("stream_mt4_nt7_w4_k128_d3_s1_r1", w3) == bench.plan_launch("stream_mt4_nt7_w4_k128_d3_s1", w3)
    w4 = synth.WORKLOADS[4]         # M4096 N8192: 512 tiles of 256 x 256, one persistent workgroup per CU
    assert bench.plan_launch("gemmpp64p_256x256x64_w4x2_g4", w4) == \
        ("gemm_pp64p_kernel", "gemm_pp64p_kernel<256, 4, false>", 256 * 512)
    assert bench.plan_launch("gemmpp64d_256x192x64_w4x2_g8", synth.WORKLOADS[3])[1] == \
        "gemm_pp64p_kernel<192, 8, true>"
    assert bench.plan_launch("gemmpp64_256x192x64_w4x2_g4", synth.WORKLOADS[3]) == \
        ("gemm_pp64_kernel", "gemm_pp64_kernel<192, 4>", 32 * 16 * 512)
    with pytest.raises(SystemExit):
        bench.plan_launch("generic", w)


def test_counters_follow_the_kernel_sources():
    """Traffic is reported only while the sources the counters were taken on
    are unchanged: the stored hash is compared with the files' hash."""
    h = bench.kernel_sources_hash("stream_kernel")
    assert isinstance(h, str) and len(h) >= 16
    assert h == bench.kernel_sources_hash("stream_kernel")
    assert h != bench.kernel_sources_hash("gemm_kernel")
