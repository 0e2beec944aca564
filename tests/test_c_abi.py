"""The C ABI used from plain C (tests/c/*.c, built by combine_shuffling_amd.build
with gcc against include/moe_shuffle.h): host calls on the CPU, and a whole
route plan / dispatch / combine on the GPU with the HIP C runtime."""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(HERE, "c", "build")


def _run(name):
    exe = os.path.join(BUILD, name)
    if not os.path.exists(exe):
        raise FileNotFoundError(f"{exe} is missing: run python -m combine_shuffling_amd.build")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    return res.stdout


def test_c_host_calls():
    if not os.path.exists(os.path.join(BUILD, "abi_host")):
        from combine_shuffling_amd import build as b
        b.build_c_tests()
    assert "abi_host ok" in _run("abi_host")


@pytest.mark.gpu
def test_c_route_dispatch_combine_on_gpu():
    assert "abi_gpu ok" in _run("abi_gpu")
