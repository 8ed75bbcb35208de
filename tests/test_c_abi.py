"""The C ABI used from plain C (tests/c_abi/zs_c_consumer.c): host calls on the
CPU; on the GPU one clipped step of a ragged shard through hipMalloc'd
buffers, checked bit for bit against the C oracle inside the same program."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c_abi"))
import build as c_abi_build  # noqa: E402


def _binary():
    return c_abi_build.BIN


def test_c_consumer_host():
    c_abi_build.build()
    r = subprocess.run([_binary(), "host"], capture_output=True, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.gpu
def test_c_consumer_gpu():
    assert os.path.exists(_binary()), "build it with __graft_entry__.build()"
    r = subprocess.run([_binary(), "gpu"], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
