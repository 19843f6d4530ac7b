"""bench.py's host logic on the CPU: the byte-for-byte check of device
outputs against the oracle's (bench.verify, run here on CPU tensors) catches
a single wrong byte and names where it is, and a run asking for more than one
GPU is refused before anything touches a GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _outputs():
    rng = np.random.default_rng(7)
    a = rng.integers(0, 2**16, 1 << 15, dtype=np.uint16)
    b = rng.integers(0, 2**32, 3001, dtype=np.uint32)
    rec = np.zeros(4, dtype=[("top1", "<f4"), ("top2", "<f4"), ("idx", "<i4"), ("reserved", "<i4")])
    rec["idx"] = [3, 1, 4, 1]
    dev = {"ring": torch.from_numpy(a.view(np.int16).copy()), "sum": torch.from_numpy(b.view(np.float32).copy()),
           "top2": torch.from_numpy(rec.view(np.uint8).copy())}
    return dev, {"ring": a, "sum": b, "top2": rec}


def test_verify_accepts_identical_bytes():
    dev, want = _outputs()
    done = bench.verify(dev, want, chunk=1000)
    assert done == {"ring": 1 << 16, "sum": 3001 * 4, "top2": 64}


@pytest.mark.parametrize("name,byte", [("ring", 0), ("ring", 65535), ("sum", 4321), ("top2", 63)])
def test_verify_names_the_first_wrong_byte(name, byte):
    dev, want = _outputs()
    flat = dev[name].view(torch.uint8).reshape(-1)
    flat[byte] ^= 0x10
    with pytest.raises(bench.Mismatch) as e:
        bench.verify(dev, want, chunk=1000)
    assert f"{name}: first differing byte at offset {byte}" in str(e.value)


def test_verify_refuses_a_size_mismatch():
    dev, want = _outputs()
    dev["sum"] = dev["sum"][:-1]
    with pytest.raises(bench.Mismatch):
        bench.verify(dev, want)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
