"""libmq and torch share one HIP runtime whatever the order they are used in.

Loading libmq before torch had imported its bundled HIP runtime put two copies of
the runtime in one process (the library's /opt/rocm one and torch's); on the GPU the
second to open the device found none.  The binding now imports torch before it loads
the library.  Checked here in a fresh process: load the library first, then import
torch, and count the HIP runtime libraries mapped.
"""

import os
import subprocess
import sys

import pytest

from block_quantized_matmul_mq_amd import mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
from block_quantized_matmul_mq_amd import mq
mq.load()
import torch
maps = open("/proc/self/maps").read().split("\n")
print(len(set(l.split()[-1] for l in maps if "libamdhip64" in l)))
"""


@pytest.mark.skipif(not os.path.exists(mq.LIB_PATH), reason="libmq.so not built")
def test_library_first_then_torch_maps_one_hip_runtime():
    out = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT)], capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout
