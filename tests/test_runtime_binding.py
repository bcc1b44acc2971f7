"""The library binds to torch's HIP runtime whatever the import order (CPU).

torch ships a HIP runtime with the same soname as the system one; the
binding loads torch before the library, so that a layer created before any
tensor exists still resolves to the runtime that owns the tensors.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_resolves_hip_runtime_from_torch_when_loaded_first():
    code = r"""
import sys
sys.path.insert(0, %r)
import mixture_experts_layer_32_amd as pkg     # no torch import before this
pkg.lib()
import torch, os
tdir = os.path.realpath(os.path.join(os.path.dirname(torch.__file__), "lib"))
maps = open("/proc/self/maps").read()
hips = sorted({l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l})
print(hips)
assert len(hips) == 1, hips
assert os.path.realpath(hips[0]).startswith(tdir), hips
""" % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
