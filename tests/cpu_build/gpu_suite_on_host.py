"""Run GPU test files on the CPU build: the Python of the GPU suite (the tests,
the harness, the binding's argument checks and marshalling) executed against
libvdn_vda_sim.so, the library's HIP sources compiled for the host.

    python tests/cpu_build/gpu_suite_on_host.py tests/test_gpu_widths.py -m gpu -k "not 768p"

torch's 'cuda' tensors become host tensors, 256-byte aligned as the GPU
allocator gives them; the binding loads the host library, and passes no
stream.  Graph capture (tests/test_gpu_graphs.py) has no host equivalent, and
the full-size cases take the emulator hours: select with -k.  What this checks
is the test code and the host side of the path, not the GPU.
"""

from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
sys.path[:0] = [ROOT, TESTS]

import pytest  # noqa: E402
import torch  # noqa: E402

from frame_wise_delta_02_amd import binding as bd  # noqa: E402
from cpu_build import build as CB  # noqa: E402
from cpu_build import sim as S  # noqa: E402

_orig = {}


def _aligned(t, copy=False):
    """The same values in a 256-byte aligned buffer (always a new one with copy,
    as a transfer to the device gives: the host array stays untouched when the
    library writes the copy)."""
    if t.numel() == 0 or (t.data_ptr() % 256 == 0 and not copy):
        return t
    es = t.element_size()
    raw = _orig["empty"](t.numel() + 256 // es + 1, dtype=t.dtype)
    off = ((-raw.data_ptr()) % 256) // es
    out = raw[off:off + t.numel()].view(t.shape)
    out.copy_(t)
    return out


def _host(dev):
    return "cpu" if isinstance(dev, (str, torch.device)) and str(dev).startswith("cuda") else dev


def install():
    bd._lib = S.load(CB.build(S.OUT, "lib"))
    bd._stream = lambda: None

    def check(x, name, dev):
        if x is not None and not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    bd._check = check
    to = torch.Tensor.to

    def to_host(self, *a, **k):
        moves = any(str(x).startswith("cuda") for x in a) or str(k.get("device", "")).startswith("cuda")
        a = tuple(_host(x) for x in a)
        if "device" in k:
            k["device"] = _host(k["device"])
        return _aligned(to(self, *a, **k).contiguous(), copy=moves)

    torch.Tensor.to = to_host
    torch.Tensor.cuda = lambda self, *a, **k: _aligned(self.contiguous(), copy=True)
    torch.cuda.synchronize = lambda *a, **k: None
    for name in ("empty", "zeros", "ones", "full", "empty_like", "zeros_like", "full_like", "from_numpy"):
        f = _orig[name] = getattr(torch, name)

        def make(f=f):
            def g(*a, **k):
                if "device" in k:
                    k["device"] = _host(k["device"])
                return _aligned(f(*a, **k))
            return g

        setattr(torch, name, make())


if __name__ == "__main__":
    install()
    sys.exit(pytest.main(sys.argv[1:] + ["-p", "no:cacheprovider", "-q", "-x", "--rootdir", ROOT]))
