"""vdn_vda_forward_noalloc against vdn_vda_forward.

The no-allocation entry point runs the same kernels with the library's own
device array as the workspace; on the same inputs its output must equal the
workspace entry point's bit for bit.  Two calls in a row, the second on a
smaller problem (so the array holds the first call's intermediates when the
second starts), each with and without the epilogue.
"""

import pytest

from frame_wise_delta_02_amd import binding as bd
from frame_wise_delta_02_amd import synth
import gpu_harness as G

pytestmark = pytest.mark.gpu

CASES = [
    # 8 heads x 40 frames x 1560 tokens at d = 64: 22.6 MiB of workspace
    synth.WORKLOADS["small_bf16"],
    # smaller: 3 heads x 17 frames x 100 tokens at d = 128, ragged tiles
    synth.WORKLOADS["768p_bf16"].scaled(name="noalloc_small", H=3, T=17, grid_h=10, grid_w=10, L=37),
]


def _same(a, b):
    import torch
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


def test_noalloc_equals_forward_on_two_calls():
    import torch
    for w in CASES:
        desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, True)
        assert bd.workspace_bytes(desc) <= 64 << 20
        x = synth.make_inputs(w)
        d = {k: G.to_device(v, w.dtype) for k, v in x.items()}
        for epi in (False, True):
            G.say(f"noalloc {w.name} epilogue={epi}")
            args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["k_text"], d["v_text"], d["beta_text"],
                    d["gate"], None)
            ref = bd.forward(*args, grid=(w.grid_h, w.grid_w), chunk=w.chunk, epilogue=epi)
            got = bd.forward_noalloc(*args, grid=(w.grid_h, w.grid_w), chunk=w.chunk, epilogue=epi)
            torch.cuda.synchronize()
            diff = (got.double() - ref.double()).abs().max().item()
            G.say(f"noalloc {w.name} epilogue={epi}: max |noalloc - forward| = {diff:.3e}")
            assert _same(got, ref), diff
