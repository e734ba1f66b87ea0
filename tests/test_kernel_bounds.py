"""Host check of every forward kernel's address ranges (tests/kernel_bounds.py)
for every problem the GPU tests, the benchmark and smoke() launch, in both scan
modes, with and without the decay bridge, the epilogue and the RMSNorm gain;
and checks that the model itself catches planted mistakes."""

import pytest

import kernel_bounds as KB
from frame_wise_delta_02_amd import synth


def _shapes():
    """(name, workload, runs prep) for every launch of the GPU suite and the benchmark."""
    import test_gpu_parity as P
    out = [(n, w, w.prep) for n, w in synth.WORKLOADS.items()]
    out += [(n, w, False) for n, w in P.EDGE.items()]
    out += [(n, w, False) for n, w in P.BRIDGE.items()]
    base = synth.WORKLOADS["long_prep_bf16"]
    out += [(n, base.scaled(name=n, **kw), True) for n, kw in P.PREP_EDGE.items()]
    out += [(n, base.scaled(name=n, **kw), True) for n, kw in P.QL2.items()]
    for dt in ("bf16", "f32"):
        out.append((f"prep_small_{dt}", base.scaled(name="ps", dtype=dt, H=2, T=9, grid_h=6, grid_w=10, L=8), True))
    out.append(("smoke", synth.WORKLOADS["768p_bf16"].scaled(name="smoke", H=2, T=16, grid_h=6, grid_w=11, L=12), False))
    out.append(("noalloc_small", synth.WORKLOADS["768p_bf16"].scaled(name="na", H=3, T=17, grid_h=10, grid_w=10, L=37),
                False))
    for h in (3, 4, 6, 8, 12, 16):  # bench.py --heads sweeps of the 768p clip
        out.append((f"768p_h{h}", synth.WORKLOADS["768p_bf16"].scaled(name="h", H=h), False))
    return out


SHAPES = _shapes()


def _prob(w, **kw):
    return KB.Prob(B=w.B, H=w.H, T=w.T, gh=w.grid_h, gw=w.grid_w, D=w.d, L=w.L, C=w.chunk, bf16=w.dtype == "bf16", **kw)


@pytest.mark.parametrize("name,w,prep", SHAPES, ids=[s[0] for s in SHAPES])
def test_forward_kernels_stay_in_bounds(name, w, prep):
    checked = 0
    for chunked in (False, True):
        for bridge in (False, True):
            for epi, gamma in ((False, False), (True, True)):
                r = KB.model_forward(_prob(w, chunked=chunked, bridge=bridge, epilogue=epi, gamma=gamma), prep=prep)
                assert not r.errors, (name, chunked, bridge, r.errors[:5])
                checked += r.checked
    assert checked > 0


def test_model_catches_planted_mistakes():
    """The checks fire: a buffer one element short, a descriptor past its
    buffer, and an offset that wraps 32 bits are all reported."""
    w = synth.WORKLOADS["768p_bf16"]
    p = _prob(w)
    S = KB.sizes(p)
    r = KB.Report()
    r.ptr("k", "q", S["q"], 0, S["q"] + 2)
    r.rsrc("k", "q", S["q"], S["q"] - 256, 512, 0, 16)
    r.rsrc("k", "q", S["q"], 0, 512, KB.U32 - 8, 16)
    assert len(r.errors) == 3
    # a frame whose token rows need more than 32-bit offsets: 4032 tokens x
    # 24 heads x 128 channels x 2 B is 24.8 MB, so 200 such frames per head row
    # stride overflow only with absurd head counts; emulate with H = 4500
    big = KB.Prob(B=1, H=4500, T=3, gh=48, gw=84, D=128, L=0)
    r2 = KB.Report()
    KB.model_readout(big, r2)
    assert any("wraps" in e for e in r2.errors)
