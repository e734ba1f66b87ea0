"""Host check of the address ranges of every kernel (forward, prep, backward
and the adjacent maps; tests/kernel_bounds.py) for every problem the GPU
tests, the benchmark and smoke() launch, in both scan modes, with and without
the decay bridge, the epilogue and the RMSNorm gain; and checks that the model
itself catches planted mistakes."""

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
    import test_gpu_widths as W  # widths between the built ones
    out += [(n, w, False) for n, w in W.CASES.items()]
    out += [(n, base.scaled(name=n, **kw), True) for n, kw in W.PREP_CASES.items()]
    return out


SHAPES = _shapes()


def _prob(w, **kw):
    """The model's problem: a width between the built ones runs at the next."""
    D = next(b for b in (16, 32, 64, 128) if b >= w.d)
    return KB.Prob(B=w.B, H=w.H, T=w.T, gh=w.grid_h, gw=w.grid_w, D=D, L=w.L, C=w.chunk, bf16=w.dtype == "bf16",
                   Du=w.d if D != w.d else 0, **kw)


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


def _bwd_shapes():
    """(name, workload, flags) for every backward launch of the GPU suite and
    the benchmark (bench.py --backward runs the 768p clip)."""
    import test_gpu_backward as GB
    out = [(n, c["w"], dict(epilogue=c.get("epilogue", True), bridge=c.get("bridge", False), gamma=c.get("gain", False)))
           for n, c in GB.CASES.items()]
    out.append(("768p", GB.BASE, {}))
    out.append(("graphs", synth.WORKLOADS["768p_bf16"].scaled(name="graphs", H=2, T=12, grid_h=5, grid_w=7, L=8), {}))
    out.append(("long_clip", synth.WORKLOADS["long_prep_bf16"], {}))
    for h in (3, 8):
        out.append((f"768p_h{h}", synth.WORKLOADS["768p_bf16"].scaled(name="h", H=h), {}))
    import test_gpu_widths as W  # widths between the built ones
    import test_gpu_training_f32 as F  # float32 inputs
    for cases in (W.BWD_CASES, F.CASES):
        out += [(n, c["w"], dict(epilogue=c.get("epilogue", True), bridge=c.get("bridge", False),
                                 gamma=c.get("gain", False))) for n, c in cases.items()]
    out.append(("stress_f32", synth.WORKLOADS["stress_f32"], {}))
    return out


BWD_SHAPES = _bwd_shapes()


@pytest.mark.parametrize("name,w,flags", BWD_SHAPES, ids=[s[0] for s in BWD_SHAPES])
def test_backward_kernels_stay_in_bounds(name, w, flags):
    """Every kernel of the three backward stages, each workspace part checked
    as a buffer of its own, with and without the epilogue and the bridge."""
    checked = 0
    for epi in (flags.get("epilogue", True), not flags.get("epilogue", True)):
        for bridge in (flags.get("bridge", False), True):
            r = KB.model_backward(_prob(w, epilogue=epi, bridge=bridge, gamma=flags.get("gamma", False) and epi,
                                        dgain=epi))
            assert not r.errors, (name, epi, bridge, r.errors[:5])
            checked += r.checked
    assert checked > 0


def test_padded_copies_are_modelled():
    """A width between the built ones adds the copies in and out, and a
    padded buffer one chunk short is reported."""
    import test_gpu_widths as W
    p = _prob(W.CASES["d48_bf16"], gamma=True)
    assert p.D == 64 and p.Du == 48
    r = KB.model_forward(p)
    assert not r.errors and r.checked
    S = KB.sizes(p)
    r2 = KB.Report()
    KB.model_copy_rows(r2, "caller q", p.B * p.T * p.U * p.H * 48 * 2, "padded q", S["q"] - 16, 96, 128, 96,
                       p.B * p.T * p.U * p.H)
    assert any("padded q" in e for e in r2.errors)
    r3 = KB.Report()
    KB.model_copy_rows(r3, "padded out", S["out"], "caller out", p.B * p.T * p.U * p.H * 48 * 2 - 2, 128, 96, 96,
                       p.B * p.T * p.U * p.H)
    assert any("caller out" in e for e in r3.errors)


def test_float32_backward_model_catches_planted_mistakes():
    """The float32 stages' buffers one element short are reported."""
    import test_gpu_training_f32 as F
    p = _prob(F.CASES["stress_d128_bridge"]["w"], bridge=True, dgain=True, gamma=True)
    assert not p.bf16
    for part in ("rstates_t", "dout", "dsq", "dq", "dgate", "dk", "dv", "dbeta", "dbeta_text", "dA", "gain"):
        S = KB.bwd_sizes(p)
        S[part] -= 4
        r = KB.Report()
        KB.model_backward_f32(p, r, S)
        KB.model_gram_bwd_f32(p, r, S)
        assert any(part in e for e in r.errors), (part, r.errors[:3])


def test_backward_slot_sizes_match_the_layout():
    """The fragment counts the kernels use fill exactly the slots the
    workspace layout sizes (readout states, gradient planes)."""
    for d in (16, 32, 64, 128):
        p = KB.Prob(B=1, H=2, T=7, gh=3, gw=4, D=d, L=2)
        S = KB.bwd_sizes(p)
        NF = KB._readout_frags(d)
        assert 2 * NF * 16 * 2 * (p.nc + 1) == S["rstates_t"]
        NFg = (d // 16) * (d // 32) * 64 if d >= 32 else 64
        assert 5 * NFg * 16 * 2 * (p.T + 1) == S["gmats"]


def test_backward_model_catches_planted_mistakes():
    """Each workspace part one slot short is reported by the kernel that
    addresses its last slot."""
    w = synth.WORKLOADS["768p_bf16"].scaled(name="m", H=2, T=12, grid_h=5, grid_w=7, L=8)
    p = _prob(w, bridge=True, dgain=True)
    dd = p.D * p.D * 4
    for part, short in (("states_r", dd), ("lam_f", dd), ("dsq", dd), ("dF", dd), ("lam_final", dd),
                        ("gmats", 5 * p.D * p.D * 2), ("rstates_t", 16), ("dout", 2), ("p32", dd), ("tmp", dd),
                        ("gain", 4), ("dgamma", 4)):
        S = KB.bwd_sizes(p)
        S[part] -= short
        r = KB.Report()
        KB.model_pack_states_t(p, r, S) if part == "rstates_t" else None
        KB.model_readout_bwd(p, r, S)
        KB.model_gram_plain(p, r, S)
        KB.model_backward_scan(p, r, S)
        if part not in ("rstates_t",):
            KB.model_backward_gram(p, r, S)
        assert any(part in e for e in r.errors), (part, r.errors[:3])


def _proj_shapes():
    """(name, workload, d_model) for every launch of the adjacent maps in the
    GPU suite and bench.py --adjacent."""
    import test_gpu_adjacent as GA
    out = [(n, w, dm) for n, (w, dm) in GA.CASES.items()]
    base = GA.BASE
    out.append(("768p", base, base.H * base.d))
    out.append(("layer", base.scaled(name="layer", B=1, T=11, grid_h=4, grid_w=6, H=2, d=64, L=8), 160))
    out.append(("graphs", base.scaled(name="graphs", H=2, T=12, grid_h=5, grid_w=7, L=8), 192))
    import test_gpu_widths as W  # the maps run at the caller's width, whatever it is
    out += [(n, w, dm) for n, (w, dm) in W.ADJ_CASES.items()]
    return out


PROJ_SHAPES = _proj_shapes()


@pytest.mark.parametrize("name,w,dm", PROJ_SHAPES, ids=[s[0] for s in PROJ_SHAPES])
def test_adjacent_maps_stay_in_bounds(name, w, dm):
    # plain products over H d channels: the caller's width, not a built one
    p = KB.Prob(B=w.B, H=w.H, T=w.T, gh=w.grid_h, gw=w.grid_w, D=w.d, L=w.L, C=w.chunk, bf16=True)
    for r in (KB.model_gates(p, dm), KB.model_out_proj(p, dm, True), KB.model_out_proj(p, dm, False)):
        assert not r.errors, (name, r.errors[:5])
        assert r.checked > 0


def test_adjacent_model_catches_planted_mistakes():
    """A gate or beta output one row short, weights without the beta rows, a
    partial-sum part one frame short: each is reported."""
    w = synth.WORKLOADS["768p_bf16"].scaled(name="m", H=2, T=5, grid_h=9, grid_w=30, L=0)
    p, dm = _prob(w), 96
    M = w.B * w.T * w.U
    for buf, short in (("gate", 2 * w.H * w.d), ("beta", 2 * w.H), ("w_gb", 2 * w.H * dm), ("partial", 4 * dm),
                       ("x", 2), ("alpha", 4)):
        real = KB.proj_sizes
        KB.proj_sizes = lambda p_, dm_, b=buf, s=short: dict(real(p_, dm_), **{b: real(p_, dm_)[b] - s})
        try:
            r = KB.model_gates(p, dm)
        finally:
            KB.proj_sizes = real
        assert any(buf in e for e in r.errors), (buf, r.errors[:3])
    assert M > 256  # several M-tiles, a ragged last one
