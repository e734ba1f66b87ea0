"""Host checks of bench.py's accounting: the algorithmic bytes and FLOP it
divides by (the figures its roofline objects report), and that it refuses
more than one GPU before touching any device."""

import os
import subprocess
import sys

import bench
from frame_wise_delta_02_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_768p_bytes():
    w = synth.WORKLOADS["768p_bf16"]
    tok = 60 * 4032 * 24
    # readout: Q and the gate logits in, O out, bfloat16, d = 128
    assert bench.algorithmic_bytes(w, "readout") == tok * 3 * 128 * 2 == 4_459_069_440
    # gram: K, V and beta of the 58 interior frames
    assert bench.algorithmic_bytes(w, "gram") == 58 * 4032 * 24 * (2 * 128 + 1) * 2
    # whole job: Q, gate and O of every frame; K, V, beta and alpha (fp32) of
    # the 58 frames the scans absorb (the anchors' are never read); the 256
    # text tokens' K, V, beta
    inner = 58 * 4032 * 24
    assert bench.job_bytes(w) == (tok * 3 * 128 * 2 + inner * (2 * 128 + 1) * 2 + 58 * 24 * 128 * 4
                                  + 256 * 24 * (2 * 128 + 1) * 2) == 7_347_787_776
    # the job's gram share is exactly the gram stage's bytes plus the text tokens
    assert bench.algorithmic_bytes(w, "gram") == inner * (2 * 128 + 1) * 2
    # matrix-core work: [A; B] is 2d x d per token of the 58 frames and the
    # text, the readout d x d per token
    assert bench.mfma_flops(w, "gram") == 2 * (inner + 24 * 256) * 2 * 128 * 128
    assert bench.mfma_flops(w, "readout") == 2 * tok * 128 * 128


def test_long_clip_prep_accounting():
    w = synth.WORKLOADS["long_prep_bf16"]
    out = w.B * w.T * w.U * w.H * w.d
    # per launch (one of K, V): 30 fp32 multiply-adds per output element
    assert bench.prep_flops(w) == 60 * out
    # both launches: K, V in and K^, V^ out in bfloat16
    assert bench.algorithmic_bytes(w, "prep") == 4 * out * 2
    # arithmetic intensity above the fp32 ridge: the prep is ALU-bound
    ridge = bench.VALU_F32_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    assert bench.prep_flops(w) / (bench.algorithmic_bytes(w, "prep") / 2) > ridge


def test_long_clip_job_bytes():
    """The long clip reads K and V of every frame (the temporal taps reach the
    anchors); the prepared K^, V^ are intermediates and are not counted."""
    w = synth.WORKLOADS["long_prep_bf16"]
    tok = 120 * 4032 * 24
    inner = 118 * 4032 * 24
    want = tok * 5 * 128 * 2 + inner * 2 + 118 * 24 * 128 * 4 + 512 * 24 * (2 * 128 + 1) * 2
    assert bench.job_bytes(w) == want == 14_894_168_064
    # no K^, V^ round trip in the job's bytes
    assert bench.job_bytes(w) < bench.algorithmic_bytes(w, "prep") + tok * 3 * 128 * 2


def test_mfma_record_fields():
    w = synth.WORKLOADS["768p_bf16"]
    r = bench.mfma_record(w, "readout", 0.5)
    assert r["peak_TFLOPs"] == 2500.0
    assert abs(r["achieved_TFLOPs"] - bench.mfma_flops(w, "readout") / 0.5e-3 / 1e12) < 0.1
    assert abs(r["frac"] - r["achieved_TFLOPs"] / 2500.0) < 1e-3
    f = synth.WORKLOADS["stress_f32"]
    assert bench.mfma_record(f, "gram", 1.0)["peak_TFLOPs"] == 157.3


def test_host_info_fields():
    h = bench.host_info()
    assert set(h) == {"cpu_model", "blas"} and h["cpu_model"] and h["blas"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_dominant_roofline_objects():
    w = synth.WORKLOADS["long_prep_bf16"]
    launch_bytes = bench.algorithmic_bytes(w, "prep") // 2
    r = bench.dominant_roofline(w, "prep", 2.5, launch_bytes, None, 2)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s" and r["peak"] == bench.VALU_F32_PEAK_TFLOPS
    assert abs(r["achieved"] - bench.prep_flops(w) / 2.5e-3 / 1e12) < 0.01
    assert abs(r["frac"] - r["achieved"] / bench.VALU_F32_PEAK_TFLOPS) < 1e-3
    assert abs(r["hbm"]["achieved"] - launch_bytes / 2.5e-3 / 1e9) < 0.1
    w = synth.WORKLOADS["768p_bf16"]
    r = bench.dominant_roofline(w, "readout", 0.9175, bench.algorithmic_bytes(w, "readout"), 123, 1)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["traffic"] == 123
    assert abs(r["achieved"] - 4860.0) < 1.0 and abs(r["frac"] - 0.6075) < 1e-4


def test_bench_names_are_defined():
    """Every name a function of bench.py reads is a local, an enclosing
    function's, a module-level name or a builtin (its GPU-only paths cannot run
    here, so this catches a name left undefined there)."""
    import builtins
    import symtable
    path = os.path.join(ROOT, "bench.py")
    top = symtable.symtable(open(path).read(), path, "exec")
    module = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    known = module | set(dir(builtins))
    missing = []

    def walk(t):
        for c in t.get_children():
            if c.get_type() == "function":
                for s in c.get_symbols():
                    if s.is_referenced() and s.is_global() and s.get_name() not in known:
                        missing.append((c.get_name(), s.get_name()))
            walk(c)

    walk(top)
    assert not missing, missing
