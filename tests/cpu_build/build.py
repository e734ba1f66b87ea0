"""Build the CPU build of the library: every source of
frame_wise_delta_02_amd/csrc compiled for the host with clang against the
emulated device environment in this folder (simt.h), as

* ``check`` -- the self-checking forward driver (check.cpp), with
  AddressSanitizer and UndefinedBehaviorSanitizer,
* ``gram_launch`` -- the forward's statistics launch alone (gram_launch.cpp),
  with both sanitizers, at any shape,
* ``libvdn_vda_sim.so`` -- the C ABI as a host library, for tests that compare
  the kernels' results with the oracle from Python, with every __shared__
  array filled with all-ones bytes before each workgroup (a kernel must write
  the LDS it reads), or
* ``libvdn_vda_sim_san.so`` -- the same with both sanitizers, linked against the
  shared sanitizer runtime (``sanitizer_runtime()``), which the loading process
  must preload.

The kernel sources are used as they are, except for the one inline-asm line of
vda_internal.h (sgpr(): v_readfirstlane_b32 into a scalar register), which is
rewritten to the readfirstlane builtin the emulator provides.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "frame_wise_delta_02_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CXX_CANDIDATES = ("/opt/rocm/llvm/bin/clang++", "/opt/rocm/lib/llvm/bin/clang++", shutil.which("clang++") or "")

SGPR_ASM = 'asm volatile("v_readfirstlane_b32 %0, %1\\n\\ts_nop 4" : "=s"(r) : "v"(v));'
SGPR_HOST = "r = __builtin_amdgcn_readfirstlane(v);"


def compiler() -> str | None:
    for c in CXX_CANDIDATES:
        if c and os.path.exists(c):
            return c
    return None


def _sources(out: str) -> list[str]:
    src = os.path.join(out, "src")
    os.makedirs(src, exist_ok=True)
    files = []
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith((".hip", ".h", ".cpp")):
            continue
        text = open(os.path.join(CSRC, f)).read()
        if f == "vda_internal.h":
            if SGPR_ASM not in text:
                raise RuntimeError("vda_internal.h: the sgpr() asm line changed; update tests/cpu_build/build.py")
            text = text.replace(SGPR_ASM, SGPR_HOST)
        if "asm volatile(\"v_" in text or "asm volatile(\"s_" in text:
            raise RuntimeError(f"{f}: inline asm the host build cannot compile")
        dst = os.path.join(src, f)
        if not os.path.exists(dst) or open(dst).read() != text:
            with open(dst, "w") as fh:
                fh.write(text)
        if f.endswith((".hip", ".cpp")):
            files.append(dst)
    return files


def sanitizer_runtime(name: str = "asan") -> str:
    """The shared sanitizer runtime a process loading libvdn_vda_sim_san.so
    (``asan``: AddressSanitizer with the UndefinedBehaviorSanitizer handlers)
    or libvdn_vda_sim_tsan.so (``tsan``) must preload."""
    r = subprocess.run([compiler(), f"-print-file-name=libclang_rt.{name}-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


KINDS = {"check": ("check", True), "lib": ("libvdn_vda_sim.so", False), "lib_san": ("libvdn_vda_sim_san.so", True),
         "selftest": ("selftest", True), "check_tsan": ("check_tsan", True), "selftest_tsan": ("selftest_tsan", True),
         "lib_tsan": ("libvdn_vda_sim_tsan.so", True), "gram_launch": ("gram_launch", True),
         "selftest_poison": ("selftest_poison", False)}


def build(out: str, kind: str) -> str:
    """Compile into ``out``; returns the path of the target ``kind`` ("check",
    "lib", "lib_san", "selftest": the emulator's own checks, selftest.cpp,
    "check_tsan" / "selftest_tsan": check.cpp / selftest.cpp with
    ThreadSanitizer on the kernels and the emulator's schedule annotated for
    it, "gram_launch": the forward's statistics launch alone, gram_launch.cpp,
    with AddressSanitizer and UndefinedBehaviorSanitizer, "selftest_poison":
    selftest.cpp with LDS poisoned before every workgroup, as the unsanitized
    library is)."""
    cxx = compiler()
    if cxx is None:
        raise RuntimeError("no clang++ for the host build")
    name, sanitize = KINDS[kind]
    files = ([] if kind.startswith("selftest") else _sources(out)) + [os.path.join(HERE, "simt.cpp")]
    os.makedirs(os.path.join(out, "src"), exist_ok=True)
    flags = ["-x", "c++", "-std=c++17", "-g", "-fPIC", "-fno-omit-frame-pointer", "-I", HERE, "-I", INCLUDE,
             "-I", os.path.join(out, "src"), "-Wno-unused-value", "-Wno-unknown-attributes",
             "-Wno-ignored-attributes"]
    tsan = kind in ("check_tsan", "selftest_tsan", "lib_tsan")
    if tsan:
        flags += ["-O1", "-fsanitize=thread"]
    elif sanitize:
        flags += ["-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    else:
        # the unsanitized library runs the parity tests: LDS poisoned before
        # every workgroup (see simt.h)
        flags += ["-O2", "-DSIMT_LDS_POISON"]
    # the sanitized executables and shared libraries share their objects
    # (-shared-libsan only chooses the runtime at link time)
    suffix = ".tsan.o" if tsan else ".san.o" if sanitize else ".o"
    headers = [os.path.join(out, "src", h) for h in os.listdir(os.path.join(out, "src")) if h.endswith(".h")]
    newest_header = max([os.path.getmtime(os.path.join(HERE, "simt.h"))] + [os.path.getmtime(h) for h in headers])

    def compile_one(f):
        o = os.path.join(out, os.path.splitext(os.path.basename(f))[0] + suffix)
        if os.path.exists(o) and os.path.getmtime(o) >= max(os.path.getmtime(f), newest_header):
            return o
        fl = flags
        if kind in ("check_tsan", "selftest_tsan", "lib_tsan") and f.endswith("simt.cpp"):
            # the emulator's bookkeeping is not instrumented; it annotates instead
            fl = [x for x in flags if x != "-fsanitize=thread"] + ["-DSIMT_TSAN"]
        r = subprocess.run([cxx, *fl, "-c", f, "-o", o], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host build of {f} failed:\n{r.stderr[-4000:]}")
        return o

    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, files))
    target = os.path.join(out, name)
    if kind in ("check", "selftest", "check_tsan", "selftest_tsan", "gram_launch", "selftest_poison"):
        main = {"check_tsan": "check.cpp", "selftest_tsan": "selftest.cpp",
                "selftest_poison": "selftest.cpp"}.get(kind, kind + ".cpp")
        cmd = [cxx, *flags[2:], os.path.join(HERE, main), *objs, "-o", target]
    else:
        cmd = [cxx, "-shared", *flags[2:], *(["-shared-libsan"] if sanitize else []), *objs, "-o", target]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {target} failed:\n{r.stderr[-4000:]}")
    return target


if __name__ == "__main__":
    import sys
    out = sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_build", "cpu_build")
    for kind in KINDS:
        print(build(out, kind))
