"""Resources of every gfx950 kernel in libvdn_vda.so, read from the code
objects the build embedded in it: registers, LDS, scratch, the largest
workgroup, and the occupancy these allow on one compute unit.

    python -m frame_wise_delta_02_amd.resources [path/to/libvdn_vda.so]

The library's .hip_fatbin section holds one offload bundle per source file;
each bundle's gfx950 code object carries the AMDGPU metadata note (YAML) that
lists its kernels.  Uses llvm-objcopy, clang-offload-bundler and llvm-readelf
from the ROCm LLVM, and c++filt for readable names when it is installed.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

import yaml

PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG, "libvdn_vda.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# One CDNA4 compute unit: four SIMDs, each with 512 unified vector registers
# per lane for a 64-wide wave (architectural and accumulation registers share
# the file, allocated in granules of 8) and at most 8 waves; 160 KiB of LDS.
SIMDS_PER_CU = 4
VGPRS_PER_SIMD_LANE = 512
VGPR_GRANULE = 8
MAX_WAVES_PER_SIMD = 8
LDS_PER_CU = 160 * 1024


def _tool(name: str) -> str:
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing")
    return path


def _run(cmd: list[str], **kw) -> subprocess.CompletedProcess:
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed:\n{r.stderr[-2000:]}")
    return r


def _metadata(code_object: str) -> dict:
    notes = _run([_tool("llvm-readelf"), "--notes", code_object]).stdout
    m = re.search(r"^\s*---\s*$(.*?)^\.\.\.\s*$", notes, re.S | re.M)
    if not m:
        raise RuntimeError(f"no AMDGPU metadata in {code_object}")
    return yaml.safe_load(m.group(1))


def _demangle(names: list[str]) -> list[str]:
    filt = shutil.which("c++filt")
    if not filt or not names:
        return names
    out = subprocess.run([filt], input="\n".join(names), capture_output=True, text=True).stdout.splitlines()
    if len(out) != len(names):
        return names
    out = [n.replace("vda::(anonymous namespace)::", "").replace("vda::", "") for n in out]
    return [re.sub(r"^void ", "", re.sub(r"\(.*", "", n)) for n in out]


def occupancy(vgprs: int, lds: int, workgroup: int) -> tuple[int, int]:
    """(waves per SIMD that the registers allow, workgroups of ``workgroup``
    threads per compute unit that registers and LDS allow together)."""
    alloc = -(-max(vgprs, 1) // VGPR_GRANULE) * VGPR_GRANULE
    waves_simd = min(MAX_WAVES_PER_SIMD, VGPRS_PER_SIMD_LANE // alloc)
    waves_wg = -(-workgroup // 64)
    by_regs = waves_simd // -(-waves_wg // SIMDS_PER_CU)
    by_lds = LDS_PER_CU // lds if lds else by_regs
    return waves_simd, min(by_regs, by_lds)


def kernels(lib: str = LIB) -> list[dict]:
    """One dict per kernel: name, symbol, vgprs (the unified count, accumulation
    registers included), agprs, sgprs, lds and scratch (bytes per lane),
    workgroup (the largest the kernel was compiled for), vgpr_spills,
    sgpr_spills, waves_per_simd, workgroups_per_cu."""
    if not os.path.exists(lib):
        raise RuntimeError(f"{lib} is missing: run `python -m frame_wise_delta_02_amd.build`")
    rows = []
    with tempfile.TemporaryDirectory() as tmp:
        fatbin = os.path.join(tmp, "fatbin")
        _run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}", lib, os.path.join(tmp, "stripped")])
        data = open(fatbin, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
        if not starts:
            raise RuntimeError(f"no offload bundle in {lib}")
        for i, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            bundle, co = os.path.join(tmp, f"b{i}"), os.path.join(tmp, f"b{i}.co")
            with open(bundle, "wb") as fh:
                fh.write(data[a:b])
            _run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={bundle}",
                  f"--targets={TARGET}", f"--output={co}"])
            for k in _metadata(co).get("amdhsa.kernels") or []:
                vgprs, lds, wg = int(k[".vgpr_count"]), int(k[".group_segment_fixed_size"]), \
                    int(k[".max_flat_workgroup_size"])
                waves_simd, per_cu = occupancy(vgprs, lds, wg)
                rows.append(dict(symbol=k[".name"], vgprs=vgprs, agprs=int(k.get(".agpr_count", 0)),
                                 sgprs=int(k[".sgpr_count"]), lds=lds,
                                 scratch=int(k[".private_segment_fixed_size"]), workgroup=wg,
                                 vgpr_spills=int(k.get(".vgpr_spill_count", 0)),
                                 sgpr_spills=int(k.get(".sgpr_spill_count", 0)),
                                 waves_per_simd=waves_simd, workgroups_per_cu=per_cu))
    for r, n in zip(rows, _demangle([r["symbol"] for r in rows])):
        r["name"] = n
    return rows


def main(argv: list[str]) -> int:
    rows = kernels(argv[1] if len(argv) > 1 else LIB)
    w = max(len(r["name"]) for r in rows)
    print(f"{'kernel':{w}}  VGPR  AGPR  SGPR  LDS bytes  scratch  workgroup  waves/SIMD  workgroups/CU")
    for r in rows:
        print(f"{r['name']:{w}}  {r['vgprs']:4d}  {r['agprs']:4d}  {r['sgprs']:4d}  {r['lds']:9d}  {r['scratch']:7d}"
              f"  {r['workgroup']:9d}  {r['waves_per_simd']:10d}  {r['workgroups_per_cu']:13d}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
