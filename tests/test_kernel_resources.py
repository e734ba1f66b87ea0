"""Resources of the gfx950 kernels as built, read from the code objects in the
in-tree libvdn_vda.so (frame_wise_delta_02_amd/resources.py): every kernel
fits one compute unit, no kernel of the forward pass, the prep or the adjacent
maps keeps anything in scratch memory, scratch appears nowhere else than where
it is known, and the 768p kernels have the occupancy their launches are
designed around."""

import shutil

import pytest

from frame_wise_delta_02_amd import resources

if shutil.which("c++filt") is None:
    pytest.skip("c++filt is needed to read the kernel names", allow_module_level=True)


@pytest.fixture(scope="module")
def kern():
    rows = resources.kernels()
    return {r["name"]: r for r in rows}


FORWARD_128 = ["gram_bf16<128, false>", "solve_sweep<128>", "gather_states<128, true>", "gather_states<128, false>",
               "prep_conv_tile<128>"] + [f"scan_rows<128, true, {m}>" for m in range(5)] + \
    [f"readout_bf16<128, {a}, {b}, {c}>" for a, b, c in [("true", "true", "true"), ("true", "false", "true"),
                                                         ("false", "false", "true"), ("true", "true", "false"),
                                                         ("true", "false", "false"), ("false", "false", "false")]]

# Kernels known to keep a private array in scratch (bytes per lane, as built):
# the float32 / d = 16 Cholesky inverse (a small register array indexed in a
# loop), and the backward pass's statistics-gradient kernel at d = 128, whose
# copy of the 160 KiB operand planes into LDS is staged through a 40-entry
# register array that does not fit beside its 490 registers.
KNOWN_SCRATCH = {"solve_mfma<16, false>": 32, "solve_mfma<32, false>": 32, "solve_mfma<64, false>": 32,
                 "solve_mfma<128, false>": 32, "gram_bwd16<128>": 656}


def test_the_forward_kernels_are_built(kern):
    missing = [n for n in FORWARD_128 if n not in kern]
    assert not missing, missing
    assert len(kern) >= 150


def test_every_kernel_fits_a_compute_unit(kern):
    for name, r in kern.items():
        assert r["lds"] <= resources.LDS_PER_CU, name
        assert r["vgprs"] <= resources.VGPRS_PER_SIMD_LANE, name
        assert r["workgroups_per_cu"] >= 1, (name, r)
        assert r["vgpr_spills"] == 0, name


def test_scratch_only_where_known(kern):
    with_scratch = {n: r["scratch"] for n, r in kern.items() if r["scratch"]}
    unknown = {n: s for n, s in with_scratch.items() if n not in KNOWN_SCRATCH}
    assert not unknown, unknown
    grown = {n: s for n, s in with_scratch.items() if s > KNOWN_SCRATCH[n]}
    assert not grown, grown


def test_no_scratch_on_the_forward_path(kern):
    for prefix in ("gram_bf16", "gram_f32", "solve_sweep", "scan_rows", "gather_states", "readout_bf16", "readout_f32",
                   "prep_conv", "prep_l2", "gemm_nt_bf16", "frame_col_sums", "frame_mean", "alpha_proj"):
        rows = [(n, r) for n, r in kern.items() if n.startswith(prefix)]
        assert rows, prefix
        for n, r in rows:
            assert r["scratch"] == 0, (n, r["scratch"])


def test_occupancy_of_the_768p_kernels(kern):
    """One statistics workgroup (8 waves, 184 registers, 64 KiB LDS) and one
    readout workgroup (8 waves, 128 KiB LDS) per compute unit; two scan
    workgroups; the inverse four."""
    assert kern["gram_bf16<128, false>"]["workgroups_per_cu"] == 1
    assert kern["gram_bf16<128, false>"]["waves_per_simd"] == 2
    for n in FORWARD_128:
        if n.startswith("readout_bf16"):
            assert kern[n]["workgroups_per_cu"] == 1, n
        if n.startswith("scan_rows"):
            assert kern[n]["workgroups_per_cu"] == 2, n
    assert kern["solve_sweep<128>"]["workgroups_per_cu"] == 4


def test_occupancy_arithmetic():
    # 512 registers per lane in granules of 8, at most 8 waves per SIMD
    assert resources.occupancy(24, 0, 256) == (8, 8)
    assert resources.occupancy(180, 65536, 512) == (2, 1)
    assert resources.occupancy(129, 0, 256) == (3, 3)
    assert resources.occupancy(512, 0, 256) == (1, 1)
    # LDS binds: 160 KiB / 40 KiB
    assert resources.occupancy(72, 40960, 256) == (7, 4)
