"""The generated gfx950 code keeps the properties the kernels are built around.
Each translation unit is compiled to AMD assembly with the library's own flags
(no GPU needed) and checked:
  - no packed-fp32 VALU instructions anywhere (the build disables them);
  - no scratch memory and no VGPR spills in any kernel;
  - every SSU update kernel moves the state with non-temporal vector loads and
    stores, reduces over dstate with DPP lane moves, and uses no matrix core;
  - the SSD front (whose C B^T tiles are a product), state-walk and scan
    kernels run on the matrix cores."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from selective_state_update_ssu_amd import build

UNITS = ["ssu_kernels_f32.hip", "ssu_kernels_bf16.hip", "ssd_kernels_bf16.hip"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa")

    def one(unit):
        path = os.path.join(str(out), unit + ".s")
        flags = [f for f in build.CXXFLAGS if f not in ("-fPIC",)]
        r = subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S",
                            os.path.join(build.CSRC, unit), "-o", path],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return unit, open(path).read()

    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(len(UNITS)) as ex:
        return dict(ex.map(one, UNITS))


def kernels(text):
    """Kernel symbol -> its instruction text."""
    out = {}
    for m in re.finditer(r"^(_Z\w+):[ \t]*(?:;.*)?$", text, re.M):
        end = text.find(".Lfunc_end", m.end())
        out[m.group(1)] = text[m.end():end]
    return out


def test_no_packed_fp32_instructions(asm):
    for unit, text in asm.items():
        assert not re.search(r"v_pk_(fma|mul|add)_f32", text), unit


def test_no_scratch_and_no_vgpr_spills(asm):
    for unit, text in asm.items():
        sizes = re.findall(r"\.private_segment_fixed_size:\s*(\d+)", text)
        spills = re.findall(r"\.vgpr_spill_count:\s*(\d+)", text)
        assert sizes and all(s == "0" for s in sizes), unit
        assert spills and all(s == "0" for s in spills), unit


@pytest.mark.parametrize("unit", ["ssu_kernels_f32.hip", "ssu_kernels_bf16.hip"])
def test_ssu_kernels_stream_state_and_reduce_across_lanes(asm, unit):
    ks = {k: v for k, v in kernels(asm[unit]).items() if "ssu_update_kernel" in k}
    assert len(ks) >= 30, len(ks)
    for name, body in ks.items():
        assert re.search(r"global_load_dwordx[24] .* nt", body), name
        assert re.search(r"global_store_dwordx[24] .* nt", body), name
        assert re.search(r"quad_perm|row_shr|row_ror|row_mirror|row_half_mirror", body), name
        assert "v_mfma" not in body, name


def test_ssd_products_on_matrix_cores(asm):
    ks = kernels(asm["ssd_kernels_bf16.hip"])
    for kind in ("ssd_front_kernel", "ssd_state_walk_kernel", "ssd_scan_kernel"):
        bodies = [b for k, b in ks.items() if kind in k]
        assert bodies, kind
        for b in bodies:
            assert "v_mfma" in b, kind
