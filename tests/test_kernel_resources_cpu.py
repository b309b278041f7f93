"""Resources of every kernel in the built library, read from the gfx950 code
object's metadata (no GPU): no kernel uses scratch memory (register spills,
a stack), and none asks for more LDS than a CU has (160 KB on MI355X).

A spill turns into scratch loads and stores: memory the runtime allocates
beside the launch, and loads the hand-counted vmcnt waits of the DMA ring do
not know about.  Keeping every kernel at zero scratch makes that whole class
of cost and fault impossible rather than something to look for."""
import os
import re
import shutil
import subprocess

import pytest

import gemm_epilogues_mlp_amd as sw

LLVM = "/opt/rocm/llvm/bin"
LDS_PER_CU = 160 * 1024


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    objcopy, bundler, readelf = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), \
        _tool("llvm-readelf")
    if not (objcopy and bundler and readelf):
        pytest.skip("ROCm LLVM tools not found")
    d = tmp_path_factory.mktemp("codeobj")
    fat, dev = str(d / "fat.bin"), str(d / "gfx950.o")
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", sw.lib_path(),
                    str(d / "copy.so")], check=True)
    subprocess.run([bundler, "--unbundle", "--type=o", f"--input={fat}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"], check=True)
    notes = subprocess.run([readelf, "--notes", dev], check=True, capture_output=True,
                           text=True).stdout
    # the metadata lists one mapping per kernel ("  - .key: value"), its
    # top-level keys at four spaces
    out, cur = [], None
    for line in notes.splitlines():
        if re.match(r"^  - \.", line):
            cur = {}
            out.append(cur)
        m = re.match(r"^  [ -] \.(\w+):\s+(.*)$", line)
        if m and cur is not None:
            cur[m.group(1)] = m.group(2).strip()
    return out


def test_every_kernel_is_listed(kernels):
    names = [k["name"] for k in kernels]
    assert len(names) == len(set(names)) and len(names) >= 40
    for part in ("tiled_kernel", "tiled_split_kernel", "tiled_persist_kernel", "skinny_kernel",
                 "packed_kernel", "f8_kernel", "f8_split_kernel", "mx_packed_kernel",
                 "gate_kernel", "quantize_mx_kernel"):
        assert any(part in n for n in names), part


def test_no_kernel_uses_scratch(kernels):
    bad = [(k["name"], k.get("private_segment_fixed_size"), k.get("vgpr_spill_count"))
           for k in kernels
           if k.get("private_segment_fixed_size") != "0" or k.get("vgpr_spill_count") != "0"
           or k.get("uses_dynamic_stack") != "false"]
    assert not bad, bad


def test_lds_fits_a_cu(kernels):
    sizes = {k["name"]: int(k["group_segment_fixed_size"]) for k in kernels}
    assert max(sizes.values()) <= LDS_PER_CU
    # the configurations' LDS figures are what their kernels allocate
    allocated = set(sizes.values())
    for i in range(sw.swiglu_config_count()):
        c = sw.swiglu_config_info(i)
        assert c["lds_bytes"] in allocated or c["lds_bytes"] == 0, c
