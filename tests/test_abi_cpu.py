"""The C ABI on a machine without a GPU: the library loads, exports every
function include/swiglu.h declares, and rejects bad calls before touching the
device.  No compute entry point runs here."""
import ctypes
import os
import re
import subprocess

import pytest

import gemm_epilogues_mlp_amd as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swiglu.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swiglu_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("swiglu_create", "swiglu_forward", "swiglu_destroy", "swiglu_forward_ex",
                 "swiglu_forward_unfused", "swiglu_pack_interleaved", "swiglu_query"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = sw.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sw.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (swiglu_\w+)", out))
    assert set(declared_functions()) <= exported


def test_library_is_built_for_gfx950():
    data = open(sw.lib_path(), "rb").read()
    assert b"gfx950" in data


def test_header_compiles_as_c():
    src = '#include "swiglu.h"\nint main(void){ return (int)swiglu_config_count(); }\n'
    cmd = ["gcc", "-std=c11", "-fsyntax-only", "-x", "c", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-"]
    r = subprocess.run(cmd, input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_null_handle_and_bad_arguments_rejected():
    lib = sw.load()
    assert lib.swiglu_forward(None, 16, 16, 16, 16, 8, 8, 8, 0, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_forward_unfused(None, 16, 16, 16, 16, 16, 8, 8, 8, -1, None) == \
        sw.ERR_INVALID_ARG
    assert lib.swiglu_forward_unfused_static(None, 16, 16, 16, 16, 8, 8, 8, -1, None) == \
        sw.ERR_INVALID_ARG
    assert lib.swiglu_pack_interleaved(None, 16, 16, 16, 8, 8, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_query(None, 8, 8, 8, 0, None, None, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_create(None, 0) == sw.ERR_INVALID_ARG
    assert lib.swiglu_destroy(None) == sw.OK
    assert lib.swiglu_config_info(-1, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_config_info(sw.swiglu_config_count(), None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_forward_fp8(None, 16, 16, 16, 8, 8, 16, 1.0, 1.0, 1.0, 0, -1, None) == \
        sw.ERR_INVALID_ARG
    assert lib.swiglu_quantize_fp8(None, 16, 16, 16, 1.0, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_pack_fp8(None, 16, 16, 16, 16, 8, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_query_fp8(None, 8, 8, 16, 0, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_forward_mx(None, 16, 16, 16, 16, 16, 8, 8, 64, 16, -1, None) == \
        sw.ERR_INVALID_ARG
    assert lib.swiglu_quantize_mx(None, 16, 16, 16, 1, 32, 16, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_pack_kmajor(None, 16, 16, 16, 8, 8, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_pack_fragments(None, 16, 16, 16, 8, 8, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_packed_bytes(72, 40) == 2 * 2 * 2 * 4096
    assert lib.swiglu_pack_fp8_fragments(None, 16, 16, 16, 8, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_fp8_packed_bytes(12, 144) == 2 * 2 * 2048
    assert lib.swiglu_pack_mx_fragments(None, 16, 16, 64, 8, None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_forward_mx_packed(None, 16, 16, 16, 16, 16, 8, 8, 64, 16, -1, None) == \
        sw.ERR_INVALID_ARG
    assert lib.swiglu_mx_packed_bytes(20, 128) == 2 * 2 * 2048
    assert lib.swiglu_mx_packed_bytes(20, 100) == 0
    assert lib.swiglu_forward_packed_splitk(None, None, None, None, 16, 72, 40, -1, 2, None, 0,
                                            None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_packed_splitk_plan(None, 16, 72, 40, None, None) == sw.ERR_INVALID_ARG


def test_splitk_workspace_bytes():
    # a 256-byte block of counters (16 bytes per slab, rounded up), then 8 KB
    # of partials per slab and piece of K
    assert sw.swiglu_packed_splitk_workspace_bytes(72, 40, 3) == 256 + 2 * 3 * 8192
    assert sw.swiglu_packed_splitk_workspace_bytes(18944, 3584, 4) == 4864 + 296 * 4 * 8192
    assert sw.swiglu_packed_splitk_workspace_bytes(2368, 3584, 1) == 768 + 37 * 8192
    assert sw.swiglu_packed_splitk_workspace_bytes(72, 0, 2) == 256 + 2 * 2 * 8192
    for bad in ((0, 40, 2), (72, -1, 2), (72, 40, 0), (72, 40, 65)):
        assert sw.swiglu_packed_splitk_workspace_bytes(*bad) == 0


def test_status_strings_and_workspace_size():
    assert sw.swiglu_status_str(0) == "ok"
    assert "unknown" in sw.swiglu_status_str(99)
    assert sw.swiglu_unfused_workspace_bytes(3, 8) == 4 * 3 * 8
    assert sw.swiglu_unfused_workspace_bytes(-1, 8) == 0


def test_config_list_is_consistent():
    n = sw.swiglu_config_count()
    assert n > 0
    seen = {sw.VARIANT_SYNC: 0, sw.VARIANT_INTERLEAVE: 0, sw.VARIANT_GEMM: 0, sw.VARIANT_FP8: 0,
            sw.VARIANT_FP8_SYNC: 0, sw.VARIANT_MXFP8: 0, sw.VARIANT_PACKED: 0,
            sw.VARIANT_FP8_PACKED: 0, sw.VARIANT_MXFP8_PACKED: 0, sw.VARIANT_MXFP8_SYNC: 0,
            sw.VARIANT_PACKED_SPLITK: 0}
    for i in range(n):
        c = sw.swiglu_config_info(i)
        assert c["id"] == i
        assert c["variant"] in seen
        seen[c["variant"]] += 1
        assert c["family"] in (0, 1, 2, 3)
        assert (c["family"] == 3) == (c["variant"] == sw.VARIANT_PACKED_SPLITK)
        if c["family"] == 3:  # decode rows, 32-deep K steps, the packed slab parts
            assert c["bm"] == 16 and c["bk"] == 32 and c["bn"] in (16, 32, 64)
        assert c["tail_split"] in (0, 4)
        if c["tail_split"]:
            assert c["family"] in (0, 2) and c["bm"] % 64 == 0 and c["bn"] % 64 == 0
        if c["family"] == 2:  # persistent: one workgroup per CU, all of LDS
            assert c["lds_bytes"] == 160 * 1024 and c["tail_split"] == 4
        # the MX streaming kernel uses no LDS (one wave, no reduction)
        assert 0 < c["lds_bytes"] <= 160 * 1024 or (c["variant"] == sw.VARIANT_MXFP8_PACKED
                                                   and c["lds_bytes"] == 0)
        assert c["waves"] * 64 <= 1024
        if c["family"] in (0, 2):
            assert c["bm"] % 32 == 0 and c["bn"] % 32 == 0
        if c["variant"] in (sw.VARIANT_FP8, sw.VARIANT_FP8_SYNC, sw.VARIANT_MXFP8,
                            sw.VARIANT_FP8_PACKED, sw.VARIANT_MXFP8_PACKED,
                            sw.VARIANT_MXFP8_SYNC):
            assert (c["family"], c["bk"]) in ((0, 64), (1, 128), (1, 64))
        if c["variant"] == sw.VARIANT_PACKED:  # streaming, 64 outputs per slab
            assert c["family"] == 1 and c["bn"] in (16, 32, 64) and c["bk"] == 32
    assert all(v > 0 for v in seen.values())


def test_create_without_device_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the GPU tests cover creation")
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_create(0)
    assert e.value.status == sw.ERR_DEVICE
