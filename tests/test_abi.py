"""The C ABI library loads and exports every entry point include/smoe.h declares
(no GPU work)."""
import ctypes
import os
import re

import quantised_routed_expert_amd as smoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "smoe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smoe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("smoe_route", "smoe_moe_decode", "smoe_moe_prefill_chunk", "smoe_ring_create",
                     "smoe_ring_acquire", "smoe_ring_release", "smoe_ring_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(smoe.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(smoe.EXPORTED) == sorted(declared_functions())


def test_host_only_queries():
    import synth
    lib = smoe.lib()
    assert lib.smoe_version() == 2
    for wl, blob, stride in ((synth.CONFIGS[0], 61440, 65536), (synth.CONFIGS[2], 10616832, 10616832),
                             (synth.Q2_WORKLOADS[0], 5898240, 5898240)):
        assert smoe.blob_bytes(wl.dims) == blob == synth.blob_sections(wl.dims)["bytes"]
        assert smoe.blob_stride(wl.dims) == stride == synth.blob_sections(wl.dims)["stride"]
        assert smoe.workspace_bytes(wl.dims, 1) > 0
    # SMOE-Q2 needs chunk 64 and d_model % 512 == 0; quant_bits must be 2 or 4
    for bad_q2 in (synth.Q2_WORKLOADS[0].dims.replace(chunk=32), synth.Dims(768, 256, 16, 4, 64, bits=2)):
        try:
            smoe.workspace_bytes(bad_q2, 1)
            raise AssertionError("expected SmoeError")
        except smoe.SmoeError as e:
            assert e.code == -1 and "Q2" in str(e)
    # a code width other than 4 (or 0) and 2 is rejected; 0 reads as SMOE-Q4
    from quantised_routed_expert_amd.binding import SmoeDims
    d = SmoeDims(4096, 1536, 128, 8, 64, 1, 1e-6, 3)
    assert lib.smoe_blob_bytes(ctypes.byref(d)) == 0
    d.quant_bits = 0
    assert lib.smoe_blob_bytes(ctypes.byref(d)) == 10616832
    d.quant_bits = 2
    assert lib.smoe_blob_bytes(ctypes.byref(d)) == 5898240
    bad = synth.CONFIGS[0].dims.replace(chunk=48)
    try:
        smoe.workspace_bytes(bad, 1)
        raise AssertionError("expected SmoeError")
    except smoe.SmoeError as e:
        assert e.code == -1 and "chunk" in str(e)
