"""The C-ABI library loads without a GPU and exports every function include/forkkv.h declares."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "forkkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(forkkv_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_all_declared_functions():
    from lora_shared_prefix_amd import forkkv
    names = declared_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(forkkv.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each of them
    assert sorted(forkkv._SIGS) == names


def test_strerror_and_pool_bytes():
    from lora_shared_prefix_amd import forkkv
    L = forkkv.lib()
    assert L.forkkv_strerror(0) == b"ok"
    assert L.forkkv_strerror(-2) == b"page pool exhausted"
    b, r = forkkv.Pool.nbytes(4096, 32768, 8, 128, 16, "bf16")
    assert b == 4096 * 2 * 8 * 16 * 128 * 2 and r == 32768 * 2 * 16 * 16 * 2
