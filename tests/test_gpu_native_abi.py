"""The C ABI used from C++ alone (tests/native/abi_gpu_check.cpp): its own
device buffers and stream, no Python marshalling.  The fused call equals the
separate calls bit for bit, exact sums come out exact, the all-gather is a
concatenation, a zero gradient leaves the weights unchanged, invalid
arguments return the documented status without writing anything, and the
workspace-free gradient norm equals the workspace form and the exact sum."""
import ctypes as C
import os

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "native", "libabi_gpu_check.so")


def test_native_caller_of_the_c_abi():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "build_native", os.path.join(ROOT, "tests", "native", "build_native.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    lib = C.CDLL(LIB)
    lib.zero_native_abi_check.argtypes = [C.c_char_p, C.c_int]
    lib.zero_native_abi_check.restype = C.c_int
    buf = C.create_string_buffer(512)
    print("native C ABI check", flush=True)
    rc = lib.zero_native_abi_check(buf, len(buf))
    assert rc == 0, buf.value.decode()
    assert buf.value == b"ok"
