"""The C ABI on the host: libsdv.so loads and exports every function include/sdv.h
declares, and host-checkable calls behave as the header states (negative status before
anything is enqueued, a message from sdv_last_error, sizes from pure host arithmetic).
No call here launches GPU work."""
import ctypes
import os
import re
import subprocess


import speculative_decoding_verify_amd as sdv
from speculative_decoding_verify_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)      # drop comments
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(sdv_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("sdv_verify_forward", "sdv_accept_greedy", "sdv_accept_sample", "sdv_kv_rollback",
              "sdv_verify_workspace_size", "sdv_sample_workspace_size", "sdv_pack_weights",
              "sdv_packed_bytes", "sdv_last_error", "sdv_abi_version", "sdv_philox_uniforms",
              "sdv_draft_tree", "sdv_draft_workspace_size", "sdv_verify_forward_noalloc",
              "sdv_pool_clear", "sdv_pool_insert", "sdv_pool_lookup"):
        assert f in names, f


def test_library_exports_every_declared_function():
    L = sdv.lib()
    names = declared_functions()
    for f in names:
        assert hasattr(L, f), f"libsdv.so does not export {f}"
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        exported = {ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln}
        missing = [f for f in names if f not in exported]
        assert not missing, missing


def test_abi_version_and_packed_sizes():
    L = sdv.lib()
    hdr = int(re.search(r"#define SDV_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.sdv_abi_version() == binding.ABI_VERSION == hdr
    # rows round up to 16, 2 bytes (bf16) / 4 bytes (fp32) per value
    assert L.sdv_packed_bytes(1, 6144, 2048) == 6144 * 2048 * 2
    assert L.sdv_packed_bytes(0, 17, 64) == 32 * 64 * 4
    assert L.sdv_packed_bytes(1, 0, 64) == 0
    assert L.sdv_packed_bytes(7, 16, 64) == 0


def test_null_arguments_are_rejected_before_launch():
    L = sdv.lib()
    st = L.sdv_verify_forward(None, None, None, None, None, 0, None)
    assert st == -1
    assert b"NULL" in L.sdv_last_error()
    st = L.sdv_kv_rollback(None, None, None, None, None, 0, None, None)
    assert st == -1
    # both move lists or neither
    st = L.sdv_accept_greedy(1, 4, 1, ctypes.c_void_p(16), None, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                             None, ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, ctypes.c_void_p(16), None,
                             None, None)
    assert st == -1
    # T above the supported maximum
    st = L.sdv_accept_greedy(1, 4096, 1, ctypes.c_void_p(16), None, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                             None, ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, None, None, None, None)
    assert st == -2


def test_workspace_sizes_are_host_arithmetic():
    L = sdv.lib()
    assert L.sdv_sample_workspace_size(0, 7, 151936) == 0
    n1 = L.sdv_sample_workspace_size(64, 7, 151936)
    n2 = L.sdv_sample_workspace_size(128, 7, 151936)
    assert 0 < n1 < n2


def test_sampling_arguments_are_checked_on_the_host():
    L = sdv.lib()
    p = ctypes.c_void_p(256)
    ws = L.sdv_sample_workspace_size(4, 3, 100)
    assert L.sdv_sample_workspace_size(4, 1025, 100) == 0           # k above the maximum
    # NULL logits, bad temperature, workspace too small: rejected before any launch
    assert L.sdv_accept_sample(4, 3, 100, None, p, p, ctypes.c_float(1.0), 7, None, p, p, None, p, ws, None,
                               None) == -1
    for t in (0.0, -1.0, float("inf"), float("nan")):
        assert L.sdv_accept_sample(4, 3, 100, p, p, p, ctypes.c_float(t), 7, None, p, p, None, p, ws, None,
                                   None) == -2
    assert L.sdv_accept_sample(4, 3, 100, p, p, p, ctypes.c_float(1.0), 7, None, p, p, None, p, ws - 1, None,
                               None) == -4
    assert L.sdv_philox_uniforms(1, None, 4, 3, None, None, None) == -1
    assert L.sdv_philox_uniforms(1, None, 0, 3, p, None, None) == -2


def test_pool_arguments_are_checked_on_the_host():
    L = sdv.lib()
    p = 256
    bad_slots = binding.SdvPool(p, p, p, p, p, 100, 1000, 4)      # n_slots not a power of two
    assert L.sdv_pool_clear(ctypes.byref(bad_slots), None) == -2
    bad_n = binding.SdvPool(p, p, p, p, p, 100, 1024, 17)         # max_n above the maximum
    assert L.sdv_pool_clear(ctypes.byref(bad_n), None) == -2
    ok = binding.SdvPool(p, p, p, p, p, 100, 1024, 4)
    assert L.sdv_pool_insert(ctypes.byref(ok), None, 3, None, None) == -1
    assert L.sdv_pool_insert(ctypes.byref(ok), ctypes.c_void_p(p), 0, None, None) == -2
    assert L.sdv_pool_lookup(ctypes.byref(ok), 0, ctypes.c_void_p(p), ctypes.c_void_p(p), 4, 4,
                             ctypes.c_void_p(p), ctypes.c_void_p(p), None, None) == -2
