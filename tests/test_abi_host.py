"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/starkv.h declares, and
reject bad arguments with the documented status before touching the device.
"""

import ctypes
import os
import re

import pytest

import rank_compressed_paged_amd as starkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "starkv.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return starkv.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(starkv_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("starkv_append", "starkv_decode", "starkv_decode_workspace_size", "starkv_status_string",
              "starkv_profile_begin", "starkv_profile_end"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_exports_are_c_symbols():
    # C linkage: the dynamic symbol table holds the plain names
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", starkv.library_path()], capture_output=True,
                         text=True).stdout
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in declared_functions():
        assert name in syms, name


def test_status_strings(lib):
    for code, tag in [(0, "OK"), (1, "INVALID_ARG"), (2, "UNSUPPORTED"), (3, "WORKSPACE"), (4, "HIP")]:
        assert tag in starkv.status_string(code)
    assert "unknown" in starkv.status_string(99)


def main_dims(**over):
    d = dict(heads=32, head_dim=128, rank_k=64, rank_v=1024, num_blocks=32768, max_blocks_per_seq=512)
    d.update(over)
    return starkv.Dims.make(**d)


def ws_size(lib, dims, batch, max_len):
    return lib.starkv_decode_workspace_size(ctypes.byref(dims), batch, max_len)


def test_workspace_size_host_only_and_monotone(lib):
    d = main_dims()
    a = ws_size(lib, d, 64, 8192)
    b = ws_size(lib, d, 64, 4096)
    c = ws_size(lib, d, 32, 8192)
    assert a > 0 and b > 0 and c > 0
    assert b <= a and c <= a
    assert a % 256 == 0
    # partial-state slots dominate: H * r_v fp16 each (z / l), at most (grid cap + batch) of them
    assert a >= (1024 + 64) * 32 * 1024 * 2
    assert ws_size(lib, d, 64, 0) > 0                       # empty batch still plans
    assert ws_size(lib, d, 0, 8192) == 0                    # invalid batch
    assert ws_size(lib, d, 64, 8192 + 1) == 0               # beyond 16 * max_blocks_per_seq
    assert ws_size(lib, main_dims(block_size=32), 64, 8192) == 0


def call_decode(lib, dims, batch=4, max_len=64, ptr=0x1000, ws_bytes=1 << 30, scale=0.1, out=0x1000):
    p = ctypes.c_void_p(ptr)
    return lib.starkv_decode(ctypes.byref(dims) if dims is not None else None, batch, max_len,
                             p, p, p, p, p, p, p, scale, p, ws_bytes, ctypes.c_void_p(out), None)


def test_decode_rejects_before_touching_the_device(lib):
    d = main_dims()
    assert call_decode(lib, None) == INVALID
    assert call_decode(lib, d, ptr=0) == INVALID                  # null pointers
    assert call_decode(lib, d, ptr=0x1008) == INVALID             # 16-byte alignment
    assert call_decode(lib, d, batch=0) == INVALID
    assert call_decode(lib, d, max_len=-1) == INVALID
    assert call_decode(lib, d, max_len=512 * 16 + 1) == INVALID
    assert call_decode(lib, d, scale=float("nan")) == INVALID
    assert call_decode(lib, main_dims(heads=0)) == INVALID
    assert call_decode(lib, main_dims(block_size=8)) == UNSUPPORTED
    assert call_decode(lib, main_dims(rank_k=48)) == UNSUPPORTED     # no kernel for this shape
    assert call_decode(lib, main_dims(rank_v=1000)) == UNSUPPORTED   # not a multiple of 32
    assert call_decode(lib, main_dims(head_dim=12)) == UNSUPPORTED
    assert call_decode(lib, d, ws_bytes=1024) == WORKSPACE


def test_grouped_heads_checks(lib):
    assert ctypes.sizeof(starkv.Dims) == 8 * 4                     # eight int32 fields, no padding
    assert call_decode(lib, main_dims(kv_heads=5)) == INVALID         # must divide the query heads
    assert call_decode(lib, main_dims(kv_heads=-1)) == INVALID
    assert call_decode(lib, main_dims(kv_heads=16), ws_bytes=1024) == WORKSPACE   # 32/16 is built
    assert call_decode(lib, main_dims(kv_heads=1)) == UNSUPPORTED     # 32 query heads per key head
    assert call_decode(lib, main_dims(heads=40, kv_heads=8)) == UNSUPPORTED   # more than 32 query heads
    assert call_decode(lib, main_dims(heads=28, kv_heads=4, rank_k=16)) == UNSUPPORTED   # grouped: r_k 32 or 64
    assert call_decode(lib, main_dims(kv_heads=8), ws_bytes=1024) == WORKSPACE   # (32, 8, 64, 1024) is built
    zero = main_dims()
    zero.num_kv_heads = 0                                             # 0 means "same as num_heads"
    assert ws_size(lib, zero, 64, 8192) == ws_size(lib, main_dims(), 64, 8192)
    # partial states are per query head: grouping does not shrink the workspace
    assert ws_size(lib, main_dims(kv_heads=8), 64, 8192) == ws_size(lib, main_dims(), 64, 8192)


def test_append_rejects_before_touching_the_device(lib):
    d = main_dims()
    p = ctypes.c_void_p(0x1000)
    args = [p] * 9
    assert lib.starkv_append(ctypes.byref(d), 0, *[ctypes.c_void_p(0)] * 9, None) == OK   # n = 0 no-op
    assert lib.starkv_append(ctypes.byref(d), -1, *args, None) == INVALID
    assert lib.starkv_append(ctypes.byref(d), 4, *[ctypes.c_void_p(0)] * 9, None) == INVALID
    bad = list(args)
    bad[0] = ctypes.c_void_p(0x1002)
    assert lib.starkv_append(ctypes.byref(d), 4, *bad, None) == INVALID
    assert lib.starkv_append(ctypes.byref(main_dims(block_size=32)), 4, *args, None) == UNSUPPORTED


def test_profile_hooks_without_launches(lib):
    starkv.profile_begin()
    ms, n = starkv.profile_end()
    assert n == 0 and ms == 0.0


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        starkv.load_library(str(tmp_path / "nope.so"))


def call_prefill(lib, dims, batch=2, rows=8, max_len=64, ptr=0x1000, ws_bytes=1 << 30, scale=0.1):
    p = ctypes.c_void_p(ptr)
    return lib.starkv_prefill(ctypes.byref(dims) if dims is not None else None, batch, rows, max_len,
                              p, p, p, p, p, p, p, p, scale, p, ws_bytes, p, None)


def test_prefill_rejects_before_touching_the_device(lib):
    d = main_dims()
    assert call_prefill(lib, None) == INVALID
    assert call_prefill(lib, d, rows=0, ptr=0) == OK                 # no queries: no-op
    assert call_prefill(lib, d, ptr=0) == INVALID
    assert call_prefill(lib, d, ptr=0x1008) == INVALID               # 16-byte alignment
    assert call_prefill(lib, d, batch=0) == INVALID
    assert call_prefill(lib, d, rows=-1) == INVALID
    assert call_prefill(lib, d, max_len=0) == INVALID
    assert call_prefill(lib, d, max_len=512 * 16 + 1) == INVALID
    assert call_prefill(lib, d, scale=float("nan")) == INVALID
    assert call_prefill(lib, main_dims(rank_k=16)) == UNSUPPORTED     # score k-steps need r_k % 32 == 0
    assert call_prefill(lib, main_dims(rank_v=128)) == UNSUPPORTED
    assert call_prefill(lib, main_dims(kv_heads=5)) == INVALID
    assert call_prefill(lib, d, ws_bytes=1024) == WORKSPACE


def test_prefill_workspace_size(lib):
    d = main_dims()
    f = lib.starkv_prefill_workspace_size
    a = f(ctypes.byref(d), 4, 2048, 8192)
    assert a > 0 and a % 256 == 0
    # q~ (fp32) and one fp32 partial state per row alone: rows * H * (r_k + r_v) * 4 bytes
    assert a >= 2048 * 32 * (64 + 1024) * 4
    assert f(ctypes.byref(d), 4, 512, 8192) < a
    assert f(ctypes.byref(d), 0, 512, 8192) == 0
    assert f(ctypes.byref(d), 4, 0, 8192) == 0
    assert f(ctypes.byref(d), 4, 512, 512 * 16 + 1) == 0


def test_check_block_tables_rejects_before_touching_the_device(lib):
    d = main_dims()
    ok_ptr = ctypes.c_void_p(256)
    f = lib.starkv_check_block_tables
    assert f(None, 4, ok_ptr, ok_ptr, ok_ptr, None) == INVALID
    assert f(ctypes.byref(d), 0, ok_ptr, ok_ptr, ok_ptr, None) == INVALID
    assert f(ctypes.byref(d), 4, None, ok_ptr, ok_ptr, None) == INVALID
    assert f(ctypes.byref(d), 4, ok_ptr, None, ok_ptr, None) == INVALID
    assert f(ctypes.byref(d), 4, ok_ptr, ok_ptr, None, None) == INVALID
    assert f(ctypes.byref(d), 4, ok_ptr, ok_ptr, ctypes.c_void_p(258), None) == INVALID   # misaligned count
    assert f(ctypes.byref(main_dims(block_size=32)), 4, ok_ptr, ok_ptr, ok_ptr, None) == UNSUPPORTED


def test_b_v_must_be_16_byte_aligned(lib):
    """Every up-projection path reads B_v rows as 16-byte vectors."""
    d = main_dims()
    p = ctypes.c_void_p(0x1000)
    bad = ctypes.c_void_p(0x1002)
    args = [p, p, bad, p, p, p, p]                     # q, b_k, b_v, k_cache, v_cache, tables, lens
    assert lib.starkv_decode(ctypes.byref(d), 4, 64, *args, 0.1, p, 1 << 30, p, None) == INVALID
    pargs = [p, p, bad, p, p, p, p, p]                 # q, b_k, b_v, pools, tables, query_start, lens
    assert lib.starkv_prefill(ctypes.byref(d), 2, 8, 64, *pargs, 0.1, p, 1 << 30, p, None) == INVALID


def test_rank_k_bounded(lib):
    assert call_decode(lib, main_dims(rank_k=264, head_dim=256)) == UNSUPPORTED
    assert ws_size(lib, main_dims(rank_k=264, head_dim=256), 4, 64) == 0


def test_every_documented_layer_shape_is_accepted(lib):
    """Multi-head layers of 1..32 heads at r_k 16/32/64 and grouped layers with
    H/H_kv <= 16 at r_k 32/64, each at r_v 256..1024, pass the host checks
    (the workspace check comes after the shape check)."""
    for rv in (256, 512, 768, 1024):
        for h in range(1, 33):
            for rk in (16, 32, 64):
                assert call_decode(lib, main_dims(heads=h, kv_heads=h, rank_k=rk, rank_v=rv),
                                   ws_bytes=1024) == WORKSPACE, (h, rk, rv)
            for kv in range(1, h):
                if h % kv or h // kv > 16:
                    continue
                for rk in (32, 64):
                    assert call_decode(lib, main_dims(heads=h, kv_heads=kv, rank_k=rk, rank_v=rv),
                                       ws_bytes=1024) == WORKSPACE, (h, kv, rk, rv)
