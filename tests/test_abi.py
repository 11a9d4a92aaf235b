"""The C ABI without a GPU: libfg8.so loads, exports every function that
include/fg8.h declares, and rejects bad arguments with the documented status
before launching anything (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fg8.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:fg8_status|size_t|const char\*|int64_t|int)\s+(\w+)\s*\(", text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    from moe_grouped_gemm_fp8_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfg8.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_header_lists_the_five_entry_points():
    names = _declared()
    for n in ("fp8_quantize", "gemm_fp8_blockscaled", "grouped_gemm_fp8_contiguous",
              "grouped_gemm_fp8_masked", "gemm_mxfp8", "fg8_gemm_workspace_bytes",
              "fg8_last_error", "fg8_version", "fp8_quantize_bf16",
              "grouped_gemm_mxfp8_contiguous", "moe_contiguous_layout_fp8",
              "fg8_moe_capacity", "grouped_gemm_fp8_contiguous_swiglu",
              "grouped_gemm_fp8_kgrouped"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in _declared():
        assert hasattr(L, n), f"{n} declared in fg8.h but not exported"
    assert L.fg8_version() == 500


P = ctypes.c_void_p


def _fake(addr):
    return P(addr)   # never dereferenced: validation fails before any launch


def test_quantize_validation(L):
    ok = _fake(0x10000)
    assert L.fp8_quantize(None, 1, 1, 128, 0, ok, ok, None) == 1
    assert b"x is NULL" in L.fg8_last_error()
    assert L.fp8_quantize(_fake(0x10004), 1, 1, 128, 0, ok, ok, None) == 1
    assert b"16-byte" in L.fg8_last_error()
    assert L.fp8_quantize(ok, 1, 1, 130, 0, ok, ok, None) == 2
    assert L.fp8_quantize(ok, 1, 1, 96, 1, ok, ok, None) == 2
    assert L.fp8_quantize(ok, 0, 1, 128, 0, ok, ok, None) == 1
    assert L.fp8_quantize(ok, 1, 1, 128, 7, ok, ok, None) == 1
    assert b"scale kind" in L.fg8_last_error()


def test_gemm_validation(L):
    ok = _fake(0x10000)
    f = L.gemm_fp8_blockscaled
    assert f(ok, ok, ok, ok, None, 0, 64, 64, 256, None, 0, None) == 1
    assert f(ok, ok, ok, ok, ok, 5, 64, 64, 256, None, 0, None) == 1
    assert f(ok, ok, ok, ok, ok, 0, 0, 64, 256, None, 0, None) == 1
    assert f(ok, ok, ok, ok, ok, 0, 64, 64, 200, None, 0, None) == 2
    assert f(ok, ok, ok, ok, ok, 0, 64, 64, 64, None, 0, None) == 2
    assert f(ok, ok, ok, ok, ok, 0, 64, 64, 1 << 24, None, 0, None) == 2
    # a split-K shape with no workspace is refused before launching
    need = L.fg8_gemm_workspace_bytes(64, 2112, 7168)
    assert need > 4096
    assert f(ok, ok, ok, ok, ok, 0, 64, 2112, 7168, None, 0, None) == 1
    assert b"workspace" in L.fg8_last_error()
    assert f(ok, ok, ok, ok, ok, 0, 64, 2112, 7168, ok, need - 1, None) == 1


def test_workspace_bytes_host_logic(L):
    assert L.fg8_gemm_workspace_bytes(4096, 7168, 2048) == 0      # enough tiles: no split
    assert L.fg8_gemm_workspace_bytes(64, 2112, 200) == 0         # invalid K
    a = L.fg8_gemm_workspace_bytes(64, 2112, 7168)
    assert (a - 4096) % (64 * 32 * 4) == 0                        # whole 64x32 FP32 tiles


def test_grouped_validation(L):
    ok = _fake(0x10000)
    c = L.grouped_gemm_fp8_contiguous
    assert c(ok, ok, ok, ok, None, ok, 0, 256, 64, 256, 4, None) == 1
    assert c(ok, ok, ok, ok, ok, ok, 0, 200, 64, 256, 4, None) == 2
    assert c(ok, ok, ok, ok, ok, ok, 0, 256, 64, 256, 0, None) == 1
    m = L.grouped_gemm_fp8_masked
    assert m(ok, ok, ok, ok, None, ok, 0, 4, 256, 64, 256, None) == 1
    assert m(ok, ok, ok, ok, ok, ok, 0, 2000, 256, 64, 256, None) == 1
    assert m(ok, ok, ok, ok, ok, ok, 0, 4, 256, 64, 100, None) == 2
    x = L.gemm_mxfp8
    assert x(ok, ok, ok, ok, None, ok, 0, 0, 64, 64, 256, None) == 1
    assert x(ok, ok, ok, ok, _fake(0x10008), ok, 0, 2, 64, 64, 256, None) == 1
    assert x(ok, ok, ok, ok, None, ok, 0, 2, 64, 64, 96, None) == 2


def test_bf16_quantize_and_mx_contiguous_validation(L):
    ok = _fake(0x10000)
    q = L.fp8_quantize_bf16
    assert q(None, 1, 1, 128, 0, ok, ok, None) == 1
    assert b"x is NULL" in L.fg8_last_error()
    assert q(_fake(0x10002), 1, 1, 128, 0, ok, ok, None) == 1
    assert q(ok, 1, 1, 100, 2, ok, ok, None) == 2
    c = L.grouped_gemm_mxfp8_contiguous
    assert c(ok, ok, ok, ok, None, ok, 0, 256, 64, 256, 4, None) == 1
    assert b"block_expert is NULL" in L.fg8_last_error()
    assert c(ok, ok, ok, ok, ok, ok, 0, 200, 64, 256, 4, None) == 2
    assert c(ok, ok, ok, ok, ok, ok, 0, 256, 64, 96, 4, None) == 2
    assert c(ok, ok, ok, ok, ok, ok, 0, 256, 64, 256, 0, None) == 1


def test_moe_capacity_host_logic(L):
    cap = L.fg8_moe_capacity
    cap.restype = ctypes.c_int64
    assert cap(8192, 8, 32) == 69632            # 65536 routed rows + 32 * 127, in 128-row blocks
    assert cap(1, 1, 1) == 128
    assert cap(5, 2, 3) == 512                   # (10 + 381) rounded up to 512
    assert cap(0, 8, 32) == 0 and cap(8, 0, 32) == 0 and cap(8, 8, 0) == 0
    assert cap(8, 8, 1025) == 0 and cap(8, 257, 4) == 0


def test_moe_layout_validation(L):
    ok = _fake(0x10000)
    f = L.moe_contiguous_layout_fp8
    f.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int64, P, P, P, P, P, P, P, P]

    def call(x=ok, bf16=0, tokens=8192, hidden=7168, ids=ok, topk=8, experts=32, m_cap=69632,
             offsets=ok):
        return f(x, bf16, tokens, hidden, ids, topk, experts, m_cap, ok, ok, ok, ok, ok, offsets,
                 ok, None)

    assert call(ids=None) == 1 and b"topk_ids is NULL" in L.fg8_last_error()
    assert call(offsets=_fake(0x10004)) == 1 and b"16-byte" in L.fg8_last_error()
    assert call(bf16=2) == 1
    assert call(tokens=0) == 1
    assert call(topk=0) == 1 and call(topk=257) == 1
    assert call(experts=0) == 1 and call(experts=1025) == 1
    assert call(hidden=7100) == 2
    assert call(m_cap=69632 - 128) == 1 and b"m_cap" in L.fg8_last_error()
    assert call(m_cap=69632 + 64) == 1


def test_swiglu_validation(L):
    ok = _fake(0x10000)
    f = L.grouped_gemm_fp8_contiguous_swiglu
    f.argtypes = [P] * 7 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, P]
    assert f(ok, ok, ok, ok, ok, None, ok, 256, 512, 512, 4, None) == 1
    assert b"q_out is NULL" in L.fg8_last_error()
    assert f(ok, ok, ok, ok, ok, ok, ok, 256, 384, 512, 4, None) == 2      # n not a multiple of 256
    assert b"gate/up" in L.fg8_last_error()
    assert f(ok, ok, ok, ok, ok, ok, ok, 200, 512, 512, 4, None) == 2      # m_total % 128
    assert f(ok, ok, ok, ok, ok, ok, ok, 256, 512, 500, 4, None) == 2      # k % 128
    assert f(ok, ok, ok, ok, ok, ok, ok, 256, 512, 512, 0, None) == 1


def test_kgrouped_and_transposed_quantize_validation(L):
    ok = _fake(0x10000)
    f = L.grouped_gemm_fp8_kgrouped
    f.argtypes = [P] * 6 + [ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                            ctypes.c_int64, P]
    assert f(ok, ok, ok, ok, None, ok, 0, 4, 256, 512, 1024, None) == 1
    assert b"k_offsets is NULL" in L.fg8_last_error()
    assert f(ok, ok, ok, ok, ok, ok, 0, 0, 256, 512, 1024, None) == 1
    assert f(ok, ok, ok, ok, ok, ok, 0, 4, 256, 512, 1000, None) == 2
    assert f(ok, ok, ok, ok, ok, ok, 0, 4, 256, 512, 1 << 24, None) == 2
    assert f(ok, ok, ok, ok, ok, ok, 3, 4, 256, 512, 1024, None) == 1
    q = L.fp8_quantize
    assert q(ok, 1, 200, 128, 3, ok, ok, None) == 2          # rows not whole groups
    assert b"transposed" in L.fg8_last_error()
    assert q(ok, 1, 256, 96, 3, ok, ok, None) == 2           # cols % 64
    assert q(ok, 1, 256, 4, 4, ok, ok, None) == 1            # unknown kind


def test_noalloc_scratch_covers_every_split_k_workspace(L):
    """gemm_fp8_blockscaled_noalloc keeps its split-K scratch in a static
    array of FG8_NOALLOC_SCRATCH_BYTES per GPU; on a 256-CU part no dense
    shape needs more (split-K is used only while the tiles fill at most one
    round, so the partials are bounded by one tile per workgroup slot)."""
    import re
    cap = int(eval(re.search(r"#define FG8_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                             open(HEADER).read()).expand(r"\1 << \2")))
    assert cap == 16 << 20
    worst = 0
    for m in (1, 7, 16, 33, 64, 65, 100, 128, 129, 200, 256, 300, 512, 1024):
        for n in (1, 64, 130, 256, 520, 1000, 2112, 4096, 7168, 16384, 24576):
            for k in (128, 512, 1024, 2048, 7168, 16384, 65536):
                need = L.fg8_gemm_workspace_bytes(m, n, k)
                worst = max(worst, need)
                assert need <= cap, (m, n, k, need)
    assert worst > 4096                       # some shapes do use split-K
    print(f"largest split-K workspace over the sweep: {worst} bytes")


def test_noalloc_validation(L):
    ok = _fake(0x10000)
    assert L.gemm_fp8_blockscaled_noalloc(None, ok, ok, ok, ok, 0, 64, 64, 128, None) == 1
    assert b"a is NULL" in L.fg8_last_error()
    assert L.gemm_fp8_blockscaled_noalloc(ok, ok, ok, ok, ok, 0, 64, 64, 200, None) == 2
    assert L.gemm_fp8_blockscaled_noalloc(ok, ok, ok, ok, ok, 7, 64, 64, 128, None) == 1
