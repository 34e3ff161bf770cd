"""The C ABI library loads, exports every function include/fa.h declares, and
rejects bad arguments on the host before any device work. CPU only: every
call here fails validation before the library touches the HIP runtime."""
import ctypes
import os
import re

import pytest

from attention_forward_online_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _header_text():
    with open(HEADER) as fh:
        text = fh.read()
    return re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def declared_functions():
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", _header_text())))


def declared_enum():
    vals = {}
    for name, val in re.findall(r"\b(FA_[A-Z0-9_]+)\s*=\s*(\d+)", _header_text()):
        vals[name] = int(val)
    return vals


def test_header_declares_the_expected_api():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"libfa.so does not export {name}"
    out = os.popen(f"nm -D --defined-only {_lib.library_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), f"{name} not a defined text symbol"


def test_library_was_built_from_the_current_sources():
    # build() records a hash of every source file and the compiler flags
    # beside libfa.so; the loader refuses a library whose hash differs
    from attention_forward_online_fa_amd import build as B
    _lib.lib()
    assert B.built_hash() == B.source_hash()
    assert set(B.SOURCES) <= set(B.source_files())
    assert HEADER in B.source_files()


def test_library_has_no_undefined_symbols_of_its_own():
    # A kernel whose host-side launch stub was not emitted shows up as an
    # undefined fa:: symbol; the library would then fail to load on any box.
    out = os.popen(f"nm -D --undefined-only {_lib.library_path()}").read()
    own = [ln for ln in out.splitlines() if "_ZN2fa" in ln or " fa_" in ln]
    assert not own, f"unresolved library symbols: {own}"


def test_enum_values_match_binding():
    e = declared_enum()
    assert e["FA_F32"] == _lib.FA_F32 and e["FA_BF16"] == _lib.FA_BF16
    for code, name in _lib.STATUS.items():
        assert e[name] == code
    m = re.search(r"#define\s+FA_MAX_SPLITS\s+(\d+)", _header_text())
    assert int(m.group(1)) == _lib.FA_MAX_SPLITS


def test_status_strings():
    lib = _lib.lib()
    assert lib.fa_status_string(0) == b"ok"
    for code in range(1, 11):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(999) == b"unknown status"


A = 0x10000          # a 16-byte aligned fake address; never dereferenced
GOOD = dict(B=1, H=4, HKV=2, Sq=64, Sk=64, D=128, scale=0.125, causal=1, window=0, dtype=1)


def call(ptrs=(A, A, A, A, A), splits=0, **over):
    a = dict(GOOD, **over)
    return _lib.lib().fa_fwd_ex(*ptrs, a["B"], a["H"], a["HKV"], a["Sq"], a["Sk"], a["D"],
                                a["scale"], a["causal"], a["window"], a["dtype"], splits, None)


@pytest.mark.parametrize("which", range(5))
def test_null_pointer(which):
    ptrs = [A] * 5
    ptrs[which] = None
    assert call(tuple(ptrs)) == 1


@pytest.mark.parametrize("over,code", [
    (dict(B=0), 2), (dict(H=0), 2), (dict(HKV=0), 2), (dict(Sq=0), 2), (dict(Sk=-3), 2),
    (dict(H=6, HKV=4), 3), (dict(H=4, HKV=3), 3),
    (dict(D=40), 4), (dict(D=8), 4), (dict(D=112), 4), (dict(D=192), 4), (dict(D=512), 4),
    (dict(dtype=3), 5), (dict(dtype=-1), 5),
    (dict(window=-1), 6), (dict(causal=2), 6),
    (dict(B=1 << 20, H=1 << 10, Sq=1 << 10), 2),
])
def test_argument_errors(over, code):
    assert call(**over) == code


def test_split_count_errors():
    assert call(splits=-1) == 10
    assert call(splits=65) == 10


@pytest.mark.parametrize("which", range(5))
def test_misaligned_buffer(which):
    ptrs = [A] * 5
    ptrs[which] = A + 4
    assert call(tuple(ptrs)) == 7


def test_plan_splits_rejects_bad_args_without_device():
    lib = _lib.lib()
    assert lib.fa_plan_splits(1, 4, 3, 64, 64, 128, 0, 0, 1) == -3
    assert lib.fa_plan_splits(1, 4, 4, 64, 64, 40, 0, 0, 1) == -4


def test_python_binding_fails_loudly_on_cpu_tensors():
    import torch
    import attention_forward_online_fa_amd as fa
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)


# ---------------------------------------------------------------- strided entry
def call_strided(qs=None, ks=None, vs=None, os_=None, **over):
    a = dict(GOOD, **over)
    arr = lambda t: None if t is None else ctypes.cast((ctypes.c_longlong * 3)(*t), ctypes.c_void_p)
    return _lib.lib().fa_fwd_strided(A, A, A, A, A, a["B"], a["H"], a["HKV"], a["Sq"], a["Sk"],
                                     a["D"], arr(qs), arr(ks), arr(vs), arr(os_), a["scale"],
                                     a["causal"], a["window"], a["dtype"], 0, None)


@pytest.mark.parametrize("kw", [
    dict(qs=(0, 128, -128)),               # negative
    dict(ks=(0, 128, 132)),                # K row stride not a multiple of D (and of 16 bytes)
    dict(vs=(8192, 128, 384 - 8)),         # V row stride not a multiple of D
    dict(qs=(8192, 128, 64)),              # row stride < D: rows overlap
    dict(os_=(8192, 3, 512)),              # head stride not a multiple of 16 bytes (bf16)
    dict(ks=(0, 128, 128 * (1 << 24))),    # key tile would span >= 2^31 bytes
    dict(os_=(8192, 0, 128)),              # O heads alias one another
    dict(os_=(0, 8192, 128), B=2),         # O batch entries alias
    dict(os_=(64 * 128, 128, 256)),        # O heads interleave with rows (head 1 row 0 = head 0 row 0.5)
])
def test_strided_rule_errors(kw):
    assert call_strided(**kw) == 11


def test_strided_other_errors_come_first():
    assert call_strided(qs=(0, 128, -128), D=40) == 4
    assert call_strided(qs=(0, 128, -128), dtype=7) == 5
    ptr_a = _lib.lib().fa_fwd_strided(None, A, A, A, A, 1, 4, 2, 64, 64, 128, None, None, None,
                                      None, 0.125, 1, 0, 1, 0, None)
    assert ptr_a == 1


def test_strided_offset_overflow_is_a_shape_error():
    assert call_strided(ks=(1 << 61, 128, 128 * 4), B=4) == 2


# ------------------------------------------------------------ block-sparse entry
def call_sparse(mask=A, mb=1, mh=1, **over):
    a = dict(GOOD, **over)
    return _lib.lib().fa_fwd_block_sparse(A, A, A, A, A, a["B"], a["H"], a["HKV"], a["Sq"],
                                          a["Sk"], a["D"], mask, mb, mh, a["scale"],
                                          a["causal"], a["window"], a["dtype"], 0, None)


def test_block_sparse_null_mask():
    assert call_sparse(mask=None) == 1


@pytest.mark.parametrize("mb,mh", [(2, 1), (0, 1), (1, 3), (1, 0), (1, 8)])
def test_block_sparse_bad_mask_axes(mb, mh):
    # GOOD: B = 1, H = 4, HKV = 2
    assert call_sparse(mb=mb, mh=mh) == 12


def test_block_sparse_shape_errors_come_first():
    assert call_sparse(D=40) == 4
    assert call_sparse(D=96) == 4       # padded head dims take no block mask
    assert call_sparse(H=4, HKV=3) == 3


def test_mask_block_constants_match_header():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    assert re.search(r"#define FA_MASK_BLOCK_Q (\d+)", src).group(1) == str(_lib.FA_MASK_BLOCK_Q)
    assert re.search(r"#define FA_MASK_BLOCK_K (\d+)", src).group(1) == str(_lib.FA_MASK_BLOCK_K)


# ---------------------------------------------------------------- backward entry
def call_bwd(ptrs=(A,) * 9, **over):
    a = dict(GOOD, **over)
    return _lib.lib().fa_bwd(*ptrs, a["B"], a["H"], a["HKV"], a["Sq"], a["Sk"], a["D"],
                             a["scale"], a["causal"], a["window"], a["dtype"], None)


@pytest.mark.parametrize("which", range(9))
def test_bwd_null_and_misaligned(which):
    ptrs = [A] * 9
    ptrs[which] = None
    assert call_bwd(tuple(ptrs)) == 1
    ptrs[which] = A + 4
    assert call_bwd(tuple(ptrs)) == 7


@pytest.mark.parametrize("over,code", [
    (dict(B=0), 2), (dict(H=6, HKV=4), 3), (dict(D=40), 4), (dict(D=512), 4), (dict(dtype=3), 5),
    (dict(window=-1), 6), (dict(causal=2), 6),
])
def test_bwd_argument_errors(over, code):
    assert call_bwd(**over) == code


def call_bwd_sparse(ptrs=(A,) * 9, mask=A, mb=1, mh=1, **over):
    a = dict(GOOD, **over)
    return _lib.lib().fa_bwd_block_sparse(*ptrs, a["B"], a["H"], a["HKV"], a["Sq"], a["Sk"],
                                          a["D"], mask, mb, mh, a["scale"], a["causal"],
                                          a["window"], a["dtype"], None)


def test_bwd_block_sparse_null_pointers():
    assert call_bwd_sparse(mask=None) == 1
    for which in range(9):
        ptrs = [A] * 9
        ptrs[which] = None
        assert call_bwd_sparse(tuple(ptrs)) == 1


@pytest.mark.parametrize("mb,mh", [(2, 1), (0, 1), (1, 3), (1, 0), (1, 8)])
def test_bwd_block_sparse_bad_mask_axes(mb, mh):
    # GOOD: B = 1, H = 4, HKV = 2
    assert call_bwd_sparse(mb=mb, mh=mh) == 12


def test_bwd_block_sparse_shape_errors():
    assert call_bwd_sparse(D=40) == 4
    assert call_bwd_sparse(D=96) == 4      # block masks: D = 64, 128 or 256
    assert call_bwd_sparse(D=32, dtype=0) == 4
    assert call_bwd_sparse(H=4, HKV=3) == 3
    assert call_bwd_sparse(H=2048, HKV=2, mh=1) == 2   # a kv head's query heads: fewer than 1024


@pytest.mark.parametrize("os_", [
    (4 * 64 * 128, 64 * 128, 128),         # contiguous [B, H, S, D]
    (64 * 4 * 128, 128, 4 * 128),          # token-major [B, S, H, D]
    (0, 64 * 128, 128),                    # B = 1: a zero batch stride is harmless
    (8 * 64 * 128, 2 * 64 * 128, 128),     # padded head stride
])
@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="valid arguments would reach a kernel launch on fake pointers")
def test_disjoint_output_strides_pass_the_stride_checks(os_):
    # valid O strides get past every stride rule; with no GPU present the call
    # then stops at the device query (FA_ERR_HIP), never FA_ERR_STRIDE
    assert call_strided(os_=os_, Sq=64, Sk=64) == 8


@pytest.mark.parametrize("D,ks", [
    (96, (0, 64 * 112, 112)),              # K row stride 112: not a multiple of 96
    (48, (0, 64 * 48, 48)),                # contiguous rows of 48
    (80, None),
    (16, (0, 64 * 16, 16)),
])
@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="valid arguments would reach a kernel launch on fake pointers")
def test_padded_head_dims_pass_the_checks(D, ks):
    # head dims 16 .. 96 take any 16-byte row stride for K and V (the padded
    # form addresses every copied chunk in full): past every check, the call
    # stops at the device query
    assert call_strided(ks=ks, D=D, Sq=64, Sk=64) == 8
    assert call(D=D) == 8
    assert call_bwd(D=D) == 8           # likewise for the backward (its workspace pool)


# -------------------------------------------------------- strided backward entry
def call_bwd_strided(strides=(None,) * 8, ptrs=(A,) * 9, **over):
    a = dict(GOOD, **over)
    arr = lambda t: None if t is None else ctypes.cast((ctypes.c_longlong * 3)(*t), ctypes.c_void_p)
    return _lib.lib().fa_bwd_strided(*ptrs, a["B"], a["H"], a["HKV"], a["Sq"], a["Sk"], a["D"],
                                     *[arr(s) for s in strides], a["scale"], a["causal"],
                                     a["window"], a["dtype"], None)


def _bwd_strides(which, st):
    s = [None] * 8
    s[which] = st
    return tuple(s)


@pytest.mark.parametrize("which,st", [
    (0, (0, 128, -128)),                   # negative
    (1, (0, 128, 100)),                    # K row stride < D
    (3, (8192, 3, 512)),                   # O head stride not a multiple of 16 bytes (bf16)
    (5, (8192, 2, 512)),                   # dQ head stride not a multiple of 16 bytes (fp32)
    (5, (8192, 0, 128)),                   # dQ heads alias one another
    (6, (0, 64 * 128, 64)),                # dK rows overlap (row stride < D)
    (7, (64 * 128, 64, 256)),              # dV head 1 starts inside head 0's rows
])
def test_bwd_strided_rule_errors(which, st):
    # GOOD: B = 1, H = 4, HKV = 2, Sq = Sk = 64, D = 128, bf16
    assert call_bwd_strided(_bwd_strides(which, st)) == 11


def test_bwd_strided_other_errors_come_first():
    assert call_bwd_strided(_bwd_strides(0, (0, 128, -128)), D=40) == 4
    assert call_bwd_strided(_bwd_strides(0, (0, 128, -128)), dtype=9) == 5
    ptrs = (None,) + (A,) * 8
    assert call_bwd_strided(ptrs=ptrs) == 1
    assert call_bwd_strided(_bwd_strides(1, (1 << 61, 128, 512)), B=4) == 2


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="valid arguments would reach a kernel launch on fake pointers")
def test_bwd_strided_token_major_passes_the_checks():
    # token-major views of every tensor (and broadcast K/V): past every stride
    # rule, the call stops at the workspace pool's device query
    tm_q = (64 * 4 * 128, 128, 4 * 128)
    tm_k = (64 * 2 * 128, 128, 2 * 128)
    assert call_bwd_strided((tm_q, tm_k, tm_k, tm_q, tm_q, tm_q, tm_k, tm_k)) == 8
    assert call_bwd_strided((None, (0, 64 * 128, 128), None, None, None, None, None, None)) == 8
