"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments before making any HIP call (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

import tiled_attention_attn_amd as taa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADER = os.path.join(INCLUDE, "attn.h")
CSRC = os.path.join(ROOT, "tiled_attention_attn_amd", "csrc")


def declared_functions(path=None):
    """Function names declared in one header, or in every header under include/."""
    paths = [path] if path else sorted(glob.glob(os.path.join(INCLUDE, "*.h")))
    names = set()
    for p in paths:
        text = re.sub(r"/\*.*?\*/", "", open(p).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**((?:attn|ikbo)_\w+)\s*\(", text,
                                flags=re.M))
    return sorted(names)


def _stale() -> bool:
    """The library is missing or older than one of its sources or headers."""
    if not os.path.exists(taa.LIB_PATH):
        return True
    built = os.path.getmtime(taa.LIB_PATH)
    srcs = glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(INCLUDE, "*.h"))
    return any(os.path.getmtime(p) > built for p in srcs)


@pytest.fixture(scope="module")
def lib():
    if _stale():   # never test an old build against new sources
        from tiled_attention_attn_amd.build import build
        build()
    return taa.load_library()


def test_header_declares_the_entry_points():
    assert declared_functions(HEADER) == ["attn_bcast_group", "attn_fwd", "attn_fwd_bcast",
                                          "attn_fwd_bcast_grouped", "attn_fwd_block_sparse",
                                          "attn_fwd_jagged", "attn_fwd_qknorm",
                                          "attn_fwd_qknorm_noalloc", "attn_strerror",
                                          "attn_version", "ikbo_linear"]
    assert declared_functions(os.path.join(INCLUDE, "attn_ceiling.h")) == [
        "attn_ceiling_copy", "attn_ceiling_exp2", "attn_ceiling_exp2_fma", "attn_ceiling_fma",
        "attn_ceiling_lds_read", "attn_ceiling_mfma16_bf16", "attn_ceiling_mfma_bf16"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.attn_version() == 106


def test_strerror_covers_every_status(lib):
    for code in (0, -1, -2, -3, -4):
        assert taa.attn_strerror(code) not in ("", "unknown status")
    assert taa.attn_strerror(12345) == "unknown status"


# A fake, 16-byte aligned, never-dereferenced device address: every case below
# must be rejected (or be an empty no-op) before the library touches it.
FAKE = ctypes.c_void_p(0x1000)
MISALIGNED = ctypes.c_void_p(0x1008)


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=2, Hkv=1, Lq=16, Lk=16, d=64, causal=0,
        kv_len=None, scale=0.0, dtype=taa.ATTN_BF16):
    return lib.attn_fwd(q, k, v, o, B, H, Hkv, Lq, Lk, d, causal, kv_len, scale, dtype, None)


def bcast(lib, c2u=FAKE, B_c=4, B_u=2, H=2, Hkv=2, Lq=16, Lk=16, d=128, scale=0.0,
          dtype=taa.ATTN_BF16):
    return lib.attn_fwd_bcast(FAKE, FAKE, FAKE, FAKE, c2u, B_c, B_u, H, Hkv, Lq, Lk, d, 0, None,
                              scale, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(d=96), taa.ATTN_EUNSUPPORTED),
    (dict(d=256), taa.ATTN_EUNSUPPORTED),
    (dict(dtype=7), taa.ATTN_EUNSUPPORTED),
    (dict(H=3, Hkv=2), taa.ATTN_EINVAL),
    (dict(Hkv=0), taa.ATTN_EINVAL),
    (dict(B=-1), taa.ATTN_EINVAL),
    (dict(Lq=-5), taa.ATTN_EINVAL),
    (dict(Lk=-1), taa.ATTN_EINVAL),
    (dict(scale=-1.0), taa.ATTN_EINVAL),
    (dict(scale=float("inf")), taa.ATTN_EINVAL),
    (dict(scale=float("nan")), taa.ATTN_EINVAL),
    (dict(q=None), taa.ATTN_EINVAL),
    (dict(o=None), taa.ATTN_EINVAL),
    (dict(k=None), taa.ATTN_EINVAL),
    (dict(q=MISALIGNED), taa.ATTN_EINVAL),
    (dict(v=MISALIGNED), taa.ATTN_EINVAL),
    (dict(B=1 << 20, H=1 << 10, Lq=1 << 20, d=128), taa.ATTN_EINVAL),   # size overflow
    (dict(Lk=(1 << 23) - 63, d=128), taa.ATTN_EINVAL),   # K/V head beyond 32-bit offsets
    (dict(B=0), taa.ATTN_OK),             # empty problems launch nothing
    (dict(Lq=0), taa.ATTN_OK),
    (dict(H=0), taa.ATTN_OK),
    (dict(B=0, q=None, o=None), taa.ATTN_OK),
])
def test_attn_fwd_argument_checks(lib, kwargs, status):
    assert fwd(lib, **kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(B_u=0), taa.ATTN_EINVAL),
    (dict(c2u=None), taa.ATTN_EINVAL),
    (dict(d=32), taa.ATTN_EUNSUPPORTED),
    (dict(H=4, Hkv=3), taa.ATTN_EINVAL),
    (dict(B_c=0, c2u=None), taa.ATTN_OK),
])
def test_attn_fwd_bcast_argument_checks(lib, kwargs, status):
    assert bcast(lib, **kwargs) == status


def bcast_grouped(lib, c2u=FAKE, order=FAKE, B_c=4, B_u=2, H=2, Hkv=2, Lq=16, Lk=16, d=128,
                  dtype=taa.ATTN_BF16):
    return lib.attn_fwd_bcast_grouped(FAKE, FAKE, FAKE, FAKE, c2u, order, B_c, B_u, H, Hkv, Lq,
                                      Lk, d, 0, None, 0.0, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(B_u=0), taa.ATTN_EINVAL),
    (dict(c2u=None), taa.ATTN_EINVAL),
    (dict(order=None), taa.ATTN_EINVAL),
    (dict(d=32), taa.ATTN_EUNSUPPORTED),
    (dict(H=4, Hkv=3), taa.ATTN_EINVAL),
    (dict(B_c=0, c2u=None, order=None), taa.ATTN_OK),
])
def test_attn_fwd_bcast_grouped_argument_checks(lib, kwargs, status):
    assert bcast_grouped(lib, **kwargs) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, -1, 2, FAKE, FAKE), taa.ATTN_EINVAL),
    ((FAKE, 4, 0, FAKE, FAKE), taa.ATTN_EINVAL),
    ((FAKE, 4, 2147483647, FAKE, FAKE), taa.ATTN_EINVAL),
    ((None, 4, 2, FAKE, FAKE), taa.ATTN_EINVAL),
    ((FAKE, 4, 2, None, FAKE), taa.ATTN_EINVAL),
    ((FAKE, 4, 2, FAKE, None), taa.ATTN_EINVAL),
    ((None, 0, 2, None, None), taa.ATTN_OK),     # nothing to group: nothing enqueued
])
def test_attn_bcast_group_argument_checks(lib, args, status):
    assert lib.attn_bcast_group(*args, None) == status


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import tiled_attention_attn_amd._binding as b
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        b.load_library(str(tmp_path / "missing.so"))


def jagged(lib, qo=FAKE, ko=FAKE, B=2, H=2, Hkv=1, max_Lq=16, max_Lk=16, d=64, scale=0.0,
           dtype=taa.ATTN_BF16):
    return lib.attn_fwd_jagged(FAKE, FAKE, FAKE, FAKE, qo, ko, B, H, Hkv, max_Lq, max_Lk, d, 0,
                               scale, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(qo=None), taa.ATTN_EINVAL),
    (dict(ko=None), taa.ATTN_EINVAL),
    (dict(d=96), taa.ATTN_EUNSUPPORTED),
    (dict(H=3, Hkv=2), taa.ATTN_EINVAL),
    (dict(B=-1), taa.ATTN_EINVAL),
    (dict(max_Lk=-1), taa.ATTN_EINVAL),
    (dict(scale=float("nan")), taa.ATTN_EINVAL),
    # packed K/V rows are Hkv*d apart: 32-bit buffer offsets bound max_Lk * Hkv
    (dict(max_Lk=(1 << 20), Hkv=8, H=8, d=128), taa.ATTN_EINVAL),
    (dict(B=0, qo=None, ko=None), taa.ATTN_OK),
    (dict(max_Lq=0, qo=None, ko=None), taa.ATTN_OK),
])
def test_attn_fwd_jagged_argument_checks(lib, kwargs, status):
    assert jagged(lib, **kwargs) == status


def sparse(lib, mask=FAKE, mask_heads=1, blk=128, B=1, H=2, Hkv=1, Lq=256, Lk=256, d=128,
           dtype=taa.ATTN_BF16):
    return lib.attn_fwd_block_sparse(FAKE, FAKE, FAKE, FAKE, mask, mask_heads, blk, B, H, Hkv, Lq,
                                     Lk, d, 0, None, 0.0, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(blk=64), taa.ATTN_EINVAL),            # not a multiple of 128
    (dict(blk=0), taa.ATTN_EINVAL),
    (dict(blk=200), taa.ATTN_EINVAL),
    (dict(mask_heads=3, H=4), taa.ATTN_EINVAL),
    (dict(mask=None), taa.ATTN_EINVAL),
    (dict(Lk=128 * 1024 + 1), taa.ATTN_EINVAL),   # 1025 key blocks
    (dict(d=96), taa.ATTN_EUNSUPPORTED),
    (dict(H=3, Hkv=2, mask_heads=3), taa.ATTN_EINVAL),
    (dict(B=0, mask=None), taa.ATTN_OK),
    (dict(Lq=0, mask=None), taa.ATTN_OK),
])
def test_attn_fwd_block_sparse_argument_checks(lib, kwargs, status):
    assert sparse(lib, **kwargs) == status


def ikbo(lib, xu=FAKE, xc=FAKE, w=FAKE, bias=None, c2u=FAKE, y=FAKE, z=FAKE, B_u=4, B_c=64,
         K_u=128, K_c=64, N=256, y_dtype=taa.ATTN_BF16):
    return lib.ikbo_linear(xu, xc, w, bias, c2u, y, z, B_u, B_c, K_u, K_c, N, y_dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(y_dtype=7), taa.ATTN_EUNSUPPORTED),
    (dict(K_u=100), taa.ATTN_EINVAL),            # rows not 16-byte multiples
    (dict(K_c=12), taa.ATTN_EINVAL),
    (dict(N=6), taa.ATTN_EINVAL),                # not a multiple of 4
    (dict(B_c=-1), taa.ATTN_EINVAL),
    (dict(B_u=0), taa.ATTN_EINVAL),              # candidates need users
    (dict(z=None), taa.ATTN_EINVAL),
    (dict(c2u=None), taa.ATTN_EINVAL),
    (dict(y=None), taa.ATTN_EINVAL),
    (dict(xu=ctypes.c_void_p(0x1008)), taa.ATTN_EINVAL),   # misaligned
    (dict(bias=ctypes.c_void_p(0x1004)), taa.ATTN_EINVAL),
    (dict(K_u=1 << 20, K_c=8), taa.ATTN_EINVAL),           # K above 2^20
    (dict(K_u=65536, K_c=0, N=16384), taa.ATTN_EINVAL),    # weight past 2^31 bytes
    (dict(K_u=0, K_c=0, N=1 << 22), taa.ATTN_EINVAL),      # bf16 tile rows past 2^31 bytes
    (dict(N=0), taa.ATTN_OK),
    (dict(B_u=0, B_c=0), taa.ATTN_OK),
    (dict(B_c=0, z=None), taa.ATTN_EINVAL),      # z is written whenever there are users
])
def test_ikbo_linear_argument_checks(lib, kwargs, status):
    assert ikbo(lib, **kwargs) == status


FAKE2 = ctypes.c_void_p(0x2000)


def qknorm(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, gq=None, gk=None, eps=1e-6, kn=FAKE2, B=1, H=2,
           Hkv=1, Lq=64, Lk=64, d=128, causal=0, dtype=taa.ATTN_BF16):
    return lib.attn_fwd_qknorm(q, k, v, o, gq, gk, eps, kn, B, H, Hkv, Lq, Lk, d, causal, None,
                               0.0, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=taa.ATTN_F32), taa.ATTN_EUNSUPPORTED),   # bf16 only
    (dict(d=96), taa.ATTN_EUNSUPPORTED),
    (dict(eps=-1.0), taa.ATTN_EINVAL),
    (dict(eps=float("inf")), taa.ATTN_EINVAL),
    (dict(kn=None), taa.ATTN_EINVAL),                    # keys need a workspace
    (dict(kn=FAKE), taa.ATTN_EINVAL),                    # ... that is not k
    (dict(gq=ctypes.c_void_p(0x1004)), taa.ATTN_EINVAL), # misaligned gain
    (dict(kn=ctypes.c_void_p(0x2008)), taa.ATTN_EINVAL),
    (dict(H=3, Hkv=2), taa.ATTN_EINVAL),                 # the attention checks apply first
    (dict(o=None), taa.ATTN_EINVAL),
    (dict(B=0, kn=None), taa.ATTN_OK),                   # nothing to compute
    (dict(Lq=0, kn=None), taa.ATTN_OK),
])
def test_attn_fwd_qknorm_argument_checks(lib, kwargs, status):
    assert qknorm(lib, **kwargs) == status


def test_ceiling_probe_argument_checks(lib):
    """The ceiling probes reject bad arguments with -1 before any HIP call; an empty copy
    launches nothing and succeeds."""
    assert lib.attn_ceiling_mfma_bf16(None, 1, FAKE, 1, 8, 1, None) == -1
    assert lib.attn_ceiling_mfma_bf16(FAKE, 0, FAKE, 1, 8, 1, None) == -1    # no operand lanes
    assert lib.attn_ceiling_mfma_bf16(FAKE, 1, FAKE, 1, 6, 1, None) == -1    # waves not 4 or 8
    assert lib.attn_ceiling_mfma_bf16(MISALIGNED, 1, FAKE, 1, 8, 1, None) == -1
    assert lib.attn_ceiling_mfma_bf16(FAKE, 1, FAKE, 0, 8, 1, None) == -1    # no workgroups
    assert lib.attn_ceiling_mfma16_bf16(None, 1, FAKE, 1, 8, 1, None) == -1
    assert lib.attn_ceiling_mfma16_bf16(FAKE, 1, FAKE, 1, 6, 1, None) == -1  # waves not 4 or 8
    assert lib.attn_ceiling_exp2(None, 1, 1, None) == -1
    assert lib.attn_ceiling_exp2(FAKE, 0, 1, None) == -1
    assert lib.attn_ceiling_fma(FAKE, 1, 0, None) == -1                      # no iterations
    assert lib.attn_ceiling_exp2_fma(None, 1, 1, None) == -1
    assert lib.attn_ceiling_exp2_fma(FAKE, 1, 0, None) == -1
    assert lib.attn_ceiling_lds_read(None, 1, 1, 0, None) == -1
    assert lib.attn_ceiling_copy(FAKE, FAKE, 17, None) == -1                 # not 16-byte units
    assert lib.attn_ceiling_copy(MISALIGNED, FAKE, 16, None) == -1
    assert lib.attn_ceiling_copy(FAKE, FAKE, 0, None) == 0


def test_qknorm_noalloc_checks_before_any_hip_call(lib):
    """The allocation-free q/k-norm call runs attn_fwd_qknorm's argument checks, then its
    workspace limit, before any HIP call."""
    f = lib.attn_fwd_qknorm_noalloc
    args = lambda B=1, H=2, Hkv=2, Lq=16, Lk=16, d=128, dtype=taa.ATTN_BF16, eps=1e-6: (  # noqa
        FAKE, FAKE, FAKE, FAKE, None, None, eps, B, H, Hkv, Lq, Lk, d, 0, None, 0.0, dtype, None)
    assert f(*args(dtype=taa.ATTN_F32)) == taa.ATTN_EUNSUPPORTED
    assert f(*args(d=96)) == taa.ATTN_EUNSUPPORTED
    assert f(*args(eps=-1.0)) == taa.ATTN_EINVAL
    assert f(*args(H=3)) == taa.ATTN_EINVAL                     # H % Hkv != 0
    assert f(*args(B=2, H=8, Hkv=8, Lk=16384)) == taa.ATTN_ESCRATCH   # 64 MiB of keys
    assert f(*args(B=0)) == taa.ATTN_OK                         # empty: nothing to launch
    assert taa.attn_strerror(taa.ATTN_ESCRATCH) not in ("", "unknown status")
