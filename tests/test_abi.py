"""CPU checks of the C ABI: the library loads, exports every function the
header declares, the ctypes structs match the C layout, and invalid arguments
return the documented error codes without launching anything."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import torch

import bit_rotated_kv_oscar_amd as oscar
from bit_rotated_kv_oscar_amd import _lib

# The calls below pass fake device addresses.  Those with otherwise valid
# arguments would launch kernels, so they only run where no GPU is visible.
NO_GPU = not torch.cuda.is_available()

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"OSCAR_API\s+[\w\s\*]*?\b(oscar_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = header_functions()
    for required in ("oscar_calibrate_rotation", "oscar_write_kv", "oscar_decode_attn",
                     "oscar_bf16_paged_decode", "oscar_prepare_rotation", "oscar_last_error"):
        assert required in names


def test_library_exports_every_header_function():
    lib = _lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (oscar_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert {n for n, _, _ in _lib.SIGNATURES} == set(header_functions())


def test_struct_layout_matches_c():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "oscar.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %d\n", sizeof(oscar_layer_cache),
        offsetof(oscar_layer_cache, group), offsetof(oscar_layer_cache, hist),
        offsetof(oscar_layer_cache, n_hist_pages), offsetof(oscar_layer_cache, bf16),
        offsetof(oscar_layer_cache, n_bf16_pages), offsetof(oscar_layer_cache, hist_pt),
        offsetof(oscar_layer_cache, hist_pt_stride), offsetof(oscar_layer_cache, bf16_pt),
        offsetof(oscar_layer_cache, status), offsetof(oscar_layer_cache, code_bits),
        sizeof(oscar_rotation), offsetof(oscar_rotation, clip), offsetof(oscar_rotation, n_heads),
        offsetof(oscar_rotation, head_clips), OSCAR_MAX_HEAD_ROTATIONS);
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    L = _lib.LayerCacheC
    expect = [ctypes.sizeof(L), L.group.offset, L.hist.offset, L.n_hist_pages.offset, L.bf16.offset,
              L.n_bf16_pages.offset, L.hist_pt.offset, L.hist_pt_stride.offset, L.bf16_pt.offset,
              L.status.offset, L.code_bits.offset, ctypes.sizeof(_lib.RotationC), _lib.RotationC.clip.offset,
              _lib.RotationC.n_heads.offset, _lib.RotationC.head_clips.offset, _lib.MAX_HEAD_ROTATIONS]
    assert vals == expect


def test_sizes():
    assert [oscar.hist_block_bytes(g) for g in (32, 64, 128)] == [1536, 1280, 1152]
    assert oscar.hist_block_bytes(48) == 0
    assert [oscar.hist_block_bytes(g, 4) for g in (32, 64, 128)] == [2560, 2304, 2176]
    assert oscar.hist_block_bytes(32, 3) == 0 and oscar.hist_block_bytes(32, 8) == 0
    assert oscar.rotation_bytes() == 196608
    assert oscar.decode_workspace_bytes(1, 32, 8, 32768) > 0
    assert oscar.decode_workspace_bytes(0, 32, 8, 32768) == 0
    assert oscar.bf16_decode_workspace_bytes(64, 32, 8, 32768) > 0


def _cache(**kw):
    c = _lib.LayerCacheC(2, 32, 0x1000, 4, 0x2000, 9, 0x3000, 1, 0x4000, 0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


ROT = _lib.RotationC(0x5000, 4.0)


def _write(c=None, rk=ROT, rv=ROT, k=0x6000, v=0x7000, cu=0x8000, lb=0x9000, batch=1, total=16, max_new=16):
    lib = _lib.load()
    c = c if c is not None else _cache()
    return lib.oscar_write_kv(ctypes.byref(c), ctypes.byref(rk), ctypes.byref(rv), k, v, cu, lb, batch,
                              total, max_new, None)


def _err():
    return _lib.load().oscar_last_error().decode()


def test_write_validation_codes():
    E = _lib
    assert _write(c=_cache(group=48)) == E.OSCAR_EUNSUPPORTED and "group" in _err()
    assert _write(c=_cache(n_kv_heads=0)) == E.OSCAR_EINVAL
    assert _write(c=_cache(hist=0)) == E.OSCAR_EINVAL
    assert _write(c=_cache(bf16_pt=0)) == E.OSCAR_EINVAL
    assert _write(c=_cache(hist_pt_stride=0)) == E.OSCAR_EINVAL
    assert _write(rk=_lib.RotationC(0x5000, float("nan"))) == E.OSCAR_EINVAL and "clip" in _err()
    assert _write(rk=_lib.RotationC(0x5000, -1.0)) == E.OSCAR_EINVAL
    assert _write(rv=_lib.RotationC(0x5000, 1e6)) == E.OSCAR_EINVAL
    assert _write(rv=_lib.RotationC(0, 1.0)) == E.OSCAR_EINVAL
    assert _write(batch=0) == E.OSCAR_EINVAL
    assert _write(max_new=32, total=16) == E.OSCAR_EINVAL
    # per-KV-head rotations: n_heads must be the cache's n_kv_heads (2 here),
    # with a valid host clip per head
    clips = (ctypes.c_float * 2)(3.0, 4.0)
    cp = ctypes.cast(clips, ctypes.POINTER(ctypes.c_float))
    assert _write(rk=_lib.RotationC(0x5000, 0.0, 3, cp)) == E.OSCAR_EINVAL and "n_heads" in _err()
    assert _write(rk=_lib.RotationC(0x5000, 0.0, -1, None)) == E.OSCAR_EINVAL and "n_heads" in _err()
    assert _write(rv=_lib.RotationC(0x5000, 0.0, 2, None)) == E.OSCAR_EINVAL and "head_clips" in _err()
    bad = (ctypes.c_float * 2)(3.0, float("inf"))
    assert _write(rv=_lib.RotationC(0x5000, 0.0, 2, ctypes.cast(bad, ctypes.POINTER(ctypes.c_float)))) == \
        E.OSCAR_EINVAL and "head_clips[1]" in _err()
    big = _cache(n_kv_heads=40)
    clips40 = (ctypes.c_float * 40)(*([2.0] * 40))
    assert _write(c=big, rk=_lib.RotationC(0x5000, 0.0, 40, ctypes.cast(clips40, ctypes.POINTER(ctypes.c_float)))) \
        == E.OSCAR_EINVAL and "at most 32" in _err()
    assert _write(k=0) == E.OSCAR_EINVAL
    assert _write(cu=0) == E.OSCAR_EINVAL
    # nothing to write: success without touching a device
    assert _write(max_new=0, total=0, k=0, v=0) == E.OSCAR_OK
    if NO_GPU:  # valid arguments, no device: refused before any launch
        assert _write() == E.OSCAR_ENODEV
        assert _write(rk=_lib.RotationC(0x5000, 0.0, 2, cp)) == E.OSCAR_ENODEV  # per-head: valid


def _decode(c=None, hq=8, batch=1, max_len=150, ws=0xA000, ws_bytes=1 << 30, scale=0.088, q=0xB000):
    lib = _lib.load()
    c = c if c is not None else _cache()
    return lib.oscar_decode_attn(ctypes.byref(c), ctypes.byref(ROT), ctypes.byref(ROT), q, hq, 0xC000, batch,
                                 max_len, scale, 0xD000, ws, ws_bytes, None)


def test_decode_validation_codes():
    E = _lib
    assert _decode(hq=7) == E.OSCAR_EUNSUPPORTED and "multiple" in _err()
    assert _decode(hq=64) == E.OSCAR_EUNSUPPORTED            # GQA 32
    assert _decode(hq=6) == E.OSCAR_EUNSUPPORTED             # GQA 3
    assert _decode(max_len=0) == E.OSCAR_EINVAL
    assert _decode(max_len=10_000) == E.OSCAR_EINVAL and "hist_pt_stride" in _err()
    assert _decode(q=0) == E.OSCAR_EINVAL
    assert _decode(scale=0.0) == E.OSCAR_EINVAL
    assert _decode(ws=0) == E.OSCAR_EWORKSPACE
    assert _decode(ws_bytes=16) == E.OSCAR_EWORKSPACE and "workspace" in _err()
    assert _decode(batch=0) == E.OSCAR_EINVAL
    if NO_GPU:
        assert _decode() == E.OSCAR_ENODEV


def test_bf16_decode_validation_codes():
    lib = _lib.load()
    E = _lib

    def call(hq=8, hkv=2, pt_stride=4, max_len=64, n_pages=8, ws_bytes=1 << 30, pt=0x1):
        return lib.oscar_bf16_paged_decode(0x1000, 0x2000, n_pages, pt, pt_stride, 0x3000, 1, max_len, hq, hkv,
                                           0.088, 0x4000, None, 0x5000, ws_bytes, None)
    assert call(hq=6, hkv=4) == E.OSCAR_EUNSUPPORTED
    assert call(pt_stride=3) == E.OSCAR_EINVAL
    assert call(n_pages=0) == E.OSCAR_EINVAL
    assert call(pt=0) == E.OSCAR_EINVAL
    assert call(ws_bytes=0) == E.OSCAR_EWORKSPACE
    if NO_GPU:
        assert call() == E.OSCAR_ENODEV


def test_calibrate_and_prepare_validation_codes():
    lib = _lib.load()
    E = _lib
    R = (ctypes.c_double * (128 * 128))()
    f = ctypes.c_float()
    W, WB = 0xE000, 1 << 40   # a workspace pointer and size that pass the size checks

    def cal(q=0x1, n=16, hq=8, hkv=2, p=0.999, ws=W, wb=WB):
        return lib.oscar_calibrate_rotation(q, 0x1, 0x1, n, hq, hkv, p, R, R, ctypes.byref(f), ctypes.byref(f),
                                            ws, wb, None)
    assert cal(q=0) == E.OSCAR_EINVAL
    assert cal(n=0) == E.OSCAR_EINVAL
    assert cal(hkv=3) == E.OSCAR_EUNSUPPORTED
    assert cal(p=1.5) == E.OSCAR_EINVAL
    assert cal(ws=0) == E.OSCAR_EWORKSPACE
    need = lib.oscar_calibrate_workspace_bytes(16, 8, 2)
    assert cal(wb=need - 1) == E.OSCAR_EWORKSPACE and "workspace" in _err()
    assert lib.oscar_prepare_rotation(0, 0x1, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_accumulate(0, 0x1, 0x1, 16, 8, 2, 0x1, W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_accumulate(0x1, 0x1, 0x1, 0, 8, 2, 0x1, W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_accumulate(0x1, 0x1, 0x1, 16, 8, 3, 0x1, W, WB, None) == E.OSCAR_EUNSUPPORTED
    assert lib.oscar_calib_accumulate(0x1, 0x1, 0x1, 16, 8, 2, 0x1, W, 1024, None) == E.OSCAR_EWORKSPACE
    assert lib.oscar_calib_accumulate_heads(0, 0x1, 0x1, 16, 8, 2, 0x1, W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_accumulate_heads(0x1, 0x1, 0x1, 70000, 8, 2, 0x1, W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_accumulate_heads(0x1, 0x1, 0x1, 16, 8, 3, 0x1, W, WB, None) == E.OSCAR_EUNSUPPORTED
    assert lib.oscar_calib_accumulate_heads(0x1, 0x1, 0x1, 16, 8, 2, 0x1, W, 1024, None) == E.OSCAR_EWORKSPACE
    assert lib.oscar_calib_rotations(0x1, 0.0, R, R, W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_rotations(0x1, float("nan"), R, R, W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_rotations(0, 10.0, R, R, W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_calib_rotations(0x1, 10.0, R, R, 0, WB, None) == E.OSCAR_EWORKSPACE
    assert lib.oscar_clip_threshold(0, 16, R, 0.999, ctypes.byref(f), W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_clip_threshold(0x1, 0, R, 0.999, ctypes.byref(f), W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_clip_threshold(0x1, 16, R, 0.0, ctypes.byref(f), W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_clip_threshold(0x1, 16, None, 0.999, ctypes.byref(f), W, WB, None) == E.OSCAR_EINVAL
    assert lib.oscar_clip_threshold(0x1, 16, R, 0.999, ctypes.byref(f), W, 100, None) == E.OSCAR_EWORKSPACE
    # no cap on the number of vectors beyond the int32 grid limit
    assert lib.oscar_clip_threshold(0x1, 1 << 31, R, 0.999, ctypes.byref(f), W, WB, None) == E.OSCAR_EINVAL
    # workspace sizes: monotone in the sizes they depend on, 0 for invalid ones
    assert lib.oscar_clip_threshold_workspace_bytes(1 << 22) > lib.oscar_clip_threshold_workspace_bytes(1 << 20) > 0
    assert lib.oscar_clip_threshold_workspace_bytes(0) == 0
    assert lib.oscar_calibrate_workspace_bytes(2048, 32, 8) > lib.oscar_calibrate_workspace_bytes(1024, 32, 8) > 0
    assert lib.oscar_calib_accumulate_workspace_bytes(0, 8, 2) == 0
    assert lib.oscar_calib_rotations_workspace_bytes() >= 3 * 128 * 128 * 8


def test_errors_raise_in_binding():
    with pytest.raises(_lib.OscarError) as ei:
        _lib.check(_write(c=_cache(group=16)))
    assert ei.value.code == _lib.OSCAR_EUNSUPPORTED


def test_profile_events_needs_both_or_neither():
    lib = _lib.load()
    assert lib.oscar_profile_events(ctypes.c_void_p(0x1000), None) == _lib.OSCAR_EINVAL and "both" in _err()
    assert lib.oscar_profile_events(None, ctypes.c_void_p(0x1000)) == _lib.OSCAR_EINVAL
    assert lib.oscar_profile_events(None, None) == _lib.OSCAR_OK


def test_extend_validation_codes():
    lib = _lib.load()
    E = _lib

    def call(c=None, hq=8, batch=1, total=16, max_new=16, max_prefix=100, scale=0.088, q=0xB000, cu=0x8000):
        c = c if c is not None else _cache()
        return lib.oscar_extend_attn(ctypes.byref(c), ctypes.byref(ROT), ctypes.byref(ROT), q, hq, 0x6000, 0x7000,
                                     cu, 0x9000, batch, total, max_new, max_prefix, scale, 0xD000, None)
    assert call(hq=6) == E.OSCAR_EUNSUPPORTED
    assert call(c=_cache(group=48)) == E.OSCAR_EUNSUPPORTED
    assert call(c=_cache(code_bits=3)) == E.OSCAR_EUNSUPPORTED and "code_bits" in _err()
    assert call(batch=0) == E.OSCAR_EINVAL
    assert call(max_new=32, total=16) == E.OSCAR_EINVAL
    assert call(max_prefix=-1) == E.OSCAR_EINVAL
    assert call(max_prefix=10_000) == E.OSCAR_EINVAL and "hist_pt_stride" in _err()
    assert call(scale=float("inf")) == E.OSCAR_EINVAL
    assert call(q=0) == E.OSCAR_EINVAL
    assert call(cu=0) == E.OSCAR_EINVAL
    assert call(max_new=0, total=0, q=0) == E.OSCAR_OK
    if NO_GPU:
        assert call() == E.OSCAR_ENODEV


def test_read_probe_validation_codes():
    lib = _lib.load()
    E = _lib
    assert lib.oscar_read_probe(0, 4096, 1, 1024, None, 0x10, None) == E.OSCAR_EINVAL        # NULL buf
    assert lib.oscar_read_probe(0x10, 4096, 1, 1024, None, 0, None) == E.OSCAR_EINVAL        # NULL sink
    assert lib.oscar_read_probe(0x10, 4096, 1, 1000, None, 0x10, None) == E.OSCAR_EINVAL     # not x16
    assert lib.oscar_read_probe(0x10, 1 << 20, 1, 8192, None, 0x10, None) == E.OSCAR_EINVAL  # > 4096
    assert lib.oscar_read_probe(0x10, 4096, 0, 1024, None, 0x10, None) == E.OSCAR_EINVAL     # no blocks
    assert lib.oscar_read_probe(0x10, 4096, 5, 1024, None, 0x10, None) == E.OSCAR_EINVAL     # past the end


def _decode_noalloc(c=None, hq=8, batch=1, max_len=150, scale=0.088, q=0xB000):
    lib = _lib.load()
    c = c if c is not None else _cache()
    return lib.oscar_decode_attn_noalloc(ctypes.byref(c), ctypes.byref(ROT), ctypes.byref(ROT), q, hq, 0xC000, batch,
                                         max_len, scale, 0xD000, None)


def test_decode_noalloc_validation_codes():
    E = _lib
    assert _lib.load().oscar_decode_noalloc_max_bytes() == 16 << 20
    assert _decode_noalloc(hq=7) == E.OSCAR_EUNSUPPORTED
    assert _decode_noalloc(max_len=0) == E.OSCAR_EINVAL
    assert _decode_noalloc(q=0) == E.OSCAR_EINVAL
    assert _decode_noalloc(batch=0) == E.OSCAR_EINVAL
    # beyond the library's scratch: more (request, KV head) units than it
    # holds, or more partials than fit -- refused before any device call
    assert _decode_noalloc(batch=4097) == E.OSCAR_EWORKSPACE and "scratch" in _err()
    big = _cache(hist_pt_stride=4096)
    assert _decode_noalloc(c=big, batch=300, max_len=60000) == E.OSCAR_EWORKSPACE
    if NO_GPU:
        assert _decode_noalloc() == E.OSCAR_ENODEV


def test_code_bits_validation():
    E = _lib
    # INT2 (0 or 2) and INT4 caches pass the cache checks of write and
    # decode (valid arguments are only sent where no device can run them)
    if NO_GPU:
        for bits in (0, 2, 4):
            assert _write(c=_cache(code_bits=bits)) == E.OSCAR_ENODEV, (bits, _err())
            assert _decode(c=_cache(code_bits=bits)) == E.OSCAR_ENODEV, (bits, _err())
    for bits in (1, 3, 8, -2):
        assert _write(c=_cache(code_bits=bits)) == E.OSCAR_EUNSUPPORTED and "code_bits" in _err()
        assert _decode(c=_cache(code_bits=bits)) == E.OSCAR_EUNSUPPORTED
    # the append step takes INT4 caches too (refused here only for want of a device)
    if NO_GPU:
        lib = _lib.load()
        c = _cache(code_bits=4)
        rc = lib.oscar_decode_step(ctypes.byref(c), ctypes.byref(ROT), ctypes.byref(ROT), 0x6000, 0x7000, 0x9000,
                                   0xB000, 8, 1, 150, 0.088, 0xD000, 0xA000, 1 << 30, None)
        assert rc == E.OSCAR_ENODEV, _err()
