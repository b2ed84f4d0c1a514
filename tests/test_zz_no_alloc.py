"""The allocation-free decode (oscar_decode_attn_noalloc, through the C ABI)
against oscar_decode_attn with a caller workspace: the same kernels and split
plan on the same cache, so the outputs agree bit for bit.  Two calls in a
row, the second with a smaller input (fewer requests, shorter contexts), so
the second reuses a scratch array that the first left behind; then a shape
beyond the scratch limit is refused with OSCAR_EWORKSPACE.  Both results are
also checked against the oracle (decode tolerance)."""
import ctypes
import math

import numpy as np
import pytest
import torch

from oracle import oscar_ref as o
from tests.parity_tools import Scenario, assert_decode_close, to_dev_bf16

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


def _gpu_case(oscar, sc):
    ref = sc.oracle_cache()
    cache = oscar.LayerCache(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, torch.from_numpy(sc.hist_pt),
                             torch.from_numpy(sc.bf16_pt), device=torch.device("cuda:0"))
    cache.hist.copy_(torch.from_numpy(ref.hist))
    cache.bf16.view(torch.int16).copy_(torch.from_numpy(ref.bf16.view(np.int16)))
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    return ref, cache, rk, rv


def _noalloc_c(oscar, cache, rk, rv, q, lens, max_len, out):
    lib = oscar._lib.load()
    c, k, v = cache.c(), rk.c(), rv.c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.oscar_decode_attn_noalloc(ctypes.byref(c), ctypes.byref(k), ctypes.byref(v),
                                         ctypes.c_void_p(q.data_ptr()), q.shape[1], ctypes.c_void_p(lens.data_ptr()),
                                         q.shape[0], max_len, SCALE, ctypes.c_void_p(out.data_ptr()), stream)


@pytest.mark.parametrize("hq,hkv,G,first,rot", [
    (32, 8, 64, [9000, 4000, 200], "random"),          # one round of workgroups: merged in the attend kernel
    (8, 2, 32, [9000, 4000, 200], "random"),
    (32, 8, 64, [300 + 97 * i for i in range(20)], "random"),  # 160 units: several rounds, separate merge kernel
    (16, 4, 64, [5000, 1200], "per_head"),             # a rotation and clip per KV head
])
def test_noalloc_decode_matches_workspace_decode_twice(hq, hkv, G, first, rot):
    import bit_rotated_kv_oscar_amd as oscar
    # first call as given; second call: 1 request of 700 tokens
    for seed, lens in ((3100 + G, first), (3200 + G, [700])):
        sc = Scenario(seed, hq, hkv, G, lens, rot=rot)
        ref, cache, rk, rv = _gpu_case(oscar, sc)
        q = to_dev_bf16(sc.q)
        L = torch.tensor(sc.lens, dtype=torch.int32, device="cuda")
        mx = max(sc.lens)
        want = oscar.decode_attn(cache, rk, rv, q, L, mx, SCALE)
        got = torch.full_like(want, float("nan"))
        rc = _noalloc_c(oscar, cache, rk, rv, q, L, mx, got)
        torch.cuda.synchronize()
        assert rc == 0, oscar._lib.load().oscar_last_error().decode()
        assert int(cache.status.item()) == 0
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g, w), f"max |diff| {np.abs(g - w).max()}"
        assert_decode_close(g, sc.oracle_decode(ref), f"noalloc decode {lens}")


def test_noalloc_decode_refuses_shapes_beyond_its_scratch():
    import bit_rotated_kv_oscar_amd as oscar
    sc = Scenario(3300, 8, 2, 64, [300])
    _, cache, rk, rv = _gpu_case(oscar, sc)
    assert oscar._lib.load().oscar_decode_noalloc_max_bytes() == 16 << 20
    # 4097 requests x 2 KV heads: more (request, KV head) units than the scratch holds
    B = 4097
    q = torch.zeros((B, 8, 128), dtype=torch.bfloat16, device="cuda")
    L = torch.full((B,), 300, dtype=torch.int32, device="cuda")
    out = torch.full((B, 8, 128), 7.0, device="cuda")
    rc = _noalloc_c(oscar, cache, rk, rv, q, L, 300, out)
    torch.cuda.synchronize()
    assert rc == oscar._lib.OSCAR_EWORKSPACE
    assert bool((out == 7.0).all())
