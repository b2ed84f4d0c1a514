"""GPU parity at the benchmark sizes, in the launch configurations that
bench.py times, on sampled outputs.

The GPU runs each whole configuration (every request and KV head, one
layer: layers are independent calls of the same shape).  The oracle cannot
redo a 32K or 100K context for every head, so it checks sampled
(request, KV head) pairs one at a time: it writes that request's tokens of
that head into a cache of its own and attends over it with the query heads
of the group.  Requests share one seeded host token array as prefixes of
different lengths (each request still has pages of its own, written by the
GPU write kernel); the 28 x 100K case shares one written request's pages
between all requests (a shared prefix), each with its own query.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import oscar_ref as o
from tests.parity_tools import (assert_decode_close, assert_history_ok, compare_history, random_rotation,
                                to_dev_bf16)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)
CLIP = 6.0


@pytest.fixture(scope="module")
def oscar():
    import bit_rotated_kv_oscar_amd as m
    return m


class FullCase:
    """Shared host tokens, rotations and per-request page tables."""

    def __init__(self, seed, hq, hkv, G, lens, shared_pages=False):
        self.hq, self.hkv, self.G = hq, hkv, G
        self.lens = np.asarray(lens, dtype=np.int64)
        self.ld = synth.LayerData(seed, 0, hq, hkv)
        self.k, self.v = self.ld.cache_kv(int(self.lens.max()))   # bf16 bits [Lmax][Hkv][128]
        self.R_K, self.R_V = random_rotation(seed), random_rotation(seed + 1)
        self.q = self.ld.decode_q(len(self.lens))
        self.shared = shared_pages
        B = len(self.lens)
        if shared_pages:
            pt1, self.n_hist_pages = synth.shuffled_page_tables(seed, 0, self.lens[:1])
            self.hist_pt = np.repeat(pt1, B, axis=0)
            self.bf16_pt = np.repeat(synth.bf16_page_tables(1, shuffle_seed=seed + 7), B, axis=0)
            self.n_bf16_pages = 9
        else:
            self.hist_pt, self.n_hist_pages = synth.shuffled_page_tables(seed, 0, self.lens)
            self.bf16_pt = synth.bf16_page_tables(B, shuffle_seed=seed + 7)
            self.n_bf16_pages = 9 * B

    def gpu(self, oscar):
        """Write every request's tokens through the GPU write kernel."""
        dev = torch.device("cuda:0")
        cache = oscar.LayerCache(self.hkv, self.G, self.n_hist_pages, self.n_bf16_pages,
                                 torch.from_numpy(self.hist_pt), torch.from_numpy(self.bf16_pt), device=dev)
        rk, rv = oscar.Rotation(self.R_K, CLIP, dev), oscar.Rotation(self.R_V, CLIP, dev)
        kd, vd = to_dev_bf16(self.k), to_dev_bf16(self.v)
        lens = self.lens[:1] if self.shared else self.lens
        idx = torch.cat([torch.arange(int(L), device=dev) for L in lens])
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
        oscar.write_kv(cache, rk, rv, kd.index_select(0, idx).contiguous(), vd.index_select(0, idx).contiguous(),
                       cu, torch.zeros(len(lens), dtype=torch.int32, device=dev), int(lens.max()))
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        return cache, rk, rv

    def oracle_out(self, b, h, q=None):
        """Oracle output of request b, query heads of KV head h: [GQA][128]."""
        L = int(self.lens[b])
        gqa = self.hq // self.hkv
        nh = synth.hist_pages_needed(L)
        ref = o.LayerCacheRef(1, self.G, nh, 9, np.arange(nh, dtype=np.int32)[None],
                              np.arange(9, dtype=np.int32)[None])
        ref.write(self.R_K, self.R_V, CLIP, CLIP, self.k[:L, h:h + 1], self.v[:L, h:h + 1],
                  np.array([0, L], np.int32), np.zeros(1, np.int32))
        qb = (self.q if q is None else q)[b:b + 1, h * gqa:(h + 1) * gqa]
        return o.decode_attn(ref, self.R_K, self.R_V, qb, [L], SCALE)[0]


def _decode(oscar, fc, cache, rk, rv):
    B = len(fc.lens)
    lens = torch.from_numpy(fc.lens.astype(np.int32)).cuda()
    L = int(fc.lens.max())
    ws = torch.zeros(oscar.decode_workspace_bytes(B, fc.hq, fc.hkv, L), dtype=torch.uint8, device="cuda")
    out = oscar.decode_attn(cache, rk, rv, to_dev_bf16(fc.q), lens, L, SCALE, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    return out.cpu().numpy()


def _check(fc, out, picks, what):
    gqa = fc.hq // fc.hkv
    for b, h in picks:
        got = out[b, h * gqa:(h + 1) * gqa]
        mx, rel = assert_decode_close(got[None], fc.oracle_out(b, h)[None], f"{what} request {b} KV head {h}")
        print(f"{what} b={b} h={h}: max abs {mx:.2e} rel {rel:.2e}", flush=True)


def test_bs1_32k_g64(oscar):
    # the default benchmark layer: 1 x 32768, 32 q / 8 KV heads, group 64
    fc = FullCase(2101, 32, 8, 64, [32768])
    cache, rk, rv = fc.gpu(oscar)
    out = _decode(oscar, fc, cache, rk, rv)
    assert np.isfinite(out).all()
    _check(fc, out, [(0, 0), (0, 5)], "bs1 32K")


def test_bs64_8k_to_32k_g64(oscar):
    # the batch-64 benchmark layer: lengths U[8192, 32768], own pages per request
    lens = synth.request_lengths(2102, 64, 8192, 32768)
    fc = FullCase(2102, 32, 8, 64, lens)
    cache, rk, rv = fc.gpu(oscar)
    out = _decode(oscar, fc, cache, rk, rv)
    assert np.isfinite(out).all()
    b_short, b_long = int(np.argmin(lens)), int(np.argmax(lens))
    _check(fc, out, [(b_short, 3), (b_long, 6), (17, 0)], "bs64")


def test_28_requests_100k_gqa8_g128(oscar):
    # 28 concurrent 100000-token requests, 64 q / 8 KV heads, group 128
    # (pages shared between requests, queries their own)
    fc = FullCase(2103, 64, 8, 128, [100000] * 28, shared_pages=True)
    cache, rk, rv = fc.gpu(oscar)
    out = _decode(oscar, fc, cache, rk, rv)
    assert np.isfinite(out).all()
    _check(fc, out, [(0, 2), (27, 2)], "28 x 100K")


def test_write_prefill_8x32k_g32(oscar):
    # the write benchmark's prefill: 8 prompts x 32768 tokens, group 32; the
    # pages of sampled (prompt, KV head) pairs against the oracle's codes
    fc = FullCase(2104, 32, 8, 32, [32768] * 8)
    cache, rk, rv = fc.gpu(oscar)
    hist = cache.hist.cpu().numpy()
    for b, h in ((0, 0), (5, 3), (7, 7)):
        L = int(fc.lens[b])
        stats = compare_history(hist[:, h:h + 1], fc.hist_pt[b:b + 1], [fc.k[:L, h:h + 1]], [fc.v[:L, h:h + 1]],
                                [L], fc.R_K, fc.R_V, CLIP, CLIP, fc.G)
        assert_history_ok(stats)
        print(f"write 8x32K b={b} h={h}: {stats}", flush=True)


def test_write_then_64_appends_decode_g32(oscar):
    # the write benchmark's decode loop: after an 8 x 32768 prefill, 64 steps
    # of write-on-append of one token per request, each followed by a decode;
    # the last step's output of sampled (request, KV head) pairs
    P, S = 32768, 64
    fc = FullCase(2105, 32, 8, 32, [P + S] * 8)
    dev = torch.device("cuda:0")
    full = fc.lens.copy()
    fc.lens = np.full(8, P)
    cache, rk, rv = fc.gpu(oscar)
    fc.lens = full
    kd, vd = to_dev_bf16(fc.k), to_dev_bf16(fc.v)
    q = to_dev_bf16(fc.q)
    ws = torch.zeros(oscar.decode_workspace_bytes(8, fc.hq, fc.hkv, P + S), dtype=torch.uint8, device=dev)
    for s in range(S):
        kn = kd[P + s].unsqueeze(0).expand(8, -1, -1).contiguous()
        vn = vd[P + s].unsqueeze(0).expand(8, -1, -1).contiguous()
        before = torch.full((8,), P + s, dtype=torch.int32, device=dev)
        out = oscar.decode_step(cache, rk, rv, kn, vn, before, q, P + S, SCALE, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    _check(fc, out.cpu().numpy(), [(1, 4), (6, 1)], "prefill + 64 appends")
