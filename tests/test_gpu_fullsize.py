"""GPU parity at the benchmark sizes, in the launch configurations that
bench.py times, on sampled outputs.

The GPU runs each whole configuration (every request and KV head, one
layer: layers are independent calls of the same shape).  The oracle cannot
redo a 32K or 100K context for every head, so it checks sampled
(request, KV head) pairs one at a time: it writes that request's tokens of
that head into a cache of its own and attends over it with the query heads
of the group.  Requests share one seeded host token array as prefixes of
different lengths, each starting at its own row offset so that no two
requests hold the same tokens (each request has pages of its own, written
by the GPU write kernel); in the INT4 28 x 100K case most requests share one
written request's pages (a shared prefix), two have pages and tokens of
their own, and every request has its own query.
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

    def __init__(self, seed, hq, hkv, G, lens, shared_pages=0, offset_step=37, bits=2):
        """shared_pages = n > 0: requests 0 .. B-n hold the pages of request 0
        (a shared prefix); the last n - 1 requests and request 0 have pages
        of their own.  Request b's tokens are rows off[b] .. off[b] + L_b of
        one seeded host array (off[b] = offset_step * b, request 0 at 0)."""
        self.hq, self.hkv, self.G, self.bits = hq, hkv, G, bits
        self.lens = np.asarray(lens, dtype=np.int64)
        B = len(self.lens)
        self.shared = int(shared_pages)
        own = self.own_requests()
        self.off = np.zeros(B, dtype=np.int64)
        self.off[own] = offset_step * np.arange(len(own))
        self.ld = synth.LayerData(seed, 0, hq, hkv)
        self.k, self.v = self.ld.cache_kv(int((self.lens + self.off).max()))  # bf16 bits [rows][Hkv][128]
        self.R_K, self.R_V = random_rotation(seed), random_rotation(seed + 1)
        self.q = self.ld.decode_q(B)
        pt_own, self.n_hist_pages = synth.shuffled_page_tables(seed, 0, self.lens[own])
        bpt_own = synth.bf16_page_tables(len(own), shuffle_seed=seed + 7)
        self.n_bf16_pages = 9 * len(own)
        slot = np.array([own.index(b) if b in own else 0 for b in range(B)])
        self.hist_pt = pt_own[slot]
        self.bf16_pt = bpt_own[slot]

    def own_requests(self):
        """Requests whose pages the GPU writes (the others share request 0's)."""
        B = len(self.lens)
        if not self.shared:
            return list(range(B))
        return [0] + list(range(B - self.shared + 1, B))

    def tokens(self, b, h=None):
        """Request b's token rows (bf16 bits [L_b][Hkv or 1][128])."""
        L, a = int(self.lens[b]), int(self.off[b])
        hs = slice(None) if h is None else slice(h, h + 1)
        return self.k[a:a + L, hs], self.v[a:a + L, hs]

    def gpu(self, oscar):
        """Write every request's tokens through the GPU write kernel."""
        dev = torch.device("cuda:0")
        cache = oscar.LayerCache(self.hkv, self.G, self.n_hist_pages, self.n_bf16_pages,
                                 torch.from_numpy(self.hist_pt), torch.from_numpy(self.bf16_pt), device=dev,
                                 code_bits=self.bits)
        rk, rv = oscar.Rotation(self.R_K, CLIP, dev), oscar.Rotation(self.R_V, CLIP, dev)
        kd, vd = to_dev_bf16(self.k), to_dev_bf16(self.v)
        own = self.own_requests()
        lens = self.lens[own]
        idx = torch.cat([torch.arange(int(self.off[b]), int(self.off[b] + self.lens[b]), device=dev) for b in own])
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
        wcache = cache
        if self.shared:
            # the write addresses the own requests' rows of the page tables
            wcache = oscar.LayerCache(self.hkv, self.G, self.n_hist_pages, self.n_bf16_pages,
                                      torch.from_numpy(self.hist_pt[own]), torch.from_numpy(self.bf16_pt[own]),
                                      device=dev, hist=cache.hist, bf16=cache.bf16, code_bits=self.bits)
            wcache.status = cache.status
        oscar.write_kv(wcache, rk, rv, kd.index_select(0, idx).contiguous(), vd.index_select(0, idx).contiguous(),
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
                              np.arange(9, dtype=np.int32)[None], bits=self.bits)
        kb, vb = self.tokens(b, h)
        ref.write(self.R_K, self.R_V, CLIP, CLIP, kb, vb, np.array([0, L], np.int32), np.zeros(1, np.int32))
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
    _check(fc, out, [(0, 0), (0, 3), (0, 5), (0, 7)], "bs1 32K")


def test_bs64_8k_to_32k_g64(oscar):
    # the batch-64 benchmark layer: lengths U[8192, 32768], own pages per request
    lens = synth.request_lengths(2102, 64, 8192, 32768)
    fc = FullCase(2102, 32, 8, 64, lens)
    cache, rk, rv = fc.gpu(oscar)
    out = _decode(oscar, fc, cache, rk, rv)
    assert np.isfinite(out).all()
    b_short, b_long = int(np.argmin(lens)), int(np.argmax(lens))
    _check(fc, out, [(b_short, 3), (b_long, 6), (17, 0), (33, 2), (48, 5), (63, 7)], "bs64")


def test_28_requests_100k_gqa8_g128(oscar):
    # 28 concurrent 100000-token requests, 64 q / 8 KV heads, group 128, as
    # the benchmark runs them: every request has pages of its own, written by
    # the GPU write kernel (request b's tokens start 1000 b rows into one
    # host array), and a query of its own
    fc = FullCase(2103, 64, 8, 128, [100000] * 28, offset_step=1000)
    assert len(fc.own_requests()) == 28 and len(np.unique(fc.hist_pt[:, 0])) == 28
    cache, rk, rv = fc.gpu(oscar)
    out = _decode(oscar, fc, cache, rk, rv)
    assert np.isfinite(out).all()
    _check(fc, out, [(0, 2), (5, 0), (13, 7), (20, 4), (26, 5), (27, 2)], "28 x 100K")


def test_int4_28_requests_100k_gqa8_g128(oscar):
    # the INT4 capacity layer (the same shape from an INT4 cache, as
    # bench.py's int4_28x100k times it): the decode of sampled pairs, and the
    # history pages of two (request, KV head) pairs against the oracle's
    # codes and meta
    fc = FullCase(2106, 64, 8, 128, [100000] * 28, shared_pages=3, offset_step=1000, bits=4)
    cache, rk, rv = fc.gpu(oscar)
    out = _decode(oscar, fc, cache, rk, rv)
    assert np.isfinite(out).all()
    _check(fc, out, [(0, 1), (14, 6), (26, 3), (27, 0)], "INT4 28 x 100K")
    hist = cache.hist.cpu().numpy()
    for b, h in ((0, 4), (27, 7)):
        kb, vb = fc.tokens(b, h)
        stats = compare_history(hist[:, h:h + 1], fc.hist_pt[b:b + 1], [kb], [vb],
                                [int(fc.lens[b])], fc.R_K, fc.R_V, CLIP, CLIP, fc.G, bits=4)
        assert_history_ok(stats)
        print(f"INT4 write b={b} h={h}: {stats}", flush=True)


def test_write_prefill_8x32k_g32(oscar):
    # the write benchmark's prefill: 8 prompts x 32768 tokens, group 32; the
    # pages of sampled (prompt, KV head) pairs against the oracle's codes
    fc = FullCase(2104, 32, 8, 32, [32768] * 8)
    cache, rk, rv = fc.gpu(oscar)
    hist = cache.hist.cpu().numpy()
    for b, h in ((0, 0), (5, 3), (7, 7)):
        L = int(fc.lens[b])
        kb, vb = fc.tokens(b, h)
        stats = compare_history(hist[:, h:h + 1], fc.hist_pt[b:b + 1], [kb], [vb],
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
    rows = torch.from_numpy(fc.off + P).to(dev)
    for s in range(S):
        kn = kd.index_select(0, rows + s).contiguous()   # request b's token at position P + s
        vn = vd.index_select(0, rows + s).contiguous()
        before = torch.full((8,), P + s, dtype=torch.int32, device=dev)
        out = oscar.decode_step(cache, rk, rv, kn, vn, before, q, P + S, SCALE, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    _check(fc, out.cpu().numpy(), [(1, 4), (6, 1)], "prefill + 64 appends")
