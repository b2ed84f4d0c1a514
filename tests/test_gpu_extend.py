"""GPU parity of the extend (chunked-prefill) attention against the oracle.

Each case writes the prefix of every request with the oracle, uploads that
cache, and runs oscar_extend_attn for the chunk that follows; both sides see
identical cache bytes.  Outputs are compared under the decode tolerance
(max |gpu - oracle| <= 2e-2, relative L2 <= 5e-3)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import oscar_ref as o
from tests.parity_tools import Scenario, assert_decode_close, to_dev_bf16

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def oscar():
    import bit_rotated_kv_oscar_amd as m
    return m


def _setup(oscar, seed, hq, hkv, G, prefix, chunk, rot="random", layer=0, bits=2):
    lens = [p + c for p, c in zip(prefix, chunk)]
    sc = Scenario(seed, hq, hkv, G, lens, rot=rot, layer=layer, bits=bits)
    ref = o.LayerCacheRef(hkv, G, sc.n_hist_pages, sc.n_bf16_pages, sc.hist_pt, sc.bf16_pt, bits=bits)
    kp = np.concatenate([t[:n] for t, n in zip(sc.tok_k, prefix)])
    vp = np.concatenate([t[:n] for t, n in zip(sc.tok_v, prefix)])
    cu_p = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int32)
    ref.write(sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, kp, vp, cu_p, np.zeros(len(prefix), np.int32))
    kn = np.concatenate([t[p:] for t, p in zip(sc.tok_k, prefix)])
    vn = np.concatenate([t[p:] for t, p in zip(sc.tok_v, prefix)])
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = sc.ld.decode_q(int(cu[-1]), stream=synth.S_EVAL_Q)
    dev = torch.device("cuda:0")
    cache = oscar.LayerCache(hkv, G, sc.n_hist_pages, sc.n_bf16_pages, torch.from_numpy(sc.hist_pt),
                             torch.from_numpy(sc.bf16_pt), device=dev, code_bits=bits)
    cache.hist.copy_(torch.from_numpy(ref.hist))
    cache.bf16.view(torch.int16).copy_(torch.from_numpy(ref.bf16.view(np.int16)))
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    return sc, ref, cache, rk, rv, q, kn, vn, cu


def _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix, max_prefix=None):
    chunk = np.diff(cu)
    out = oscar.extend_attn(cache, rk, rv, to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn),
                            torch.from_numpy(cu).cuda(), torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                            int(chunk.max()), max(prefix) if max_prefix is None else max_prefix, SCALE)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("G", [32, 64, 128])
def test_extend_ragged_prefixes_and_chunks(oscar, G):
    # prefixes: none, inside the sink, sink only, ring only, exactly sink +
    # window, one history token, several pages; chunks: ragged tiles, one
    # token, whole tiles
    prefix = [0, 5, 16, 100, 144, 145, 300, 700]
    chunk = [37, 16, 1, 50, 17, 33, 64, 20]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2000 + G, 8, 2, G, prefix, chunk)
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    assert int(cache.status.item()) == 0
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out, exp, f"extend G={G}")


@pytest.mark.parametrize("G", [32, 64, 128])
def test_extend_int4_ragged_prefixes_and_chunks(oscar, G):
    # the same shapes over an INT4 history (16-level codes, 1 KB code areas)
    prefix = [0, 5, 16, 100, 144, 145, 300, 700]
    chunk = [37, 16, 1, 50, 17, 33, 64, 20]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2050 + G, 8, 2, G, prefix, chunk, bits=4)
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    assert int(cache.status.item()) == 0
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    mx, rel = assert_decode_close(out, exp, f"extend INT4 G={G}")
    print(f"extend INT4 G={G} max abs {mx:.2e} rel {rel:.2e}")


def test_extend_int4_gqa8_calibrated(oscar):
    prefix, chunk = [2500, 170], [48, 33]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2060, 16, 2, 64, prefix, chunk, rot="calibrated", bits=4)
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    assert int(cache.status.item()) == 0
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out, exp, "extend INT4 GQA 8 calibrated")


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (16, 2)])
def test_extend_gqa_groups(oscar, hq, hkv):
    prefix, chunk = [260, 31], [40, 70]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2100 + hq, hq, hkv, 64, prefix, chunk)
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out, exp, f"extend hq={hq} hkv={hkv}")


def test_extend_calibrated_long_prefix(oscar):
    # calibrated rotations and clips, a prefix of many history pages
    prefix, chunk = [2500], [48]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2200, 8, 2, 64, prefix, chunk, rot="calibrated")
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out, exp, "extend calibrated")


def test_extend_single_token_matches_decode_without_history(oscar):
    # one new token over a prefix with no history equals the decode after
    # appending it (both read the same bf16 values)
    prefix, chunk = [0, 15, 100, 143], [1, 1, 1, 1]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2300, 8, 2, 32, prefix, chunk)
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    oscar.write_kv(cache, rk, rv, to_dev_bf16(kn), to_dev_bf16(vn), torch.from_numpy(cu).cuda(),
                   torch.tensor(prefix, dtype=torch.int32, device="cuda"), 1)
    lens = torch.tensor([p + 1 for p in prefix], dtype=torch.int32, device="cuda")
    dec = oscar.decode_attn(cache, rk, rv, to_dev_bf16(q), lens, 144, SCALE)
    torch.cuda.synchronize()
    assert_decode_close(out, dec.cpu().numpy(), "extend vs decode after append")
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out, exp, "extend single token")


def test_extend_bad_page_and_length_are_flagged(oscar):
    prefix, chunk = [400, 200], [20, 20]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2400, 8, 2, 64, prefix, chunk)
    # request 0: a history page id past the pool; request 1 is untouched
    pt = sc.hist_pt.copy()
    pt[0, 3] = sc.n_hist_pages + 5
    cache.hist_pt.copy_(torch.from_numpy(pt))
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    assert int(cache.status.item()) & oscar._lib.STATUS_BAD_PAGE
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out[cu[1]:cu[2]], exp[cu[1]:cu[2]], "extend request beside a bad page")
    # a prefix length above max_prefix: flagged, rows left as they were
    cache.status.zero_()
    cache.hist_pt.copy_(torch.from_numpy(sc.hist_pt))
    sentinel = torch.full((int(cu[-1]), 8, 128), 7.0, device="cuda")
    oscar.extend_attn(cache, rk, rv, to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn), torch.from_numpy(cu).cuda(),
                      torch.tensor(prefix, dtype=torch.int32, device="cuda"), 20, 300, SCALE, out=sentinel)
    torch.cuda.synchronize()
    assert int(cache.status.item()) & oscar._lib.STATUS_BAD_LEN
    s = sentinel.cpu().numpy()
    assert np.all(s[:cu[1]] == 7.0)
    assert_decode_close(s[cu[1]:], exp[cu[1]:], "extend request beside a bad length")


@pytest.mark.parametrize("G", [64, 128])
def test_extend_history_page_counts(oscar, G):
    # histories of 1 to 7 full pages, with and without a partial last page,
    # and a longer one: every phase of the history loop's page slots
    prefix = [144 + 16 * k + r for k, r in [(1, 0), (2, 5), (3, 0), (4, 15), (5, 0), (6, 1), (7, 0), (13, 9)]]
    chunk = [16, 3, 20, 1, 33, 16, 7, 25]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2450 + G, 8, 2, G, prefix, chunk)
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    assert int(cache.status.item()) == 0
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out, exp, f"extend page counts G={G}")


def test_extend_bad_page_in_each_slot(oscar):
    # request r < 7 has a bad id at history page r of its 6 full pages and
    # a partial seventh; request 7 is untouched and exact
    prefix, chunk = [144 + 16 * 6 + 3] * 8, [5] * 8
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2470, 8, 2, 64, prefix, chunk)
    pt = sc.hist_pt.copy()
    for r in range(7):
        pt[r, r] = sc.n_hist_pages + 1 + r
    cache.hist_pt.copy_(torch.from_numpy(pt))
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    assert int(cache.status.item()) & oscar._lib.STATUS_BAD_PAGE
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert np.all(np.isfinite(out))
    assert_decode_close(out[cu[7]:], exp[cu[7]:], "extend request beside bad pages")


def test_extend_bench_shape_sampled_rows(oscar):
    # the timed shape of the extend workload (one layer): Hq 32 / Hkv 8, G 64,
    # prefix 28672 + chunk 4096, in the launch the benchmark uses; rows at the
    # chunk's start, tile edges and end are checked against the oracle
    import time
    t0 = time.time()
    L0, n = 28672, 4096
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2500, 32, 8, 64, [L0], [n])
    print(f"setup {time.time() - t0:.1f} s", flush=True)
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, [L0])
    assert int(cache.status.item()) == 0
    rows = [0, 1, 15, 16, 2047, 2048, 4079, 4095]
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, [L0], SCALE, rows=rows)
    print(f"oracle done {time.time() - t0:.1f} s", flush=True)
    assert_decode_close(out[rows], exp, "extend bench shape")


def test_extend_rows_past_total_tokens_are_flagged(oscar):
    # cu_new runs past the rows of q / k_new / v_new / out for request 1:
    # flagged OSCAR_STATUS_BAD_LEN, its rows never read or written; request
    # 0 is computed as usual
    prefix, chunk = [300, 250], [20, 20]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2410, 8, 2, 64, prefix, chunk)
    bad_cu = np.array([0, 20, 45], dtype=np.int32)          # 45 > T = 40
    sentinel = torch.full((40, 8, 128), 7.0, device="cuda")
    oscar.extend_attn(cache, rk, rv, to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn),
                      torch.from_numpy(bad_cu).cuda(), torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                      25, max(prefix), SCALE, out=sentinel)
    torch.cuda.synchronize()
    assert int(cache.status.item()) & oscar._lib.STATUS_BAD_LEN
    s = sentinel.cpu().numpy()
    assert np.all(s[20:] == 7.0)
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(s[:20], exp[:20], "extend request beside rows past the end")
    # a negative first offset is flagged the same way
    cache.status.zero_()
    neg_cu = np.array([-5, 15, 40], dtype=np.int32)
    sentinel.fill_(7.0)
    oscar.extend_attn(cache, rk, rv, to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn),
                      torch.from_numpy(neg_cu).cuda(), torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                      25, max(prefix), SCALE, out=sentinel)
    torch.cuda.synchronize()
    assert int(cache.status.item()) & oscar._lib.STATUS_BAD_LEN


def test_extend_unused_ring_entries_are_not_looked_up(oscar):
    # prefixes that fill the window only in part: ring pages without a
    # visible token have table entry -1; nothing is flagged, results exact
    prefix, chunk = [20, 100, 140], [9, 30, 12]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2420, 8, 2, 32, prefix, chunk)
    bpt = sc.bf16_pt.copy()
    for b, L0 in enumerate(prefix):
        for rp in range(8):
            slots = [16 * rp + t for t in range(16)]
            # slot s holds position L0 - 128 + ((s - L0) mod 128); visible iff >= 16
            if not any(L0 - 128 + ((s - L0) % 128) >= 16 for s in slots):
                bpt[b, 1 + rp] = -1
    assert (bpt == -1).sum() >= 6
    cache.bf16_pt.copy_(torch.from_numpy(bpt))
    out = _run(oscar, cache, rk, rv, q, kn, vn, cu, prefix)
    assert int(cache.status.item()) == 0
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out, exp, "extend with unset ring entries")


@pytest.mark.parametrize("q_mult,sm_scale", [(400.0, 1.0), (1e-3, SCALE)])
def test_extend_large_and_small_query_norms(oscar, q_mult, sm_scale):
    # q R_K sm_scale log2(e) far above the fp16 range of the history operand
    # (x400 at sm_scale 1), or so small that an unscaled low part would be
    # subnormal: the power-of-two guard keeps both exact to the tolerance
    prefix, chunk = [600, 350], [24, 17]
    sc, ref, cache, rk, rv, q, kn, vn, cu = _setup(oscar, 2430, 8, 2, 64, prefix, chunk)
    qf = synth.bf16_to_f64(q) * q_mult
    qb = synth.bf16_bits(qf.astype(np.float32))
    out = oscar.extend_attn(cache, rk, rv, to_dev_bf16(qb), to_dev_bf16(kn), to_dev_bf16(vn),
                            torch.from_numpy(cu).cuda(), torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                            int(np.diff(cu).max()), max(prefix), sm_scale)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, qb, kn, vn, cu, prefix, sm_scale)
    assert_decode_close(got, exp, f"extend q x{q_mult} sm_scale {sm_scale}")
