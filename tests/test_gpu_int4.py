"""GPU parity of the INT4 history variant against the fp64 oracle.

The INT4 cache is the pages' 4-bit comparison point ([nl] §4 "Schaalbaarheid",
[fr] §4 "Évolutivité": the INT4 and BF16 caches are the baselines that run
out of memory at 28 requests of 100K tokens).  Same pipeline as INT2 with
16-level codes (include/oscar.h, INT4 codes); the write is compared with the
oracle-written pool under the rules of tests/parity_tools.py (INT4 form),
the decode on oracle-written bytes.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oscar_ref as o
from tests.parity_tools import (Scenario, assert_decode_close, assert_history_ok, bf16_pool_bits,
                                compare_history, decode_error, to_dev_bf16)
from tests.test_gpu_parity import _prefix_cache, check_raw_rows, gpu_cache, gpu_decode, gpu_rotations, gpu_write

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def oscar():
    import bit_rotated_kv_oscar_amd as m
    return m


# ------------------------------------------------------------------ write


@pytest.mark.parametrize("G", [32, 64, 128])
def test_int4_write_ragged_batch(oscar, G):
    lens = [1, 16, 17, 144, 145, 160, 161, 300, 1000]
    sc = Scenario(2200 + G, 8, 2, G, lens, bits=4)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc)
    assert cache.hist.shape[2] == o.hist_block_bytes(G, 4)
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, G, bits=4)
    print("int4 write stats", stats)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), ref)


def test_int4_write_calibrated_single_layer(oscar):
    sc = Scenario(2301, 8, 2, 32, [4096], rot="calibrated", bits=4)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc)
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, sc.G, bits=4)
    print("int4 write stats", stats)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), ref)


def test_int4_write_chunks_and_appends(oscar):
    # uneven chunks, one longer than the recent window, then single-token
    # appends: ring tokens leave the window into INT4 pages whose other rows
    # are already there (the V dwords mix four rows: read-modify-write)
    lens = [700, 433]
    chunks = [0, 100, 250, 400] + list(range(401, 440)) + [600, 700]
    sc = Scenario(2302, 8, 2, 64, lens, bits=4)
    ref = sc.oracle_cache(chunks)
    cache = gpu_cache(oscar, sc)
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv, chunks)
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, sc.G, bits=4)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), ref)


# ------------------------------------------------------------------ decode


@pytest.mark.parametrize("G", [32, 64, 128])
def test_int4_decode_ragged_batch(oscar, G):
    lens = [1, 15, 16, 17, 100, 144, 145, 146, 159, 160, 161, 777, 2049]
    sc = Scenario(2400 + G, 8, 2, G, lens, bits=4)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    out = gpu_decode(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    mx, rel = assert_decode_close(out, sc.oracle_decode(ref))
    print(f"int4 G={G} max abs {mx:.2e} rel {rel:.2e}")


@pytest.mark.parametrize("hq,hkv,G", [(4, 4, 64), (16, 2, 128), (16, 2, 32), (2, 1, 32)])
def test_int4_decode_gqa_groups(oscar, hq, hkv, G):
    sc = Scenario(2500 + hq + G, hq, hkv, G, [300, 1500], bits=4)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    mx, rel = assert_decode_close(gpu_decode(oscar, sc, cache, rk, rv), sc.oracle_decode(ref), f"{hq}/{hkv}")
    print(f"int4 {hq}/{hkv} G={G} max abs {mx:.2e} rel {rel:.2e}")


def test_int4_decode_calibrated_closer_than_int2(oscar):
    # the same calibrated tokens decoded from INT4 and from INT2 pools: both
    # match their own oracle, and INT4 lands closer to the unquantised
    # attention
    errs = {}
    for bits in (2, 4):
        sc = Scenario(2600, 8, 2, 32, [4096], rot="calibrated", bits=bits)
        ref = sc.oracle_cache()
        cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
        rk, rv = gpu_rotations(oscar, sc)
        out = gpu_decode(oscar, sc, cache, rk, rv)
        assert_decode_close(out, sc.oracle_decode(ref), f"bits={bits}")
        exact = o.attention(o.bf16_to_f64(sc.q)[0], o.bf16_to_f64(sc.k), o.bf16_to_f64(sc.v), SCALE)
        errs[bits] = decode_error(out[0], exact)[1]
    print("rel error vs unquantised attention", errs)
    assert errs[4] < 0.5 * errs[2]


def test_int4_decode_many_splits_and_merge_kernel(oscar):
    # one request at 20K (125 history splits per head, fused merge in
    # several register windows), then 24 requests x 8 KV heads (192 units,
    # more than half the CUs: the separate merge kernel); the workspace's
    # counters return to zero
    L = 20000
    sc = Scenario(2700, 8, 2, 64, [L], bits=4)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    ws = torch.zeros(oscar.decode_workspace_bytes(1, 8, 2, L), dtype=torch.uint8, device="cuda")
    expect = sc.oracle_decode(ref)
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    for rep in range(2):
        out = oscar.decode_attn(cache, rk, rv, to_dev_bf16(sc.q), lens, L, SCALE, workspace=ws)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        assert_decode_close(out.cpu().numpy(), expect, f"many splits, call {rep}")
        assert int(ws[-256:].count_nonzero().item()) == 0

    lens2 = [int(x) for x in np.random.default_rng(5).integers(150, 700, size=24)]
    sc2 = Scenario(2701, 32, 8, 128, lens2, bits=4)
    ref2 = sc2.oracle_cache()
    cache2 = gpu_cache(oscar, sc2, hist=ref2.hist, bf16=ref2.bf16)
    rk2, rv2 = gpu_rotations(oscar, sc2)
    out2 = gpu_decode(oscar, sc2, cache2, rk2, rv2)
    assert int(cache2.status.item()) == 0
    mx, rel = assert_decode_close(out2, sc2.oracle_decode(ref2), "24 x 8 units")
    print(f"int4 merge-kernel path max abs {mx:.2e} rel {rel:.2e}")


def test_int4_gpu_write_then_decode(oscar):
    # the decode reads what the INT4 write kernel stored
    sc = Scenario(2800, 8, 2, 64, [3000, 700, 145], bits=4)
    cache = gpu_cache(oscar, sc)
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv)
    out = gpu_decode(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    assert_decode_close(out, sc.oracle_decode(sc.oracle_cache()), "write then decode")


def test_int4_noalloc_matches_workspace_decode(oscar):
    sc = Scenario(2900, 8, 2, 32, [5000, 1000], bits=4)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    lens = torch.tensor(sc.lens, dtype=torch.int32, device="cuda")
    q = to_dev_bf16(sc.q)
    a = oscar.decode_attn(cache, rk, rv, q, lens, max(sc.lens), SCALE)
    b = oscar.decode_attn_noalloc(cache, rk, rv, q, lens, max(sc.lens), SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_int4_bad_page_flagged_not_followed(oscar):
    sc = Scenario(3000, 8, 2, 64, [600], bits=4)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    cache.hist_pt[0, 3] = sc.n_hist_pages + 1000
    rk, rv = gpu_rotations(oscar, sc)
    out = gpu_decode(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) & 1
    assert np.isfinite(out).all()


# ------------------------------------------------------------------ append + decode


def _last_tokens(sc, s):
    k = np.stack([t[L - s] for t, L in zip(sc.tok_k, sc.lens)])
    v = np.stack([t[L - s] for t, L in zip(sc.tok_v, sc.lens)])
    return to_dev_bf16(k), to_dev_bf16(v)


@pytest.mark.parametrize("G,rot", [(32, "random"), (64, "random"), (128, "random"), (32, "identity")])
def test_int4_decode_step_appends_then_decodes(oscar, G, rot):
    # the token at position L-129 leaves the window into an INT4 page
    # whenever L - 1 >= 144 (its K dwords written whole, its V nibbles
    # merged into dwords shared with three other rows); with the identity
    # rotation many steps fall exactly halfway between levels
    lens = [1, 16, 17, 143, 144, 145, 146, 160, 161, 500, 1201]
    sc = Scenario(3200 + G, 8, 2, G, lens, rot=rot, bits=4)
    pre = _prefix_cache(sc, 1)
    full = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=pre.hist, bf16=pre.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    k1, v1 = _last_tokens(sc, 1)
    before = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    out = oscar.decode_step(cache, rk, rv, k1, v1, before, to_dev_bf16(sc.q), max(lens), SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, G, bits=4)
    assert_history_ok(stats)
    if rot == "identity":
        assert stats.get("code_in_band", 0) == 0, stats
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), full)
    assert_decode_close(out.cpu().numpy(), sc.oracle_decode(full), f"int4 decode_step G={G} {rot}")


def test_int4_decode_step_many_steps(oscar):
    # 40 consecutive steps: evicted tokens fill INT4 history pages row by row
    lens = [330, 200, 150]
    steps = 40
    sc = Scenario(3300, 8, 2, 64, lens, bits=4)
    pre = _prefix_cache(sc, steps)
    full = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=pre.hist, bf16=pre.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    ws = torch.zeros(oscar.decode_workspace_bytes(len(lens), 8, 2, max(lens)), dtype=torch.uint8, device="cuda")
    q = to_dev_bf16(sc.q)
    for s in range(steps, 0, -1):
        k_s, v_s = _last_tokens(sc, s)
        before = torch.tensor([L - s for L in lens], dtype=torch.int32, device="cuda")
        out = oscar.decode_step(cache, rk, rv, k_s, v_s, before, q, max(lens), SCALE, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, 64, bits=4)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), full)
    assert_decode_close(out.cpu().numpy(), sc.oracle_decode(full), "int4 decode_step x40")
