"""GPU parity of per-KV-head rotations (the optional extension of the pages'
per-layer rotation): every KV head written, decoded and extended with its
own R and clip, against the oracle with the same per-head rotations; a cache
written with equal per-head rotations is the per-layer cache bit for bit;
per-head calibration against the oracle's."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import oscar_ref as o
from tests.parity_tools import (Scenario, assert_decode_close, assert_history_ok, bf16_pool_bits,
                                compare_history, to_dev_bf16)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def oscar():
    import bit_rotated_kv_oscar_amd as m
    return m


def _cache(oscar, sc, hist=None, bf16=None):
    c = oscar.LayerCache(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, torch.from_numpy(sc.hist_pt),
                         torch.from_numpy(sc.bf16_pt), device=torch.device("cuda:0"), code_bits=sc.bits)
    if hist is not None:
        c.hist.copy_(torch.from_numpy(hist))
    if bf16 is not None:
        c.bf16.view(torch.int16).copy_(torch.from_numpy(bf16.view(np.int16)))
    return c


def _write(oscar, sc, cache, rk, rv, chunks=None):
    for cu, lb, k, v in sc.write_calls(chunks):
        n = np.diff(cu)
        oscar.write_kv(cache, rk, rv, to_dev_bf16(k), to_dev_bf16(v), torch.from_numpy(cu).cuda(),
                       torch.from_numpy(lb).cuda(), int(n.max()) if n.size else 0)
    torch.cuda.synchronize()


def _decode(oscar, sc, cache, rk, rv):
    lens = torch.tensor(sc.lens, dtype=torch.int32, device="cuda")
    out = oscar.decode_attn(cache, rk, rv, to_dev_bf16(sc.q), lens, max(sc.lens), SCALE)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_raw(sc, gpu_bf16, ref):
    for b, L in enumerate(sc.lens):
        for p in range(L):
            w, idx = o.storage_of(p, L)
            if w == "hist":
                continue
            pg, row = ref._bf16_row(b, w, idx)
            assert np.array_equal(gpu_bf16[pg, :, :, row, :], ref.bf16[pg, :, :, row, :]), (b, p)


@pytest.mark.parametrize("G,bits", [(32, 2), (64, 2), (128, 2), (64, 4)])
def test_per_head_write_matches_oracle(oscar, G, bits):
    lens = [1, 145, 161, 300, 1000]
    sc = Scenario(3000 + G + bits, 8, 4, G, lens, rot="per_head", bits=bits)
    ref = sc.oracle_cache()
    cache = _cache(oscar, sc)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    _write(oscar, sc, cache, rk, rv, chunks=[0, 150, 151, 400, 1000])
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, G, bits=bits)
    print(f"G={G} bits={bits}", stats, flush=True)
    assert_history_ok(stats)
    _check_raw(sc, bf16_pool_bits(cache.bf16), ref)
    # the decode of the GPU-written cache against the oracle's
    assert_decode_close(_decode(oscar, sc, cache, rk, rv), sc.oracle_decode(ref), f"per-head G={G} bits={bits}")


@pytest.mark.parametrize("hq,hkv,G", [(8, 4, 32), (8, 2, 64), (32, 4, 128), (4, 4, 64)])
def test_per_head_decode_matches_oracle(oscar, hq, hkv, G):
    # the oracle's cache bytes on the device: the decode alone, per-head R
    lens = [1, 17, 145, 146, 700, 2049]
    sc = Scenario(3100 + hq + G, hq, hkv, G, lens, rot="per_head")
    ref = sc.oracle_cache()
    cache = _cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    out = _decode(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    mx, rel = assert_decode_close(out, sc.oracle_decode(ref), f"per-head decode {hq}/{hkv} G={G}")
    print(f"{hq}/{hkv} G={G}: max abs {mx:.2e} rel {rel:.2e}", flush=True)


def test_per_head_decode_batch64_several_rounds(oscar):
    # enough units for the several-round split plan and its merge kernel
    lens = list(synth.request_lengths(3150, 64, 300, 3000))
    sc = Scenario(3150, 16, 4, 64, lens, rot="per_head")
    ref = sc.oracle_cache()
    cache = _cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    assert_decode_close(_decode(oscar, sc, cache, rk, rv), sc.oracle_decode(ref), "per-head batch 64")


def _prefix(sc, drop):
    ref = o.LayerCacheRef(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, sc.hist_pt, sc.bf16_pt, bits=sc.bits)
    keep = [max(0, L - drop) for L in sc.lens]
    kp = np.concatenate([t[:n] for t, n in zip(sc.tok_k, keep)])
    vp = np.concatenate([t[:n] for t, n in zip(sc.tok_v, keep)])
    cu = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
    ref.write(sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, kp, vp, cu, np.zeros(len(keep), np.int32))
    return ref


@pytest.mark.parametrize("bits", [2, 4])
def test_per_head_decode_step_matches_oracle(oscar, bits):
    # the appended token pushes position L-129 out of the window: the raw
    # workgroup quantises it with its own head's R and clip
    lens = [1, 144, 145, 146, 161, 500, 1201]
    sc = Scenario(3200 + bits, 8, 4, 64, lens, rot="per_head", bits=bits)
    pre = _prefix(sc, 1)
    full = sc.oracle_cache()
    cache = _cache(oscar, sc, hist=pre.hist, bf16=pre.bf16)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    k_last = np.stack([t[-1] for t in sc.tok_k])
    v_last = np.stack([t[-1] for t in sc.tok_v])
    before = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    out = oscar.decode_step(cache, rk, rv, to_dev_bf16(k_last), to_dev_bf16(v_last), before, to_dev_bf16(sc.q),
                            max(lens), SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, sc.G, bits=bits)
    assert_history_ok(stats)
    _check_raw(sc, bf16_pool_bits(cache.bf16), full)
    assert_decode_close(out.cpu().numpy(), sc.oracle_decode(full), f"per-head decode_step bits={bits}")


@pytest.mark.parametrize("G", [32, 64])
def test_per_head_extend_matches_oracle(oscar, G):
    prefix, chunk = [0, 20, 150, 700], [5, 33, 17, 40]
    lens = [p + c for p, c in zip(prefix, chunk)]
    sc = Scenario(3300 + G, 8, 2, G, lens, rot="per_head")
    ref = o.LayerCacheRef(sc.hkv, G, sc.n_hist_pages, sc.n_bf16_pages, sc.hist_pt, sc.bf16_pt)
    kp = np.concatenate([t[:n] for t, n in zip(sc.tok_k, prefix)])
    vp = np.concatenate([t[:n] for t, n in zip(sc.tok_v, prefix)])
    cu_p = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int32)
    ref.write(sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, kp, vp, cu_p, np.zeros(len(prefix), np.int32))
    kn = np.concatenate([t[p:] for t, p in zip(sc.tok_k, prefix)])
    vn = np.concatenate([t[p:] for t, p in zip(sc.tok_v, prefix)])
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = sc.ld.decode_q(int(cu[-1]), stream=synth.S_EVAL_Q)
    cache = _cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    out = oscar.extend_attn(cache, rk, rv, to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn),
                            torch.from_numpy(cu).cuda(), torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                            int(max(chunk)), max(prefix), SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    exp = o.extend_attn(ref, sc.R_K, sc.R_V, q, kn, vn, cu, prefix, SCALE)
    assert_decode_close(out.cpu().numpy(), exp, f"per-head extend G={G}")


def test_mixed_per_head_k_and_layer_v(oscar):
    # R_K per head, one R_V for the layer (each rotation chooses its form)
    lens = [145, 600, 1500]
    sc = Scenario(3400, 8, 4, 64, lens, rot="per_head")
    sc.R_V, sc.clip_v = sc.R_V[0], 5.0
    ref = sc.oracle_cache()
    cache = _cache(oscar, sc)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    _write(oscar, sc, cache, rk, rv)
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, sc.G)
    assert_history_ok(stats)
    assert_decode_close(_decode(oscar, sc, cache, rk, rv), sc.oracle_decode(ref), "mixed per-head K")


def test_equal_per_head_rotations_reproduce_the_layer_cache(oscar):
    # the per-head write (one head per workgroup) and the per-layer write
    # (four heads per workgroup) do the same arithmetic per head: identical
    # bytes, and identical decodes
    lens = [1, 150, 777, 2000]
    sc = Scenario(3500, 8, 4, 32, lens)
    a, b = _cache(oscar, sc), _cache(oscar, sc)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    RK4, RV4 = np.stack([sc.R_K] * 4), np.stack([sc.R_V] * 4)
    rk4, rv4 = oscar.Rotation(RK4, [sc.clip_k] * 4), oscar.Rotation(RV4, [sc.clip_v] * 4)
    _write(oscar, sc, a, rk, rv)
    _write(oscar, sc, b, rk4, rv4)
    assert torch.equal(a.hist, b.hist) and torch.equal(a.bf16, b.bf16)
    assert np.array_equal(_decode(oscar, sc, a, rk, rv), _decode(oscar, sc, b, rk4, rv4))


def test_per_head_calibration_matches_oracle(oscar):
    ld = synth.LayerData(3600, 0, 8, 2)
    qc, kc, vc = ld.calibration(1024)
    R_K, R_V, ck, cv = oscar.calibrate_per_head(to_dev_bf16(qc), to_dev_bf16(kc), to_dev_bf16(vc))
    cal = o.calibrate_per_head(*(o.bf16_to_f64(x) for x in (qc, kc, vc)))
    assert R_K.shape == (2, 128, 128)
    assert np.abs(R_K.numpy() - cal["R_K"]).max() < 1e-8
    assert np.abs(R_V.numpy() - cal["R_V"]).max() < 1e-8
    for h in range(2):
        assert abs(ck[h] - cal["clip_K"][h]) <= 1e-6 * cal["clip_K"][h]
        assert abs(cv[h] - cal["clip_V"][h]) <= 1e-6 * cal["clip_V"][h]
    # the two heads' rotations differ (their query groups differ)
    assert np.abs(cal["R_K"][0] - cal["R_K"][1]).max() > 1e-3


def test_per_head_calibrated_decode_step_loop(oscar):
    # per-head calibrated rotations through 24 steps of append + decode
    lens0 = [150, 900]
    S = 24
    sc = Scenario(3700, 8, 2, 64, [L + S for L in lens0], rot="per_head_calibrated", n_cal=512)
    pre = _prefix(sc, S)
    cache = _cache(oscar, sc, hist=pre.hist, bf16=pre.bf16)
    rk, rv = oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)
    for s in range(S):
        kn = np.stack([t[L + s] for t, L in zip(sc.tok_k, lens0)])
        vn = np.stack([t[L + s] for t, L in zip(sc.tok_v, lens0)])
        before = torch.tensor([L + s for L in lens0], dtype=torch.int32, device="cuda")
        out = oscar.decode_step(cache, rk, rv, to_dev_bf16(kn), to_dev_bf16(vn), before, to_dev_bf16(sc.q),
                                max(sc.lens), SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    full = sc.oracle_cache()
    assert_decode_close(out.cpu().numpy(), sc.oracle_decode(full), "per-head calibrated loop")
