"""GPU parity of liboscar against the fp64 oracle (through the C ABI).

Every case builds seeded inputs with synth/, runs the oracle on the CPU and the
HIP kernels on cuda:0, and compares under the rules of tests/parity_tools.py.
Decode cases feed the oracle-written cache to the GPU, so both sides attend
over identical bytes; write cases compare the GPU-written pools with the
oracle-written ones.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import oscar_ref as o
from tests.parity_tools import (Scenario, assert_decode_close, assert_history_ok, bf16_pool_bits,
                                compare_history, decode_error, random_rotation, to_dev_bf16)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def oscar():
    import bit_rotated_kv_oscar_amd as m
    return m


def gpu_cache(oscar, sc: Scenario, hist=None, bf16=None):
    dev = torch.device("cuda:0")
    c = oscar.LayerCache(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, torch.from_numpy(sc.hist_pt),
                         torch.from_numpy(sc.bf16_pt), device=dev, code_bits=sc.bits)
    if hist is not None:
        c.hist.copy_(torch.from_numpy(hist))
    if bf16 is not None:
        c.bf16.view(torch.int16).copy_(torch.from_numpy(bf16.view(np.int16)))
    return c


def gpu_rotations(oscar, sc: Scenario):
    return oscar.Rotation(sc.R_K, sc.clip_k), oscar.Rotation(sc.R_V, sc.clip_v)


def gpu_write(oscar, sc: Scenario, cache, rk, rv, chunks=None):
    for cu, lb, k, v in sc.write_calls(chunks):
        n = np.diff(cu)
        oscar.write_kv(cache, rk, rv, to_dev_bf16(k), to_dev_bf16(v), torch.from_numpy(cu).cuda(),
                       torch.from_numpy(lb).cuda(), int(n.max()) if n.size else 0)
    torch.cuda.synchronize()


def gpu_decode(oscar, sc: Scenario, cache, rk, rv):
    lens = torch.tensor(sc.lens, dtype=torch.int32, device="cuda")
    out = oscar.decode_attn(cache, rk, rv, to_dev_bf16(sc.q), lens, max(sc.lens), SCALE)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_raw_rows(sc: Scenario, gpu_bf16: np.ndarray, ref: o.LayerCacheRef):
    """Sink and ring rows in use must be bit-identical."""
    for b, L in enumerate(sc.lens):
        for p in range(L):
            w, idx = o.storage_of(p, L)
            if w == "hist":
                continue
            pg, row = ref._bf16_row(b, w, idx)
            assert np.array_equal(gpu_bf16[pg, :, :, row, :], ref.bf16[pg, :, :, row, :]), (b, p)


# ------------------------------------------------------------------ forms


def test_prepare_rotation_forms(oscar):
    R = np.linalg.qr(np.random.default_rng(3).standard_normal((128, 128)))[0]
    rot = oscar.Rotation(R, 5.0)
    f = rot.forms.cpu().numpy()
    R32 = f[0:65536].view(np.float32).reshape(128, 128)
    RT32 = f[65536:131072].view(np.float32).reshape(128, 128)
    hi = f[131072:163840].view(np.float16).reshape(128, 128).astype(np.float64)
    lo = f[163840:196608].view(np.float16).reshape(128, 128).astype(np.float64)
    assert np.array_equal(R32, R.astype(np.float32))
    assert np.array_equal(RT32, R32.T)
    assert np.abs(hi.T + lo.T / 2048 - R).max() < 2.0 ** -22


# ------------------------------------------------------------------ write


def test_write_single_layer_calibrated_g32(oscar):
    # one layer: 8 query / 2 KV heads, 4096 tokens (16 sink + 128 recent + 3952 history), G = 32
    sc = Scenario(100, 8, 2, 32, [4096], rot="calibrated")
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc)
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, sc.G)
    print("write stats", stats)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), ref)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_write_ragged_batch(oscar, G):
    lens = [1, 16, 17, 144, 145, 160, 161, 300, 1000]
    sc = Scenario(200 + G, 8, 2, G, lens)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc)
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, G)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), ref)


def test_write_chunks_and_appends(oscar):
    # prefill in uneven chunks (one longer than the recent window), then
    # single-token appends: ring tokens leave the window and are quantised
    lens = [700, 433]
    chunks = [0, 100, 250, 400] + list(range(401, 440)) + [600, 700]
    sc = Scenario(300, 8, 2, 64, lens)
    ref = sc.oracle_cache(chunks)
    cache = gpu_cache(oscar, sc)
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv, chunks)
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, sc.G)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), ref)


def test_write_bad_page_id_is_flagged_and_skipped(oscar):
    # one history page id of request 0 points outside the pool: the kernel
    # flags it, writes nothing for that page, and writes every other page
    sc = Scenario(310, 8, 2, 32, [1000, 600])
    cache = gpu_cache(oscar, sc)
    cache.hist.fill_(0xAB)
    bad_j = 5
    cache.hist_pt[0, bad_j] = sc.n_hist_pages + 1000
    rk, rv = gpu_rotations(oscar, sc)
    gpu_write(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) & 1
    gh = cache.hist.cpu().numpy()
    # the page the oracle would have used holds no history of request 0
    assert np.all(gh[sc.hist_pt[0, bad_j]] == 0xAB)
    hist0 = np.arange(o.N_SINK, sc.lens[0] - o.N_RECENT)
    keep0 = hist0[(hist0 - o.N_SINK) // o.PAGE != bad_j]
    hist1 = np.arange(o.N_SINK, sc.lens[1] - o.N_RECENT)
    stats = compare_history(gh, sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens, sc.R_K, sc.R_V, sc.clip_k, sc.clip_v,
                            sc.G, positions=[keep0, hist1])
    assert_history_ok(stats)


# ------------------------------------------------------------------ decode


@pytest.mark.parametrize("G", [32, 64, 128])
def test_decode_ragged_batch(oscar, G):
    lens = [1, 15, 16, 17, 100, 144, 145, 146, 159, 160, 161, 777, 2049]
    sc = Scenario(400 + G, 8, 2, G, lens)
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    out = gpu_decode(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) == 0
    mx, rel = assert_decode_close(out, sc.oracle_decode(ref))
    print(f"G={G} max abs {mx:.2e} rel {rel:.2e}")


def test_decode_single_layer_calibrated(oscar):
    sc = Scenario(101, 8, 2, 32, [4096], rot="calibrated")
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    out = gpu_decode(oscar, sc, cache, rk, rv)
    mx, rel = assert_decode_close(out, sc.oracle_decode(ref))
    print(f"max abs {mx:.2e} rel {rel:.2e}")


def test_decode_mha_and_gqa8(oscar):
    for hq, hkv in ((4, 4), (16, 2)):
        sc = Scenario(500 + hq, hq, hkv, 64, [300, 1500])
        ref = sc.oracle_cache()
        cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
        rk, rv = gpu_rotations(oscar, sc)
        assert_decode_close(gpu_decode(oscar, sc, cache, rk, rv), sc.oracle_decode(ref), f"{hq}/{hkv}")


def test_decode_deterministic(oscar):
    sc = Scenario(600, 8, 2, 64, [3000, 200])
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    a = gpu_decode(oscar, sc, cache, rk, rv)
    b = gpu_decode(oscar, sc, cache, rk, rv)
    assert np.array_equal(a, b)


def test_decode_shared_prefix_pages(oscar):
    # request 1 reuses request 0's first two history pages (same tokens)
    L = 400
    sc = Scenario(700, 8, 2, 32, [L, L])
    for arr in (sc.k, sc.v):
        arr[L:L + 176] = arr[:176]
    sc.tok_k = [sc.k[:L], sc.k[L:]]
    sc.tok_v = [sc.v[:L], sc.v[L:]]
    sc.hist_pt[1, :2] = sc.hist_pt[0, :2]
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    assert_decode_close(gpu_decode(oscar, sc, cache, rk, rv), sc.oracle_decode(ref))


def test_decode_many_splits_reuses_workspace(oscar):
    # one request over 2 KV heads at 20K: 125 history splits per head, so the
    # merging workgroup sums its partials in several register windows; the
    # workspace is filled with zeros once, and every call leaves its merge
    # counters (the last bytes) at zero again
    L = 20000
    sc = Scenario(1500, 8, 2, 64, [L])
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    need = oscar.decode_workspace_bytes(1, 8, 2, L)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    expect = sc.oracle_decode(ref)
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    q = to_dev_bf16(sc.q)
    for rep in range(3):
        out = oscar.decode_attn(cache, rk, rv, q, lens, L, SCALE, workspace=ws)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        assert_decode_close(out.cpu().numpy(), expect, f"many splits, call {rep}")
        assert int(ws[-256:].count_nonzero().item()) == 0


def test_bad_page_ids_are_flagged_not_followed(oscar):
    sc = Scenario(800, 8, 2, 64, [600])
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    cache.hist_pt[0, 3] = sc.n_hist_pages + 1000   # outside the pool
    rk, rv = gpu_rotations(oscar, sc)
    out = gpu_decode(oscar, sc, cache, rk, rv)
    assert int(cache.status.item()) & 1
    assert np.isfinite(out).all()


# ------------------------------------------------------------------ BF16 baseline


def test_bf16_paged_decode(oscar):
    lens = [1, 16, 17, 300, 1024, 4097]
    hq, hkv = 8, 2
    ld = synth.LayerData(900, 0, hq, hkv)
    k, v = ld.cache_kv(sum(lens))
    pt, npages = synth.shuffled_page_tables(900, 0, lens, n_pages_fn=lambda L: (L + 15) // 16)
    pages = np.zeros((npages, hkv, 2, 16, 128), dtype=np.uint16)
    off = 0
    for b, L in enumerate(lens):
        p = np.arange(L)
        pages[pt[b, p // 16], :, 0, p % 16] = k[off:off + L]
        pages[pt[b, p // 16], :, 1, p % 16] = v[off:off + L]
        off += L
    q = ld.decode_q(len(lens))
    ref = o.bf16_paged_decode(q, pages, pt, lens, SCALE)
    import bit_rotated_kv_oscar_amd as m
    kv = to_dev_bf16(pages)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = m.bf16_paged_decode(to_dev_bf16(q), kv, torch.from_numpy(pt).cuda(),
                              torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), SCALE,
                              status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_decode_close(out.cpu().numpy(), ref, "bf16")


# ------------------------------------------------------------------ calibration


def test_calibration_matches_oracle(oscar):
    ld = synth.LayerData(1000, 0, 8, 2)
    qc, kc, vc = ld.calibration(2048)
    R_K, R_V, ck, cv = oscar.calibrate_rotation(to_dev_bf16(qc), to_dev_bf16(kc), to_dev_bf16(vc), 0.999)
    R_K, R_V = R_K.numpy(), R_V.numpy()
    q, k, v = (o.bf16_to_f64(x) for x in (qc, kc, vc))
    cal = o.calibrate(q, k, v)
    H, P = o.hadamard(), o.bitrev_permutation()
    for R, C in ((R_K, o.query_covariance(q)), (R_V, o.score_covariance(q, k, v))):
        assert np.abs(R.T @ R - np.eye(128)).max() < 1e-12
        lam = np.sort(np.linalg.eigvalsh(C))[::-1]
        assert np.abs(R.T @ C @ R - P @ H @ np.diag(lam) @ H @ P).max() < 1e-10 * np.abs(C).max()
    assert np.abs(R_K - cal["R_K"]).max() < 1e-8
    assert np.abs(R_V - cal["R_V"]).max() < 1e-8
    assert abs(ck - cal["clip_K"]) <= 1e-6 * cal["clip_K"]
    assert abs(cv - cal["clip_V"]) <= 1e-6 * cal["clip_V"]


def test_calibration_over_sequences_matches_oracle(oscar):
    # three calibration sequences of different lengths, moments accumulated
    # on the device, rotations and clips against the oracle's pooled ones
    seqs_bits = []
    for i, n in enumerate((700, 1024, 300)):
        ld = synth.LayerData(1300 + i, 0, 8, 2)
        seqs_bits.append(ld.calibration(n))
    sums = torch.zeros((2, 128, 128), dtype=torch.float64, device="cuda")
    count = 0
    for qc, kc, vc in seqs_bits:
        count += oscar.calib_accumulate(to_dev_bf16(qc), to_dev_bf16(kc), to_dev_bf16(vc), sums)
    R_K, R_V = oscar.calib_rotations(sums, count)
    k_all = to_dev_bf16(np.concatenate([k for _, k, _ in seqs_bits]))
    v_all = to_dev_bf16(np.concatenate([v for _, _, v in seqs_bits]))
    ck = oscar.clip_threshold(k_all, R_K)
    cv = oscar.clip_threshold(v_all, R_V)
    cal = o.calibrate_sequences([tuple(o.bf16_to_f64(x) for x in sb) for sb in seqs_bits])
    assert count == (700 + 1024 + 300) * 8
    R_K, R_V = R_K.numpy(), R_V.numpy()
    for R, C in ((R_K, cal["C_Q"]), (R_V, cal["C_S"])):
        assert np.abs(R.T @ R - np.eye(128)).max() < 1e-12
        lam = np.sort(np.linalg.eigvalsh(C))[::-1]
        H, P = o.hadamard(), o.bitrev_permutation()
        assert np.abs(R.T @ C @ R - P @ H @ np.diag(lam) @ H @ P).max() < 1e-10 * np.abs(C).max()
    assert np.abs(R_K - cal["R_K"]).max() < 1e-8
    assert np.abs(R_V - cal["R_V"]).max() < 1e-8
    assert abs(ck - cal["clip_K"]) <= 1e-6 * cal["clip_K"]
    assert abs(cv - cal["clip_V"]) <= 1e-6 * cal["clip_V"]


# ------------------------------------------------------------------ decode step


def _prefix_cache(sc: Scenario, drop: int):
    """Oracle cache holding all but the last `drop` tokens of every request."""
    ref = o.LayerCacheRef(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, sc.hist_pt, sc.bf16_pt, bits=sc.bits)
    keep = [max(0, L - drop) for L in sc.lens]
    kp = np.concatenate([t[:n] for t, n in zip(sc.tok_k, keep)])
    vp = np.concatenate([t[:n] for t, n in zip(sc.tok_v, keep)])
    cu = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
    ref.write(sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, kp, vp, cu, np.zeros(len(keep), np.int32))
    return ref


@pytest.mark.parametrize("G", [32, 64, 128])
def test_decode_step_appends_then_decodes(oscar, G):
    # lengths after the step; the appended token pushes position L-129 out of
    # the window whenever L - 1 >= 144
    lens = [1, 16, 17, 143, 144, 145, 146, 160, 161, 500, 1201]
    sc = Scenario(1100 + G, 8, 2, G, lens)
    pre = _prefix_cache(sc, 1)
    full = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=pre.hist, bf16=pre.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    k_last = np.stack([t[-1] for t in sc.tok_k])
    v_last = np.stack([t[-1] for t in sc.tok_v])
    before = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    out = oscar.decode_step(cache, rk, rv, to_dev_bf16(k_last), to_dev_bf16(v_last), before, to_dev_bf16(sc.q),
                            max(lens), SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, G)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), full)
    assert_decode_close(out.cpu().numpy(), sc.oracle_decode(full), f"decode_step G={G}")


@pytest.mark.parametrize("rot", ["hadamard", "identity"])
def test_decode_step_rotation_variants(oscar, rot):
    # write-on-append under the pages' comparison rotations (unrotated bf16
    # values put many quantisation steps exactly halfway between levels)
    lens = [145, 146, 161, 500, 1201]
    sc = Scenario(1150, 8, 2, 32, lens, rot=rot)
    pre = _prefix_cache(sc, 1)
    full = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=pre.hist, bf16=pre.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    k_last = np.stack([t[-1] for t in sc.tok_k])
    v_last = np.stack([t[-1] for t in sc.tok_v])
    before = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    out = oscar.decode_step(cache, rk, rv, to_dev_bf16(k_last), to_dev_bf16(v_last), before, to_dev_bf16(sc.q),
                            max(lens), SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, 32)
    assert_history_ok(stats)
    assert stats.get("code_in_band", 0) == 0, stats
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), full)
    assert_decode_close(out.cpu().numpy(), sc.oracle_decode(full), f"decode_step ({rot})")


def test_decode_step_many_steps(oscar):
    # 40 consecutive steps: ring slots are reused and evicted tokens fill two
    # history pages row by row
    lens = [330, 200, 150]
    steps = 40
    sc = Scenario(1200, 8, 2, 64, lens)
    pre = _prefix_cache(sc, steps)
    full = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=pre.hist, bf16=pre.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    ws = torch.zeros(oscar.decode_workspace_bytes(len(lens), 8, 2, max(lens)), dtype=torch.uint8, device="cuda")
    q = to_dev_bf16(sc.q)
    for s in range(steps, 0, -1):
        k_s = np.stack([t[L - s] for t, L in zip(sc.tok_k, lens)])
        v_s = np.stack([t[L - s] for t, L in zip(sc.tok_v, lens)])
        before = torch.tensor([L - s for L in lens], dtype=torch.int32, device="cuda")
        out = oscar.decode_step(cache, rk, rv, to_dev_bf16(k_s), to_dev_bf16(v_s), before, q, max(lens), SCALE,
                                workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                            sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, 64)
    assert_history_ok(stats)
    check_raw_rows(sc, bf16_pool_bits(cache.bf16), full)
    assert_decode_close(out.cpu().numpy(), sc.oracle_decode(full), "decode_step x40")


def test_bf16_decode_reuses_workspace(oscar):
    # one workspace, filled once, serves repeated calls
    lens = [700, 33]
    ld = synth.LayerData(1300, 0, 8, 2)
    k, v = ld.cache_kv(sum(lens))
    pt, npages = synth.shuffled_page_tables(1300, 0, lens, n_pages_fn=lambda L: (L + 15) // 16)
    pages = np.zeros((npages, 2, 2, 16, 128), dtype=np.uint16)
    off = 0
    for b, L in enumerate(lens):
        p = np.arange(L)
        pages[pt[b, p // 16], :, 0, p % 16] = k[off:off + L]
        pages[pt[b, p // 16], :, 1, p % 16] = v[off:off + L]
        off += L
    q = ld.decode_q(len(lens))
    ref = o.bf16_paged_decode(q, pages, pt, lens, SCALE)
    ws = torch.zeros(oscar.bf16_decode_workspace_bytes(2, 8, 2, max(lens)), dtype=torch.uint8, device="cuda")
    args = (to_dev_bf16(q), to_dev_bf16(pages), torch.from_numpy(pt).cuda(),
            torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), SCALE)
    for _ in range(3):
        out = oscar.bf16_paged_decode(*args, workspace=ws)
        torch.cuda.synchronize()
        assert_decode_close(out.cpu().numpy(), ref, "bf16 repeated")
        assert int(ws[-256:].count_nonzero().item()) == 0   # merge counters back at zero


def test_bf16_decode_one_round_many_splits(oscar):
    # one request at 20K over 2 KV heads: one round of workgroups, 125
    # splits per head, merged inside the kernel in several register windows
    L, hq, hkv = 20000, 8, 2
    ld = synth.LayerData(1350, 0, hq, hkv)
    k, v = ld.cache_kv(L)
    pt, npages = synth.shuffled_page_tables(1350, 0, [L], n_pages_fn=lambda n: (n + 15) // 16)
    pages = np.zeros((npages, hkv, 2, 16, 128), dtype=np.uint16)
    p = np.arange(L)
    pages[pt[0, p // 16], :, 0, p % 16] = k
    pages[pt[0, p // 16], :, 1, p % 16] = v
    q = ld.decode_q(1)
    ref = o.bf16_paged_decode(q, pages, pt, [L], SCALE)
    ws = torch.zeros(oscar.bf16_decode_workspace_bytes(1, hq, hkv, L), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        out = oscar.bf16_paged_decode(to_dev_bf16(q), to_dev_bf16(pages), torch.from_numpy(pt).cuda(),
                                      torch.tensor([L], dtype=torch.int32, device="cuda"), L, SCALE, workspace=ws)
        torch.cuda.synchronize()
        assert_decode_close(out.cpu().numpy(), ref, "bf16 one round")
        assert int(ws[-256:].count_nonzero().item()) == 0


# ------------------------------------------------------------------ long splits


def _shared_page_batch(sc: Scenario, ref: o.LayerCacheRef, batch: int):
    """`batch` requests of sc.lens[0] tokens that all read the pages of
    request 0 (page tables repeated), with their own queries."""
    hist_pt = np.repeat(sc.hist_pt[:1], batch, axis=0)
    bf16_pt = np.repeat(sc.bf16_pt[:1], batch, axis=0)
    q = sc.ld.decode_q(batch)
    return hist_pt, bf16_pt, q


def test_decode_more_than_64_pages_per_wave(oscar):
    # 16 requests x 8 KV heads = 128 (request, head) units: one round with one
    # history split per unit, so each of the 8 waves walks 554 / 8 > 64 pages
    L, B = 9000, 16
    sc = Scenario(1300, 32, 8, 64, [L])
    ref = sc.oracle_cache()
    hist_pt, bf16_pt, q = _shared_page_batch(sc, ref, B)
    dev = torch.device("cuda:0")
    cache = oscar.LayerCache(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, torch.from_numpy(hist_pt),
                             torch.from_numpy(bf16_pt), device=dev)
    cache.hist.copy_(torch.from_numpy(ref.hist))
    cache.bf16.view(torch.int16).copy_(torch.from_numpy(ref.bf16.view(np.int16)))
    rk, rv = gpu_rotations(oscar, sc)
    out = oscar.decode_attn(cache, rk, rv, to_dev_bf16(q), torch.full((B,), L, dtype=torch.int32, device=dev),
                            L, SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    got = out.cpu().numpy()
    pick = [0, 9, 15]
    ref.hist_pt = hist_pt[:len(pick)]
    ref.bf16_pt = bf16_pt[:len(pick)]
    expect = o.decode_attn(ref, sc.R_K, sc.R_V, q[pick], [L] * len(pick), SCALE)
    assert_decode_close(got[pick], expect, "int2 long split")


@pytest.mark.parametrize("hq,hkv,G", [(32, 8, 64), (64, 8, 128), (16, 8, 64), (8, 8, 128)])
def test_decode_several_rounds_fp4_scores(oscar, hq, hkv, G):
    # 24 requests x 8 KV heads = 192 (request, head) units, more than one
    # round holds: the several-round plan, whose INT2 scores (one or two
    # scale groups per head) run on the fp8 x fp4 matrix-core products.
    _several_rounds_case(oscar, hq, hkv, G)


def test_decode_gqa8_g32(oscar):
    # GQA 8 with four scale groups per head: 32 (head, group) pairs per KV
    # head, the widest score fragment (fp16 products; these instances keep
    # part of their state in scratch), in one round and in several rounds
    sc = Scenario(1750, 16, 2, 32, [300, 1500])
    ref = sc.oracle_cache()
    cache = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
    rk, rv = gpu_rotations(oscar, sc)
    assert_decode_close(gpu_decode(oscar, sc, cache, rk, rv), sc.oracle_decode(ref), "16/2 G 32")
    _several_rounds_case(oscar, 64, 8, 32)


def _several_rounds_case(oscar, hq, hkv, G):
    # Requests read request 0's pages as prefixes of ragged lengths (partial
    # last pages, one or no history page), each with its own query.
    L, B = 2500, 24
    sc = Scenario(1700 + hq + G, hq, hkv, G, [L])
    ref = sc.oracle_cache()
    hist_pt, bf16_pt, q = _shared_page_batch(sc, ref, B)
    rng = np.random.default_rng(1701)
    lens = np.concatenate([[L, 2049, 160, 161, 144, 150, 1000], rng.integers(145, L, B - 7)]).astype(np.int32)
    dev = torch.device("cuda:0")
    cache = oscar.LayerCache(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, torch.from_numpy(hist_pt),
                             torch.from_numpy(bf16_pt), device=dev)
    cache.hist.copy_(torch.from_numpy(ref.hist))
    cache.bf16.view(torch.int16).copy_(torch.from_numpy(ref.bf16.view(np.int16)))
    rk, rv = gpu_rotations(oscar, sc)
    out = oscar.decode_attn(cache, rk, rv, to_dev_bf16(q), torch.from_numpy(lens).to(dev), L, SCALE)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    got = out.cpu().numpy()
    pick = [0, 1, 2, 3, 5, 6, 11, 23]
    ref.hist_pt = hist_pt[:len(pick)]
    ref.bf16_pt = bf16_pt[:len(pick)]
    expect = o.decode_attn(ref, sc.R_K, sc.R_V, q[pick], [int(lens[b]) for b in pick], SCALE)
    mx, rel = assert_decode_close(got[pick], expect, f"several rounds {hq}/{hkv} G {G}")
    print(f"several rounds {hq}/{hkv} G={G}: max abs {mx:.2e} rel {rel:.2e}")


@pytest.mark.parametrize("q_mult,sm_scale", [(400.0, 1.0), (1e-3, SCALE), (0.0, SCALE)])
def test_decode_several_rounds_fp4_scores_query_norms(oscar, q_mult, sm_scale):
    # the fp8 parts of q R_K take their exponents from each (head, group)'s
    # largest value: scores far beyond the fp16 range (x400 at sm_scale 1),
    # tiny queries, and every third query head all zero (no parts: uniform
    # attention) beside normal ones
    L, B = 1200, 24
    sc = Scenario(1800, 32, 8, 64, [L])
    ref = sc.oracle_cache()
    hist_pt, bf16_pt, q = _shared_page_batch(sc, ref, B)
    qf = synth.bf16_to_f64(q) * (q_mult if q_mult else 1.0)
    if q_mult == 0.0:
        qf[:, ::3] = 0.0  # every third query head all zero
    q = synth.bf16_bits(qf.astype(np.float32))
    lens = np.full(B, L, dtype=np.int32)
    lens[1::2] = 700
    dev = torch.device("cuda:0")
    cache = oscar.LayerCache(sc.hkv, sc.G, sc.n_hist_pages, sc.n_bf16_pages, torch.from_numpy(hist_pt),
                             torch.from_numpy(bf16_pt), device=dev)
    cache.hist.copy_(torch.from_numpy(ref.hist))
    cache.bf16.view(torch.int16).copy_(torch.from_numpy(ref.bf16.view(np.int16)))
    rk, rv = gpu_rotations(oscar, sc)
    out = oscar.decode_attn(cache, rk, rv, to_dev_bf16(q), torch.from_numpy(lens).to(dev), L, sm_scale)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    pick = [0, 1, 7, 22]
    ref.hist_pt = hist_pt[:len(pick)]
    ref.bf16_pt = bf16_pt[:len(pick)]
    expect = o.decode_attn(ref, sc.R_K, sc.R_V, q[pick], [int(lens[b]) for b in pick], sm_scale)
    mx, rel = assert_decode_close(got[pick], expect, f"several rounds q x{q_mult} sm_scale {sm_scale}")
    print(f"several rounds q x{q_mult}: max abs {mx:.2e} rel {rel:.2e}")


def test_bf16_decode_more_than_64_pages_per_wave(oscar):
    # 40 requests x 8 KV heads = 320 units: one split per unit, 563 / 8 > 64
    # pages per wave; all requests read the same pages
    L, B, hq, hkv = 9000, 40, 32, 8
    ld = synth.LayerData(1400, 0, hq, hkv)
    k, v = ld.cache_kv(L)
    pt1, npages = synth.shuffled_page_tables(1400, 0, [L], n_pages_fn=lambda n: (n + 15) // 16)
    pages = np.zeros((npages, hkv, 2, 16, 128), dtype=np.uint16)
    p = np.arange(L)
    pages[pt1[0, p // 16], :, 0, p % 16] = k
    pages[pt1[0, p // 16], :, 1, p % 16] = v
    pt = np.repeat(pt1, B, axis=0)
    q = ld.decode_q(B)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = oscar.bf16_paged_decode(to_dev_bf16(q), to_dev_bf16(pages), torch.from_numpy(pt).cuda(),
                                  torch.full((B,), L, dtype=torch.int32, device="cuda"), L, SCALE,
                                  status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    pick = [0, 21, 39]
    expect = o.bf16_paged_decode(q[pick], pages, pt[:len(pick)], [L] * len(pick), SCALE)
    assert_decode_close(out.cpu().numpy()[pick], expect, "bf16 long split")


def test_clip_threshold_exact_order_statistics_past_2_20_vectors(oscar):
    # R = I and integer values 0..250 (exact in bf16): the 0.999 and 0.5
    # quantiles (type 7) follow from the value counts in closed form; 2^20 + 3
    # vectors (134M values, past the former host-sort cap) go through the
    # device radix selection, and ties (each value ~535K times) exercise the
    # equal-neighbour case
    n = (1 << 20) + 3
    idx = torch.arange(n * 128, device="cuda", dtype=torch.int64)
    vals = (idx % 251).to(torch.float32)
    x = vals.to(torch.bfloat16).view(n, 128)
    counts = np.bincount((np.arange(n * 128, dtype=np.int64) % 251), minlength=251)
    cum = np.cumsum(counts)

    def order_stat(r):  # 0-based rank -> value
        return float(np.searchsorted(cum, r, side="right"))

    for p in (0.999, 0.5, 1.0, 1e-9):
        h = (n * 128 - 1) * p
        lo = int(np.floor(h))
        a = order_stat(lo)
        b = order_stat(min(lo + 1, n * 128 - 1))
        t = h - lo
        want = b - (b - a) * (1 - t) if t >= 0.5 else a + (b - a) * t
        got = oscar.clip_threshold(x, torch.eye(128, dtype=torch.float64), p)
        assert got == np.float32(want), (p, got, want)
    # a general rotation on a smaller set: the oracle's numpy quantile
    R = random_rotation(77)
    xs = to_dev_bf16(synth.bf16_bits(np.random.default_rng(3).standard_normal((3000, 128)).astype(np.float32) * 3))
    xf = synth.bf16_to_f64(xs.view(torch.int16).cpu().numpy().view(np.uint16))
    want = o.clip_threshold(xf, R, 0.999)
    got = oscar.clip_threshold(xs, torch.from_numpy(R), 0.999)
    assert abs(got - want) <= 1e-6 * want


def test_calibration_reports_an_unconverged_eigen_iteration(oscar, monkeypatch):
    # the sweep limit forced to 1 (diagnostic hook): the iteration stops
    # before its tolerance and both calibration entry points say so
    ld = synth.LayerData(41, 0, 8, 2)
    qc, kc, vc = (to_dev_bf16(x) for x in ld.calibration(256))
    monkeypatch.setenv("OSCAR_JACOBI_SWEEPS", "1")
    with pytest.raises(oscar.OscarError) as ei:
        oscar.calibrate_rotation(qc, kc, vc, 0.999)
    assert ei.value.code == oscar._lib.OSCAR_EINVAL and "converge" in str(ei.value)
    sums = torch.zeros((2, 128, 128), dtype=torch.float64, device="cuda")
    count = oscar.calib_accumulate(qc, kc, vc, sums)
    with pytest.raises(oscar.OscarError) as ei:
        oscar.calib_rotations(sums, count)
    assert "converge" in str(ei.value)
    # back at the default limit the same inputs calibrate
    monkeypatch.delenv("OSCAR_JACOBI_SWEEPS")
    R_K, R_V, ck, cv = oscar.calibrate_rotation(qc, kc, vc, 0.999)
    assert np.abs(R_K.numpy().T @ R_K.numpy() - np.eye(128)).max() < 1e-12
