"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, invariants of the construction, hand-derived bytes of the documented
storage format (tests/golden/), brute force in plain Python on tiny inputs, or
special cases that reduce to a textbook routine.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import oscar_ref as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- Hadamard


def fwht(x):
    """Textbook fast Walsh-Hadamard butterfly (natural order), unnormalised."""
    x = np.array(x, dtype=np.float64)
    n = x.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x


def test_hadamard_orthonormal_symmetric():
    H = o.hadamard()
    assert np.abs(H @ H.T - np.eye(128)).max() <= 1e-15
    assert np.array_equal(H, H.T)
    np.testing.assert_allclose(H[0], 2.0 ** -3.5, rtol=3e-16, atol=0)
    np.testing.assert_allclose(np.abs(H), 2.0 ** -3.5, rtol=3e-16, atol=0)


def test_hadamard_equals_butterfly():
    x = RNG.standard_normal((5, 128))
    np.testing.assert_allclose(x @ o.hadamard(), fwht(x) / math.sqrt(128), rtol=0, atol=1e-13)


# ------------------------------------------------------------- bit reversal


def test_bitrev_table():
    table = {0: 0, 1: 64, 2: 32, 3: 96, 5: 80, 6: 48, 127: 127, 64: 1}
    for i, r in table.items():
        assert o.bitrev(i) == r


def test_bitrev_permutation_identities():
    P = o.bitrev_permutation()
    H = o.hadamard()
    assert np.array_equal(P @ P, np.eye(128))      # involution
    assert np.array_equal(P, P.T)
    assert P.sum(axis=0).tolist() == [1.0] * 128 and P.sum(axis=1).tolist() == [1.0] * 128
    assert np.abs(P @ H @ P - H).max() == 0.0
    assert np.abs(H @ P - P @ H).max() == 0.0
    # x P moves channel j to position bitrev(j)?  (x P)[j] = sum_i x[i] P[i][j] = x[bitrev(j)]
    x = np.arange(128.0)
    assert np.array_equal(x @ P, np.array([o.bitrev(j) for j in range(128)], dtype=float))


# -------------------------------------------------------------- calibration


def test_query_covariance_closed_form():
    # q rows are scaled basis vectors: C_Q is diagonal with alpha^2 / (N*Hq)
    n, hq = 128, 2
    q = np.zeros((n, hq, 128))
    alpha = np.arange(1, 129, dtype=float)
    for i in range(n):
        q[i, 0, i] = alpha[i]
    C = o.query_covariance(q)
    np.testing.assert_allclose(np.diag(C), alpha ** 2 / (n * hq), rtol=1e-15)
    assert np.abs(C - np.diag(np.diag(C))).max() == 0.0


def test_query_covariance_converges_to_sigma():
    lam = synth.layer_lambda(7, 0)
    q = RNG.standard_normal((20000, 4, 128)) * np.sqrt(lam)
    C = o.query_covariance(q)
    # 80000 samples: relative error of each diagonal entry ~ sqrt(2/80000) = 0.5%
    np.testing.assert_allclose(np.diag(C), lam, rtol=0.03)
    assert np.abs(C - np.diag(np.diag(C))).max() < 0.05 * lam.max()


def test_score_covariance_single_token():
    # N = 1: the only probability is 1, so o = v and C_S = mean_h v_g v_g^T
    hq, hkv = 4, 2
    q = RNG.standard_normal((1, hq, 128))
    k = RNG.standard_normal((1, hkv, 128))
    v = RNG.standard_normal((1, hkv, 128))
    expect = sum(np.outer(v[0, h // 2], v[0, h // 2]) for h in range(hq)) / hq
    np.testing.assert_allclose(o.score_covariance(q, k, v), expect, rtol=1e-14, atol=1e-14)


def test_causal_attention_two_tokens_by_hand():
    d = 128
    q = RNG.standard_normal((2, 1, d))
    k = RNG.standard_normal((2, 1, d))
    v = RNG.standard_normal((2, 1, d))
    out = o.causal_attention_outputs(q, k, v)
    # token 0 sees only itself; token 1 weighs keys 0 and 1
    s0 = sum(q[1, 0, i] * k[0, 0, i] for i in range(d)) / math.sqrt(d)
    s1 = sum(q[1, 0, i] * k[1, 0, i] for i in range(d)) / math.sqrt(d)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(out[0, 0], v[0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[1, 0], w0 * v[0, 0] + (1 - w0) * v[1, 0], rtol=1e-13, atol=1e-13)


def test_causal_attention_gqa_map():
    n, hq, hkv = 6, 4, 2
    q = RNG.standard_normal((n, hq, 128))
    k = RNG.standard_normal((n, hkv, 128))
    v = RNG.standard_normal((n, hkv, 128))
    out = o.causal_attention_outputs(q, k, v)
    for h in range(hq):
        g = h // 2
        single = o.causal_attention_outputs(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1])
        np.testing.assert_allclose(out[:, h], single[:, 0], rtol=1e-14, atol=1e-14)


def test_score_covariance_matches_literal_form():
    # (S V)^T (S V) / N per head equals the page's V^T S^T S V / N with S the
    # explicit causal probability matrix built in plain loops
    n = 5
    q = RNG.standard_normal((n, 1, 128))
    k = RNG.standard_normal((n, 1, 128))
    v = RNG.standard_normal((n, 1, 128))
    S = np.zeros((n, n))
    for i in range(n):
        logits = [float(q[i, 0] @ k[j, 0]) / math.sqrt(128) for j in range(i + 1)]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        for j in range(i + 1):
            S[i, j] = w[j] / sum(w)
    V = v[:, 0, :]
    np.testing.assert_allclose(o.score_covariance(q, k, v), V.T @ S.T @ S @ V / n, rtol=1e-12, atol=1e-13)


def test_eigenbasis_diagonal_sorts_and_signs():
    vals = RNG.permutation(np.arange(1.0, 129.0))
    U = o.eigenbasis(np.diag(vals))
    order = np.argsort(-vals)
    expect = np.eye(128)[:, order]
    assert np.array_equal(U, expect)


def test_eigenbasis_sign_rule():
    Q, _ = np.linalg.qr(RNG.standard_normal((128, 128)))
    lam = np.linspace(10, 1, 128)
    C = Q @ np.diag(lam) @ Q.T
    U = o.eigenbasis(C)
    for j in range(128):
        col = Q[:, j] * np.sign(Q[np.argmax(np.abs(Q[:, j])), j])
        np.testing.assert_allclose(U[:, j], col, atol=1e-10)
        assert U[np.argmax(np.abs(U[:, j])), j] > 0


@pytest.fixture(scope="module")
def calibrated():
    ld = synth.LayerData(11, 0, 8, 2)
    qb, kb, vb = ld.calibration(512)
    q, k, v = (o.bf16_to_f64(x) for x in (qb, kb, vb))
    cal = o.calibrate(q, k, v)
    return q, k, v, cal


def test_rotation_orthogonal(calibrated):
    _, _, _, cal = calibrated
    for R in (cal["R_K"], cal["R_V"]):
        assert np.abs(R.T @ R - np.eye(128)).max() <= 1e-12


def test_rotation_diagonalises_then_mixes(calibrated):
    # R^T C R = P H Lambda H P, independent of eigenvector signs
    q, k, v, cal = calibrated
    H, P = o.hadamard(), o.bitrev_permutation()
    for C, R in ((o.query_covariance(q), cal["R_K"]), (o.score_covariance(q, k, v), cal["R_V"])):
        lam = np.sort(np.linalg.eigvalsh(C))[::-1]
        lhs = R.T @ C @ R
        rhs = P @ H @ np.diag(lam) @ H @ P
        assert np.abs(lhs - rhs).max() <= 1e-12 * np.abs(C).max() * 128


def test_rotation_equalises_importance(calibrated):
    # diag(R_K^T C_Q R_K) = tr(C_Q)/128 for every channel (the Hadamard factor
    # equalises the importance metric, [nl]/[fr] section 2.2.A)
    q, _, _, cal = calibrated
    C = o.query_covariance(q)
    d = np.diag(cal["R_K"].T @ C @ cal["R_K"])
    np.testing.assert_allclose(d, np.trace(C) / 128, rtol=1e-12)


def test_rotation_preserves_dot_products(calibrated):
    q, k, _, cal = calibrated
    R = cal["R_K"]
    a, b = q[:50, 0], k[:50, 0]
    np.testing.assert_allclose(np.sum((a @ R) * (b @ R), axis=1), np.sum(a * b, axis=1), rtol=1e-12, atol=1e-12)


def test_clip_quantile_closed_form():
    # |values| 1..1024, quantile 0.999: h = 1023*0.999 = 1021.977 -> 1022.977
    x = -np.arange(1.0, 1025.0).reshape(8, 1, 128)
    assert abs(o.clip_threshold(x, np.eye(128), 0.999) - (1.0 + 0.999 * 1023.0)) < 1e-9
    assert o.clip_threshold(x, np.eye(128), 1.0) == 1024.0


def test_clip_uses_rotated_values():
    # with a rotation that maps e_0 to (1,1,..)/sqrt(128) the quantile sees the
    # rotated magnitudes, not the raw ones
    x = np.zeros((1, 1, 128))
    x[0, 0, 0] = math.sqrt(128.0)
    assert abs(o.clip_threshold(x, o.hadamard(), 0.5) - 1.0) < 1e-12


# ---------------------------------------------------------------- quantiser


def _group_input(vals, G=32):
    x = np.zeros((1, 128))
    x[0, :G] = vals
    return x


def test_quantizer_hand_cases():
    I = np.eye(128)
    # levels
    q = o.quantize(_group_input(np.tile([0, 1, 2, 3], 8)), I, 1000.0, 32)
    assert q["zero"][0, 0] == 0 and q["scale"][0, 0] == 1
    assert q["codes"][0, :32].tolist() == [0, 1, 2, 3] * 8
    # centred
    q = o.quantize(_group_input(np.tile([-1.5, -0.5, 0.5, 1.5], 8)), I, 1000.0, 32)
    assert q["zero"][0, 0] == -1.5 and q["scale"][0, 0] == 1
    assert q["codes"][0, :32].tolist() == [0, 1, 2, 3] * 8
    # constant group: scale 0, codes 0, dequantised value = zero
    q = o.quantize(_group_input(np.full(32, 0.75)), I, 1000.0, 32)
    assert q["scale"][0, 0] == 0 and q["zero"][0, 0] == 0.75
    assert q["codes"][0, :32].tolist() == [0] * 32
    assert np.all(o.dequantize(q["codes"], q["scale"], q["zero"], 32)[0, :32] == 0.75)
    # clipped maximum
    vals = np.array([50.0] + [float(i % 3) for i in range(31)])
    q = o.quantize(_group_input(vals), I, 4.0, 32)
    assert q["xc"][0, 0] == 4.0
    assert q["zero"][0, 0] == 0.0 and float(q["scale"][0, 0]) == 1.3330078125
    assert q["codes"][0, 0] == 3
    # fp16 rounding of the zero
    q = o.quantize(_group_input(np.array([0.1] + [0.5] * 31)), I, 1000.0, 32)
    assert float(q["zero"][0, 0]) == 0.0999755859375
    # ties round to even
    q = o.quantize(_group_input(np.array([0.0, 3.0, 1.5, 2.5, 0.5] + [1.0] * 27)), I, 1000.0, 32)
    assert q["codes"][0, 2:5].tolist() == [2, 2, 0]


def test_quantizer_golden_file_consistent():
    g = _golden("quantizer_cases.json")
    names = [c["name"] for c in g["cases"]]
    assert names == ["levels", "centered", "constant", "clipped", "fp16 zero", "tie to even"]


def test_quantizer_invariants_random():
    x = synth.bf16_to_f64(synth.bf16_bits(RNG.standard_normal((400, 128)).astype(np.float32) * 3))
    R, _ = np.linalg.qr(RNG.standard_normal((128, 128)))
    for G in (32, 64, 128):
        q = o.quantize(x, R, 5.0, G)
        c, s, z = q["codes"], q["scale"].astype(float), q["zero"].astype(float)
        assert c.min() >= 0 and c.max() <= 3
        xh = o.dequantize(c, q["scale"], q["zero"], G)
        ng = 128 // G
        err = np.abs(q["xc"] - xh).reshape(-1, ng, G)
        # half a step plus fp16 rounding slack of the zero and of the scale (x3)
        slack = np.abs(q["xc"]).reshape(-1, ng, G).max(axis=2) * 2.0 ** -10
        assert np.all(err.max(axis=2) <= s / 2 + 4 * slack + 1e-12)
        g = q["xc"].reshape(-1, ng, G)
        cg = c.reshape(-1, ng, G)
        amin = np.argmin(g, axis=2)
        amax = np.argmax(g, axis=2)
        assert np.all(np.take_along_axis(cg, amin[..., None], 2) == 0)
        assert np.all(np.take_along_axis(cg, amax[..., None], 2) == 3)


def test_quantizer_identity_is_textbook_minmax():
    # R = I and no clipping: per-token asymmetric min-max INT2 written out
    # element by element in plain Python
    x = synth.bf16_to_f64(synth.bf16_bits(RNG.standard_normal((6, 128)).astype(np.float32)))
    for G in (32, 64, 128):
        q = o.quantize(x, np.eye(128), 1e9, G)
        for n in range(x.shape[0]):
            for g in range(128 // G):
                vals = [float(v) for v in x[n, g * G:(g + 1) * G]]
                lo, hi = min(vals), max(vals)
                z = float(np.float16(lo))
                s = float(np.float16((hi - lo) / 3))
                for i, val in enumerate(vals):
                    t = (val - z) / s
                    r = math.floor(t + 0.5)
                    if t + 0.5 == r and r % 2 == 1:   # exact tie -> even
                        r -= 1
                    assert q["codes"][n, g * G + i] == min(3, max(0, r))


# ------------------------------------------------------------------ packing


def test_pack_roundtrip_and_bijection():
    c = RNG.integers(0, 4, size=(7, 16, 128)).astype(np.uint8)
    for kind in "KV":
        assert np.array_equal(o.unpack_codes(o.pack_codes(c, kind), kind), c)
        # every bit of the 512-byte area is used by exactly one code
        ones = np.full((1, 16, 128), 3, dtype=np.uint8)
        assert np.all(o.pack_codes(ones, kind) == 0xFF)


def test_pack_hand_derived_bytes():
    g = _golden("pack_bytes.json")
    for case in g["cases"]:
        c = np.zeros((16, 128), dtype=np.uint8)
        c[case["row"], case["channel"]] = case["code"]
        area = o.pack_codes(c, case["kind"])
        expect = np.zeros(512, dtype=np.uint8)
        expect[case["byte"]] = case["value"]
        assert np.array_equal(area, expect), case["derivation"]
    for case in g["meta_cases"]:
        ng = 128 // case["G"]
        s = np.zeros((16, ng), dtype=np.float16)
        z = np.zeros((16, ng), dtype=np.float16)
        s[case["row"], case["group"]] = case["scale"]
        z[case["row"], case["group"]] = case["zero"]
        area = o.pack_meta(s, z)
        assert area.shape == (64 * ng,)
        for k, v in case["bytes"].items():
            assert area[int(k)] == v
        s2, z2 = o.unpack_meta(area, case["G"])
        assert np.array_equal(s2, s) and np.array_equal(z2, z)


def test_block_sizes():
    assert [o.hist_block_bytes(G) for G in (32, 64, 128)] == [1536, 1280, 1152]
    assert [o.hist_block_bytes(G, 4) for G in (32, 64, 128)] == [2560, 2304, 2176]


# ------------------------------------------------------------- INT4 variant


def test_int4_quantizer_hand_cases():
    I = np.eye(128)
    # sixteen levels, each value its own code
    q = o.quantize(_group_input(np.tile(np.arange(16.0), 2)), I, 1000.0, 32, bits=4)
    assert q["zero"][0, 0] == 0 and q["scale"][0, 0] == 1
    assert q["codes"][0, :32].tolist() == list(range(16)) * 2
    # the INT2 quantiser on the same group spreads the range over 3 steps
    q2 = o.quantize(_group_input(np.tile(np.arange(16.0), 2)), I, 1000.0, 32)
    assert q2["scale"][0, 0] == 5 and q2["codes"][0, :16].tolist() == [0] * 3 + [1] * 5 + [2] * 5 + [3] * 3
    # ties round to even: range 0..15 gives step 1; 2.5 -> 2, 3.5 -> 4, 14.5 -> 14
    q = o.quantize(_group_input(np.array([0.0, 15.0, 2.5, 3.5, 14.5] + [1.0] * 27)), I, 1000.0, 32, bits=4)
    assert q["codes"][0, 2:5].tolist() == [2, 4, 14]
    # clipped maximum: range [0, 4] over 15 steps, fp16 step 0.26660156...
    vals = np.array([50.0] + [float(i % 3) for i in range(31)])
    q = o.quantize(_group_input(vals), I, 4.0, 32, bits=4)
    assert float(q["scale"][0, 0]) == float(np.float16(4.0 / 15.0)) == 0.2666015625
    assert q["codes"][0, 0] == 15
    # x = 1 sits at 1/0.2666015625 = 3.7509... steps -> 4; x = 2 at 7.50183 -> 8
    assert q["codes"][0, 1:4].tolist() == [0, 4, 8]
    # constant group
    q = o.quantize(_group_input(np.full(32, -0.25)), I, 1000.0, 32, bits=4)
    assert q["scale"][0, 0] == 0 and q["codes"][0, :32].tolist() == [0] * 32
    assert np.all(o.dequantize(q["codes"], q["scale"], q["zero"], 32)[0, :32] == -0.25)


def test_int4_quantizer_invariants_random():
    x = synth.bf16_to_f64(synth.bf16_bits(RNG.standard_normal((400, 128)).astype(np.float32) * 3))
    R, _ = np.linalg.qr(RNG.standard_normal((128, 128)))
    for G in (32, 64, 128):
        q = o.quantize(x, R, 5.0, G, bits=4)
        c, s = q["codes"], q["scale"].astype(float)
        assert c.min() == 0 and c.max() == 15
        xh = o.dequantize(c, q["scale"], q["zero"], G)
        ng = 128 // G
        err = np.abs(q["xc"] - xh).reshape(-1, ng, G)
        slack = np.abs(q["xc"]).reshape(-1, ng, G).max(axis=2) * 2.0 ** -10
        assert np.all(err.max(axis=2) <= s / 2 + 16 * slack + 1e-12)
        g = q["xc"].reshape(-1, ng, G)
        cg = c.reshape(-1, ng, G)
        assert np.all(np.take_along_axis(cg, np.argmin(g, axis=2)[..., None], 2) == 0)
        assert np.all(np.take_along_axis(cg, np.argmax(g, axis=2)[..., None], 2) == 15)
        # four bits quantise the same rotated values more finely than two
        q2 = o.quantize(x, R, 5.0, G)
        e4 = np.linalg.norm(q["xc"] - xh)
        e2 = np.linalg.norm(q2["xc"] - o.dequantize(q2["codes"], q2["scale"], q2["zero"], G))
        assert e4 < 0.3 * e2


def test_int4_quantizer_identity_is_textbook_minmax():
    x = synth.bf16_to_f64(synth.bf16_bits(RNG.standard_normal((6, 128)).astype(np.float32)))
    for G in (32, 128):
        q = o.quantize(x, np.eye(128), 1e9, G, bits=4)
        for n in range(x.shape[0]):
            for g in range(128 // G):
                vals = [float(v) for v in x[n, g * G:(g + 1) * G]]
                lo, hi = min(vals), max(vals)
                z = float(np.float16(lo))
                s = float(np.float16((hi - lo) / 15))
                for i, val in enumerate(vals):
                    t = (val - z) / s
                    r = math.floor(t + 0.5)
                    if t + 0.5 == r and r % 2 == 1:
                        r -= 1
                    assert q["codes"][n, g * G + i] == min(15, max(0, r))


def test_int4_pack_roundtrip_and_bijection():
    c = RNG.integers(0, 16, size=(7, 16, 128)).astype(np.uint8)
    for kind in "KV":
        area = o.pack_codes(c, kind, 4)
        assert area.shape == (7, 1024)
        assert np.array_equal(o.unpack_codes(area, kind, 4), c)
        assert np.all(o.pack_codes(np.full((1, 16, 128), 15, dtype=np.uint8), kind, 4) == 0xFF)


def test_int4_pack_hand_derived_bytes():
    g = _golden("pack_bytes_int4.json")
    for case in g["cases"]:
        c = np.zeros((16, 128), dtype=np.uint8)
        c[case["row"], case["channel"]] = case["code"]
        expect = np.zeros(1024, dtype=np.uint8)
        for k, v in case["bytes"].items():
            expect[int(k)] = v
        assert np.array_equal(o.pack_codes(c, case["kind"], 4), expect), case["derivation"]
    for case in g["dword_cases"]:
        c = np.zeros((16, 128), dtype=np.uint8)
        for row, ch, code in case["codes"]:
            c[row, ch] = code
        expect = np.zeros(1024, dtype=np.uint8)
        for k, v in case["bytes"].items():
            expect[int(k)] = v
        assert np.array_equal(o.pack_codes(c, case["kind"], 4), expect), case["derivation"]


# ------------------------------------------------------------------- layout


def test_storage_of_boundaries():
    assert o.storage_of(0, 1) == ("sink", 0)
    assert o.storage_of(15, 16) == ("sink", 15)
    assert o.storage_of(16, 17) == ("ring", 16)
    assert o.storage_of(143, 144) == ("ring", 15)
    assert o.storage_of(16, 145) == ("hist", 0)     # first token to leave the window
    assert o.storage_of(17, 145) == ("ring", 17)
    assert o.storage_of(144, 145) == ("ring", 16)   # takes the freed slot
    assert o.storage_of(31, 160) == ("hist", 15)
    assert o.storage_of(32, 161) == ("hist", 16)    # second history page
    for L in (1, 16, 17, 144, 145, 160, 161, 4096):
        kinds = [o.storage_of(p, L)[0] for p in range(L)]
        n_ring = min(128, max(0, L - 16))
        assert kinds.count("sink") == min(L, 16)
        assert kinds.count("ring") == n_ring
        assert kinds.count("hist") == max(0, L - 144)
        slots = [o.storage_of(p, L)[1] for p in range(L) if o.storage_of(p, L)[0] == "ring"]
        assert len(set(slots)) == len(slots)


def _make_cache(L_max, hkv=2, G=32, batch=1, seed=3, bits=2):
    n_hist = max(1, (max(0, L_max - 144) + 15) // 16)
    pt, npool = synth.shuffled_page_tables(seed, 0, [L_max] * batch, n_pool_pages=n_hist * batch + 3)
    bpt = synth.bf16_page_tables(batch, shuffle_seed=seed)
    return o.LayerCacheRef(hkv, G, npool, 9 * batch, pt, bpt, bits=bits)


def _rot(seed=5):
    R, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((128, 128)))
    return R


@pytest.mark.parametrize("L,bits", [(1, 2), (16, 2), (17, 2), (144, 2), (145, 2), (160, 2), (161, 2),
                                    (300, 2), (145, 4), (300, 4)])
def test_prefill_equals_token_by_token(L, bits):
    ld = synth.LayerData(21, 0, 4, 2)
    k, v = ld.cache_kv(L)
    R = _rot()
    a = _make_cache(L, bits=bits)
    a.write(R, R.T, 4.0, 3.0, k, v, [0, L], [0])
    b = _make_cache(L, bits=bits)
    for p in range(L):
        b.write(R, R.T, 4.0, 3.0, k[p:p + 1], v[p:p + 1], [0, 1], [p])
    assert np.array_equal(a.hist, b.hist)
    Ka, Va = a.gather(0, L, R, R.T)
    Kb, Vb = b.gather(0, L, R, R.T)
    assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)


def test_chunked_writes_equal_one_shot():
    L = 500
    ld = synth.LayerData(22, 0, 4, 2)
    k, v = ld.cache_kv(L)
    R = _rot(6)
    a = _make_cache(L, G=64)
    a.write(R, R, 5.0, 5.0, k, v, [0, L], [0])
    b = _make_cache(L, G=64)
    cuts = [0, 10, 150, 151, 400, 500]   # chunks longer than the window evict many ring tokens
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        b.write(R, R, 5.0, 5.0, k[lo:hi], v[lo:hi], [0, hi - lo], [lo])
    assert np.array_equal(a.hist, b.hist)
    for L_ in (L,):
        Ka, Va = a.gather(0, L_, R, R)
        Kb, Vb = b.gather(0, L_, R, R)
        assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)


def test_gather_raw_tokens_exact_and_history_close():
    L = 200
    ld = synth.LayerData(23, 0, 4, 2)
    k, v = ld.cache_kv(L)
    R = _rot(7)
    c = _make_cache(L, G=32)
    c.write(R, R, 1e4, 1e4, k, v, [0, L], [0])
    K, V = c.gather(0, L, R, R)
    kf, vf = synth.bf16_to_f64(k), synth.bf16_to_f64(v)
    raw = [p for p in range(L) if o.storage_of(p, L)[0] != "hist"]
    hist = [p for p in range(L) if o.storage_of(p, L)[0] == "hist"]
    assert np.array_equal(K[raw], kf[raw]) and np.array_equal(V[raw], vf[raw])
    # history: error of each rotated coordinate <= half a step (+ fp16 slack);
    # an orthogonal R keeps the Euclidean norm of the error
    for X, Xh in ((kf, K), (vf, V)):
        err = np.linalg.norm((X[hist] - Xh[hist]).reshape(len(hist), 2, 128), axis=2)
        q = o.quantize(X[hist].reshape(-1, 128), R, 1e4, 32)
        bound = np.sqrt(np.sum(((q["scale"].astype(float) / 2 + 0.01) ** 2) * 32, axis=1)).reshape(len(hist), 2)
        assert np.all(err <= bound)


# ------------------------------------------------------------------- decode


def _brute_attention(q, K, V, scale):
    """Plain-Python softmax attention of one head."""
    logits = [sum(q[i] * K[t][i] for i in range(len(q))) * scale for t in range(len(K))]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    tot = sum(w)
    return [sum(w[t] * V[t][i] for t in range(len(K))) / tot for i in range(len(q))]


def test_attention_brute_force_tiny():
    for L in (1, 2, 7, 20):
        q = RNG.standard_normal((4, 128))
        K = RNG.standard_normal((L, 2, 128))
        V = RNG.standard_normal((L, 2, 128))
        out = o.attention(q, K, V, 0.1)
        for h in range(4):
            ref = _brute_attention(q[h].tolist(), K[:, h // 2].tolist(), V[:, h // 2].tolist(), 0.1)
            np.testing.assert_allclose(out[h], ref, rtol=1e-12, atol=1e-12)


def _filled(L, batch=1, hkv=2, hq=8, G=32, seed=31, R=None, Rv=None, clip=(6.0, 6.0), bits=2):
    ld = synth.LayerData(seed, 0, hq, hkv)
    k, v = ld.cache_kv(L * batch)
    R = _rot(8) if R is None else R
    Rv = R if Rv is None else Rv
    c = _make_cache(L, hkv=hkv, G=G, batch=batch, seed=seed, bits=bits)
    cu = [L * i for i in range(batch + 1)]
    c.write(R, Rv, clip[0], clip[1], k, v, cu, [0] * batch)
    return c, k, v, ld.decode_q(batch), R, Rv


def test_decode_single_token_returns_v():
    c, k, v, q, R, Rv = _filled(1)
    out = o.decode_attn(c, R, Rv, q, [1], 0.088)
    vf = synth.bf16_to_f64(v)
    for h in range(8):
        assert np.array_equal(out[0, h], vf[0, h // 4])


def test_decode_equal_keys_average_values():
    L = 40
    ld = synth.LayerData(32, 0, 8, 2)
    k, v = ld.cache_kv(L)
    k[:] = k[0]
    c = _make_cache(L)
    R = np.eye(128)
    c.write(R, R, 1e4, 1e4, k, v, [0, L], [0])
    out = o.decode_attn(c, R, R, ld.decode_q(1), [L], 0.088)
    vf = synth.bf16_to_f64(v)
    for h in range(8):
        np.testing.assert_allclose(out[0, h], vf[:, h // 4].mean(axis=0), rtol=1e-12, atol=1e-12)


def test_decode_without_history_equals_bf16_decode():
    for L in (1, 16, 17, 100, 144):
        c, k, v, q, R, Rv = _filled(L)
        out = o.decode_attn(c, R, Rv, q, [L], 0.088)
        pages = np.zeros(((L + 15) // 16, 2, 2, 16, 128), dtype=np.uint16)
        for p in range(L):
            pages[p // 16, :, 0, p % 16] = k[p]
            pages[p // 16, :, 1, p % 16] = v[p]
        pt = np.arange(pages.shape[0], dtype=np.int32)[None]
        ref = o.bf16_paged_decode(q, pages, pt, [L], 0.088)
        np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_decode_lossless_history_pins_rotation_direction():
    # R = a cyclic channel shift (orthogonal, not symmetric).  Each rotated
    # group holds only the values {z, z+s, z+2s, z+3s} with fp16-exact s, z,
    # so quantisation is lossless and the INT2 decode must equal the BF16
    # decode of the same tokens: a transposed R on either side breaks this.
    L = 180
    shift = np.roll(np.eye(128), 5, axis=1)
    rng = np.random.default_rng(99)
    k = np.zeros((L, 2, 128), dtype=np.float32)
    v = np.zeros((L, 2, 128), dtype=np.float32)
    for X in (k, v):
        lv = rng.integers(0, 4, size=(L, 2, 128)).astype(np.float32)
        lv[..., 0::32] = 0
        lv[..., 1::32] = 3
        X[:] = (lv * 0.5 - 1.0) @ shift.T  # x R = levels
    kb, vb = synth.bf16_bits(k), synth.bf16_bits(v)
    c = _make_cache(L)
    c.write(shift, shift, 100.0, 100.0, kb, vb, [0, L], [0])
    q = synth.LayerData(5, 0, 8, 2).decode_q(1)
    out = o.decode_attn(c, shift, shift, q, [L], 0.088)
    pages = np.zeros(((L + 15) // 16, 2, 2, 16, 128), dtype=np.uint16)
    for p in range(L):
        pages[p // 16, :, 0, p % 16] = kb[p]
        pages[p // 16, :, 1, p % 16] = vb[p]
    ref = o.bf16_paged_decode(q, pages, np.arange(pages.shape[0], dtype=np.int32)[None], [L], 0.088)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # and the same cache read with R^T in place of R is far off
    bad = o.decode_attn(c, shift.T, shift.T, q, [L], 0.088)
    assert np.abs(bad - ref).max() > 0.1


def test_decode_mha_and_gqa_agree_when_heads_repeat():
    L = 200
    c, k, v, q, R, Rv = _filled(L, hkv=2, hq=2)
    out_mha = o.decode_attn(c, R, Rv, q, [L], 0.088)
    # GQA with 4 query heads where heads 0,1 repeat query 0 and heads 2,3 query 1
    q4 = np.repeat(q, 2, axis=1)
    out_gqa = o.decode_attn(c, R, Rv, q4, [L], 0.088)
    np.testing.assert_allclose(out_gqa[0, 0::2], out_mha[0], rtol=0, atol=0)


def test_decode_page_permutation_invariant():
    L = 260
    c, k, v, q, R, Rv = _filled(L, G=64)
    out = o.decode_attn(c, R, Rv, q, [L], 0.088)
    perm = np.random.default_rng(4).permutation(c.hist.shape[0])
    c2 = o.LayerCacheRef(2, 64, c.hist.shape[0], 9, perm[c.hist_pt], c.bf16_pt)
    c2.hist[perm] = c.hist
    c2.bf16[:] = c.bf16
    out2 = o.decode_attn(c2, R, Rv, q, [L], 0.088)
    assert np.array_equal(out, out2)


def test_decode_shared_prefix_pages():
    # two requests with the same first 176 tokens share history pages 0-1
    L = 300
    ld = synth.LayerData(41, 0, 8, 2)
    k, v = ld.cache_kv(2 * L)
    k[L:L + 176] = k[:176]
    v[L:L + 176] = v[:176]
    R = _rot(9)
    n_hist = (L - 144 + 15) // 16
    pt = np.array([np.arange(n_hist), np.r_[0, 1, np.arange(n_hist, 2 * n_hist - 2)]], dtype=np.int32)
    bpt = synth.bf16_page_tables(2)
    shared = o.LayerCacheRef(2, 32, 2 * n_hist, 18, pt, bpt)
    shared.write(R, R, 6.0, 6.0, k[:L], v[:L], [0, L], [0])
    shared.write(R, R, 6.0, 6.0, k[L:], v[L:], [0, 0, L], [0, 0])   # request 1 rewrites pages 0-1 identically
    sep = o.LayerCacheRef(2, 32, 2 * n_hist, 18,
                          np.array([np.arange(n_hist), np.arange(n_hist, 2 * n_hist)], dtype=np.int32), bpt)
    sep.write(R, R, 6.0, 6.0, k, v, [0, L, 2 * L], [0, 0])
    q = ld.decode_q(2)
    np.testing.assert_array_equal(o.decode_attn(shared, R, R, q, [L, L], 0.088),
                                  o.decode_attn(sep, R, R, q, [L, L], 0.088))


def test_decode_brute_force_with_history():
    # the whole decode (dequantise + inverse rotation + softmax) against a
    # plain-Python evaluation that reads codes bit by bit from the bytes
    L = 170
    c, k, v, q, R, Rv = _filled(L, hkv=1, hq=2, G=64, clip=(3.0, 2.5))
    out = o.decode_attn(c, R, Rv, q, [L], 0.1)
    qf = synth.bf16_to_f64(q)[0]
    kf, vf = synth.bf16_to_f64(k), synth.bf16_to_f64(v)
    LO, HI = o.LO_BIT, o.HI_BIT

    def code_at(area, kind, t, ch):
        for lane in range(64):
            a, qq = lane % 16, lane // 16
            for d in range(2):
                for u in range(8):
                    if kind == "K":
                        hits = [(a, 32 * (2 * d + u // 4) + 8 * qq + 2 * (u % 4), LO[u]),
                                (a, 32 * (2 * d + u // 4) + 8 * qq + 2 * (u % 4) + 1, HI[u])]
                    else:
                        cc, t0 = 16 * (4 * d + u // 2) + a, 4 * qq + 2 * (u % 2)
                        hits = [(t0, cc, LO[u]), (t0 + 1, cc, HI[u])]
                    for tt, c2, bit in hits:
                        if tt == t and c2 == ch:
                            word = int.from_bytes(bytes(area[8 * lane + 4 * d:8 * lane + 4 * d + 4]), "little")
                            return (word >> bit) & 3
        raise AssertionError

    def vec(kind, p):
        h = p - 16
        blk = c.hist[c.hist_pt[0, h // 16], 0]
        off = 0 if kind == "K" else 512 + 128
        meta = blk[off + 512: off + 512 + 128].view(np.float16)
        xr = []
        for ch in range(128):
            g = ch // 64
            s, z = float(meta[2 * (16 * g + h % 16)]), float(meta[2 * (16 * g + h % 16) + 1])
            xr.append(code_at(blk[off:off + 512], kind, h % 16, ch) * s + z)
        Rm = R if kind == "K" else Rv
        return [sum(xr[j] * Rm[i, j] for j in range(128)) for i in range(128)]

    Ks, Vs = [], []
    for p in range(L):
        if o.storage_of(p, L)[0] == "hist":
            Ks.append(vec("K", p))
            Vs.append(vec("V", p))
        else:
            Ks.append(kf[p, 0].tolist())
            Vs.append(vf[p, 0].tolist())
    for h in range(2):
        ref = _brute_attention(qf[h].tolist(), Ks, Vs, 0.1)
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-11, atol=1e-11)


def test_int4_decode_lossless_history_pins_rotation_direction():
    # as for INT2, with sixteen levels per group: each rotated group holds
    # only z + k s, k = 0..15, with both ends present, so INT4 storage is
    # lossless and the decode equals the BF16 decode of the same tokens
    L = 200
    shift = np.roll(np.eye(128), 9, axis=1)
    rng = np.random.default_rng(98)
    k = np.zeros((L, 2, 128), dtype=np.float32)
    v = np.zeros((L, 2, 128), dtype=np.float32)
    for X in (k, v):
        lv = rng.integers(0, 16, size=(L, 2, 128)).astype(np.float32)
        lv[..., 0::64] = 0
        lv[..., 1::64] = 15
        X[:] = (lv * 0.25 - 2.0) @ shift.T
    kb, vb = synth.bf16_bits(k), synth.bf16_bits(v)
    c = _make_cache(L, G=64, bits=4)
    c.write(shift, shift, 100.0, 100.0, kb, vb, [0, L], [0])
    q = synth.LayerData(6, 0, 8, 2).decode_q(1)
    out = o.decode_attn(c, shift, shift, q, [L], 0.088)
    pages = np.zeros(((L + 15) // 16, 2, 2, 16, 128), dtype=np.uint16)
    for p in range(L):
        pages[p // 16, :, 0, p % 16] = kb[p]
        pages[p // 16, :, 1, p % 16] = vb[p]
    ref = o.bf16_paged_decode(q, pages, np.arange(pages.shape[0], dtype=np.int32)[None], [L], 0.088)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    bad = o.decode_attn(c, shift.T, shift.T, q, [L], 0.088)
    assert np.abs(bad - ref).max() > 0.1


def test_int4_decode_brute_force_with_history():
    # INT4 decode against a plain-Python evaluation that finds each 4-bit
    # code by scanning the layout's (lane, dword, nibble) enumeration
    L = 166
    c, k, v, q, R, Rv = _filled(L, hkv=1, hq=2, G=32, clip=(3.0, 2.5), bits=4)
    out = o.decode_attn(c, R, Rv, q, [L], 0.1)
    qf = synth.bf16_to_f64(q)[0]
    kf, vf = synth.bf16_to_f64(k), synth.bf16_to_f64(v)

    def code_at(area, kind, t, ch):
        for lane in range(64):
            a, qq = lane % 16, lane // 16
            for i in range(4):
                for e in range(8):
                    if kind == "K":
                        tt, c2 = a, 32 * i + 8 * qq + 2 * (e % 4) + e // 4
                    else:
                        tt, c2 = 4 * qq + 2 * (e % 2) + e // 4, 16 * (2 * i + (e // 2) % 2) + a
                    if tt == t and c2 == ch:
                        word = int.from_bytes(bytes(area[16 * lane + 4 * i:16 * lane + 4 * i + 4]), "little")
                        return (word >> (4 * e)) & 15
        raise AssertionError

    def vec(kind, p):
        h = p - 16
        blk = c.hist[c.hist_pt[0, h // 16], 0]
        off = 0 if kind == "K" else 1024 + 256
        meta = blk[off + 1024: off + 1024 + 256].view(np.float16)
        xr = []
        for ch in range(128):
            g = ch // 32
            s, z = float(meta[2 * (16 * g + h % 16)]), float(meta[2 * (16 * g + h % 16) + 1])
            xr.append(code_at(blk[off:off + 1024], kind, h % 16, ch) * s + z)
        Rm = R if kind == "K" else Rv
        return [sum(xr[j] * Rm[i, j] for j in range(128)) for i in range(128)]

    Ks, Vs = [], []
    for p in range(L):
        if o.storage_of(p, L)[0] == "hist":
            Ks.append(vec("K", p))
            Vs.append(vec("V", p))
        else:
            Ks.append(kf[p, 0].tolist())
            Vs.append(vf[p, 0].tolist())
    for h in range(2):
        ref = _brute_attention(qf[h].tolist(), Ks, Vs, 0.1)
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-11, atol=1e-11)


def test_int4_history_closer_than_int2():
    # the same tokens stored at four bits (no clipping) decode closer to the
    # unquantised attention than at two bits
    L = 400
    outs = {}
    for bits in (2, 4):
        c, k, v, q, R, Rv = _filled(L, bits=bits, seed=33, clip=(1e4, 1e4))
        outs[bits] = o.decode_attn(c, R, Rv, q, [L], 0.088)
    kf, vf = synth.bf16_to_f64(k), synth.bf16_to_f64(v)
    ref = o.attention(synth.bf16_to_f64(q)[0], kf, vf, 0.088)
    e2 = np.abs(outs[2][0] - ref).max()
    e4 = np.abs(outs[4][0] - ref).max()
    assert e4 < 0.5 * e2


# ------------------------------------------------------- rotation variants


def test_sorted_diagonal_query_covariance_gives_hadamard_only():
    # q_n = sqrt(N lambda_n) e_n makes C_Q exactly diag(lambda); with distinct
    # descending lambda the eigenbasis is the identity (largest entry
    # positive), so OSCAR's R_K is the data-oblivious H P_br
    lam = np.sort(10.0 ** RNG.uniform(-2, 1, 128))[::-1]
    q = np.zeros((128, 1, 128))
    q[np.arange(128), 0, np.arange(128)] = np.sqrt(128 * lam)
    C = o.query_covariance(q)
    assert np.abs(C - np.diag(lam)).max() < 1e-12
    R = o.compose_rotation(o.eigenbasis(C))
    assert np.abs(R - o.hadamard_only_rotation()).max() < 1e-12
    assert np.abs(o.hadamard_only_rotation().T @ o.hadamard_only_rotation() - np.eye(128)).max() < 1e-14
    assert np.array_equal(o.identity_rotation(), np.eye(128))


def test_hadamard_only_equalises_only_diagonal_importance():
    # for a diagonal C_Q every Hadamard column sees tr(C_Q)/128; a dense C_Q
    # breaks that for H P_br but not for OSCAR's U_Q H P_br
    lam = 10.0 ** RNG.uniform(-2, 1, 128)
    Hp = o.hadamard_only_rotation()
    d = np.diag(Hp.T @ np.diag(lam) @ Hp)
    assert np.abs(d - lam.sum() / 128).max() < 1e-12
    B = np.linalg.qr(RNG.standard_normal((128, 128)))[0]
    C = B @ np.diag(lam) @ B.T
    d_h = np.diag(Hp.T @ C @ Hp)
    R = o.compose_rotation(o.eigenbasis(C))
    d_o = np.diag(R.T @ C @ R)
    assert np.abs(d_o - np.trace(C) / 128).max() < 1e-11
    assert d_h.max() / d_h.min() > 1.5


def test_logit_distortion_hand_values():
    q = np.zeros((2, 128))
    q[0, :2] = [1.0, 2.0]
    q[1, 1] = 1.0
    K = RNG.standard_normal((2, 1, 128))
    dK = np.zeros((2, 1, 128))
    dK[0, 0, :2] = [3.0, -1.0]     # head 0: (3 - 2)^2 = 1, head 1: 1
    dK[1, 0, 1] = 2.0              # head 0: 4^2 = 16, head 1: 2^2 = 4
    assert o.logit_distortion(q, K, K) == 0.0
    assert abs(o.logit_distortion(q, K, K - dK) - (1 + 1 + 16 + 4) / 4) < 1e-12
    # GQA: query heads 0, 1 read KV head 0, heads 2, 3 KV head 1
    q4 = np.zeros((4, 128))
    q4[:, 0] = [1.0, 2.0, 3.0, 4.0]
    K2 = np.zeros((1, 2, 128))
    Kh = K2.copy()
    Kh[0, 0, 0] = -1.0
    Kh[0, 1, 0] = -2.0
    assert abs(o.logit_distortion(q4, K2, Kh) - (1 + 4 + 36 + 64) / 4) < 1e-12


def test_logit_distortion_rotation_invariant():
    # (q R) . (dk R) = q . dk for orthogonal R: the diagnostic reads the same
    # in either basis, and a transposed operand breaks the identity
    R = np.linalg.qr(RNG.standard_normal((128, 128)))[0]
    q = RNG.standard_normal((8, 128))
    K = RNG.standard_normal((40, 2, 128))
    Kh = K + 0.1 * RNG.standard_normal(K.shape)
    a = o.logit_distortion(q, K, Kh)
    b = o.logit_distortion(q @ R, K @ R, Kh @ R)
    assert abs(a - b) < 1e-12 * a
    assert abs(o.logit_distortion(q @ R.T, K @ R, Kh @ R) - a) > 1e-3 * a


def test_relative_l2_hand_value():
    assert abs(o.relative_l2(np.array([3.0, 4.0]), np.array([0.0, 5.0])) - math.sqrt(10) / 5) < 1e-15


def test_identity_rotation_outliers_dominate_int2_error():
    # [nl]/[fr] §2.1: a x20 outlier channel sets the range of its group under
    # plain INT2; spreading it over the channels (any orthogonal mixing such
    # as H P_br) shrinks the per-group range and the reconstruction error
    g = np.random.default_rng(77)
    x = g.standard_normal((256, 128))
    x[:, 5] *= 20.0
    err = {}
    for name, R in (("identity", o.identity_rotation()), ("hadamard", o.hadamard_only_rotation())):
        clip = o.clip_threshold(x, R, 0.999)
        qq = o.quantize(x, R, clip, 32)
        xh = o.dequantize(qq["codes"], qq["scale"], qq["zero"], 32) @ R.T
        err[name] = o.relative_l2(xh, x)
    assert err["hadamard"] < 0.8 * err["identity"], err


# ------------------------------------------------ calibration over sequences


def test_calibration_over_sequences_pools_query_moments():
    # C_Q has no attention in it: pooling sequences equals one concatenation
    g = np.random.default_rng(41)
    seqs = [(g.standard_normal((n, 4, 128)), g.standard_normal((n, 2, 128)), g.standard_normal((n, 2, 128)))
            for n in (5, 9, 3)]
    cal = o.calibrate_sequences(seqs)
    q_all = np.concatenate([q for q, _, _ in seqs])
    assert np.abs(cal["C_Q"] - o.query_covariance(q_all)).max() < 1e-13


def test_calibration_over_single_token_sequences_closed_form():
    # a one-token sequence attends to itself only: o = v of its KV head, so
    # C_S is the mean of v v^T over sequences and query heads
    g = np.random.default_rng(42)
    hq, hkv = 4, 2
    seqs = [(g.standard_normal((1, hq, 128)), g.standard_normal((1, hkv, 128)), g.standard_normal((1, hkv, 128)))
            for _ in range(7)]
    cal = o.calibrate_sequences(seqs)
    C = np.zeros((128, 128))
    for _, _, v in seqs:
        for h in range(hq):
            x = v[0, h // (hq // hkv)]
            C += np.outer(x, x)
    assert np.abs(cal["C_S"] - C / (7 * hq)).max() < 1e-13
    # the clips cover the vectors of every sequence
    k_all = np.concatenate([k for _, k, _ in seqs]).reshape(-1, 128)
    ref = float(np.quantile(np.abs(k_all @ cal["R_K"]), 0.999, method="linear"))
    assert abs(cal["clip_K"] - ref) < 1e-12 * ref


# ------------------------------------------------------------------ extend


def _sdpa_rows(q, K, V, first_pos, sm_scale):
    """Library attention (torch's scaled_dot_product_attention, fp64, CPU):
    query row i sits at position first_pos + i and sees keys 0 .. first_pos + i.
    q [T][Hq][128], K/V [L][Hkv][128] -> [T][Hq][128]."""
    import torch
    T, hq = q.shape[0], q.shape[1]
    gqa = hq // K.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(gqa, 0)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(gqa, 0)[None]
    mask = torch.arange(K.shape[0])[None, :] <= (first_pos + torch.arange(T))[:, None]
    o_ = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sm_scale)
    return o_[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv", [(8, 2), (2, 2), (8, 1)])
def test_extend_without_prefix_is_causal_attention(hq, hkv):
    # empty prefix: the chunk attends causally to itself, textbook attention
    T = 37
    ld = synth.LayerData(31, 0, hq, hkv)
    k, v = ld.cache_kv(T)
    q = ld.decode_q(T)
    c = _make_cache(T, hkv=hkv)
    R = _rot()
    out = o.extend_attn(c, R, R.T, q, k, v, [0, T], [0], 0.088)
    ref = _sdpa_rows(o.bf16_to_f64(q), o.bf16_to_f64(k), o.bf16_to_f64(v), 0, 0.088)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_extend_lossless_prefix_equals_full_causal_attention():
    # A prefix with sink, INT2 history and recent window, quantised losslessly
    # (rotated values on the grid z + c s, see the decode pin above), so the
    # extend over the cached prefix plus the raw chunk equals plain causal
    # attention over all tokens, row by row.  Two requests with different
    # prefix lengths share one call.
    lens0, T = [180, 150], [23, 9]
    # different shifts for K and V: swapping R_K and R_V breaks the equality
    shift_k, shift_v = np.roll(np.eye(128), 5, axis=1), np.roll(np.eye(128), 9, axis=1)
    rng = np.random.default_rng(41)
    tot = [a + t for a, t in zip(lens0, T)]
    kv = []
    for shift in (shift_k, shift_v):
        lv = rng.integers(0, 4, size=(sum(tot), 2, 128)).astype(np.float32)
        lv[..., 0::32] = 0
        lv[..., 1::32] = 3
        kv.append(synth.bf16_bits((lv * 0.5 - 1.0) @ shift.T))
    k, v = kv
    q = synth.LayerData(6, 0, 8, 2).decode_q(sum(T))
    c = _make_cache(max(lens0), batch=2)
    starts = np.concatenate([[0], np.cumsum(tot)])
    pre_k = np.concatenate([k[starts[b]:starts[b] + lens0[b]] for b in range(2)])
    pre_v = np.concatenate([v[starts[b]:starts[b] + lens0[b]] for b in range(2)])
    c.write(shift_k, shift_v, 100.0, 100.0, pre_k, pre_v, [0, lens0[0], sum(lens0)], [0, 0])
    new_k = np.concatenate([k[starts[b] + lens0[b]:starts[b + 1]] for b in range(2)])
    new_v = np.concatenate([v[starts[b] + lens0[b]:starts[b + 1]] for b in range(2)])
    cu = [0, T[0], sum(T)]
    out = o.extend_attn(c, shift_k, shift_v, q, new_k, new_v, cu, lens0, 0.088)
    for b in range(2):
        K = o.bf16_to_f64(k[starts[b]:starts[b + 1]])
        V = o.bf16_to_f64(v[starts[b]:starts[b + 1]])
        ref = _sdpa_rows(o.bf16_to_f64(q[cu[b]:cu[b + 1]]), K, V, lens0[b], 0.088)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=1e-12, atol=1e-12)


def test_extend_single_token_short_prefix_equals_decode_after_append():
    # no history involved (L0 + 1 <= 144): one new token equals the decode of
    # the cache after that token is appended
    for L0 in (0, 15, 16, 100, 143):
        c, k, v, q, R, Rv = _filled(L0 + 1)
        pre = _make_cache(L0 + 1)
        pre.write(R, Rv, 4.0, 3.0, k[:L0], v[:L0], [0, L0], [0])
        out = o.extend_attn(pre, R, Rv, q, k[L0:L0 + 1], v[L0:L0 + 1], [0, 1], [L0], 0.088)
        ref = o.decode_attn(c, R, Rv, q, [L0 + 1], 0.088)
        np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_extend_selected_rows_equal_full_rows():
    prefix, T = 170, 21
    c, k, v, q, R, Rv = _filled(prefix + T)
    pre = _make_cache(prefix + T)
    pre.write(R, Rv, 6.0, 6.0, k[:prefix], v[:prefix], [0, prefix], [0])
    qs = synth.LayerData(8, 0, 8, 2).decode_q(T)
    full = o.extend_attn(pre, R, Rv, qs, k[prefix:], v[prefix:], [0, T], [prefix], 0.088)
    rows = [20, 0, 7]
    part = o.extend_attn(pre, R, Rv, qs, k[prefix:], v[prefix:], [0, T], [prefix], 0.088, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


# ------------------------------------------------- pins added for the gaps


def test_bf16_to_f64_fixed_values():
    # bf16 = the top 16 bits of an IEEE binary32: sign, 8 exponent bits
    # (bias 127), 7 fraction bits; values by hand from that definition
    cases = {
        0x3F80: 1.0,                      # 0 01111111 0000000
        0xC000: -2.0,                     # 1 10000000 0000000
        0x4049: 2.0 * (1 + 73 / 128),     # 0 10000000 1001001 = 3.140625
        0x0001: 2.0 ** -133,              # smallest subnormal: 2^-126 * 2^-7
        0x0080: 2.0 ** -126,              # smallest normal
        0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,  # largest finite
        0x3E00: 0.125,                    # 0 01111100 0000000
        0xBF40: -0.75,                    # 1 01111110 1000000
    }
    got = o.bf16_to_f64(np.array(list(cases), dtype=np.uint16))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    z = o.bf16_to_f64(np.array([0x8000, 0x7F80, 0xFF80], dtype=np.uint16))
    assert z[0] == 0.0 and math.copysign(1.0, z[0]) < 0
    assert z[1] == math.inf and z[2] == -math.inf


def test_bf16_paged_decode_follows_page_table():
    # the request's pages sit at permuted positions of a pool that also holds
    # decoy pages; the last page is partial, so which physical page is last
    # matters too.  The result must be attention over the tokens in logical
    # order (gathered here by hand), and reading the pool in its own order or
    # ignoring the partial page must differ from it.
    rng = np.random.default_rng(77)
    L, hq, hkv = 75, 4, 2
    n_log = (L + 15) // 16                      # 5 logical pages, last holds 11 rows
    pool = synth.bf16_bits(rng.standard_normal((12, hkv, 2, 16, 128)).astype(np.float32))
    perm = np.array([9, 2, 11, 0, 6], dtype=np.int32)
    pt = np.full((1, 8), -1, dtype=np.int32)
    pt[0, :n_log] = perm
    q = synth.bf16_bits(rng.standard_normal((1, hq, 128)).astype(np.float32))
    got = o.bf16_paged_decode(q, pool, pt, [L], 0.088)
    # by hand: token p is row p % 16 of page perm[p // 16]
    K = np.empty((L, hkv, 128))
    V = np.empty((L, hkv, 128))
    for p in range(L):
        for h in range(hkv):
            K[p, h] = synth.bf16_to_f64(pool[perm[p // 16], h, 0, p % 16])
            V[p, h] = synth.bf16_to_f64(pool[perm[p // 16], h, 1, p % 16])
    qf = synth.bf16_to_f64(q[0])
    for h in range(hq):
        g = h // (hq // hkv)
        logits = [float(np.dot(qf[h], K[p, g])) * 0.088 for p in range(L)]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        ref = sum(w[p] * V[p, g] for p in range(L)) / sum(w)
        np.testing.assert_allclose(got[0, h], ref, rtol=1e-12, atol=1e-12)
    # an identity table over the same pool gives a different answer
    ident = o.bf16_paged_decode(q, pool, np.arange(8, dtype=np.int32)[None], [L], 0.088)
    assert np.abs(ident - got).max() > 1e-3
    # the permuted table equals the identity table over a pool permuted the same way
    pool2 = pool.copy()
    pool2[:n_log] = pool[perm]
    same = o.bf16_paged_decode(q, pool2, np.arange(8, dtype=np.int32)[None], [L], 0.088)
    np.testing.assert_allclose(same, got, rtol=1e-13, atol=1e-13)


def test_calibrate_clip_wiring():
    # clip_K is the 0.999 quantile (type 7) of |k R_K| and clip_V that of
    # |v R_V| ([nl]/[fr] section 2.2.A: one clip per layer and tensor from
    # the rotated calibration values).  V is drawn at three times the scale
    # of K, so a swap of k and v, or of R_K and R_V, gives other numbers.
    ld = synth.LayerData(31, 0, 4, 2)
    qb, kb, vb = ld.calibration(300)
    q, k = o.bf16_to_f64(qb), o.bf16_to_f64(kb)
    v = 3.0 * o.bf16_to_f64(vb)
    cal = o.calibrate(q, k, v)

    def q999(x):
        # type 7 by hand: sorted values, h = (n - 1) p, linear interpolation
        s = np.sort(np.abs(x).ravel())
        h = (s.size - 1) * 0.999
        f = int(math.floor(h))
        return s[f] + (h - f) * (s[min(f + 1, s.size - 1)] - s[f])

    kr = k.reshape(-1, 128) @ cal["R_K"]
    vr = v.reshape(-1, 128) @ cal["R_V"]
    assert abs(cal["clip_K"] - q999(kr)) <= 1e-12 * q999(kr)
    assert abs(cal["clip_V"] - q999(vr)) <= 1e-12 * q999(vr)
    # the alternatives a wiring mistake would produce are far from these
    assert abs(q999(k.reshape(-1, 128) @ cal["R_V"]) - cal["clip_K"]) > 1e-2 * cal["clip_K"]
    assert abs(q999(v.reshape(-1, 128) @ cal["R_K"]) - cal["clip_V"]) > 1e-2 * cal["clip_V"]
    assert cal["clip_V"] > 2.0 * cal["clip_K"]


# ---- per-KV-head rotations (an extension of the per-layer rule): each head
# must behave exactly as a one-head layer with that head's R and clip

def _one_head_cache(ref, h, L):
    """A one-head cache with request 0's page tables of ref."""
    return o.LayerCacheRef(1, ref.G, ref.hist.shape[0], ref.bf16.shape[0], ref.hist_pt, ref.bf16_pt, bits=ref.bits)


@pytest.mark.parametrize("bits", [2, 4])
def test_per_head_rotation_with_equal_heads_matches_shared(bits):
    L, hkv, hq = 400, 2, 8
    ld = synth.LayerData(41, 0, hq, hkv)
    k, v = ld.cache_kv(L)
    R, Rv = _rot(11), _rot(12)
    a = _make_cache(L, hkv=hkv, G=64, bits=bits)
    a.write(R, Rv, 4.0, 3.0, k, v, [0, L], [0])
    b = _make_cache(L, hkv=hkv, G=64, bits=bits)
    b.write(np.stack([R, R]), np.stack([Rv, Rv]), [4.0, 4.0], [3.0, 3.0], k, v, [0, L], [0])
    assert np.array_equal(a.hist, b.hist) and np.array_equal(a.bf16, b.bf16)
    q = ld.decode_q(1)
    assert np.array_equal(o.decode_attn(a, R, Rv, q, [L], 0.1), o.decode_attn(b, np.stack([R, R]),
                                                                               np.stack([Rv, Rv]), q, [L], 0.1))


@pytest.mark.parametrize("bits", [2, 4])
def test_per_head_rotation_is_each_head_as_its_own_layer(bits):
    # heads with different R and clips: head h's bytes and decode equal those
    # of a one-head layer that holds only head h's tokens, written with the
    # shared (per-layer) rule and R[h], clip[h]
    L, hkv, hq = 420, 3, 6
    gqa = hq // hkv
    ld = synth.LayerData(42, 0, hq, hkv)
    k, v = ld.cache_kv(L)
    RK = np.stack([_rot(20 + h) for h in range(hkv)])
    RV = np.stack([_rot(30 + h) for h in range(hkv)])
    ck, cv = [3.0, 5.0, 7.0], [2.5, 4.0, 6.5]
    ref = _make_cache(L, hkv=hkv, G=32, bits=bits)
    ref.write(RK, RV, ck, cv, k, v, [0, L], [0])
    q = ld.decode_q(1)
    out = o.decode_attn(ref, RK, RV, q, [L], 0.09)
    for h in range(hkv):
        one = _one_head_cache(ref, h, L)
        one.write(RK[h], RV[h], ck[h], cv[h], k[:, h:h + 1], v[:, h:h + 1], [0, L], [0])
        assert np.array_equal(one.hist[:, 0], ref.hist[:, h])
        assert np.array_equal(one.bf16[:, 0], ref.bf16[:, h])
        exp = o.decode_attn(one, RK[h], RV[h], q[:, h * gqa:(h + 1) * gqa], [L], 0.09)
        assert np.array_equal(out[:, h * gqa:(h + 1) * gqa], exp)
    # and another head's R would not do: head 1 written with R[0] differs
    wrong = _one_head_cache(ref, 1, L)
    wrong.write(RK[0], RV[0], ck[1], cv[1], k[:, 1:2], v[:, 1:2], [0, L], [0])
    assert not np.array_equal(wrong.hist[:, 0], ref.hist[:, 1])


def test_per_head_extend_is_each_head_as_its_own_layer():
    L0, n, hkv, hq = 300, 7, 2, 4
    gqa = hq // hkv
    ld = synth.LayerData(43, 0, hq, hkv)
    k, v = ld.cache_kv(L0 + n)
    RK = np.stack([_rot(50 + h) for h in range(hkv)])
    RV = np.stack([_rot(60 + h) for h in range(hkv)])
    ck, cv = [4.0, 6.0], [3.0, 5.0]
    ref = _make_cache(L0 + n, hkv=hkv, G=64)
    ref.write(RK, RV, ck, cv, k[:L0], v[:L0], [0, L0], [0])
    q = ld.decode_q(n)
    out = o.extend_attn(ref, RK, RV, q, k[L0:], v[L0:], [0, n], [L0], 0.1)
    for h in range(hkv):
        one = _one_head_cache(ref, h, L0)
        one.write(RK[h], RV[h], ck[h], cv[h], k[:L0, h:h + 1], v[:L0, h:h + 1], [0, L0], [0])
        exp = o.extend_attn(one, RK[h], RV[h], q[:, h * gqa:(h + 1) * gqa], k[L0:, h:h + 1], v[L0:, h:h + 1],
                            [0, n], [L0], 0.1)
        assert np.array_equal(out[:, h * gqa:(h + 1) * gqa], exp)


def test_calibrate_per_head_one_kv_head_is_the_layer_rule():
    ld = synth.LayerData(44, 0, 4, 1)
    q, k, v = (synth.bf16_to_f64(x) for x in ld.calibration(96))
    a = o.calibrate(q, k, v)
    b = o.calibrate_per_head(q, k, v)
    assert np.allclose(b["R_K"][0], a["R_K"], atol=1e-12) and np.allclose(b["R_V"][0], a["R_V"], atol=1e-12)
    assert b["clip_K"][0] == pytest.approx(a["clip_K"], rel=1e-13)
    assert b["clip_V"][0] == pytest.approx(a["clip_V"], rel=1e-13)


def test_calibrate_per_head_uses_each_groups_queries_and_vectors():
    # two KV heads, two query heads each.  Group 0's queries carry most of
    # their energy in channel 3, group 1's in channel 70: the leading
    # eigenvector of head h's C_Q is e_3 / e_70, so R_K[h] (H P_br)^T has that
    # first column.  KV head 1's vectors are three times head 0's: with equal
    # R_K (queries of equal moments) its clip is exactly three times larger.
    rng = np.random.default_rng(7)
    N = 64
    q = rng.standard_normal((N, 4, 128)) * 0.1
    q[:, 0:2, 3] += rng.standard_normal((N, 2)) * 5.0
    q[:, 2:4, 70] += rng.standard_normal((N, 2)) * 5.0
    k0 = rng.standard_normal((N, 1, 128))
    k = np.concatenate([k0, 3.0 * k0], axis=1)
    v = rng.standard_normal((N, 2, 128))
    c = o.calibrate_per_head(q, k, v)
    HP = o.hadamard() @ o.bitrev_permutation()
    for h, ch in ((0, 3), (1, 70)):
        U = c["R_K"][h] @ HP.T
        assert np.argmax(np.abs(U[:, 0])) == ch and U[ch, 0] > 0.99
    # equal query moments for both groups: equal R_K, clips in ratio 3
    q2 = q.copy()
    q2[:, 2:4] = q2[:, 0:2]
    c2 = o.calibrate_per_head(q2, k, v)
    assert np.allclose(c2["R_K"][0], c2["R_K"][1], atol=1e-12)
    assert c2["clip_K"][1] == pytest.approx(3.0 * c2["clip_K"][0], rel=1e-12)
    # C_S of a group comes from its own outputs: with V of head 1 zero, its
    # outputs are zero and every head-1 moment vanishes (R_V[1] is then the
    # eigenbasis of the zero matrix, the identity order), head 0 unaffected
    v3 = v.copy()
    v3[:, 1] = 0.0
    c3 = o.calibrate_per_head(q, k, v3)
    assert np.allclose(c3["R_V"][0], c["R_V"][0], atol=1e-12)
    assert c3["clip_V"][1] == 0.0
