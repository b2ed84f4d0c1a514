"""The pages' rotation comparison through the same kernels: OSCAR's
calibrated R = U H P_br against the data-oblivious Hadamard-only R = H P_br
(QuaRot-style) and the identity (plain INT2) ([abs]; [nl]/[fr] §2.1).

Each variant is parity-checked like any other rotation (GPU write against
the oracle's codes and meta, GPU decode over the oracle-written cache), its
clip from the library's oscar_clip_threshold against the oracle's, and its
distortion reported: the query-weighted logit distortion E[(q . dk)^2] of the
history keys over 64 held-out queries, the relative error of the history
values, and the GPU decode output against attention over the unquantised
cache.  The workload is the single-layer 4096-token shape (8 query / 2 KV
heads, G 32), with the default diagonal query covariance and with a dense
one (query channels correlated through a random orthogonal basis).
"""
import json
import math

import numpy as np
import pytest
import torch

import synth
from oracle import oscar_ref as o
from tests.parity_tools import Scenario, assert_decode_close, assert_history_ok, compare_history, to_dev_bf16
from tests.test_gpu_parity import gpu_cache, gpu_decode, gpu_rotations, gpu_write

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def oscar():
    import bit_rotated_kv_oscar_amd as m
    return m


@pytest.mark.parametrize("dense", [False, True])
def test_rotation_variants(oscar, dense):
    results = {}
    for rot in ("calibrated", "hadamard", "identity"):
        print(f"variant {rot} dense_q={dense}", flush=True)
        sc = Scenario(900 + int(dense), 8, 2, 32, [4096], rot=rot, dense_q=dense)
        if rot != "calibrated":
            _, kc, vc = sc.ld.calibration(2048)
            R = torch.from_numpy(sc.R_K)
            ck = oscar.clip_threshold(to_dev_bf16(kc), R)
            cv = oscar.clip_threshold(to_dev_bf16(vc), R)
            assert abs(ck - sc.clip_k) <= 1e-6 * sc.clip_k and abs(cv - sc.clip_v) <= 1e-6 * sc.clip_v
        ref = sc.oracle_cache()
        # write parity
        cache = gpu_cache(oscar, sc)
        rk, rv = gpu_rotations(oscar, sc)
        gpu_write(oscar, sc, cache, rk, rv)
        assert int(cache.status.item()) == 0
        stats = compare_history(cache.hist.cpu().numpy(), sc.hist_pt, sc.tok_k, sc.tok_v, sc.lens,
                                sc.R_K, sc.R_V, sc.clip_k, sc.clip_v, sc.G)
        assert_history_ok(stats)
        # decode parity over the oracle-written cache
        cache_ref = gpu_cache(oscar, sc, hist=ref.hist, bf16=ref.bf16)
        out = gpu_decode(oscar, sc, cache_ref, rk, rv)
        assert_decode_close(out, sc.oracle_decode(ref), f"decode ({rot})")
        # distortion of the history tokens and of the output
        L = sc.lens[0]
        K, V = ref.gather(0, L, sc.R_K, sc.R_V)
        Kx, Vx = o.bf16_to_f64(sc.tok_k[0]), o.bf16_to_f64(sc.tok_v[0])
        hist = slice(o.N_SINK, L - o.N_RECENT)
        qe = o.bf16_to_f64(sc.ld.decode_q(64, stream=synth.S_EVAL_Q))
        dist = float(np.mean([o.logit_distortion(qe[i], Kx[hist], K[hist]) for i in range(qe.shape[0])]))
        exact = o.attention(o.bf16_to_f64(sc.q)[0], Kx, Vx, SCALE)
        results[rot] = {"clip_k": round(sc.clip_k, 4), "clip_v": round(sc.clip_v, 4),
                        "logit_distortion": round(dist, 6),
                        "k_rel_err": round(o.relative_l2(K[hist], Kx[hist]), 5),
                        "v_rel_err": round(o.relative_l2(V[hist], Vx[hist]), 5),
                        "decode_rel_err_vs_unquantised": round(o.relative_l2(out[0], exact), 5)}
    print("VARIANTS " + json.dumps({"dense_q": dense, "results": results}), flush=True)
    # the outlier channels (x20) set the range of their groups without a
    # rotation: plain INT2 reconstructs the keys worst ([nl]/[fr] §2.1)
    assert results["identity"]["k_rel_err"] > results["hadamard"]["k_rel_err"]
    assert results["identity"]["k_rel_err"] > results["calibrated"]["k_rel_err"]
