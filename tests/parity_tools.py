"""Helpers of the GPU parity tests: build seeded scenarios on both sides and
compare results under the tolerances of the workload's specification.

Write parity (two levels):
  1. fp16 scale and zero equal the oracle's, except where the GPU's value is
     the fp16 rounding of some value within the fp32 error bound of the
     kernel of the oracle's unrounded one (one fp16 step across a nearby
     midpoint in general; several steps only near zero, where fp16 steps
     shrink below the bound).  The kernel rotates with
     exact fp16 x fp16 products summed in fp32: R = R_hi + 2^-11 R_lo with
     both parts fp16 (R carried to 2^-22 relative, i.e. 4u), the x R_hi and
     x R_lo sums of 128 products each accumulated in fp32, and one fused
     multiply-add joining them; so each rotated value carries at most
     (n+6) u sum_i |x_i R_ij| of error (n = 128, u = 2^-24; Higham,
     "Accuracy and Stability of Numerical Algorithms", section 3.1: n u for
     the sum, 4u for R's representation, one rounding for the join, one
     more covering the x R_lo sum); the zero inherits that bound, the scale
     (max - min)/3 a third of two of them plus two roundings;
  2. codes equal the oracle's codes recomputed with the GPU's scale and zero,
     except where the oracle's t = (xc - z)/s lies within 1e-4 code units of
     a rounding boundary k + 1/2; at most 1e-5 of all codes may differ.
INT4 history (15 steps per group instead of 3): the same rules with the
scale's bound divided by 15 (the kernel multiplies by fp32(1/15), which
carries one more rounding of up to one ulp than fp32(1/3): three roundings
of (max - min)/15 instead of two) and a code band 5 times wider, since a
step 5 times smaller turns the same rotation error into 5 times as many
code units.
Decode parity: max |gpu - oracle| <= 2e-2 and ||gpu - oracle||_2 /
||oracle||_2 <= 5e-3 over all (request, head, channel).
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import oscar_ref as o

ABS_TOL = 2e-2
REL_L2_TOL = 5e-3
CODE_BAND = 1e-4
CODE_RATE = 1e-5
ROT_BOUND = (128 + 6) * 2.0 ** -24


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_pool_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def random_rotation(seed: int) -> np.ndarray:
    R, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((128, 128)))
    return R


def calibrated(ld: synth.LayerData, n_cal: int = 2048):
    """Oracle calibration of a layer; clips rounded to fp32 (what the kernels use)."""
    qc, kc, vc = ld.calibration(n_cal)
    cal = o.calibrate(o.bf16_to_f64(qc), o.bf16_to_f64(kc), o.bf16_to_f64(vc))
    return cal["R_K"], cal["R_V"], float(np.float32(cal["clip_K"])), float(np.float32(cal["clip_V"]))


def decode_error(gpu: np.ndarray, ref: np.ndarray):
    d = gpu.astype(np.float64) - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))


def assert_decode_close(gpu: np.ndarray, ref: np.ndarray, what: str = "decode"):
    mx, rel = decode_error(gpu, ref)
    assert mx <= ABS_TOL and rel <= REL_L2_TOL, f"{what}: max abs {mx:.3e}, rel L2 {rel:.3e}"
    return mx, rel


def _f16_neighbours_ok(gpu: np.ndarray, ref: np.ndarray, unrounded: np.ndarray, tol: np.ndarray) -> np.ndarray:
    """True where gpu == ref, or gpu is the fp16 rounding of some value within
    tol of the unrounded fp64 one, i.e. lies between the roundings of
    unrounded - tol and unrounded + tol.  Where tol is below half an fp16
    step this is the adjacent value across a midpoint within tol; near zero
    (fp16 steps of 2^-24) the kernel's rotation error can span several."""
    g = gpu.astype(np.float16)
    r = ref.astype(np.float16)
    same = g.view(np.uint16) == r.view(np.uint16)
    lo = o.f16_round(unrounded - tol).astype(np.float64)
    hi = o.f16_round(unrounded + tol).astype(np.float64)
    gv = g.astype(np.float64)
    return same | ((gv >= lo) & (gv <= hi))


def compare_history(gpu_hist: np.ndarray, hist_pt: np.ndarray, tokens_k, tokens_v, lens,
                    R_K, R_V, clip_k, clip_v, G: int, positions=None, bits: int = 2) -> dict:
    """Two-level comparison of every history row of every request.

    tokens_k/v[b]: bf16 bits [L_b][Hkv][128] of request b (all positions).
    R_K / R_V with clip_k / clip_v: the layer's rotation and clip, or one per
    KV head ([Hkv][128][128] and [Hkv]).
    positions[b] (optional): subset of history positions to check.
    bits: code width of the pool (2 or 4).
    """
    steps = float(o.levels(bits))
    band = CODE_BAND * steps / 3.0
    n_round = 2 if bits == 2 else 3
    stats = {"codes": 0, "raw_code_mismatch": 0, "code_out_of_band": 0, "meta": 0,
             "meta_differ": 0, "meta_out_of_tol": 0}
    hkv = gpu_hist.shape[1]
    for b, L in enumerate(lens):
        hist_p = np.arange(o.N_SINK, max(o.N_SINK, L - o.N_RECENT))
        if positions is not None:
            hist_p = np.asarray(positions[b])
        if hist_p.size == 0:
            continue
        hidx = hist_p - o.N_SINK
        pids = hist_pt[b, hidx // o.PAGE]
        rows = hidx % o.PAGE
        for kind, toks, R_all, clip_all in (("K", tokens_k[b], R_K, clip_k), ("V", tokens_v[b], R_V, clip_v)):
            for h in range(hkv):
                R, clip = o.head_rotation(R_all, clip_all, h)  # the layer's, or head h's own
                x = o.bf16_to_f64(toks[hist_p, h, :])
                q = o.quantize(x, R, clip, G, bits)
                areas = o.split_block(gpu_hist[pids, h], G, bits)
                codes_all = o.unpack_codes(areas[kind.lower() + "_codes"], kind, bits)   # [n][16][128]
                s_all, z_all = o.unpack_meta(areas[kind.lower() + "_meta"], G)
                ar = np.arange(len(rows))
                gc, gs, gz = codes_all[ar, rows], s_all[ar, rows], z_all[ar, rows]
                ng = 128 // G
                xg = q["xc"].reshape(-1, ng, G)
                lo, hi = xg.min(axis=2), xg.max(axis=2)
                err = (ROT_BOUND * (np.abs(x) @ np.abs(R))).reshape(-1, ng, G).max(axis=2)
                u = 2.0 ** -24
                ok_z = _f16_neighbours_ok(gz, q["zero"], lo, err)
                ok_s = _f16_neighbours_ok(gs, q["scale"], (hi - lo) / steps,
                                          (2 * err + u * (hi - lo)) / steps + (n_round - 1) * u * (hi - lo) / steps)
                stats["meta"] += 2 * gs.size
                stats["meta_differ"] += int((gs != q["scale"]).sum() + (gz != q["zero"]).sum())
                stats["meta_out_of_tol"] += int((~ok_s).sum() + (~ok_z).sum())
                ref_codes, t = o.codes_from_meta(q["xc"], gs, gz, G, bits)
                diff = gc != ref_codes
                frac = t - np.floor(t)
                near = np.abs(frac - 0.5) < band
                stats["codes"] += gc.size
                stats["raw_code_mismatch"] += int((gc != q["codes"]).sum())
                stats["code_out_of_band"] += int((diff & ~np.nan_to_num(near, nan=False)).sum())
                stats.setdefault("code_in_band", 0)
                stats["code_in_band"] += int((diff & np.nan_to_num(near, nan=False)).sum())
    return stats


META_RATE = 1e-3


def assert_history_ok(stats: dict):
    """No meta outside the midpoint rule, no code flip outside the 1e-4 band,
    in-band flips at a rate <= 1e-5 (at least one allowed in small cases),
    and at most 1e-3 of the fp16 scales and zeros differing from the
    oracle's at all (at least two allowed in small cases): the midpoint
    rule admits a wide window near zero, this ceiling bounds how often it
    may be used."""
    assert stats["meta_out_of_tol"] == 0, stats
    assert stats["meta_differ"] <= max(2, META_RATE * stats["meta"]), stats
    assert stats["code_out_of_band"] == 0, stats
    assert stats.get("code_in_band", 0) <= max(1, CODE_RATE * stats["codes"]), stats


class Scenario:
    """Seeded requests written by the oracle (numpy pools) with shuffled page tables."""

    def __init__(self, seed: int, hq: int, hkv: int, G: int, lens, rot="random", n_cal=2048, layer=0,
                 spare_pages=3, dense_q=False, bits=2):
        self.seed, self.hq, self.hkv, self.G, self.bits = seed, hq, hkv, G, bits
        self.lens = [int(x) for x in lens]
        self.ld = synth.LayerData(seed, layer, hq, hkv, dense_q=dense_q)
        if rot == "calibrated":
            self.R_K, self.R_V, self.clip_k, self.clip_v = calibrated(self.ld, n_cal)
        elif rot in ("hadamard", "identity"):
            # the pages' data-oblivious comparisons: one fixed R for K and V,
            # clips by the same quantile rule from the calibration tokens
            R = o.hadamard_only_rotation() if rot == "hadamard" else o.identity_rotation()
            _, kc, vc = self.ld.calibration(n_cal)
            self.R_K = self.R_V = R
            self.clip_k = float(np.float32(o.clip_threshold(o.bf16_to_f64(kc), R)))
            self.clip_v = float(np.float32(o.clip_threshold(o.bf16_to_f64(vc), R)))
        elif rot == "per_head":
            # a random rotation and a clip of its own for every KV head
            self.R_K = np.stack([random_rotation(seed + 10 * h) for h in range(hkv)])
            self.R_V = np.stack([random_rotation(seed + 10 * h + 1) for h in range(hkv)])
            self.clip_k = [4.5 + 0.75 * h for h in range(hkv)]
            self.clip_v = [3.5 + 0.5 * h for h in range(hkv)]
        elif rot == "per_head_calibrated":
            qc, kc, vc = self.ld.calibration(n_cal)
            cal = o.calibrate_per_head(*(o.bf16_to_f64(x) for x in (qc, kc, vc)))
            self.R_K, self.R_V = cal["R_K"], cal["R_V"]
            self.clip_k = [float(np.float32(c)) for c in cal["clip_K"]]
            self.clip_v = [float(np.float32(c)) for c in cal["clip_V"]]
        else:
            self.R_K, self.R_V = random_rotation(seed), random_rotation(seed + 1)
            self.clip_k = self.clip_v = 6.0
        total = sum(self.lens)
        k, v = self.ld.cache_kv(total)
        cu = np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32)
        self.k, self.v, self.cu = k, v, cu
        self.tok_k = [k[cu[b]:cu[b + 1]] for b in range(len(self.lens))]
        self.tok_v = [v[cu[b]:cu[b + 1]] for b in range(len(self.lens))]
        need = sum(synth.hist_pages_needed(L) for L in self.lens)
        self.hist_pt, self.n_hist_pages = synth.shuffled_page_tables(seed, layer, self.lens,
                                                                     n_pool_pages=need + spare_pages)
        self.bf16_pt = synth.bf16_page_tables(len(self.lens), shuffle_seed=seed + 7)
        self.n_bf16_pages = 9 * len(self.lens)
        self.q = self.ld.decode_q(len(self.lens))

    def oracle_cache(self, chunks=None) -> o.LayerCacheRef:
        ref = o.LayerCacheRef(self.hkv, self.G, self.n_hist_pages, self.n_bf16_pages, self.hist_pt, self.bf16_pt,
                              bits=self.bits)
        for cu, lb, k, v in self.write_calls(chunks):
            ref.write(self.R_K, self.R_V, self.clip_k, self.clip_v, k, v, cu, lb)
        return ref

    def write_calls(self, chunks=None):
        """Write calls (cu_new, len_before, k rows, v rows).  chunks: list of
        cut lists per call shared by all requests (positions), default one call."""
        if chunks is None:
            return [(self.cu, np.zeros(len(self.lens), np.int32), self.k, self.v)]
        calls = []
        for lo, hi in zip(chunks[:-1], chunks[1:]):
            ks, vs, cu, lb = [], [], [0], []
            for b, L in enumerate(self.lens):
                a, e = min(lo, L), min(hi, L)
                ks.append(self.tok_k[b][a:e])
                vs.append(self.tok_v[b][a:e])
                cu.append(cu[-1] + (e - a))
                lb.append(a)
            calls.append((np.array(cu, np.int32), np.array(lb, np.int32), np.concatenate(ks), np.concatenate(vs)))
        return calls

    def oracle_decode(self, ref: o.LayerCacheRef, sm_scale=None) -> np.ndarray:
        sm_scale = sm_scale or 1.0 / np.sqrt(128)
        return o.decode_attn(ref, self.R_K, self.R_V, self.q, self.lens, sm_scale)
