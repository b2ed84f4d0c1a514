"""Plain fp64 CPU oracle of the OSCAR KV write and mixed-precision decode.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the GPU library and
imports nothing from it; it is slow and written to be checked by eye.

Sources (cited by page and section):
  [abs] arXiv:2605.17757 v2 abstract ("OSCAR: Offline Spectral
        Covariance-Aware Rotation for 2-bit KV Cache Quantization");
  [nl]  gist.science/nl technical summary, sections 1-2;
  [fr]  gist.science/fr technical summary, sections 1-2.

Readings where the pages are silent or garbled (each is listed in the design
notes of this repository):
  * row vectors: x_rot = x R, inverse x_rot R^T;
  * C_Q is the uncentred mean outer product q q^T, pooled over all query heads
    of the layer (the pages print "q_n^T q_n", which as written is a scalar);
  * S in C_S holds causal softmax probabilities (scale 1/sqrt(128)); query
    head h reads KV head h // (Hq/Hkv); C_S is pooled over query heads;
  * eigenvalues descending; each eigenvector's largest-|entry| positive
    (lowest index on ties);
  * H is the Sylvester Hadamard matrix divided by sqrt(128); P_br[i][j] = 1
    iff i = bitrev7(j);
  * one symmetric clip per layer and tensor: the 0.999 quantile (linear
    interpolation, "type 7") of |x R| over calibration tokens, heads and
    channels;
  * per-layer R and clip, as the pages fix them; per-KV-head R and clip is
    an optional extension, the same rules applied to each KV head's own
    data (its query heads' moments, its vectors' quantile);
  * clip first, then per-token groups of G consecutive rotated channels,
    asymmetric min-max INT2 with fp16 scale and zero, codes from the stored
    (fp16-rounded) scale and zero, round half to even, all codes 0 when the
    fp16 scale is 0; the INT4 variant is the same with 16 levels
    (scale = (max - min)/15), the bit width being the only difference;
  * sink = first 16 tokens, recent = last 128 tokens (exact sliding window),
    both raw bf16 and unrotated; history in between;
  * decode: one query per request over all cached tokens, no mask, fp64;
  * extend: new tokens see the cached prefix as it stands plus the chunk's
    own earlier tokens at bf16 (the chunk is written afterwards), fp64.
"""
from __future__ import annotations

import numpy as np

D = 128
PAGE = 16
N_SINK = 16
N_RECENT = 128
BF16_PAGES_PER_REQ = 9


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_to_f64(u) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_round(x) -> np.ndarray:
    """Round float64 to the nearest fp16 (ties to even), returned as float16."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


# --------------------------------------------------------------------------
# the fixed factors of the rotation  ([nl] §2.2.A, [fr] §2.2.A.3)
# --------------------------------------------------------------------------

def hadamard(n: int = D) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix: H[i][j] = (-1)^popcount(i&j)/sqrt(n).

    [nl]/[fr] §2.2.A: the Hadamard factor equalises the importance metric
    over channels and spreads outlier energy.
    """
    i = np.arange(n)
    parity = np.zeros((n, n), dtype=np.int64)
    anded = i[:, None] & i[None, :]
    for b in range(int(np.log2(n))):
        parity ^= (anded >> b) & 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(n)


def bitrev(i: int, bits: int = 7) -> int:
    """Reverse the low `bits` bits of i."""
    r = 0
    for _ in range(bits):
        r = (r << 1) | (i & 1)
        i >>= 1
    return r


def bitrev_permutation(n: int = D) -> np.ndarray:
    """P_br with P[i][j] = 1 iff i = bitrev(j) ([nl]/[fr] §2.2.A: interleaves
    high- and low-variance channels so every quantisation group sees a
    balanced range)."""
    bits = int(np.log2(n))
    P = np.zeros((n, n))
    for j in range(n):
        P[bitrev(j, bits), j] = 1.0
    return P


# --------------------------------------------------------------------------
# offline calibration  ([nl] §2.1-2.2.A, [fr] §2.1-2.2.A, [abs])
# --------------------------------------------------------------------------

def query_covariance(q: np.ndarray) -> np.ndarray:
    """C_Q: mean over tokens and query heads of the outer product q q^T.

    q: float64 [N][Hq][d].  Logit distortion is governed by the query second
    moment ([nl]/[fr] §2.1; estimate in §2.2.A).
    """
    x = q.reshape(-1, q.shape[-1])
    return x.T @ x / x.shape[0]


def causal_attention_outputs(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             sm_scale: float | None = None) -> np.ndarray:
    """O = S V per query head, S the causal softmax(q K^T * sm_scale).

    q: [N][Hq][d], k, v: [N][Hkv][d]; query head h reads KV head
    h // (Hq/Hkv).  Returns [N][Hq][d].
    """
    n, hq, d = q.shape
    hkv = k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.empty_like(q)
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    for h in range(hq):
        g = h // (hq // hkv)
        logits = (q[:, h, :] @ k[:, g, :].T) * sm_scale
        logits[future] = -np.inf
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def score_covariance(q, k, v, sm_scale=None) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V, pooled over query heads: the mean outer
    product of the attention outputs S V ([nl]/[fr] §2.1 value target,
    §2.2.A estimate)."""
    o = causal_attention_outputs(q, k, v, sm_scale)
    x = o.reshape(-1, o.shape[-1])
    return x.T @ x / x.shape[0]


def eigenbasis(C: np.ndarray) -> np.ndarray:
    """Eigenbasis U of a symmetric C ([nl]/[fr] §2.2.A "rotation derivation"):
    columns sorted by descending eigenvalue, each column's largest-magnitude
    entry made positive (first index on ties)."""
    w, U = np.linalg.eigh(C)
    order = np.argsort(-w, kind="stable")
    U = U[:, order].copy()
    for j in range(U.shape[1]):
        i = int(np.argmax(np.abs(U[:, j])))
        if U[i, j] < 0:
            U[:, j] = -U[:, j]
    return U


def compose_rotation(U: np.ndarray) -> np.ndarray:
    """R = U H P_br ([nl] §2.2.A "Formule", [fr] §2.2.A.3)."""
    n = U.shape[0]
    return U @ hadamard(n) @ bitrev_permutation(n)


def quantile_linear(values: np.ndarray, p: float) -> float:
    """Quantile with linear interpolation between order statistics (type 7):
    h = (n-1) p, result = x[floor h] + (h - floor h)(x[floor h + 1] - x[floor h])."""
    return float(np.quantile(np.asarray(values, dtype=np.float64).ravel(), p, method="linear"))


def clip_threshold(x: np.ndarray, R: np.ndarray, quantile: float = 0.999) -> float:
    """Per-layer clip: quantile of |x R| over all tokens, heads and channels of
    the calibration set ([nl]/[fr] §2.2.A "clipping thresholds")."""
    xr = x.reshape(-1, x.shape[-1]) @ R
    return quantile_linear(np.abs(xr), quantile)


def calibrate(q, k, v, clip_quantile: float = 0.999) -> dict:
    """Full offline calibration of one layer.  q, k, v float64 (bf16 values)."""
    U_Q = eigenbasis(query_covariance(q))
    U_S = eigenbasis(score_covariance(q, k, v))
    R_K = compose_rotation(U_Q)
    R_V = compose_rotation(U_S)
    return {"R_K": R_K, "R_V": R_V,
            "clip_K": clip_threshold(k, R_K, clip_quantile),
            "clip_V": clip_threshold(v, R_V, clip_quantile)}


def calibrate_per_head(q, k, v, clip_quantile: float = 0.999) -> dict:
    """Per-KV-head calibration (an extension of the per-layer rule): KV head
    h gets R_K[h], R_V[h] from C_Q and C_S over the query heads that read it
    (h * Hq/Hkv .. +Hq/Hkv-1, each attending to KV head h as in the layer),
    and clips from its own K and V vectors.  Returns R_K, R_V [Hkv][128][128]
    and clip_K, clip_V [Hkv]."""
    hq, hkv = q.shape[1], k.shape[1]
    gqa = hq // hkv
    o = causal_attention_outputs(q, k, v)
    out = {"R_K": [], "R_V": [], "clip_K": [], "clip_V": []}
    for h in range(hkv):
        qs = q[:, h * gqa:(h + 1) * gqa]
        os_ = o[:, h * gqa:(h + 1) * gqa].reshape(-1, D)
        R_K = compose_rotation(eigenbasis(query_covariance(qs)))
        R_V = compose_rotation(eigenbasis(os_.T @ os_ / os_.shape[0]))
        out["R_K"].append(R_K)
        out["R_V"].append(R_V)
        out["clip_K"].append(clip_threshold(k[:, h], R_K, clip_quantile))
        out["clip_V"].append(clip_threshold(v[:, h], R_V, clip_quantile))
    return {key: np.asarray(val) for key, val in out.items()}


def head_rotation(R, clip, h: int):
    """KV head h's rotation and clip: R [128][128] and a scalar clip are
    shared by every head (the per-layer rotation); R [Hkv][128][128] with
    clip [Hkv] give head h its own."""
    R = np.asarray(R, dtype=np.float64)
    if R.ndim == 2:
        return R, None if clip is None else float(clip)
    return R[h], None if clip is None else float(np.asarray(clip, dtype=np.float64)[h])


def calibrate_sequences(seqs, clip_quantile: float = 0.999) -> dict:
    """Calibration over several sequences (list of (q, k, v) float64 arrays,
    q [N_s][Hq][128], k, v [N_s][Hkv][128]): C_Q and C_S are means over every
    token and query head of all sequences, each sequence's attention causal
    within itself; R and the clips as in calibrate, the clips over the
    vectors of all sequences ([nl]/[fr] §2.2.A: moments of a calibration
    set)."""
    hq = seqs[0][0].shape[1]
    weights = [q.shape[0] * hq for q, _, _ in seqs]
    total = float(sum(weights))
    C_Q = sum(w * query_covariance(q) for w, (q, _, _) in zip(weights, seqs)) / total
    C_S = sum(w * score_covariance(q, k, v) for w, (q, k, v) in zip(weights, seqs)) / total
    R_K = compose_rotation(eigenbasis(C_Q))
    R_V = compose_rotation(eigenbasis(C_S))
    k_all = np.concatenate([k for _, k, _ in seqs])
    v_all = np.concatenate([v for _, _, v in seqs])
    return {"R_K": R_K, "R_V": R_V, "C_Q": C_Q, "C_S": C_S,
            "clip_K": clip_threshold(k_all, R_K, clip_quantile),
            "clip_V": clip_threshold(v_all, R_V, clip_quantile)}


# --------------------------------------------------------------------------
# rotation variants and distortion diagnostics ([abs]: OSCAR against
# Hadamard-only, QuaRot-style INT2; [nl]/[fr] §2.1: data-oblivious Hadamard
# rotations and naive INT2, whose outliers dominate the quantisation scale)
# --------------------------------------------------------------------------

def hadamard_only_rotation(n: int = D) -> np.ndarray:
    """The data-oblivious rotation R = H P_br: OSCAR's composition without a
    covariance eigenbasis (U = I)."""
    return hadamard(n) @ bitrev_permutation(n)


def identity_rotation(n: int = D) -> np.ndarray:
    """No rotation: plain per-token INT2 of the raw channels."""
    return np.eye(n)


def logit_distortion(q: np.ndarray, K: np.ndarray, K_hat: np.ndarray) -> float:
    """Query-weighted logit distortion: the mean over query heads h and tokens
    t of (q_h . (K[t, g(h)] - K_hat[t, g(h)]))^2 with g(h) = h // (Hq/Hkv),
    the error the attention logits see.  q: [Hq][128]; K, K_hat: [L][Hkv][128]."""
    hq, hkv = q.shape[0], K.shape[1]
    dK = K - K_hat
    total = 0.0
    for h in range(hq):
        g = h // (hq // hkv)
        total += float(((dK[:, g, :] @ q[h]) ** 2).sum())
    return total / (hq * K.shape[0])


def relative_l2(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_2 / ||ref||_2 over all entries."""
    return float(np.linalg.norm(np.asarray(x, np.float64) - ref) / np.linalg.norm(ref))


# --------------------------------------------------------------------------
# the INT2 quantiser  ([nl]/[fr] §1 four levels, §2.2.B rotate + clip + INT2)
# and its INT4 variant (16 levels; the INT4 baseline the pages compare
# against, [nl] §4 / [fr] §4)
# --------------------------------------------------------------------------

def levels(bits: int) -> int:
    """Highest code of a bits-wide quantiser: 3 (INT2) or 15 (INT4)."""
    assert bits in (2, 4)
    return (1 << bits) - 1


def quantize(x: np.ndarray, R: np.ndarray, clip: float, G: int, bits: int = 2) -> dict:
    """Rotate, clip and quantise vectors.

    x: float64 [n][128] (bf16 values).  Returns codes uint8 [n][128], scale
    and zero float16 [n][128/G], the clipped rotated values xc [n][128] and
    t = (xc - zero)/scale in code units (NaN where scale == 0).  The scale
    spreads a group's range over levels(bits) steps.
    """
    n = x.shape[0]
    ng = D // G
    xc = np.clip(x @ R, -clip, clip)
    g = xc.reshape(n, ng, G)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    zero = f16_round(lo)
    scale = f16_round((hi - lo) / float(levels(bits)))
    codes, t = codes_from_meta(xc, scale, zero, G, bits)
    return {"codes": codes, "scale": scale, "zero": zero, "xc": xc, "t": t}


def codes_from_meta(xc: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int, bits: int = 2):
    """Codes of clipped rotated values for a given fp16 (scale, zero):
    clamp(rint((xc - z)/s), 0, levels(bits)), 0 where s == 0."""
    n = xc.shape[0]
    ng = D // G
    s = scale.astype(np.float64)[:, :, None]
    z = zero.astype(np.float64)[:, :, None]
    g = xc.reshape(n, ng, G)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s > 0, (g - z) / np.where(s > 0, s, 1.0), np.nan)
    c = np.where(s > 0, np.clip(np.rint(np.nan_to_num(t)), 0, levels(bits)), 0).astype(np.uint8)
    return c.reshape(n, D), t.reshape(n, D)


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int) -> np.ndarray:
    """Rotated-basis values c*s + z, float64 [n][128]."""
    n = codes.shape[0]
    ng = D // G
    c = codes.reshape(n, ng, G).astype(np.float64)
    return (c * scale.astype(np.float64)[:, :, None] + zero.astype(np.float64)[:, :, None]).reshape(n, D)


# --------------------------------------------------------------------------
# storage format of a history block (defined in include/oscar.h)
# --------------------------------------------------------------------------

LO_BIT = (8, 6, 12, 10, 4, 2, 16, 14)
HI_BIT = (24, 22, 28, 26, 20, 18, 0, 30)


def code_area_bytes(bits: int = 2) -> int:
    """Bytes of one code area: 16 tokens x 128 channels x bits."""
    return PAGE * D * bits // 8


def hist_block_bytes(G: int, bits: int = 2) -> int:
    return 2 * code_area_bytes(bits) + 128 * (D // G)


def _code_bit_tables_int4(kind: str):
    """(byte index, shift) [16 rows][128 channels] of every 4-bit code of an
    INT4 code area (1024 bytes, 256 dwords; dword w = 4 l + i of lane l,
    a = l % 16, q = l / 16; nibble e = 0..7 of a dword at bits 4 e .. 4 e + 3):
      K: a = token t; dword i = kb (0..3), nibble e holds channel
         32 kb + 8 q + 2 (e % 4) + e / 4 of token t;
      V: a = channel offset m; dword i = d (0..3), nibble e holds channel
         16 (2 d + (e / 2) % 2) + m, token 4 q + 2 (e % 2) + e / 4.
    Nibbles e and e + 4 thus hold neighbouring channels (K) or tokens (V)."""
    byte_idx = np.full((PAGE, D), -1, dtype=np.int64)
    shift = np.full((PAGE, D), -1, dtype=np.int64)
    for lane in range(64):
        a, q = lane % 16, lane // 16
        for i in range(4):
            word = 4 * lane + i
            for e in range(8):
                if kind == "K":
                    t, c = a, 32 * i + 8 * q + 2 * (e % 4) + e // 4
                else:
                    t, c = 4 * q + 2 * (e % 2) + e // 4, 16 * (2 * i + (e // 2) % 2) + a
                assert byte_idx[t, c] < 0
                byte_idx[t, c] = 4 * word + e // 2
                shift[t, c] = 4 * (e % 2)
    assert (byte_idx >= 0).all()
    return byte_idx, shift


def _code_bit_tables(kind: str):
    """(byte index, shift) [16 rows][128 channels] of every code of a code area."""
    byte_idx = np.full((PAGE, D), -1, dtype=np.int64)
    shift = np.full((PAGE, D), -1, dtype=np.int64)
    for lane in range(64):
        a, q = lane % 16, lane // 16
        for d in range(2):
            word = 2 * lane + d
            for u in range(8):
                if kind == "K":
                    t0, c0 = a, 32 * (2 * d + u // 4) + 8 * q + 2 * (u % 4)
                    cells = ((t0, c0, LO_BIT[u]), (t0, c0 + 1, HI_BIT[u]))
                else:
                    c, t0 = 16 * (4 * d + u // 2) + a, 4 * q + 2 * (u % 2)
                    cells = ((t0, c, LO_BIT[u]), (t0 + 1, c, HI_BIT[u]))
                for t, c, bit in cells:
                    assert byte_idx[t, c] < 0
                    byte_idx[t, c] = 4 * word + bit // 8
                    shift[t, c] = bit % 8
    assert (byte_idx >= 0).all()
    return byte_idx, shift


_TABLES = {(2, "K"): _code_bit_tables("K"), (2, "V"): _code_bit_tables("V"),
           (4, "K"): _code_bit_tables_int4("K"), (4, "V"): _code_bit_tables_int4("V")}


def pack_codes(codes: np.ndarray, kind: str, bits: int = 2) -> np.ndarray:
    """codes uint8 [..., 16, 128] (0..levels(bits)) -> code areas uint8
    [..., code_area_bytes(bits)]."""
    byte_idx, shift = _TABLES[(bits, kind)]
    nb, mask = code_area_bytes(bits), levels(bits)
    lead = codes.shape[:-2]
    out = np.zeros(lead + (nb,), dtype=np.uint8)
    flat_out = out.reshape(-1, nb)
    flat_c = codes.reshape(-1, PAGE, D).astype(np.uint8)
    for t in range(PAGE):
        for c in range(D):
            flat_out[:, byte_idx[t, c]] |= ((flat_c[:, t, c] & mask) << np.uint8(shift[t, c])).astype(np.uint8)
    return out


def unpack_codes(area: np.ndarray, kind: str, bits: int = 2) -> np.ndarray:
    """code areas uint8 [..., code_area_bytes(bits)] -> codes uint8 [..., 16, 128]."""
    byte_idx, shift = _TABLES[(bits, kind)]
    return (area[..., byte_idx] >> shift.astype(np.uint8)) & levels(bits)


def pack_meta(scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """scale, zero float16 [..., 16 rows, NG] -> meta areas uint8 [..., 64*NG]:
    entry (g, t) at byte 4*(16 g + t), scale then zero."""
    s = np.swapaxes(scale.astype(np.float16), -1, -2)  # [..., NG, 16]
    z = np.swapaxes(zero.astype(np.float16), -1, -2)
    pair = np.stack([s, z], axis=-1)                  # [..., NG, 16, 2]
    return pair.view(np.uint8).reshape(scale.shape[:-2] + (-1,))


def unpack_meta(area: np.ndarray, G: int):
    """meta areas uint8 [..., 64*NG] -> (scale, zero) float16 [..., 16, NG]."""
    ng = D // G
    pair = np.ascontiguousarray(area).view(np.float16).reshape(area.shape[:-1] + (ng, PAGE, 2))
    return np.swapaxes(pair[..., 0], -1, -2), np.swapaxes(pair[..., 1], -1, -2)


def split_block(block: np.ndarray, G: int, bits: int = 2) -> dict:
    """Views of the four areas of history blocks uint8 [..., B_hist(G, bits)]."""
    m = 64 * (D // G)
    a = code_area_bytes(bits)
    return {"k_codes": block[..., 0:a], "k_meta": block[..., a:a + m],
            "v_codes": block[..., a + m:2 * a + m], "v_meta": block[..., 2 * a + m:2 * a + 2 * m]}


# --------------------------------------------------------------------------
# the mixed-precision paged cache  ([nl]/[fr] §2.2.B)
# --------------------------------------------------------------------------

def storage_of(p: int, L: int):
    """Where position p of a request of length L lives: ('sink', row),
    ('hist', history index h = p - 16) or ('ring', slot)."""
    if p < N_SINK:
        return ("sink", p)
    if p < L - N_RECENT:
        return ("hist", p - N_SINK)
    return ("ring", p % N_RECENT)


class LayerCacheRef:
    """One layer's cache as numpy pools with page tables (formats of oscar.h);
    bits = 2 (INT2 history) or 4 (INT4)."""

    def __init__(self, n_kv_heads: int, G: int, n_hist_pages: int, n_bf16_pages: int,
                 hist_pt: np.ndarray, bf16_pt: np.ndarray, bits: int = 2):
        self.hkv, self.G, self.bits = n_kv_heads, G, bits
        self.hist = np.zeros((n_hist_pages, n_kv_heads, hist_block_bytes(G, bits)), dtype=np.uint8)
        self.bf16 = np.zeros((n_bf16_pages, n_kv_heads, 2, PAGE, D), dtype=np.uint16)
        self.hist_pt = np.asarray(hist_pt, dtype=np.int32)
        self.bf16_pt = np.asarray(bf16_pt, dtype=np.int32)

    # ---- raw bf16 rows
    def _bf16_row(self, b: int, where: str, idx: int):
        if where == "sink":
            return self.bf16_pt[b, 0], idx
        return self.bf16_pt[b, 1 + idx // PAGE], idx % PAGE

    def write(self, rot_k: np.ndarray, rot_v: np.ndarray, clip_k: float, clip_v: float,
              k_new: np.ndarray, v_new: np.ndarray, cu_new, len_before) -> None:
        """Append tokens (the write of [abs] and [nl]/[fr] §2.2.B).

        rot_k / rot_v with clip_k / clip_v: one R [128][128] and clip for
        the layer, or per KV head R [Hkv][128][128] and clips [Hkv].
        k_new, v_new: bf16 bits [T][Hkv][128].  Request b receives rows
        cu_new[b]..cu_new[b+1]-1 at positions len_before[b]... .  Ring tokens
        that leave the recent window are quantised into history.
        """
        G = self.G
        for b in range(len(len_before)):
            L0 = int(len_before[b])
            n = int(cu_new[b + 1]) - int(cu_new[b])
            L = L0 + n
            # tokens whose storage may change: the old ring tokens (positions
            # max(16, L0-128) .. L0-1) and all new tokens.  Old ring rows are
            # read before anything is written.
            src = {}
            for p in range(max(N_SINK, L0 - N_RECENT), L0):
                w, idx = storage_of(p, L0)
                assert w == "ring"
                pg, row = self._bf16_row(b, "ring", idx)
                src[p] = (self.bf16[pg, :, 0, row, :].copy(), self.bf16[pg, :, 1, row, :].copy())
            for i in range(n):
                r = int(cu_new[b]) + i
                src[L0 + i] = (k_new[r].copy(), v_new[r].copy())
            hist_pos = []
            for p in sorted(src):
                w, idx = storage_of(p, L)
                kx, vx = src[p]
                if w == "hist":
                    hist_pos.append((p, idx))
                    continue
                if p < L0 and w == "ring":
                    continue  # stays where it is
                pg, row = self._bf16_row(b, w, idx)
                self.bf16[pg, :, 0, row, :] = kx
                self.bf16[pg, :, 1, row, :] = vx
            if not hist_pos:
                continue
            # quantise every history-bound token, then store them page by page
            hidx = np.array([idx for _, idx in hist_pos])
            pages, rows = hidx // PAGE, hidx % PAGE
            upages = np.unique(pages)
            slot = np.searchsorted(upages, pages)
            pids = self.hist_pt[b, upages]
            xs = {"k": np.stack([bf16_to_f64(src[p][0]) for p, _ in hist_pos]),  # [n][Hkv][128]
                  "v": np.stack([bf16_to_f64(src[p][1]) for p, _ in hist_pos])}
            rot = {"k": (rot_k, clip_k), "v": (rot_v, clip_v)}
            for h in range(self.hkv):
                blocks = self.hist[pids, h].copy()          # [P][block]
                areas = split_block(blocks, G, self.bits)
                for kind in ("k", "v"):
                    R, clip = head_rotation(*rot[kind], h)
                    qq = quantize(xs[kind][:, h, :], R, clip, G, self.bits)
                    codes = unpack_codes(areas[kind + "_codes"], kind.upper(), self.bits)
                    sc, zr = unpack_meta(areas[kind + "_meta"], G)
                    sc, zr = sc.copy(), zr.copy()
                    codes[slot, rows] = qq["codes"]
                    sc[slot, rows] = qq["scale"]
                    zr[slot, rows] = qq["zero"]
                    areas[kind + "_codes"][:] = pack_codes(codes, kind.upper(), self.bits)
                    areas[kind + "_meta"][:] = pack_meta(sc, zr)
                self.hist[pids, h] = blocks

    # ---- reconstruction for the decode
    def gather(self, b: int, L: int, rot_k: np.ndarray, rot_v: np.ndarray):
        """K, V float64 [L][Hkv][128] of request b, history inverse-rotated
        back to the original basis (dequantise, then x_rot R^T; R per layer
        [128][128] or per KV head [Hkv][128][128])."""
        G = self.G
        K = np.empty((L, self.hkv, D))
        V = np.empty((L, self.hkv, D))
        where = [storage_of(p, L) for p in range(L)]
        raw = [(p, self._bf16_row(b, w, idx)) for p, (w, idx) in enumerate(where) if w != "hist"]
        if raw:
            pos = np.array([p for p, _ in raw])
            pg = np.array([r[0] for _, r in raw])
            row = np.array([r[1] for _, r in raw])
            K[pos] = bf16_to_f64(self.bf16[pg, :, 0, row, :])
            V[pos] = bf16_to_f64(self.bf16[pg, :, 1, row, :])
        hist = [(p, idx) for p, (w, idx) in enumerate(where) if w == "hist"]
        if hist:
            pos = np.array([p for p, _ in hist])
            hidx = np.array([idx for _, idx in hist])
            pages, rows = hidx // PAGE, hidx % PAGE
            upages = np.unique(pages)
            slot = np.searchsorted(upages, pages)
            pids = self.hist_pt[b, upages]
            for h in range(self.hkv):
                areas = split_block(self.hist[pids, h], G, self.bits)
                for kind, Rh, out in (("k", rot_k, K), ("v", rot_v, V)):
                    R, _ = head_rotation(Rh, None, h)
                    c = unpack_codes(areas[kind + "_codes"], kind.upper(), self.bits)      # [P][16][128]
                    sc, zr = unpack_meta(areas[kind + "_meta"], G)             # [P][16][NG]
                    n = c.shape[0] * PAGE
                    x = dequantize(c.reshape(n, D), sc.reshape(n, -1), zr.reshape(n, -1), G) @ R.T
                    out[pos, h] = x.reshape(-1, PAGE, D)[slot, rows]
        return K, V


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(q K^T * sm_scale) V for one request, fp64.

    q: [Hq][128]; K, V: [L][Hkv][128]; query head h reads KV head
    h // (Hq/Hkv).  Returns [Hq][128].
    """
    hq, hkv = q.shape[0], K.shape[1]
    out = np.empty((hq, q.shape[1]))
    for h in range(hq):
        g = h // (hq // hkv)
        logits = (K[:, g, :] @ q[h]) * sm_scale
        w = np.exp(logits - logits.max())
        out[h] = (w / w.sum()) @ V[:, g, :]
    return out


def decode_attn(cache: LayerCacheRef, rot_k, rot_v, q_bits: np.ndarray, seq_lens,
                sm_scale: float) -> np.ndarray:
    """Decode attention over the mixed-precision cache ([nl]/[fr] §2.2.B):
    every history token is dequantised and inverse-rotated, then plain
    softmax attention over all seq_lens[b] tokens.  Returns [B][Hq][128]."""
    q = bf16_to_f64(q_bits)
    out = np.empty(q.shape)
    for b in range(q.shape[0]):
        K, V = cache.gather(b, int(seq_lens[b]), rot_k, rot_v)
        out[b] = attention(q[b], K, V, sm_scale)
    return out


def extend_attn(cache: LayerCacheRef, rot_k, rot_v, q_bits: np.ndarray, k_new: np.ndarray,
                v_new: np.ndarray, cu_new, len_before, sm_scale: float, rows=None) -> np.ndarray:
    """Chunked-prefill ("extend") attention of new tokens over a cached prefix
    ([abs]: paged layouts with prefix caching; [nl]/[fr] section 2.2.B: the
    fused kernel reads the INT2 history, dequantises and inverse-rotates it).

    Request b's prefix is the cache as it stands, len_before[b] tokens: sink,
    INT2 history and recent window, each read as the decode reads it.  Its
    new tokens are rows cu_new[b] .. cu_new[b+1]-1 of q_bits / k_new / v_new
    (bf16 bits, [T][Hq or Hkv][128]), at positions len_before[b] + i; new
    token i attends to the whole prefix and to new tokens 0..i at full bf16
    precision (causal).  The chunk is not written here.  Returns
    [T][Hq][128] fp64; with rows (indices into the T rows) only those rows
    are computed and returned, in that order."""
    q = bf16_to_f64(q_bits)
    out = np.empty(q.shape)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(len(len_before)):
        L0 = int(len_before[b])
        r0, r1 = int(cu_new[b]), int(cu_new[b + 1])
        if want is not None and not any(r0 <= r < r1 for r in want):
            continue
        Kp, Vp = cache.gather(b, L0, rot_k, rot_v)
        Kn, Vn = bf16_to_f64(k_new[r0:r1]), bf16_to_f64(v_new[r0:r1])
        for i in range(r1 - r0):
            if want is not None and r0 + i not in want:
                continue
            K = np.concatenate([Kp, Kn[:i + 1]])
            V = np.concatenate([Vp, Vn[:i + 1]])
            out[r0 + i] = attention(q[r0 + i], K, V, sm_scale)
    return out if rows is None else out[np.asarray(rows, dtype=np.int64)]


def bf16_paged_decode(q_bits, kv_pages, pt, seq_lens, sm_scale) -> np.ndarray:
    """Plain BF16 paged decode: token p of request b is row p%16 of page
    pt[b][p//16] (kv_pages bf16 bits [pages][Hkv][2][16][128])."""
    q = bf16_to_f64(q_bits)
    out = np.empty(q.shape)
    for b in range(q.shape[0]):
        L = int(seq_lens[b])
        p = np.arange(L)
        pages = np.asarray(pt[b])[p // PAGE]
        K = bf16_to_f64(kv_pages[pages, :, 0, p % PAGE, :])
        V = bf16_to_f64(kv_pages[pages, :, 1, p % PAGE, :])
        out[b] = attention(q[b], K, V, sm_scale)
    return out
