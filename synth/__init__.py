"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, clipping, quantisation or attention).  The
recipe follows the workload descriptions used throughout this repository:

* K, V ~ N(0, 1), with 4 outlier channels per (layer, KV head) scaled by 20,
  drawn without replacement; the same channels serve calibration and cache
  tokens.
* Q ~ N(0, diag(lam)) with lam_i = 10**u_i, u_i ~ U(-2, 1) (log-uniform in
  [0.01, 10]); one lam per layer, shared by its query heads.  The optional
  dense variant draws Q ~ N(0, B diag(lam) B^T) with B a seeded random
  orthogonal basis (correlated query channels).
* Every float is rounded to bf16 (round to nearest even from fp32) and handed
  over as uint16 bit patterns.
* Every stream has its own seed: numpy PCG64 seeded by
  SeedSequence([base_seed, layer, stream_id]).
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
PAGE = 16
N_SINK = 16
N_RECENT = 128

# stream ids of SeedSequence([base, layer, stream])
S_SIGMA, S_OUTLIER, S_CAL_Q, S_CAL_K, S_CAL_V = 0, 1, 2, 3, 4
S_CACHE_K, S_CACHE_V, S_DEC_Q, S_PAGES, S_LENS, S_NEW_K, S_NEW_V = 5, 6, 7, 8, 9, 10, 11
S_BASIS, S_EVAL_Q = 12, 13


def rng(base_seed: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([base_seed, layer, stream])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def layer_lambda(base_seed: int, layer: int) -> np.ndarray:
    u = rng(base_seed, layer, S_SIGMA).uniform(-2.0, 1.0, size=HEAD_DIM)
    return 10.0 ** u


def outlier_channels(base_seed: int, layer: int, n_kv_heads: int) -> np.ndarray:
    g = rng(base_seed, layer, S_OUTLIER)
    return np.stack([g.choice(HEAD_DIM, size=4, replace=False) for _ in range(n_kv_heads)])


def kv_f32(g: np.random.Generator, n: int, outliers: np.ndarray) -> np.ndarray:
    """[n][Hkv][128] fp32 with the outlier channels of each head scaled x20."""
    hkv = outliers.shape[0]
    x = g.standard_normal((n, hkv, HEAD_DIM), dtype=np.float32)
    for h in range(hkv):
        x[:, h, outliers[h]] *= 20.0
    return x


def q_f32(g: np.random.Generator, n: int, n_q_heads: int, lam: np.ndarray, basis=None) -> np.ndarray:
    z = g.standard_normal((n, n_q_heads, HEAD_DIM), dtype=np.float32)
    y = z * np.sqrt(lam).astype(np.float32)
    if basis is not None:
        y = (y.astype(np.float64) @ basis.T).astype(np.float32)
    return y


def random_basis(base_seed: int, layer: int) -> np.ndarray:
    """A seeded random orthogonal 128 x 128 matrix (the Q factor of a Gaussian
    matrix, columns signed by the diagonal of R)."""
    a = rng(base_seed, layer, S_BASIS).standard_normal((HEAD_DIM, HEAD_DIM))
    qm, r = np.linalg.qr(a)
    return qm * np.sign(np.diag(r))


class LayerData:
    """All seeded host inputs of one layer of one workload."""

    def __init__(self, base_seed: int, layer: int, n_q_heads: int, n_kv_heads: int, dense_q: bool = False):
        self.base_seed, self.layer = base_seed, layer
        self.hq, self.hkv = n_q_heads, n_kv_heads
        self.lam = layer_lambda(base_seed, layer)
        self.outliers = outlier_channels(base_seed, layer, n_kv_heads)
        self.basis = random_basis(base_seed, layer) if dense_q else None

    def calibration(self, n_tokens: int):
        """(q, k, v) bf16 bits: [N][Hq][128], [N][Hkv][128], [N][Hkv][128]."""
        q = bf16_bits(q_f32(rng(self.base_seed, self.layer, S_CAL_Q), n_tokens, self.hq, self.lam, self.basis))
        k = bf16_bits(kv_f32(rng(self.base_seed, self.layer, S_CAL_K), n_tokens, self.outliers))
        v = bf16_bits(kv_f32(rng(self.base_seed, self.layer, S_CAL_V), n_tokens, self.outliers))
        return q, k, v

    def cache_kv(self, n_tokens: int, stream_k: int = S_CACHE_K, stream_v: int = S_CACHE_V):
        """(k, v) bf16 bits [n_tokens][Hkv][128] (all requests concatenated)."""
        k = bf16_bits(kv_f32(rng(self.base_seed, self.layer, stream_k), n_tokens, self.outliers))
        v = bf16_bits(kv_f32(rng(self.base_seed, self.layer, stream_v), n_tokens, self.outliers))
        return k, v

    def decode_q(self, batch: int, stream: int = S_DEC_Q):
        return bf16_bits(q_f32(rng(self.base_seed, self.layer, stream), batch, self.hq, self.lam, self.basis))


def hist_pages_needed(seq_len: int) -> int:
    """History pages a request of this length occupies."""
    n_hist = max(0, seq_len - N_SINK - N_RECENT)
    return (n_hist + PAGE - 1) // PAGE


def shuffled_page_tables(base_seed: int, layer: int, lens, n_pool_pages: int | None = None,
                         stride: int | None = None, n_pages_fn=hist_pages_needed):
    """Page tables for requests of the given lengths drawn from one pool.

    Pages of all requests are taken from a seeded random permutation of the
    pool, so pages of different requests interleave.  Returns
    (table int32 [B][stride], n_pool_pages); unused entries are 0.
    """
    need = [n_pages_fn(int(L)) for L in lens]
    total = int(sum(need))
    if n_pool_pages is None:
        n_pool_pages = max(total, 1)
    if stride is None:
        stride = max(max(need) if need else 1, 1)
    perm = rng(base_seed, layer, S_PAGES).permutation(n_pool_pages)[:total]
    table = np.zeros((len(lens), stride), dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, n_pool_pages


def bf16_page_tables(batch: int, first_page: int = 0, shuffle_seed: int | None = None):
    """BF16 page tables [B][9]: one sink page and 8 ring pages per request."""
    ids = np.arange(first_page, first_page + 9 * batch, dtype=np.int32)
    if shuffle_seed is not None:
        ids = first_page + rng(shuffle_seed, 0, S_PAGES).permutation(9 * batch).astype(np.int32)
    return ids.reshape(batch, 9)


def request_lengths(base_seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Integer lengths uniform in [lo, hi] (inclusive)."""
    return rng(base_seed, 0, S_LENS).integers(lo, hi + 1, size=batch).astype(np.int32)


# ---------------------------------------------------------------- on device
# Bulk generators for benchmark-sized workloads: the same distributions as
# above, drawn with torch's seeded device generator instead of numpy.

def device_generator(base_seed: int, layer: int, stream: int, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([base_seed, layer, stream]).generate_state(1)[0]))
    return g


def kv_device(gen, n: int, outliers: np.ndarray, device="cuda", out=None, work=None):
    """bf16 [n][Hkv][128] ~ N(0, 1) with the outlier channels scaled x20.
    out (bf16) and work (fp32), both with at least n * Hkv * 128 elements,
    optionally receive the values and hold the fp32 draw (no allocation)."""
    import torch
    hkv = outliers.shape[0]
    scale = torch.ones((hkv, HEAD_DIM), dtype=torch.float32)
    for h in range(hkv):
        scale[h, torch.as_tensor(outliers[h])] = 20.0
    shape = (n, hkv, HEAD_DIM)
    if work is not None:
        x = work.view(-1)[: n * hkv * HEAD_DIM].view(shape)
        torch.randn(shape, generator=gen, device=device, dtype=torch.float32, out=x)
    else:
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x.mul_(scale.to(device))
    if out is not None:
        y = out.view(-1)[: n * hkv * HEAD_DIM].view(shape)
        y.copy_(x)
        return y
    return x.to(torch.bfloat16)


def q_device(gen, n: int, n_q_heads: int, lam: np.ndarray, device="cuda"):
    """bf16 [n][Hq][128] ~ N(0, diag(lam))."""
    import torch
    z = torch.randn((n, n_q_heads, HEAD_DIM), generator=gen, device=device, dtype=torch.float32)
    z.mul_(torch.as_tensor(np.sqrt(lam), dtype=torch.float32, device=device))
    return z.to(torch.bfloat16)
