// Extend (chunked-prefill) attention over the mixed-precision cache: the new
// tokens of a request attend to its cached prefix -- BF16 sink and recent
// window, INT2 history read through dequantisation in the rotated basis -- and
// causally to the chunk's own tokens at bf16 ([abs]: paged KV layouts with
// prefix caching; [nl]/[fr] §2.2.B: the fused kernel unpacks, dequantises
// and inverse-rotates the INT2 history inside the attention).
//
// One wave per (request, query head, tile of 16 new tokens); the waves of a
// workgroup are query heads of one KV head (GQA), so they read the same keys
// at about the same time and the repeats are served by the caches.  Per tile
// of 16 keys the wave forms the 16 x 16 score block as S^T = K Q^T on the
// matrix cores (lane l holds query l%16 and keys 4(l/16)..+3), keeps an
// online softmax per query, and accumulates O^T = V^T P^T on the matrix cores
// with P^T taken straight from the score registers:
//   history (INT2) tiles: A = the stored 2-bit codes expanded to exact fp16
//     integers, B = q R_K (scores) or p s_V (values) split into fp16 high and
//     low parts, so each product is exact and the sums are fp32; scale and
//     zero of a group enter per key: score = sum_g s_g (q_g . c_g) + z_g
//     sum(q_g), value = sum_t p_t s_t c_t + (sum_t p_t z_t);
//   BF16 tiles (sink, ring, chunk): A = raw bf16 rows, B = q (bf16, exact)
//     or p split into bf16 high and low parts.
// The history accumulator stays in the rotated basis and is brought back with
// R_V^T once per query at the end.
#include <cmath>

#include "attn_common.h"

namespace oscar {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct ExtendArgs {
  const uint8_t *hist;
  int64_t n_hist_pages;
  const uint16_t *bf16;
  int64_t n_bf16_pages;
  const int32_t *hist_pt;
  int hist_pt_stride;
  const int32_t *bf16_pt;
  uint32_t *status;
  const float *rk;   // fp32 R_K[i][j] at i*128 + j
  const float *rvt;  // fp32 R_V[j][c] at c*128 + j
  const uint16_t *q, *k_new, *v_new;
  const int32_t *cu_new, *len_before;
  int hq, hkv, max_new, max_prefix;
  float scale_log2;  // sm_scale * log2(e)
  float *out;
};

constexpr int EXT_TILE = 16;

__device__ inline float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// bf16 bits of x, round to nearest even (x finite)
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// x = hi + lo with hi, lo bf16 (lo carries the rounding error of hi)
__device__ inline void split_bf16(const float (&x)[4], s16x4 &hi, s16x4 &lo) {
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = bf16_rne(x[j]);
    hi[j] = short(h);
    lo[j] = short(bf16_rne(x[j] - __uint_as_float(h << 16)));
  }
}
__device__ inline void split_f16(const float (&x)[4], f16x4 &hi, f16x4 &lo) {
  for (int j = 0; j < 4; ++j) {
    const _Float16 h = _Float16(x[j]);
    hi[j] = h;
    lo[j] = _Float16(x[j] - float(h));
  }
}

// exact code values 0..3 from the expanded operands (1 + c/4, 1 + c/16)
__device__ inline f16x8 codes_k(uint32_t w0, uint32_t w1, int kb) {
  const f16x8 m = {4, 4, 16, 16, 4, 4, 16, 16};
  return expand_k(w0, w1, kb) * m - m;
}
__device__ inline f16x4 codes_v(uint32_t w0, uint32_t w1, int r) {
  const f16x4 m = {4, 4, 16, 16};
  return expand_v(w0, w1, r) * m - m;
}

template <int NG>
struct ExtState {
  f32x4 acc_r[8];  // history part, rotated basis: channel 16 b + 4 (l/16) + r
  f32x4 acc_p[8];  // BF16 part: channel 32 (b/2) + 2 (4 (l/16) + r) + b%2
  float zacc[NG];  // sum_t p_t z_t of the lane's keys, per group
  float m, l;      // running max (log2 units) of the lane's query; lane-partial sum
};

// Online softmax over one tile: s[r] = scaled score of key 4(l/16)+r for the
// lane's query (-inf where masked); p[r] receives the probabilities relative
// to the updated running max, and every accumulator is rescaled.
template <int NG>
__device__ inline void softmax_tile(ExtState<NG> &st, const float (&s)[4], float (&p)[4]) {
  float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  const float mn = fmaxf(st.m, mx);
  const float ref = mn == -INFINITY ? 0.f : mn;
  const float alpha = exp2f(st.m - ref);
  float sum = 0.f;
  for (int r = 0; r < 4; ++r) {
    p[r] = exp2f(s[r] - ref);
    sum += p[r];
  }
  st.l = st.l * alpha + sum;
  st.m = mn;
  for (int b = 0; b < 8; ++b) {
    st.acc_r[b] *= alpha;
    st.acc_p[b] *= alpha;
  }
  for (int g = 0; g < NG; ++g) st.zacc[g] *= alpha;
}

// One tile of 16 raw bf16 keys: key t's K row at kp + t * stride (elements),
// V row at vp + t * stride, for t < nrows; rows t >= nrows are not read (their
// loads repeat row 0).  valid(t, i) says whether key t is visible to query i
// of the tile, valid(t, -1) whether key t exists at all.
template <int NG, class Valid>
__device__ inline void bf16_tile(ExtState<NG> &st, const uint16_t *kp, const uint16_t *vp, int64_t stride,
                                 int nrows, const bf16x8 (&qb)[4], float scale_log2, int lane, Valid valid) {
  const int kq = lane >> 4, m = lane & 15;
  // scores S^T[t][i] = K[t] . q[i]
  f32x4 d = {0.f, 0.f, 0.f, 0.f};
  const uint16_t *krow = kp + int64_t(m < nrows ? m : 0) * stride + 8 * kq;
  for (int kb = 0; kb < 4; ++kb) {
    const u32x4 u = *reinterpret_cast<const u32x4 *>(krow + 32 * kb);
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), qb[kb], d, 0, 0, 0);
  }
  bool ok[4];
  float s[4], p[4];
  for (int r = 0; r < 4; ++r) {
    ok[r] = valid(4 * kq + r, m);
    s[r] = ok[r] ? d[r] * scale_log2 : -INFINITY;
  }
  softmax_tile(st, s, p);
  s16x4 phi, plo;
  split_bf16(p, phi, plo);
  // O^T += V^T P^T; lane (m, kq) of the block pair (2c, 2c+1) holds channels
  // 32c + 2m and 32c + 2m + 1 of keys 4kq .. 4kq+3
  for (int c = 0; c < 4; ++c) {
    uint32_t u[4];
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * kq + j < nrows ? 4 * kq + j : 0;
      const uint32_t x = *reinterpret_cast<const uint32_t *>(vp + int64_t(t) * stride + 32 * c + 2 * m);
      u[j] = valid(4 * kq + j, -1) ? x : 0u;  // absent rows may hold anything
    }
    const uint32_t e0 = __builtin_amdgcn_perm(u[1], u[0], 0x05040100u);
    const uint32_t e1 = __builtin_amdgcn_perm(u[3], u[2], 0x05040100u);
    const uint32_t o0 = __builtin_amdgcn_perm(u[1], u[0], 0x07060302u);
    const uint32_t o1 = __builtin_amdgcn_perm(u[3], u[2], 0x07060302u);
    const s16x4 ae = __builtin_bit_cast(s16x4, u32x2{e0, e1});
    const s16x4 ao = __builtin_bit_cast(s16x4, u32x2{o0, o1});
    st.acc_p[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, phi, st.acc_p[2 * c], 0, 0, 0);
    st.acc_p[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, plo, st.acc_p[2 * c], 0, 0, 0);
    st.acc_p[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, phi, st.acc_p[2 * c + 1], 0, 0, 0);
    st.acc_p[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, plo, st.acc_p[2 * c + 1], 0, 0, 0);
  }
}

// One INT2 history page (block of one KV head), rows < n_valid.
template <int G>
__device__ inline void hist_tile(ExtState<D / G> &st, const uint8_t *blk, int n_valid, const f16x8 (&qh)[4],
                                 const f16x8 (&ql)[4], const float (&qs)[D / G], float scale_log2, int lane) {
  constexpr int NG = D / G;
  const int kq = lane >> 4;
  const u32x2 kc = *reinterpret_cast<const u32x2 *>(blk + k_codes_off(G) + 8 * lane);
  const u32x2 vc = *reinterpret_cast<const u32x2 *>(blk + v_codes_off(G) + 8 * lane);
  u32x4 km[NG], vm[NG];
  for (int g = 0; g < NG; ++g) {
    km[g] = *reinterpret_cast<const u32x4 *>(blk + k_meta_off(G) + 4 * (16 * g + 4 * kq));
    vm[g] = *reinterpret_cast<const u32x4 *>(blk + v_meta_off(G) + 4 * (16 * g + 4 * kq));
  }
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < NG; ++g) {
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    for (int kb = g * G / 32; kb < (g + 1) * G / 32; ++kb) {
      const f16x8 c = codes_k(kc[0], kc[1], kb);
      d = mfma_k(c, ql[kb], d);
      d = mfma_k(c, qh[kb], d);
    }
    for (int r = 0; r < 4; ++r) s[r] += lo_f16(km[g][r]) * d[r] + hi_f16(km[g][r]) * qs[g];
  }
  bool ok[4];
  float p[4];
  for (int r = 0; r < 4; ++r) {
    ok[r] = 4 * kq + r < n_valid;
    s[r] = ok[r] ? s[r] * scale_log2 : -INFINITY;
  }
  softmax_tile(st, s, p);
  for (int g = 0; g < NG; ++g) {
    float ps[4];
    for (int r = 0; r < 4; ++r) {
      ps[r] = ok[r] ? p[r] * lo_f16(vm[g][r]) : 0.f;
      st.zacc[g] += ok[r] ? p[r] * hi_f16(vm[g][r]) : 0.f;
    }
    f16x4 bh, bl;
    split_f16(ps, bh, bl);
    for (int b = g * G / 16; b < (g + 1) * G / 16; ++b) {
      const f16x4 a = codes_v(vc[0], vc[1], b);
      st.acc_r[b] = mfma_v(a, bl, st.acc_r[b]);
      st.acc_r[b] = mfma_v(a, bh, st.acc_r[b]);
    }
  }
}

template <int GQA, int G>
__global__ void __launch_bounds__(64 * (GQA < 4 ? GQA : 4)) extend_kernel(ExtendArgs a) {
  constexpr int WAVES = GQA < 4 ? GQA : 4;
  constexpr int NG = D / G;
  __shared__ float buf_all[WAVES][EXT_TILE * D];
  const int lane = threadIdx.x & 63, w = wave_id();
  float *buf = buf_all[w];
  const int b = __builtin_amdgcn_workgroup_id_z();
  const int h = __builtin_amdgcn_workgroup_id_y() * WAVES + w;
  const int kh = h / GQA;
  const int t0 = __builtin_amdgcn_workgroup_id_x() * EXT_TILE;
  const int r0 = __builtin_amdgcn_readfirstlane(a.cu_new[b]);
  const int n = __builtin_amdgcn_readfirstlane(a.cu_new[b + 1]) - r0;
  const int L0 = __builtin_amdgcn_readfirstlane(a.len_before[b]);
  if (n < 0 || n > a.max_new || L0 < 0 || L0 > a.max_prefix) {
    if (t0 == 0 && threadIdx.x == 0 && __builtin_amdgcn_workgroup_id_y() == 0) flag_status(a.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  if (t0 >= n) return;
  const int m = lane & 15, kq = lane >> 4;
  const int qi = t0 + m;                          // this lane's query (chunk index)
  const int qrow = r0 + (qi < n ? qi : n - 1);    // a valid row for loads

  // ---- q: bf16 B operands (lane: query m, channels 32 kb + 8 kq .. +7), and
  // fp32 copies in buf[c][16] for the rotation
  bf16x8 qb[4];
  const uint16_t *qp = a.q + (int64_t(qrow) * a.hq + h) * D + 8 * kq;
  for (int kb = 0; kb < 4; ++kb) {
    const u32x4 u = *reinterpret_cast<const u32x4 *>(qp + 32 * kb);
    qb[kb] = __builtin_bit_cast(bf16x8, u);
    for (int e = 0; e < 4; ++e) {
      buf[(32 * kb + 8 * kq + 2 * e) * EXT_TILE + m] = __uint_as_float(u[e] << 16);
      buf[(32 * kb + 8 * kq + 2 * e + 1) * EXT_TILE + m] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  // q R_K: lane computes channels 2 lane, 2 lane + 1 of all 16 queries
  float qr[EXT_TILE][2];
  for (int i = 0; i < EXT_TILE; ++i) qr[i][0] = qr[i][1] = 0.f;
#pragma unroll 2
  for (int c = 0; c < D; ++c) {
    const float2 r = *reinterpret_cast<const float2 *>(a.rk + c * D + 2 * lane);
    for (int i4 = 0; i4 < EXT_TILE / 4; ++i4) {
      const float4 x = *reinterpret_cast<const float4 *>(buf + c * EXT_TILE + 4 * i4);
      const float xs[4] = {x.x, x.y, x.z, x.w};
      for (int e = 0; e < 4; ++e) {
        qr[4 * i4 + e][0] = fmaf(xs[e], r.x, qr[4 * i4 + e][0]);
        qr[4 * i4 + e][1] = fmaf(xs[e], r.y, qr[4 * i4 + e][1]);
      }
    }
  }
  __syncthreads();
  for (int i = 0; i < EXT_TILE; ++i) *reinterpret_cast<float2 *>(buf + i * D + 2 * lane) = make_float2(qr[i][0], qr[i][1]);
  __syncthreads();
  f16x8 qh[4], ql[4];
  float qs[NG];
  for (int g = 0; g < NG; ++g) qs[g] = 0.f;
  for (int kb = 0; kb < 4; ++kb) {
    for (int e = 0; e < 8; ++e) {
      const float x = buf[m * D + 32 * kb + 8 * kq + e];
      const _Float16 hi = _Float16(x);
      qh[kb][e] = hi;
      ql[kb][e] = _Float16(x - float(hi));
      qs[(32 * kb) / G] += x;
    }
  }
  for (int g = 0; g < NG; ++g) {
    qs[g] += shfl_xor(qs[g], 16);
    qs[g] += shfl_xor(qs[g], 32);
  }

  ExtState<NG> st;
  for (int i = 0; i < 8; ++i) st.acc_r[i] = st.acc_p[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < NG; ++g) st.zacc[g] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;

  const int32_t *bpt = a.bf16_pt + int64_t(b) * BF16_PT;
  const int64_t page_elems = int64_t(2) * PAGE * D;  // K and V of one head
  auto bf16_page = [&](int e, const uint16_t *&kp) -> bool {
    const int pid = __builtin_amdgcn_readfirstlane(bpt[e]);
    if (pid < 0 || pid >= a.n_bf16_pages) {
      if (lane == 0) flag_status(a.status, OSCAR_STATUS_BAD_PAGE);
      return false;
    }
    kp = a.bf16 + (int64_t(pid) * a.hkv + kh) * page_elems;
    return true;
  };

  // ---- prefix: sink page
  if (L0 > 0) {
    const uint16_t *kp;
    if (bf16_page(0, kp)) {
      const int ns = L0 < N_SINK ? L0 : N_SINK;
      bf16_tile(st, kp, kp + PAGE * D, D, PAGE, qb, a.scale_log2, lane, [&](int t, int) { return t < ns; });
    }
  }
  // ---- prefix: INT2 history pages
  const int nht = n_hist_tokens(L0), nhp = n_hist_pages(L0);
  const int32_t *hpt = a.hist_pt + int64_t(b) * a.hist_pt_stride;
  const int blk_bytes = hist_block_bytes(G);
#pragma unroll 1
  for (int j = 0; j < nhp; ++j) {
    const int pid = __builtin_amdgcn_readfirstlane(hpt[j]);
    if (pid < 0 || pid >= a.n_hist_pages) {
      if (lane == 0) flag_status(a.status, OSCAR_STATUS_BAD_PAGE);
      continue;
    }
    const uint8_t *blk = a.hist + (int64_t(pid) * a.hkv + kh) * blk_bytes;
    const int nv = nht - PAGE * j < PAGE ? nht - PAGE * j : PAGE;
    hist_tile<G>(st, blk, nv, qh, ql, qs, a.scale_log2, lane);
  }
  // ---- prefix: recent window (ring slot s holds position L0 - 128 + ((s - L0) mod 128))
  if (L0 > N_SINK) {
#pragma unroll 1
    for (int rp = 0; rp < N_RECENT / PAGE; ++rp) {
      const uint16_t *kp;
      if (!bf16_page(1 + rp, kp)) continue;
      bf16_tile(st, kp, kp + PAGE * D, D, PAGE, qb, a.scale_log2, lane, [&](int t, int) {
        const int s = PAGE * rp + t;
        const int pos = L0 - N_RECENT + (((s - L0) % N_RECENT) + N_RECENT) % N_RECENT;
        return pos >= N_SINK;
      });
    }
  }
  // ---- the chunk itself, causal: key j visible to query i iff j <= i
  const int64_t nstride = int64_t(a.hkv) * D;
#pragma unroll 1
  for (int j0 = 0; j0 <= t0; j0 += EXT_TILE) {
    const int nk = n - j0 < EXT_TILE ? n - j0 : EXT_TILE;  // keys of this tile that exist
    const uint16_t *kp = a.k_new + (int64_t(r0 + j0) * a.hkv + kh) * D;
    const uint16_t *vp = a.v_new + (int64_t(r0 + j0) * a.hkv + kh) * D;
    bf16_tile(st, kp, vp, nstride, nk, qb, a.scale_log2, lane, [&](int t, int i) {
      return t < nk && (i < 0 || j0 + t <= t0 + i);
    });
  }

  // ---- epilogue: totals over the four lanes of each query
  st.l += shfl_xor(st.l, 16);
  st.l += shfl_xor(st.l, 32);
  for (int g = 0; g < NG; ++g) {
    st.zacc[g] += shfl_xor(st.zacc[g], 16);
    st.zacc[g] += shfl_xor(st.zacc[g], 32);
  }
  // rotated part (+ zero-point sums) into buf[c][16], then times R_V^T
  __syncthreads();
  for (int bb = 0; bb < 8; ++bb)
    for (int r = 0; r < 4; ++r) {
      const int c = 16 * bb + 4 * kq + r;
      buf[c * EXT_TILE + m] = st.acc_r[bb][r] + st.zacc[c / G];
    }
  __syncthreads();
  float o[EXT_TILE][2];
  for (int i = 0; i < EXT_TILE; ++i) o[i][0] = o[i][1] = 0.f;
#pragma unroll 2
  for (int c = 0; c < D; ++c) {
    const float2 r = *reinterpret_cast<const float2 *>(a.rvt + c * D + 2 * lane);
    for (int i4 = 0; i4 < EXT_TILE / 4; ++i4) {
      const float4 x = *reinterpret_cast<const float4 *>(buf + c * EXT_TILE + 4 * i4);
      const float xs[4] = {x.x, x.y, x.z, x.w};
      for (int e = 0; e < 4; ++e) {
        o[4 * i4 + e][0] = fmaf(xs[e], r.x, o[4 * i4 + e][0]);
        o[4 * i4 + e][1] = fmaf(xs[e], r.y, o[4 * i4 + e][1]);
      }
    }
  }
  __syncthreads();
  // BF16 part into buf[c][16]
  for (int bb = 0; bb < 8; ++bb)
    for (int r = 0; r < 4; ++r) {
      const int c = 32 * (bb >> 1) + 2 * (4 * kq + r) + (bb & 1);
      buf[c * EXT_TILE + m] = st.acc_p[bb][r];
    }
  __syncthreads();
  const float inv = 1.f / st.l;
  for (int jj = 0; jj < 2; ++jj)
    for (int i = 0; i < EXT_TILE; ++i) o[i][jj] += buf[(2 * lane + jj) * EXT_TILE + i];
  for (int i = 0; i < EXT_TILE; ++i) {
    if (t0 + i >= n) break;
    const float s = lane_value(inv, i);
    *reinterpret_cast<float2 *>(a.out + (int64_t(r0 + t0 + i) * a.hq + h) * D + 2 * lane) =
        make_float2(o[i][0] * s, o[i][1] * s);
  }
}

template <int GQA>
hipError_t launch_gqa(const ExtendArgs &a, int G, int batch, int max_new, hipStream_t s) {
  constexpr int WAVES = GQA < 4 ? GQA : 4;
  const dim3 grid((max_new + EXT_TILE - 1) / EXT_TILE, a.hq / WAVES, batch);
  const KernelEvents ev = take_profile_events();
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, grid, dim3(64 * WAVES), 0, s, ev.before, ev.after, 0, a);
  };
  if (G == 32) go(extend_kernel<GQA, 32>);
  else if (G == 64) go(extend_kernel<GQA, 64>);
  else go(extend_kernel<GQA, 128>);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_extend(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q, int n_q_heads,
                         const uint16_t *k_new, const uint16_t *v_new, const int32_t *cu_new,
                         const int32_t *len_before, int batch, int max_new, int max_prefix, float sm_scale,
                         float *out, hipStream_t s) {
  ExtendArgs a;
  a.hist = c.hist;
  a.n_hist_pages = c.n_hist_pages;
  a.bf16 = c.bf16;
  a.n_bf16_pages = c.n_bf16_pages;
  a.hist_pt = c.hist_pt;
  a.hist_pt_stride = c.hist_pt_stride;
  a.bf16_pt = c.bf16_pt;
  a.status = c.status;
  a.rk = reinterpret_cast<const float *>(rk.forms + FORM_R);
  a.rvt = reinterpret_cast<const float *>(rv.forms + FORM_RT);
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cu_new = cu_new;
  a.len_before = len_before;
  a.hq = n_q_heads;
  a.hkv = c.n_kv_heads;
  a.max_new = max_new;
  a.max_prefix = max_prefix;
  a.scale_log2 = sm_scale * LOG2E;
  a.out = out;
  switch (n_q_heads / c.n_kv_heads) {
    case 1: return launch_gqa<1>(a, c.group, batch, max_new, s);
    case 2: return launch_gqa<2>(a, c.group, batch, max_new, s);
    case 4: return launch_gqa<4>(a, c.group, batch, max_new, s);
    default: return launch_gqa<8>(a, c.group, batch, max_new, s);
  }
}

}  // namespace oscar
