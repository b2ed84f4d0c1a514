// Extend (chunked-prefill) attention over the mixed-precision cache: the new
// tokens of a request attend to its cached prefix -- BF16 sink and recent
// window, INT2 (or INT4) history read through dequantisation in the rotated
// basis -- and
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
//   history (INT2) tiles: A = the stored 2-bit codes expanded to fp16 1 + c w
//     (w = 1/4 or 1/16, the decode's expansion), B = q R_K / w split into
//     fp16 high and low parts (scores: exact products, fp32 sums, the
//     constant 1 taken off per group) or p s_V / w scaled by a power of two
//     and rounded to fp16 once (values: one rounding per weight); scale and
//     zero of a group enter per key: score = sum_g s_g (q_g . c_g) + z_g
//     sum(q_g), value = sum_t p_t s_t c_t + (sum_t p_t z_t);
//   BF16 tiles (sink, ring, chunk): A = raw bf16 rows, B = q (bf16, exact)
//     or p split into bf16 high and low parts.
// The history accumulator stays in the rotated basis and is brought back with
// R_V^T once per query at the end.
#include <cmath>
#include <type_traits>

#include "attn_common.h"

namespace oscar {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct ExtendArgs {
  const uint8_t *hist;
  int n_hist_pages;  // below 2^31 (page ids are int32): scalar compares
  const uint16_t *bf16;
  int n_bf16_pages;
  const int32_t *hist_pt;
  int hist_pt_stride;
  const int32_t *bf16_pt;
  uint32_t *status;
  const float *rk;   // fp32 R_K[i][j] at i*128 + j
  const float *rvt;  // fp32 R_V[j][c] at c*128 + j
  int64_t rk_stride, rv_stride;  // floats between KV heads' forms (0: one rotation for the layer)
  const uint16_t *q, *k_new, *v_new;
  const int32_t *cu_new, *len_before;
  int hq, hkv, max_new, max_prefix;
  int64_t total_tokens;  // rows of q / k_new / v_new / out
  float scale_log2;  // sm_scale * log2(e)
  float pv_scale;    // power of two: p s_V pv_scale stays below 2^15 (fp16 operand)
  float pk4, pk16;   // log2(4 pv_scale), log2(16 pv_scale): the PV weights of the history rows
  uint32_t ex_m4, ex_m16, ex_e;  // code expansion constants 0x03000300, 0x00C000C0, 0x3C003C00
  uint32_t ex_mn;                // INT4 expansion mask 0x03C003C0
  int bits;                      // history code width (2 or 4)
  float *out;
};

constexpr int EXT_TILE = 16;

// Max / sum over the four lanes l, l^16, l^32, l^48 that hold one query
// (row swaps between lanes, no LDS round trip); every one of them receives it.
__device__ inline float lanes4_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float lanes4_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

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

// Online-softmax state of one part of the keys: the BF16 keys (sink, window,
// chunk; acc = O^T in the original basis) or the INT2 history (acc = O^T in
// the rotated basis, cacc = the column sums of the PV operands per group,
// which the expansion's constant 1 adds to acc, and the zero-point sums per
// group).  The two parts are merged at the end, so only one part's
// accumulators are live at a time.
// History tiles (NZ > 0) keep two classes of the lane's four keys, rows 0, 1
// and rows 2, 3: their probabilities come out of the exponential already
// multiplied by the PV operand's power-of-two weight 2^off_a / 2^off_b (INT2:
// pv_scale * 4 / pv_scale * 16; INT4: pv_scale * 16 for both), and their
// sums (l / lb, zacc / zb) are taken per class and unweighted at the end.
template <int NZ>
struct SoftState {
  static constexpr int NZ1 = NZ > 0 ? NZ : 1;
  f32x4 acc[8];
  f32x4 cacc[NZ1];
  float zacc[NZ1], zb[NZ1];     // sum_t p_t z_t of the lane's keys, per group (rows 0, 1 / 2, 3)
  float m, l, lb;               // running max (log2 units) of the lane's query; lane-partial sums
  float thr, nref, nrb;         // m + LAZY_TH (the raise test); off_a - m and off_b - m (off - 0 while m = -inf)
  float offa, offb;             // the classes' weights, log2
  __device__ void init(float off_a = 0.f, float off_b = 0.f) {
    for (int b = 0; b < 8; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < NZ1; ++g) {
      cacc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      zacc[g] = zb[g] = 0.f;
    }
    m = -INFINITY;
    l = lb = 0.f;
    thr = -INFINITY;
    offa = off_a;
    offb = off_b;
    nref = off_a;
    nrb = off_b;
  }
};

// Online softmax over one tile: s[r] * sc = score of key 4(l/16)+r for the
// lane's query in log2 units (-inf where masked; sc > 0); p[r] receives the
// probabilities relative to the running max.  The running max is raised
// only when a score exceeds it by more than 2^LAZY_TH (so p <= 2^LAZY_TH);
// the accumulators are rescaled only in the waves where some query's max was
// raised.
template <int NZ>
__device__ inline void softmax_tile(SoftState<NZ> &st, const float (&s)[4], float (&p)[4], float sc = 1.f) {
  // the lane's own four keys decide whether any query may need a new max
  // (the four lanes of a query share its running max); the query's max over
  // its 16 keys is formed only then
  const float lmx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * sc;
  if (__builtin_amdgcn_ballot_w64(lmx > st.thr)) {  // false while both are -inf
    const float mx = lanes4_max(lmx);
    const bool raise = mx > st.thr;
    const float mn = raise ? mx : st.m;
    const float alpha = raise ? __builtin_amdgcn_exp2f(st.m - mn) : 1.f;  // st.m = -inf: 0
    st.l *= alpha;
    if constexpr (NZ > 0) st.lb *= alpha;
    for (int b = 0; b < 8; ++b) st.acc[b] *= alpha;
    for (int g = 0; g < NZ; ++g) {
      st.cacc[g] *= alpha;
      st.zacc[g] *= alpha;
      st.zb[g] *= alpha;
    }
    st.m = mn;
    st.thr = mn + LAZY_TH;
    const float base = mn == -INFINITY ? 0.f : -mn;
    st.nref = base + st.offa;
    st.nrb = base + st.offb;
  }
  if constexpr (NZ > 0) {
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sc, r < 2 ? st.nref : st.nrb));
    st.l += p[0] + p[1];
    st.lb += p[2] + p[3];
  } else {
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sc, st.nref));
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
  }
}

// One tile of 16 raw bf16 keys: key t's K row at kp + t * stride (elements),
// V row at vp + t * stride, for t < nrows; rows t >= nrows are not read (their
// loads repeat row 0).  valid(t, i) says whether key t is visible to query i
// of the tile, valid(t, -1) whether key t exists at all.
template <class Valid>
__device__ inline void bf16_tile(SoftState<0> &st, const uint16_t *kp, const uint16_t *vp, int64_t stride,
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
    st.acc[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, phi, st.acc[2 * c], 0, 0, 0);
    st.acc[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, plo, st.acc[2 * c], 0, 0, 0);
    st.acc[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, phi, st.acc[2 * c + 1], 0, 0, 0);
    st.acc[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, plo, st.acc[2 * c + 1], 0, 0, 0);
  }
}

// One history page (block of one KV head): the lane's code dwords (INT2: 8
// bytes per tensor, INT4: 16) and the scale / zero entries of its four keys
// per group.
template <int NG, int BITS>
struct HistData {
  typedef typename std::conditional<BITS == 2, u32x2, u32x4>::type Codes;
  Codes kc, vc;
  u32x4 km[NG], vm[NG];
};

template <int G, int BITS>
__device__ inline void hist_load(HistData<D / G, BITS> &hd, const uint8_t *blk, int lane) {
  typedef typename HistData<D / G, BITS>::Codes Codes;
  const int kq = lane >> 4;
  hd.kc = *reinterpret_cast<const Codes *>(blk + k_codes_off(G, BITS) + sizeof(Codes) * lane);
  hd.vc = *reinterpret_cast<const Codes *>(blk + v_codes_off(G, BITS) + sizeof(Codes) * lane);
  for (int g = 0; g < D / G; ++g) {
    hd.km[g] = *reinterpret_cast<const u32x4 *>(blk + k_meta_off(G, BITS) + 4 * (16 * g + 4 * kq));
    hd.vm[g] = *reinterpret_cast<const u32x4 *>(blk + v_meta_off(G, BITS) + 4 * (16 * g + 4 * kq));
  }
}

// Attention over one loaded history page.  MASKED: only rows < n_valid
// exist (the others, and their meta, may hold anything), so their scores are
// -inf and their value operands zero; a full page (every row written) runs
// without the masks.
template <int G, int BITS, bool MASKED>
__device__ inline void hist_tile(SoftState<D / G> &st, const HistData<D / G, BITS> &hd, int n_valid,
                                 const f16x8 (&qh)[4], const f16x8 (&ql)[4], const float (&qs)[D / G],
                                 const float (&qoff)[D / G], float inv_kqs, float pv_scale, const Expander &ex,
                                 const Expander4 &ex4, int lane) {
  constexpr int NG = D / G;
  const int kq = lane >> 4;
  float s[4];
  for (int g = 0; g < NG; ++g) {
    // starts at minus the sum of the operands: the expansion's constant 1
    // comes off in the accumulator, d = sum_c c q_c (q carries 1/w, the
    // softmax scale and kqs)
    f32x4 d = {-qoff[g], -qoff[g], -qoff[g], -qoff[g]};
    for (int kb = g * G / 32; kb < (g + 1) * G / 32; ++kb) {
      // 1 + c w: INT2 w = 1/4 or 1/16, INT4 w = 1/16
      f16x8 x;
      if constexpr (BITS == 2)
        x = ex.k(hd.kc[0], hd.kc[1], kb);
      else
        x = ex4.k(hd.kc[kb]);
      d = mfma_k(x, ql[kb], d);
      d = mfma_k(x, qh[kb], d);
    }
    // s += z_g qs_g + s_g d (two mixed-precision FMAs on the packed meta)
    for (int r = 0; r < 4; ++r) {
      const float t = fmaf(hi_f16(hd.km[g][r]), qs[g], g == 0 ? 0.f : s[r]);
      s[r] = fmaf(lo_f16(hd.km[g][r]), d[r], t);
    }
  }
  bool ok[4];
  float p[4];
  for (int r = 0; r < 4; ++r) {
    ok[r] = !MASKED || 4 * kq + r < n_valid;
    s[r] = ok[r] ? s[r] : -INFINITY;
  }
  softmax_tile(st, s, p, inv_kqs);  // scores in kqs units
  // A = 1 + c w (INT2: w = 1/4 for rows 0, 1 of the lane's four keys, 1/16
  // for rows 2, 3; INT4: 1/16), B = fp16(p s k / w): the product is B + c p s k; the column
  // sums of B come off at the end (cacc: the same B against an all-ones
  // operand), the zero points enter as sum_t p_t z_t
  // (p carries the weight already: the softmax state's class offsets)
  const f16x4 ones = as_f16x4(0x3C003C00u, 0x3C003C00u);
  for (int g = 0; g < NG; ++g) {
    f16x4 bp;
    for (int r = 0; r < 4; ++r) {
      bp[r] = _Float16(ok[r] ? fmaf(p[r], lo_f16(hd.vm[g][r]), 0.f) : 0.f);  // one v_fma_mixlo_f16
      float &z = r < 2 ? st.zacc[g] : st.zb[g];
      z = ok[r] ? fmaf(p[r], hi_f16(hd.vm[g][r]), z) : z;
    }
    st.cacc[g] = mfma_v(ones, bp, st.cacc[g]);
    for (int b = g * G / 16; b < (g + 1) * G / 16; ++b) {
      if constexpr (BITS == 2)
        st.acc[b] = mfma_v(ex.v(hd.vc[0], hd.vc[1], b), bp, st.acc[b]);
      else
        st.acc[b] = mfma_v(ex4.v(hd.vc[b >> 1], b & 1), bp, st.acc[b]);
    }
  }
}

template <int GQA, int G, int BITS>
__global__ void __launch_bounds__(64 * (GQA < 4 ? GQA : 4)) __attribute__((amdgpu_waves_per_eu(2)))
extend_kernel(ExtendArgs a) {
  constexpr int WAVES = GQA < 4 ? GQA : 4;
  constexpr int NG = D / G;
  __shared__ float buf_all[WAVES][2][EXT_TILE * D];
  const int lane = threadIdx.x & 63, w = wave_id();
  float *buf = buf_all[w][0];   // q staging, then the history part of the output
  float *bufp = buf_all[w][1];  // the BF16 part of the output
  const int b = __builtin_amdgcn_workgroup_id_z();
  const int h = __builtin_amdgcn_workgroup_id_y() * WAVES + w;
  const int kh = h / GQA;
  const int t0 = __builtin_amdgcn_workgroup_id_x() * EXT_TILE;
  const int r0 = __builtin_amdgcn_readfirstlane(a.cu_new[b]);
  const int n = __builtin_amdgcn_readfirstlane(a.cu_new[b + 1]) - r0;
  const int L0 = __builtin_amdgcn_readfirstlane(a.len_before[b]);
  // the request's rows must lie inside the total_tokens rows of the inputs
  // and the output (no access outside them), its counts inside the bounds
  // the grid was sized for
  if (r0 < 0 || n < 0 || n > a.max_new || int64_t(r0) + n > a.total_tokens || L0 < 0 || L0 > a.max_prefix) {
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
    const float2 r = *reinterpret_cast<const float2 *>(a.rk + kh * a.rk_stride + c * D + 2 * lane);
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
  // history operands: y = q R_K sm_scale log2(e) kqs / w (w = 1/4 or 1/16
  // per element, the weight of the code expansion) as fp16 high + low
  // parts; kqs is a power of two that brings the wave's largest |y| into
  // (2^13, 2^14]: no fp16 overflow for large q or sm_scale, and the low
  // parts stay normal numbers for the elements that matter; scores come out
  // in kqs units and are multiplied by 1/kqs.  qs = sum of the scaled q per
  // group (zero points), qoff = sum of the operands as used (the
  // expansion's constant 1), both in kqs units.
  float amax = 0.f;
  for (int kb = 0; kb < 4; ++kb)
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(buf[m * D + 32 * kb + 8 * kq + e]));
  amax = wave_max(amax) * a.scale_log2 * 16.f;
  float kqs = 1.f;
  if (amax > 0.f && amax < INFINITY) {
    int ex;
    (void)frexpf(amax, &ex);              // amax in [2^(ex-1), 2^ex)
    kqs = ldexpf(1.f, 14 - ex);           // amax kqs in [2^13, 2^14)
  }
  const float inv_kqs = 1.f / kqs;
  f16x8 qh[4], ql[4];
  float qs[NG], qoff[NG];
  for (int g = 0; g < NG; ++g) qs[g] = qoff[g] = 0.f;
  for (int kb = 0; kb < 4; ++kb) {
    for (int e = 0; e < 8; ++e) {
      const float x = buf[m * D + 32 * kb + 8 * kq + e] * a.scale_log2 * kqs;
      const float y = x * ((BITS == 4 || (e & 2)) ? 16.f : 4.f);
      const _Float16 hi = _Float16(y);
      const _Float16 lo = _Float16(y - float(hi));
      qh[kb][e] = hi;
      ql[kb][e] = lo;
      qs[(32 * kb) / G] += x;
      qoff[(32 * kb) / G] += float(hi) + float(lo);
    }
  }
  for (int g = 0; g < NG; ++g) {
    qs[g] = lanes4_sum(qs[g]);
    qoff[g] = lanes4_sum(qoff[g]);
  }

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

  // ======== BF16 keys: sink, recent window, the chunk
  SoftState<0> sp;
  sp.init();
  if (L0 > 0) {
    const uint16_t *kp;
    if (bf16_page(0, kp)) {
      const int ns = L0 < N_SINK ? L0 : N_SINK;
      bf16_tile(sp, kp, kp + PAGE * D, D, PAGE, qb, a.scale_log2, lane, [&](int t, int) { return t < ns; });
    }
  }
  // ring slot s holds position L0 - 128 + ((s - L0) mod 128)
  if (L0 > N_SINK) {
#pragma unroll 1
    for (int rp = 0; rp < N_RECENT / PAGE; ++rp) {
      // a ring page without a visible token is never looked up (its table
      // entry may be unset while the window is still filling)
      if (!raw_valid_rows(L0, 1 + rp)) continue;
      const uint16_t *kp;
      if (!bf16_page(1 + rp, kp)) continue;
      bf16_tile(sp, kp, kp + PAGE * D, D, PAGE, qb, a.scale_log2, lane, [&](int t, int) {
        const int s = PAGE * rp + t;
        const int pos = L0 - N_RECENT + (((s - L0) % N_RECENT) + N_RECENT) % N_RECENT;
        return pos >= N_SINK;
      });
    }
  }
  // the chunk itself, causal: key j visible to query i iff j <= i
  const int64_t nstride = int64_t(a.hkv) * D;
#pragma unroll 1
  for (int j0 = 0; j0 <= t0; j0 += EXT_TILE) {
    const int nk = n - j0 < EXT_TILE ? n - j0 : EXT_TILE;  // keys of this tile that exist
    const uint16_t *kp = a.k_new + (int64_t(r0 + j0) * a.hkv + kh) * D;
    const uint16_t *vp = a.v_new + (int64_t(r0 + j0) * a.hkv + kh) * D;
    bf16_tile(sp, kp, vp, nstride, nk, qb, a.scale_log2, lane, [&](int t, int i) {
      return t < nk && (i < 0 || j0 + t <= t0 + i);
    });
  }
  // park the BF16 accumulator in LDS (bufp[c][16], unnormalised)
  for (int bb = 0; bb < 8; ++bb)
    for (int r = 0; r < 4; ++r) {
      const int c = 32 * (bb >> 1) + 2 * (4 * kq + r) + (bb & 1);
      bufp[c * EXT_TILE + m] = sp.acc[bb][r];
    }
  const float m1 = sp.m, l1 = lanes4_sum(sp.l);

  // ======== history pages (INT2 or INT4)
  const float pv_unscale = 1.f / a.pv_scale;
  SoftState<NG> sh;
  // rows 0, 1 of an INT2 page carry weight 4 pv_scale, rows 2, 3 (and every
  // INT4 row) 16 pv_scale
  sh.init(BITS == 2 ? a.pk4 : a.pk16, a.pk16);
  Expander ex;
  ex.m4 = a.ex_m4;
  ex.m16 = a.ex_m16;
  ex.e = a.ex_e;
  // the exponent pattern in a VGPR, the masks in SGPRs: one v_and_or_b32
  // per expanded register (the empty asm emits nothing)
  asm volatile("" : "+v"(ex.e));
  Expander4 ex4;
  ex4.m = a.ex_mn;
  ex4.e = ex.e;
  const int nht = n_hist_tokens(L0), nhp = n_hist_pages(L0);
  const int32_t *hpt = a.hist_pt + int64_t(b) * a.hist_pt_stride;
  const int blk_bytes = hist_block_bytes(G, BITS);
  // page ids 64 at a time (lane i: page j0 + i, -1 past the end); the next
  // page's data is loaded while the current one is computed
  auto page_block = [&](int pid) -> const uint8_t * { return a.hist + (int64_t(pid) * a.hkv + kh) * blk_bytes; };
  auto bad_page = [&](int pid) { return pid < 0 || pid >= a.n_hist_pages; };
  if (nhp > 0) {
    int ids = lane < nhp ? hpt[lane] : -1;
    // page j's id and data; a bad page is never read
    auto page_id = [&](int j) {
      if (j > 0 && (j & 63) == 0) ids = j + lane < nhp ? hpt[j + lane] : -1;
      return __builtin_amdgcn_readlane(ids, j & 63);
    };
    // full pages (every row written) run unmasked; only the last page can
    // be partial, and it runs after the loop
    auto run_full = [&](int pid, const HistData<NG, BITS> &hd) {
      if (bad_page(pid)) {
        if (lane == 0) flag_status(a.status, OSCAR_STATUS_BAD_PAGE);
        return;
      }
      hist_tile<G, BITS, false>(sh, hd, PAGE, qh, ql, qs, qoff, inv_kqs, a.pv_scale, ex, ex4, lane);
    };
    const int nfull = nht / PAGE;
    HistData<NG, BITS> d0, d1;
    int p0 = page_id(0), p1 = -1;
    if (!bad_page(p0)) hist_load<G, BITS>(d0, page_block(p0), lane);
    int j = 0;
#pragma unroll 1
    for (; j + 2 <= nfull; j += 2) {
      // d0 holds page j; page j + 1 goes to d1, page j + 2 to d0
      if (j + 1 < nhp) {
        p1 = page_id(j + 1);
        if (!bad_page(p1)) hist_load<G, BITS>(d1, page_block(p1), lane);
      }
      run_full(p0, d0);
      if (j + 2 < nhp) {
        p0 = page_id(j + 2);
        if (!bad_page(p0)) hist_load<G, BITS>(d0, page_block(p0), lane);
      }
      run_full(p1, d1);
    }
    // the partial last page, if any
    auto run_last = [&](int jj, int pid, const HistData<NG, BITS> &hd) {
      if (bad_page(pid)) {
        if (lane == 0) flag_status(a.status, OSCAR_STATUS_BAD_PAGE);
        return;
      }
      hist_tile<G, BITS, true>(sh, hd, nht - PAGE * jj, qh, ql, qs, qoff, inv_kqs, a.pv_scale, ex, ex4, lane);
    };
    if (j < nfull) {
      // one full page left (in d0), maybe followed by the partial page (d1)
      const bool more = j + 1 < nhp;
      if (more) {
        p1 = page_id(j + 1);
        if (!bad_page(p1)) hist_load<G, BITS>(d1, page_block(p1), lane);
      }
      run_full(p0, d0);
      if (more) run_last(j + 1, p1, d1);
    } else if (j < nhp) {
      run_last(j, p0, d0);  // in d0
    }
  }

  // ======== merge: o = (f2 (acc_r + z) R_V^T + f1 acc_p) / (f1 l1 + f2 l2)
  // the two classes' sums without their weights
  const float ua = exp2f(-sh.offa), ub = exp2f(-sh.offb);
  const float l2 = lanes4_sum(fmaf(sh.l, ua, sh.lb * ub));
  for (int g = 0; g < NG; ++g) sh.zacc[g] = lanes4_sum(fmaf(sh.zacc[g], ua, sh.zb[g] * ub));
  const float mm = fmaxf(m1, sh.m);  // finite: every query sees at least itself
  const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
  const float f2 = sh.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sh.m - mm);
  const float inv = 1.f / (f1 * l1 + f2 * l2);
  for (int bb = 0; bb < 8; ++bb)
    for (int r = 0; r < 4; ++r) {
      const int c = 16 * bb + 4 * kq + r;
      buf[c * EXT_TILE + m] = fmaf(sh.acc[bb][r] - sh.cacc[c / G][r], pv_unscale, sh.zacc[c / G]) * f2;
    }
  __syncthreads();
  float o[EXT_TILE][2];
  for (int i = 0; i < EXT_TILE; ++i) o[i][0] = o[i][1] = 0.f;
#pragma unroll 2
  for (int c = 0; c < D; ++c) {
    const float2 r = *reinterpret_cast<const float2 *>(a.rvt + kh * a.rv_stride + c * D + 2 * lane);
    for (int i4 = 0; i4 < EXT_TILE / 4; ++i4) {
      const float4 x = *reinterpret_cast<const float4 *>(buf + c * EXT_TILE + 4 * i4);
      const float xs[4] = {x.x, x.y, x.z, x.w};
      for (int e = 0; e < 4; ++e) {
        o[4 * i4 + e][0] = fmaf(xs[e], r.x, o[4 * i4 + e][0]);
        o[4 * i4 + e][1] = fmaf(xs[e], r.y, o[4 * i4 + e][1]);
      }
    }
  }
  for (int i = 0; i < EXT_TILE; ++i) {
    if (t0 + i >= n) break;
    const float fi = lane_value(f1, i), si = lane_value(inv, i);
    const float p0 = bufp[(2 * lane) * EXT_TILE + i], p1 = bufp[(2 * lane + 1) * EXT_TILE + i];
    *reinterpret_cast<float2 *>(a.out + (int64_t(r0 + t0 + i) * a.hq + h) * D + 2 * lane) =
        make_float2(fmaf(fi, p0, o[i][0]) * si, fmaf(fi, p1, o[i][1]) * si);
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
  const bool int4 = a.bits == 4;
  if (G == 32) int4 ? go(extend_kernel<GQA, 32, 4>) : go(extend_kernel<GQA, 32, 2>);
  else if (G == 64) int4 ? go(extend_kernel<GQA, 64, 4>) : go(extend_kernel<GQA, 64, 2>);
  else int4 ? go(extend_kernel<GQA, 128, 4>) : go(extend_kernel<GQA, 128, 2>);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_extend(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q, int n_q_heads,
                         const uint16_t *k_new, const uint16_t *v_new, const int32_t *cu_new,
                         const int32_t *len_before, int batch, int64_t total_tokens, int max_new,
                         int max_prefix, float sm_scale, float *out, hipStream_t s) {
  ExtendArgs a;
  a.hist = c.hist;
  a.n_hist_pages = int(c.n_hist_pages);
  a.bf16 = c.bf16;
  a.n_bf16_pages = int(c.n_bf16_pages);
  a.hist_pt = c.hist_pt;
  a.hist_pt_stride = c.hist_pt_stride;
  a.bf16_pt = c.bf16_pt;
  a.status = c.status;
  a.rk = reinterpret_cast<const float *>(rk.forms + FORM_R);
  a.rvt = reinterpret_cast<const float *>(rv.forms + FORM_RT);
  a.rk_stride = rk.stride / 4;
  a.rv_stride = rv.stride / 4;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cu_new = cu_new;
  a.len_before = len_before;
  a.hq = n_q_heads;
  a.hkv = c.n_kv_heads;
  a.max_new = max_new;
  a.max_prefix = max_prefix;
  a.total_tokens = total_tokens;
  a.scale_log2 = sm_scale * LOG2E;
  // p <= 2^LAZY_TH, s_V <= 2 clip_V / 3, 1/w <= 16: the fp16 operand
  // p s_V k / w stays in [2^14, 2^15) at its largest
  float k = 1.f;
  const float vmax = exp2f(LAZY_TH) * 16.f * (2.f * rv.clip / 3.f);
  while (vmax * k > 32768.f) k *= 0.5f;
  while (vmax * k * 2.f <= 32768.f && k < 65536.f) k *= 2.f;
  a.pv_scale = k;
  a.pk4 = std::log2(4.f * k);
  a.pk16 = std::log2(16.f * k);
  a.ex_m4 = 0x03000300u;
  a.ex_m16 = 0x00C000C0u;
  a.ex_e = 0x3C003C00u;
  a.ex_mn = 0x03C003C0u;
  a.bits = cache_bits(c);
  a.out = out;
  switch (n_q_heads / c.n_kv_heads) {
    case 1: return launch_gqa<1>(a, c.group, batch, max_new, s);
    case 2: return launch_gqa<2>(a, c.group, batch, max_new, s);
    case 4: return launch_gqa<4>(a, c.group, batch, max_new, s);
    default: return launch_gqa<8>(a, c.group, batch, max_new, s);
  }
}

}  // namespace oscar
