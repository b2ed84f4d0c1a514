// Mixed-precision paged decode attention over the OSCAR cache.
//
// OSCAR online phase (gist.science nl/fr technical summaries, section 2.2.B:
// one fused kernel unpacks, dequantises, undoes the rotation and attends over
// the INT2 history on paged storage with prefix caching; arXiv:2605.17757 v2
// abstract: batch-1 decode gains come from cutting KV memory traffic).
//
// The rotation is never undone per token: history keys stay in the rotated
// basis and are scored against q R_K (R orthogonal keeps q.k), and the
// history part of the output is rotated back by R_V^T once per (request,
// query head) in the merge.  Per-group scale s and zero z are factored out of
// both contractions, so the matrix cores see the 2-bit codes as exact fp16
// values:
//   score_t = sum_g s_tg (q_g . c_tg) + z_tg sum_{i in g} q_i
//   o       = sum_g [ sum_t (p_t s_tg) c_tg ] + sum_t p_t z_tg
//
// Kernels, in stream order:
//   qprep:  per (request, KV head): q_rot = q R_K * sm_scale * log2(e) for the
//           query heads of the group, laid out as the B operand of the score
//           MFMAs (fp16 high + low parts), with the column sums that cancel
//           the code expansion's constant and the per-group sums of q_rot.
//   split:  one workgroup (4 waves) per (request, KV head, split).  Split 0
//           attends over the raw BF16 sink + recent pages; split s >= 1 over
//           history pages, each wave taking every 4th page.  Writes an
//           unnormalised partial (o[128], m, l) per query head.
//   merge:  LSE-combines the splits, rotates the history part back with
//           R_V^T, adds the raw part and normalises (fp32 out).
#include "attn_common.h"

namespace oscar {

constexpr int FRAG_DW = 32;  // dwords per lane of the q fragment block

// Column layout of the score and PV accumulators for a GQA group of GQA heads
// and NG scale groups: column n = h + GQA * (part + 2 * cg); part 0/1 = fp16
// high/low part of the fp32 operand, cg = which of the CG groups sharing an
// accumulator.  NA accumulators cover the NG groups.
template <int GQA, int NG>
struct Cols {
  static constexpr int CG0 = 16 / (2 * GQA);
  static constexpr int CG = CG0 < NG ? CG0 : NG;
  static constexpr int NA = (NG + CG - 1) / CG;
  static constexpr int G = D / NG;
  __device__ static int grp_of_kblock(int k) { return (32 * k) / G; }   // 32-channel block
  __device__ static int grp_of_rblock(int r) { return (16 * r) / G; }   // 16-channel block
};

SplitPlan plan_int2_splits(int batch, int n_kv_heads, int max_seq_len) {
  const int pages = n_hist_pages(max_seq_len);
  SplitPlan p;
  if (pages == 0) {
    p.pages_per_split = WAVES;
    p.n_splits = 0;
    return p;
  }
  // about 1024 workgroups per launch for the longest request (4 per CU)
  const int64_t total = int64_t(pages) * batch * n_kv_heads;
  int64_t pw = (total + int64_t(WAVES) * 1024 - 1) / (int64_t(WAVES) * 1024);
  if (pw < 2) pw = 2;
  if (pw > 32) pw = 32;
  p.pages_per_split = int(pw) * WAVES;
  p.n_splits = (pages + p.pages_per_split - 1) / p.pages_per_split;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static size_t frag_bytes(int batch, int hkv) { return align256(size_t(batch) * hkv * FRAG_DW * 64 * 4); }

size_t decode_int2_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  const SplitPlan p = plan_int2_splits(batch, n_kv_heads, max_seq_len);
  return frag_bytes(batch, n_kv_heads) +
         align256(size_t(batch) * n_q_heads * (1 + p.n_splits) * PART_STRIDE * sizeof(float));
}

struct DecodeArgs {
  oscar_layer_cache c;
  const uint8_t *fk, *fv;
  const uint16_t *q;
  const int32_t *seq_lens;
  int n_q_heads, max_seq_len, pages_per_split, n_splits;
  float sm_scale;
  float pv_scale, pv_unscale;  // 2^k and 2^-k applied to the PV operand
  uint32_t *frag;              // [B][Hkv][FRAG_DW][64]
  float *parts;                // [B][Hq][1 + n_splits][PART_STRIDE]
  float *out;
};

__device__ inline bool valid_len(int L, int max_len) { return L >= 1 && L <= max_len; }

// ------------------------------------------------------------------ qprep

template <int GQA, int NG>
__global__ void __launch_bounds__(256) qprep_kernel(DecodeArgs a) {
  using C = Cols<GQA, NG>;
  const int hk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ float qs[GQA][D];   // bf16 query, fp32
  __shared__ float qr[GQA][D];   // q R_K * sm_scale * log2(e)
  __shared__ float qz[GQA][NG];  // per-group sums of qr
  __shared__ float red[256];
  for (int e = tid; e < GQA * D; e += 256)
    qs[e / D][e % D] = bf16_to_f32(a.q[(int64_t(b) * a.n_q_heads + hk * GQA) * D + e]);
  __syncthreads();
  const float *R = reinterpret_cast<const float *>(a.fk + FORM_R);
  const float sc = a.sm_scale * LOG2E;
  float amax = 0.f;
  for (int e = tid; e < GQA * D; e += 256) {
    const int h = e / D, j = e % D;
    float s = 0.f;
    for (int i = 0; i < D; ++i) s = fmaf(qs[h][i], R[i * D + j], s);
    qr[h][j] = s * sc;
    amax = fmaxf(amax, fabsf(s * sc));
  }
  red[tid] = amax;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  // the B operand holds qr * 16 at most: scale down by a power of two if that
  // would leave the fp16 range (never for ordinary queries)
  float kq = 1.f;
  while (red[0] * 16.f * kq > 16384.f) kq *= 0.5f;
  if (tid < GQA * NG) {
    const int h = tid / NG, g = tid % NG;
    float s = 0.f;
    for (int i = 0; i < C::G; ++i) s += qr[h][g * C::G + i];
    qz[h][g] = s;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid, n = lane & 15, qd = lane >> 4;
    const int h = n % GQA, part = (n / GQA) & 1, cg = n / (2 * GQA);
    const bool ncol = cg < C::CG;
    uint32_t *fr = a.frag + (int64_t(b) * a.c.n_kv_heads + hk) * FRAG_DW * 64;
    // value of the B operand at (channel c, column n)
    auto bval = [&](int c) -> _Float16 {
      const int g = (32 * (c / 32)) / C::G;
      if (!ncol || (g % C::CG) != cg) return _Float16(0.f);
      const float mult = ((c & 3) < 2) ? 4.f : 16.f;
      const float x = qr[h][c] * mult * kq;
      const _Float16 hi = _Float16(x);
      return part ? _Float16(x - float(hi)) : hi;
    };
    for (int k = 0; k < 4; ++k)
      for (int v = 0; v < 4; ++v) {
        const int c0 = 32 * k + 8 * qd + 2 * v;
        const uint16_t lo16 = __builtin_bit_cast(uint16_t, bval(c0));
        const uint16_t hi16 = __builtin_bit_cast(uint16_t, bval(c0 + 1));
        fr[(4 * k + v) * 64 + lane] = uint32_t(lo16) | (uint32_t(hi16) << 16);
      }
    for (int ai = 0; ai < C::NA; ++ai) {
      // minus the column sum of B over the channel blocks of accumulator ai
      float cs = 0.f;
      for (int c = 0; c < D; ++c)
        if (C::grp_of_kblock(c / 32) / C::CG == ai) cs += float(bval(c));
      fr[(16 + ai) * 64 + lane] = __float_as_uint(-cs);
      const int g = ai * C::CG + cg;
      const float zq = (ncol && part == 0 && g < NG) ? qz[h][g] : 0.f;
      fr[(16 + C::NA + ai) * 64 + lane] = __float_as_uint(zq);
    }
    fr[(16 + 2 * C::NA) * 64 + lane] = __float_as_uint(1.f / kq);
  }
}

// ------------------------------------------------------------------ split

// One wave over history pages j = j0 + wave, j0 + wave + WAVES, ... < j1.
template <int GQA, int NG>
__device__ void history_wave(const DecodeArgs &a, int b, int hk, int L, int j0, int j1, int wave,
                             int lane, float *o_lds, float *m_lds, float *l_lds) {
  using C = Cols<GQA, NG>;
  constexpr int NA = C::NA;
  const oscar_layer_cache &c = a.c;
  const int n = lane & 15, qd = lane >> 4;
  const int h = n % GQA, part = (n / GQA) & 1, cg = n / (2 * GQA);
  const bool ncol = cg < C::CG;
  const int blk_bytes = hist_block_bytes(C::G);
  const int kmeta = k_meta_off(C::G), vcode = v_codes_off(C::G), vmeta = v_meta_off(C::G);
  const int nh = n_hist_tokens(L);

  const uint32_t *fr = a.frag + (int64_t(b) * c.n_kv_heads + hk) * FRAG_DW * 64;
  f16x8 bq[4];
  for (int k = 0; k < 4; ++k)
    bq[k] = as_f16x8(fr[(4 * k) * 64 + lane], fr[(4 * k + 1) * 64 + lane], fr[(4 * k + 2) * 64 + lane],
                     fr[(4 * k + 3) * 64 + lane]);
  float cinit[NA], zq[NA];
  int goff[NA];
  bool gval[NA];
  for (int ai = 0; ai < NA; ++ai) {
    cinit[ai] = __uint_as_float(fr[(16 + ai) * 64 + lane]);
    zq[ai] = __uint_as_float(fr[(16 + NA + ai) * 64 + lane]);
    const int g = ai * C::CG + cg;
    gval[ai] = ncol && g < NG;
    goff[ai] = 64 * (g < NG ? g : NG - 1) + 16 * qd;
  }
  const float inv_kq = __uint_as_float(fr[(16 + 2 * NA) * 64 + lane]);

  float m_run = -INFINITY, l_run = 0.f;
  float corr[NA], zacc[NA];
  f32x4 acc[8];
  for (int r = 0; r < 8; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ai = 0; ai < NA; ++ai) corr[ai] = zacc[ai] = 0.f;

  for (int j = j0 + wave; j < j1; j += WAVES) {
    const int pid = __builtin_amdgcn_readfirstlane(c.hist_pt[int64_t(b) * c.hist_pt_stride + j]);
    if (pid < 0 || pid >= c.n_hist_pages) {
      if (lane == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
      continue;
    }
    const uint8_t *blk = c.hist + (int64_t(pid) * c.n_kv_heads + hk) * blk_bytes;
    const u32x2 kc = *reinterpret_cast<const u32x2 *>(blk + 8 * lane);
    const u32x2 vc = *reinterpret_cast<const u32x2 *>(blk + vcode + 8 * lane);
    u32x4 km[NA], vm[NA];
    for (int ai = 0; ai < NA; ++ai) {
      km[ai] = *reinterpret_cast<const u32x4 *>(blk + kmeta + goff[ai]);
      vm[ai] = *reinterpret_cast<const u32x4 *>(blk + vmeta + goff[ai]);
    }
    const int nvalid = min(PAGE, nh - PAGE * j);

    // ---- scores: D[t][n] = sum_c code_tc q'_cn, per accumulator
    f32x4 dacc[NA];
    for (int ai = 0; ai < NA; ++ai) dacc[ai] = f32x4{cinit[ai], cinit[ai], cinit[ai], cinit[ai]};
    for (int k = 0; k < 4; ++k) {
      const int ai = C::grp_of_kblock(k) / C::CG;
      dacc[ai] = mfma_k(expand_k(kc[0], kc[1], k), bq[k], dacc[ai]);
    }
    float sc[4];
    float mx = -INFINITY;
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
      for (int ai = 0; ai < NA; ++ai) {
        const uint32_t sz = km[ai][i];
        v = fmaf(lo_f16(sz) * inv_kq, dacc[ai][i], fmaf(hi_f16(sz), zq[ai], v));
      }
      if constexpr (GQA < 16) v += row_ror<GQA>(v);
      if constexpr (2 * GQA < 16) v += row_ror<2 * GQA>(v);
      if constexpr (4 * GQA < 16) v += row_ror<4 * GQA>(v);
      if constexpr (8 * GQA < 16) v += row_ror<8 * GQA>(v);
      sc[i] = (4 * qd + i < nvalid) ? v : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    // ---- online softmax, max raised lazily
    if (__any(mx > m_run + LAZY_TH)) {
      const float mm = quad_max(fmaxf(mx, m_run));
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mm);
      for (int r = 0; r < 8; ++r) acc[r] *= alpha;
      for (int ai = 0; ai < NA; ++ai) {
        corr[ai] *= alpha;
        zacc[ai] *= alpha;
      }
      l_run *= alpha;
      m_run = mm;
    }
    float p[4];
    for (int i = 0; i < 4; ++i) {
      p[i] = (sc[i] == -INFINITY) ? 0.f : fast_exp2(sc[i] - m_run);
      l_run += p[i];
    }
    // ---- PV operand: p * s * (1/w) * 2^k as fp16 high / low parts
    f16x4 bp[NA];
    for (int ai = 0; ai < NA; ++ai) {
      _Float16 e[4];
      for (int i = 0; i < 4; ++i) {
        const uint32_t sz = vm[ai][i];
        const bool ok = gval[ai] && (4 * qd + i < nvalid);
        const float mult = (i < 2) ? 4.f : 16.f;
        const float x = ok ? p[i] * lo_f16(sz) * (mult * a.pv_scale) : 0.f;
        const _Float16 hi = _Float16(x);
        e[i] = part ? _Float16(x - float(hi)) : hi;
        corr[ai] += float(e[i]);
        zacc[ai] = ok ? fmaf(p[i], hi_f16(sz), zacc[ai]) : zacc[ai];
      }
      bp[ai] = f16x4{e[0], e[1], e[2], e[3]};
    }
    for (int r = 0; r < 8; ++r) {
      const int ai = C::grp_of_rblock(r) / C::CG;
      acc[r] = mfma_v(expand_v(vc[0], vc[1], r), bp[ai], acc[r]);
    }
  }

  // ---- this wave's o[h][c], m[h], l[h] into LDS
  const float lt = quad_sum(l_run);
  for (int ai = 0; ai < NA; ++ai) {
    corr[ai] = quad_sum(corr[ai]);
    zacc[ai] = quad_sum(zacc[ai]);
  }
  for (int r = 0; r < 8; ++r) {
    const int g = C::grp_of_rblock(r);
    const int ai = g / C::CG;
    for (int i = 0; i < 4; ++i) {
      float v = acc[r][i] - corr[ai];
      v += row_ror<16 - GQA>(v);  // add the low-part column n + GQA
      if (part == 0 && ncol && cg == g % C::CG)
        o_lds[h * D + 16 * r + 4 * qd + i] = fmaf(v, a.pv_unscale, zacc[ai]);
    }
  }
  if (qd == 0 && n < GQA) {
    m_lds[n] = m_run;
    l_lds[n] = lt;
  }
}

// Raw (BF16) sink + recent pages of one request: page 0 = sink, pages 1..8 =
// ring; slot s of the ring holds a live token iff its position is in the
// recent window.
__device__ inline uint32_t raw_valid_rows(int L, int page) {
  uint32_t m = 0;
  for (int r = 0; r < PAGE; ++r) {
    bool ok;
    if (page == 0) {
      ok = r < L && r < N_SINK;
    } else {
      const int s = PAGE * (page - 1) + r;
      ok = (L >= N_RAW) || (s >= N_SINK && s < L) || (s < N_SINK && s + N_RECENT < L);
    }
    m |= uint32_t(ok) << r;
  }
  return m;
}

template <int GQA, int NG>
__global__ void __launch_bounds__(WAVES * 64) split_kernel(DecodeArgs a) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const oscar_layer_cache &c = a.c;
  const int L = a.seq_lens[b];
  __shared__ float o_lds[WAVES * GQA * D];
  __shared__ float m_lds[WAVES * GQA], l_lds[WAVES * GQA];
  if (!valid_len(L, a.max_seq_len)) {
    if (tid == 0 && split == 0 && hk == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  float *o_w = o_lds + wave * GQA * D;
  if (split == 0) {
    Bf16Wave<GQA> st;
    st.init(a.q + (int64_t(b) * a.n_q_heads + hk * GQA) * D, a.sm_scale, lane);
    for (int pg = wave; pg < BF16_PT; pg += WAVES) {
      const uint32_t valid = raw_valid_rows(L, pg);
      if (!valid) continue;
      const int page = c.bf16_pt[b * BF16_PT + pg];
      if (page < 0 || page >= c.n_bf16_pages) {
        if (lane == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
        continue;
      }
      const uint16_t *base = c.bf16 + (int64_t(page) * c.n_kv_heads + hk) * 2 * PAGE * D;
      st.page(base, base + PAGE * D, valid, lane);
    }
    st.finish(o_w, m_lds + wave * GQA, l_lds + wave * GQA, lane);
  } else {
    const int pages = n_hist_pages(L);
    const int j0 = (split - 1) * a.pages_per_split;
    const int j1 = min(pages, j0 + a.pages_per_split);
    history_wave<GQA, NG>(a, b, hk, L, j0, j1, wave, lane, o_w, m_lds + wave * GQA, l_lds + wave * GQA);
  }
  __syncthreads();
  float *part0 = a.parts + ((int64_t(b) * a.n_q_heads + hk * GQA) * (1 + a.n_splits) + split) * PART_STRIDE;
  combine_waves<GQA>(o_lds, m_lds, l_lds, part0, int64_t(1 + a.n_splits) * PART_STRIDE, tid);
}

// ------------------------------------------------------------------ merge

__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_lens[b];
  float *o = a.out + (int64_t(b) * a.n_q_heads + hq) * D;
  if (!valid_len(L, a.max_seq_len)) {
    if (tid < D) o[tid] = 0.f;
    return;
  }
  const int used = 1 + (n_hist_pages(L) + a.pages_per_split - 1) / a.pages_per_split;
  const float *parts = a.parts + (int64_t(b) * a.n_q_heads + hq) * (1 + a.n_splits) * PART_STRIDE;
  __shared__ float w_s[1024];
  __shared__ float red[256];
  __shared__ float rot[2][D];
  // max over splits
  float m = -INFINITY;
  for (int s = tid; s < used; s += 256) m = fmaxf(m, parts[s * PART_STRIDE + D]);
  red[tid] = m;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  const float mst = red[0];
  __syncthreads();
  float l = 0.f;
  for (int s = tid; s < used; s += 256) {
    const float ms = parts[s * PART_STRIDE + D];
    const float w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - mst);
    if (s < 1024) w_s[s] = w;
    l = fmaf(w, parts[s * PART_STRIDE + D + 1], l);
  }
  red[tid] = l;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const float lsum = red[0];
  // history splits 1..used-1 in two halves, channel = tid % 128
  const int ch = tid & (D - 1), half = tid >> 7;
  float acc = 0.f;
  for (int s = 1 + half; s < used; s += 2) {
    const float ms = parts[s * PART_STRIDE + D];
    const float w = s < 1024 ? w_s[s] : ((ms == -INFINITY) ? 0.f : fast_exp2(ms - mst));
    acc = fmaf(w, parts[s * PART_STRIDE + ch], acc);
  }
  rot[half][ch] = acc;
  __syncthreads();
  if (tid < D) {
    const float *RT = reinterpret_cast<const float *>(a.fv + FORM_RT);
    float back = 0.f;  // (rot R_V^T)[tid] = sum_i rot[i] R_V[tid][i]
    for (int i = 0; i < D; ++i) back = fmaf(rot[0][i] + rot[1][i], RT[i * D + tid], back);
    const float plain = w_s[0] * parts[tid];
    o[tid] = (back + plain) / lsum;
  }
}

// ------------------------------------------------------------------ launch

template <int GQA, int NG>
static hipError_t launch_t(const DecodeArgs &a, int batch, int hkv, hipStream_t s) {
  hipLaunchKernelGGL((qprep_kernel<GQA, NG>), dim3(hkv, batch), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((split_kernel<GQA, NG>), dim3(1 + a.n_splits, hkv, batch), dim3(WAVES * 64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.n_q_heads, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int GQA>
static hipError_t launch_g(const DecodeArgs &a, int G, int batch, int hkv, hipStream_t s) {
  switch (G) {
    case 32: return launch_t<GQA, 4>(a, batch, hkv, s);
    case 64: return launch_t<GQA, 2>(a, batch, hkv, s);
    default: return launch_t<GQA, 1>(a, batch, hkv, s);
  }
}

hipError_t launch_decode_int2(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q,
                              int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                              float sm_scale, float *out, void *ws, hipStream_t s) {
  const SplitPlan p = plan_int2_splits(batch, c.n_kv_heads, max_seq_len);
  DecodeArgs a;
  a.c = c;
  a.fk = rk.forms;
  a.fv = rv.forms;
  a.q = q;
  a.seq_lens = seq_lens;
  a.n_q_heads = n_q_heads;
  a.max_seq_len = max_seq_len;
  a.pages_per_split = p.pages_per_split;
  a.n_splits = p.n_splits;
  a.sm_scale = sm_scale;
  // PV operand scale: p <= 2^LAZY_TH, s <= 2 clip / 3, 1/w <= 16; keep the
  // largest value under 2^15
  float k = 1.f;
  const float vmax = 8.f * 16.f * (2.f * rv.clip / 3.f);
  while (vmax * k > 32768.f) k *= 0.5f;
  while (vmax * k * 2.f <= 32768.f && k < 65536.f) k *= 2.f;
  a.pv_scale = k;
  a.pv_unscale = 1.f / k;
  a.frag = static_cast<uint32_t *>(ws);
  a.parts = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + frag_bytes(batch, c.n_kv_heads));
  a.out = out;
  const int gqa = n_q_heads / c.n_kv_heads;
  switch (gqa) {
    case 1: return launch_g<1>(a, c.group, batch, c.n_kv_heads, s);
    case 2: return launch_g<2>(a, c.group, batch, c.n_kv_heads, s);
    case 4: return launch_g<4>(a, c.group, batch, c.n_kv_heads, s);
    case 8: return launch_g<8>(a, c.group, batch, c.n_kv_heads, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
