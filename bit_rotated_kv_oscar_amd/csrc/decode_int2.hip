// Mixed-precision paged decode attention over the OSCAR cache, and the
// write-on-append of one token per request.
//
// OSCAR online phase (gist.science nl/fr technical summaries, section 2.2.B:
// one fused kernel unpacks, dequantises, undoes the rotation and attends over
// the INT2 history on paged storage with prefix caching; arXiv:2605.17757 v2
// abstract: fused write and decode kernels, batch-1 decode gains from cutting
// KV memory traffic).
//
// The rotation is never undone per token: history keys stay in the rotated
// basis and are scored against q R_K (R orthogonal keeps q.k), and the
// history part of the output is rotated back by R_V^T once per (request,
// query head).  Per-group scale s and zero z are factored out of both
// contractions so the matrix cores see the 2-bit codes as exact fp16 values:
//   score_t = sum_g s_tg (q_g . c_tg) + z_tg sum_{i in g} q_i
//   o       = sum_g [ sum_t (p_t s_tg) c_tg ] + sum_t p_t z_tg
//
// Three kernels per call, in stream order:
//   prologue (one block per (request, KV head)):
//     - optional append: the token leaving the recent window (position
//       L-128 when L >= 144) is read from its ring slot, rotated, clipped,
//       quantised and stored in history; the new token takes the slot;
//     - q_rot = q R_K * sm_scale * log2(e) for the query heads of the group,
//       laid out as the B operand of the score MFMAs (fp16 high + low parts)
//       with the column sums that cancel the code expansion's constant and
//       the per-group sums of q_rot.
//   attend (one workgroup of 8 waves per (request, KV head, split)):
//     split 0 attends over the raw BF16 sink + recent pages, split s >= 1
//     over history pages (wave w takes every 8th page of the split, page ids
//     preloaded, next page's loads issued before the current page computes).
//     Each workgroup writes an unnormalised partial (o[128], m, l) per query
//     head.
//   merge (one block per (request, KV head)): LSE-combines the partials,
//     rotates the history part back with R_V^T, adds the raw part and
//     normalises (fp32 out).  A kernel boundary, not an in-kernel fence, makes
//     the partials visible: the L2 caches of the eight XCDs are not coherent
//     with each other, and a device-scope fence writes back and invalidates
//     the whole L2.
#include <cmath>
#include <type_traits>

#include "attn_common.h"

namespace oscar {

constexpr int AW = 8;                // waves per attend workgroup
constexpr int FRAG_DW = 32;          // dwords per lane of the q fragment block
constexpr int PRO_THREADS = 512;     // prologue block: K half + V half
constexpr int MAX_SPLITS = 255;      // history splits per (request, KV head)

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
  __device__ static constexpr int grp_of_kblock(int k) { return (32 * k) / G; }  // 32-channel block
  __device__ static constexpr int grp_of_rblock(int r) { return (16 * r) / G; }  // 16-channel block
};

SplitPlan plan_int2_splits(int batch, int n_kv_heads, int max_seq_len) {
  const int pages = n_hist_pages(max_seq_len);
  SplitPlan p;
  if (pages == 0) {
    p.pages_per_split = AW;
    p.n_splits = 0;
    return p;
  }
  // Resident attend workgroups: two per CU on 256 CUs.  When every unit
  // (request, KV head) fits in one round with at least one history split,
  // spread each unit's pages over as many splits as that round holds (its
  // raw workgroup included); otherwise use splits of 8 pages per wave.
  const int64_t units = int64_t(batch) * n_kv_heads;
  const int64_t slots = 2 * 256;
  int64_t pps;
  if (slots - units >= units) {
    const int64_t per_unit = (slots - units) / units;
    pps = (pages + per_unit - 1) / per_unit;
  } else {
    pps = 8 * AW;
  }
  if (pps < AW) pps = AW;
  const int64_t min_pps = (pages + MAX_SPLITS - 1) / MAX_SPLITS;  // bounds the merge's LDS
  if (pps < min_pps) pps = min_pps;
  p.pages_per_split = int(pps);
  p.n_splits = int((pages + pps - 1) / pps);
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
static size_t frag_bytes(int batch, int hkv) { return align256(size_t(batch) * hkv * FRAG_DW * 64 * 4); }

size_t decode_int2_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  const SplitPlan p = plan_int2_splits(batch, n_kv_heads, max_seq_len);
  return frag_bytes(batch, n_kv_heads) +
         align256(size_t(batch) * n_q_heads * (1 + p.n_splits) * PART_STRIDE * sizeof(float));
}

struct StepArgs {
  oscar_layer_cache c;
  const uint8_t *fk, *fv;
  float clip_k, clip_v;
  // append (may be null: no append)
  const uint16_t *k_new, *v_new;  // [B][Hkv][128]
  const int32_t *len_before;      // [B]: the new token goes to position len_before[b]
  // decode (q may be null: append only)
  const uint16_t *q;
  const int32_t *seq_lens;        // [B] after the append
  int n_q_heads, max_seq_len, pages_per_split, n_splits;
  float sm_scale;
  float pv_scale, pv_unscale;     // 2^k and 2^-k applied to the PV operand
  float pk01, pk23;               // log2(4 * 2^k), log2(16 * 2^k): PV factors of tokens 4q+{0,1}, 4q+{2,3}
  uint32_t ex_m4, ex_m16, ex_e;   // code expansion constants 0x03000300, 0x00C000C0, 0x3C003C00
  uint32_t *frag;                 // [B][Hkv][FRAG_DW][64]
  float *parts;                   // [B][Hq][1 + n_splits][PART_STRIDE]
  float *out;                     // [B][Hq][128]
};

__device__ inline bool valid_len(int L, int max_len) { return L >= 1 && L <= max_len; }

// ------------------------------------------------------------------ prologue

// Quantise one rotated vector (128 values in LDS, already in y) into history
// row `row` of the block at `blk` (K or V area), G channels per group.
// Threads t < 128 of the half take part; `codes` is LDS scratch.
__device__ inline void store_int2_row(const float *y, float clip, int G, bool is_v, uint8_t *blk, int row,
                                      uint8_t *codes, float *sz_lds, int t) {
  const int ng = D / G;
  if (t < ng) {
    float lo = fminf(fmaxf(y[t * G], -clip), clip), hi = lo;
    for (int i = 1; i < G; ++i) {
      const float v = fminf(fmaxf(y[t * G + i], -clip), clip);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    sz_lds[2 * t] = __half2float(__float2half_rn((hi - lo) / 3.0f));
    sz_lds[2 * t + 1] = __half2float(__float2half_rn(lo));
  }
  __syncthreads();
  if (t < D) {
    const float v = fminf(fmaxf(y[t], -clip), clip);
    const float s = sz_lds[2 * (t / G)], z = sz_lds[2 * (t / G) + 1];
    codes[t] = s > 0.f ? uint8_t(min(3, max(0, int(rintf((v - z) / s))))) : uint8_t(0);
  }
  __syncthreads();
  uint32_t *area = reinterpret_cast<uint32_t *>(blk + (is_v ? v_codes_off(G) : k_codes_off(G)));
  if (!is_v) {
    // the 8 dwords of token `row`: lanes 16q + row, halves d
    if (t < 8) {
      const int q = t >> 1, d = t & 1;
      uint32_t w = 0;
      for (int u = 0; u < 8; ++u) {
        const int c0 = 32 * (2 * d + u / 4) + 8 * q + 2 * (u % 4);
        w |= uint32_t(codes[c0]) << slot_lo(u);
        w |= uint32_t(codes[c0 + 1]) << slot_hi(u);
      }
      area[2 * (16 * q + row) + d] = w;
    }
  } else {
    // token `row` owns 4 codes in each of 32 dwords (lanes 16 (row/4) + m, halves d)
    if (t < 32) {
      const int m = t & 15, d = t >> 4, q = row >> 2, jj = (row & 3) >> 1;
      const int bit_sel = row & 1;
      uint32_t w = 0, mask = 0;
      for (int rr = 0; rr < 4; ++rr) {
        const int u = 2 * rr + jj;
        const int c = 16 * (4 * d + rr) + m;
        const int bit = bit_sel ? slot_hi(u) : slot_lo(u);
        w |= uint32_t(codes[c]) << bit;
        mask |= 3u << bit;
      }
      uint32_t *p = area + 2 * (16 * q + m) + d;
      *p = (*p & ~mask) | w;
    }
  }
  if (t < ng) {
    __half2 *meta = reinterpret_cast<__half2 *>(blk + (is_v ? v_meta_off(G) : k_meta_off(G)));
    meta[PAGE * t + row] = __halves2half2(__float2half_rn(sz_lds[2 * t]), __float2half_rn(sz_lds[2 * t + 1]));
  }
}

template <int GQA, int NG>
__global__ void __launch_bounds__(PRO_THREADS) prologue_kernel(StepArgs a) {
  using C = Cols<GQA, NG>;
  constexpr int G = C::G;
  const int hk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int half = tid >> 8, t = tid & 255;  // half 0: K (and the query), 1: V
  const oscar_layer_cache &c = a.c;
  const int hkv = c.n_kv_heads;
  __shared__ float xin[2][GQA + 1][D];       // [half][vector][channel]
  __shared__ float yout[2][GQA + 1][D];
  __shared__ float part_lds[2][2 * (GQA + 1) * D];
  __shared__ uint8_t codes[2][D];
  __shared__ float sz_lds[2][8];
  __shared__ float red[256];
  __shared__ int evict_s;

  // R^T rows for this thread (output channel jx, inputs 64 hf .. 64 hf + 63),
  // loaded first so they overlap the dependent loads below
  const bool want_q = a.q != nullptr;
  const int jx = t & (D - 1), hf = t >> 7;
  f32x4 rr[16];
  if ((half == 0 && want_q) || a.k_new) {
    const float *RT = reinterpret_cast<const float *>((half ? a.fv : a.fk) + FORM_RT) + jx * D + 64 * hf;
#pragma unroll
    for (int i4 = 0; i4 < 16; ++i4) rr[i4] = *reinterpret_cast<const f32x4 *>(RT + 4 * i4);
  }

  // ---------------- append (optional)
  int evict_pos = -1;  // position leaving the ring, or -1
  uint8_t *evict_blk = nullptr;
  if (a.k_new) {
    const int L0 = a.len_before[b];
    if (L0 < 0 || L0 >= (1 << 30)) {
      if (tid == 0 && hk == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
    } else {
      const uint16_t *src = (half ? a.v_new : a.k_new) + (int64_t(b) * hkv + hk) * D;
      int page, row;
      if (L0 < N_SINK) {
        page = c.bf16_pt[b * BF16_PT];
        row = L0;
      } else {
        const int slot = L0 % N_RECENT;
        page = c.bf16_pt[b * BF16_PT + 1 + slot / PAGE];
        row = slot % PAGE;
        if (L0 >= N_RAW) evict_pos = L0 - N_RECENT;
      }
      const bool page_ok = page >= 0 && page < c.n_bf16_pages;
      uint16_t *ring = page_ok ? c.bf16 + ((int64_t(page) * hkv + hk) * 2 + half) * (PAGE * D) + row * D : nullptr;
      if (evict_pos >= 0) {
        const int hj = (evict_pos - N_SINK) / PAGE;
        const int pid = hj < c.hist_pt_stride ? c.hist_pt[int64_t(b) * c.hist_pt_stride + hj] : -1;
        if (pid >= 0 && pid < c.n_hist_pages && page_ok)
          evict_blk = c.hist + (int64_t(pid) * hkv + hk) * hist_block_bytes(G);
        else if (t == 0 && half == 0)
          flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
        if (t < D) xin[half][GQA][t] = (evict_blk && ring) ? bf16_to_f32(ring[t]) : 0.f;
      } else if (!page_ok && t == 0 && half == 0) {
        flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
      }
      __syncthreads();  // the evicted row is read before the slot is overwritten
      if (ring && t < D) ring[t] = src[t];
    }
  }
  // ---------------- query (K half)
  if (want_q && half == 0) {
    for (int e = t; e < GQA * D; e += 256)
      xin[0][e / D][e % D] = bf16_to_f32(a.q[(int64_t(b) * a.n_q_heads + hk * GQA) * D + e]);
  }
  if (want_q) {
    const int L = a.k_new ? a.len_before[b] + 1 : a.seq_lens[b];
    if (!valid_len(L, a.max_seq_len)) {  // attend skips this request: zero its output here
      if (tid == 0 && hk == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
      for (int e = tid; e < GQA * D; e += PRO_THREADS)
        a.out[(int64_t(b) * a.n_q_heads + hk * GQA) * D + e] = 0.f;
    }
  }
  if (tid == 0) evict_s = evict_blk ? 1 : 0;
  __syncthreads();
  // ---------------- rotations: K half rotates q heads + evicted k, V half the evicted v
  {
    // both halves run the same code path (uniform barriers); unused vectors are zero
    float acc[GQA + 1];
#pragma unroll
    for (int v = 0; v <= GQA; ++v) acc[v] = 0.f;
    const bool need = (half == 0 && want_q) || evict_s;
    if (need) {
#pragma unroll
      for (int i4 = 0; i4 < 16; ++i4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 64 * hf + 4 * i4 + e;
#pragma unroll
          for (int v = 0; v <= GQA; ++v) acc[v] = fmaf(xin[half][v][i], rr[i4][e], acc[v]);
        }
    }
#pragma unroll
    for (int v = 0; v <= GQA; ++v) part_lds[half][(hf * (GQA + 1) + v) * D + jx] = acc[v];
    __syncthreads();
    if (t < D)
#pragma unroll
      for (int v = 0; v <= GQA; ++v)
        yout[half][v][t] = part_lds[half][v * D + t] + part_lds[half][(GQA + 1 + v) * D + t];
    __syncthreads();
  }
  // ---------------- quantise the evicted token into history
  if (evict_s) {
    const int hrow = (evict_pos - N_SINK) % PAGE;
    store_int2_row(yout[half][GQA], half ? a.clip_v : a.clip_k, G, half == 1, evict_blk, hrow, codes[half],
                   sz_lds[half], t);
  }
  // ---------------- q fragments (K half builds them; both halves share the barrier)
  const float sc = a.sm_scale * LOG2E;
  float amax = 0.f;
  if (want_q && half == 0)
    for (int e = t; e < GQA * D; e += 256) amax = fmaxf(amax, fabsf(yout[0][e / D][e % D] * sc));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((t & 63) == 0 && half == 0) red[t >> 6] = amax;
  __syncthreads();
  if (!want_q || half == 1) return;  // no block barrier below this point
  const float gmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float kq = 1.f;
  while (gmax * 16.f * kq > 16384.f) kq *= 0.5f;
  if (t >= 64) return;
  const int lane = t, n = lane & 15, qd = lane >> 4;
  const int h = n % GQA, part = (n / GQA) & 1, cg = n / (2 * GQA);
  const bool ncol = cg < C::CG;
  uint32_t *fr = a.frag + (int64_t(b) * hkv + hk) * FRAG_DW * 64;
  auto bval = [&](int ch) -> _Float16 {
    const int g = ch / G;
    if (!ncol || (g % C::CG) != cg) return _Float16(0.f);
    const float mult = ((ch & 3) < 2) ? 4.f : 16.f;
    const float x = yout[0][h][ch] * sc * mult * kq;
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
    float cs = 0.f;  // column sum of B over the channel blocks of accumulator ai
    for (int ch = 0; ch < D; ++ch)
      if ((ch / G) / C::CG == ai) cs += float(bval(ch));
    fr[(16 + ai) * 64 + lane] = __float_as_uint(-cs);
    const int g = ai * C::CG + cg;
    float zq = 0.f;  // per-group sum of q_rot, in the kq units of the B operand
    if (ncol && part == 0 && g < NG)
      for (int i = 0; i < G; ++i) zq += yout[0][h][g * G + i] * sc;
    fr[(16 + C::NA + ai) * 64 + lane] = __float_as_uint(zq * kq);
  }
  fr[(16 + 2 * C::NA) * 64 + lane] = __float_as_uint(1.f / kq);
}

// ------------------------------------------------------------------ attend

template <int NA>
struct PageLoads {
  u32x2 kc, vc;
  u32x4 km[NA], vm[NA];
};

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ inline h2v as_h2(uint32_t w) { return __builtin_bit_cast(h2v, w); }

// (x & m) | e.  m and e arrive as kernel arguments, so the compiler cannot
// fold them into literals and forms one v_and_or_b32 (a VOP3 instruction,
// which takes no literal on gfx950) instead of an AND and an OR; plain C++
// keeps the compiler's hazard tracking between these writes and the matrix
// instructions that read them.
__device__ inline uint32_t and_or(uint32_t x, uint32_t m, uint32_t e) { return (x & m) | e; }

struct Expander {
  uint32_t m4, m16, e;  // 0x03000300, 0x00C000C0, 0x3C003C00
  __device__ f16x8 k(uint32_t w0, uint32_t w1, int kb) const {
    const uint32_t w = (kb < 2) ? w0 : w1;
    const uint32_t x0 = (kb & 1) ? (w << 4) : w;
    const uint32_t x1 = (kb & 1) ? rotr8(w) : (w >> 4);
    return as_f16x8(and_or(x0, m4, e), and_or(x0, m16, e), and_or(x1, m4, e), and_or(x1, m16, e));
  }
  __device__ f16x4 v(uint32_t w0, uint32_t w1, int r) const {
    const uint32_t w = (r < 4) ? w0 : w1;
    const int s = r & 3;
    const uint32_t x = s == 0 ? w : s == 1 ? (w >> 4) : s == 2 ? (w << 4) : rotr8(w);
    return as_f16x4(and_or(x, m4, e), and_or(x, m16, e));
  }
};

// One wave over its history pages j = j0 + wave + AW*i, i < npw.
//
// Lane (n = l%16, quad qd = l/16) holds column n = (h, part, cg) of the score
// and PV accumulators and tokens 4qd..4qd+3 of each page.  Probabilities are
// kept pre-multiplied by 2^k01 (tokens 4qd, 4qd+1) or 2^k23 (tokens 4qd+2,
// 4qd+3), the 1/w weights of the V code expansion times the PV operand
// scale, folded into the exponent; l and the z sums keep the two classes
// apart and undo the factors once at the end.
template <int GQA, int NG>
__device__ void history_wave(const StepArgs &a, int b, int hk, int L, int j0, int j1, int wave, int lane,
                             const uint32_t *frag_lds, float *o_lds, float *m_lds, float *l_lds) {
  using C = Cols<GQA, NG>;
  constexpr int NA = C::NA;
  const oscar_layer_cache &c = a.c;
  const int n = lane & 15, qd = lane >> 4;
  const int h = n % GQA, part = (n / GQA) & 1, cg = n / (2 * GQA);
  const bool ncol = cg < C::CG;
  const int blk_bytes = hist_block_bytes(C::G);
  const int kmeta = k_meta_off(C::G), vcode = v_codes_off(C::G), vmeta = v_meta_off(C::G);
  const int nh = n_hist_tokens(L);
  const int npw = j1 > j0 + wave ? (j1 - j0 - wave + AW - 1) / AW : 0;

  f16x8 bq[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    bq[k] = as_f16x8(frag_lds[(4 * k) * 64 + lane], frag_lds[(4 * k + 1) * 64 + lane],
                     frag_lds[(4 * k + 2) * 64 + lane], frag_lds[(4 * k + 3) * 64 + lane]);
  float cinit[NA], zq[NA];
  int goff[NA];
#pragma unroll
  for (int ai = 0; ai < NA; ++ai) {
    cinit[ai] = __uint_as_float(frag_lds[(16 + ai) * 64 + lane]);
    zq[ai] = __uint_as_float(frag_lds[(16 + NA + ai) * 64 + lane]);
    const int g = ai * C::CG + cg;
    goff[ai] = 64 * (g < NG ? g : NG - 1) + 16 * qd;
  }
  const float inv_kq = __uint_as_float(frag_lds[(16 + 2 * NA) * 64 + lane]);
  const float k01 = a.pk01, k23 = a.pk23;  // log2 of the two PV factors
  Expander ex;
  ex.m4 = a.ex_m4;
  ex.m16 = a.ex_m16;
  ex.e = a.ex_e;
  // keep the exponent pattern in a VGPR (the mask stays in an SGPR): then one
  // v_and_or_b32 per expanded register.  The empty asm emits no instruction.
  asm volatile("" : "+v"(ex.e));
  // lanes holding the low fp16 part of the operands
  const bool lo_lane = part == 1;

  int my_pid = -1;
  if (lane < npw) my_pid = c.hist_pt[int64_t(b) * c.hist_pt_stride + j0 + wave + AW * lane];

  float m_run = -INFINITY, l01 = 0.f, l23 = 0.f;
  float corr[NA], z01[NA], z23[NA];
  f32x4 acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ai = 0; ai < NA; ++ai) corr[ai] = z01[ai] = z23[ai] = 0.f;

  auto issue = [&](int i, PageLoads<NA> &ld) -> bool {
    const int pid = __builtin_amdgcn_readlane(my_pid, i);
    if (pid < 0 || pid >= c.n_hist_pages) return false;
    const uint8_t *blk = c.hist + (int64_t(pid) * c.n_kv_heads + hk) * blk_bytes;
    ld.kc = *reinterpret_cast<const u32x2 *>(blk + 8 * lane);
    ld.vc = *reinterpret_cast<const u32x2 *>(blk + vcode + 8 * lane);
#pragma unroll
    for (int ai = 0; ai < NA; ++ai) {
      ld.km[ai] = *reinterpret_cast<const u32x4 *>(blk + kmeta + goff[ai]);
      ld.vm[ai] = *reinterpret_cast<const u32x4 *>(blk + vmeta + goff[ai]);
    }
    return true;
  };

  // one page; PARTIAL: rows >= nvalid are absent (their bits may be anything)
  auto page = [&](const PageLoads<NA> &ld, int nvalid, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    // ---- scores (kq units): D[t][n] = sum_c code_tc q'_cn
    f32x4 dacc[NA];
#pragma unroll
    for (int ai = 0; ai < NA; ++ai) dacc[ai] = f32x4{cinit[ai], cinit[ai], cinit[ai], cinit[ai]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ai = C::grp_of_kblock(k) / C::CG;
      dacc[ai] = mfma_k(ex.k(ld.kc[0], ld.kc[1], k), bq[k], dacc[ai]);
    }
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int ai = 0; ai < NA; ++ai) {
        const h2v sz = as_h2(ld.km[ai][i]);
        v = fmaf(float(sz.x), dacc[ai][i], fmaf(float(sz.y), zq[ai], v));
      }
      if constexpr (GQA < 16) v += row_ror<GQA>(v);
      if constexpr (2 * GQA < 16) v += row_ror<2 * GQA>(v);
      if constexpr (4 * GQA < 16) v += row_ror<4 * GQA>(v);
      if constexpr (8 * GQA < 16) v += row_ror<8 * GQA>(v);
      if constexpr (PARTIAL) v = (4 * qd + i < nvalid) ? v : -INFINITY;
      sc[i] = v;
      mx = fmaxf(mx, v);
    }
    // ---- online softmax, max raised lazily (true log2 units)
    mx *= inv_kq;
    if (__any(mx > m_run + LAZY_TH)) {
      const float mm = quad_max(fmaxf(mx, m_run));
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mm);
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] *= alpha;
#pragma unroll
      for (int ai = 0; ai < NA; ++ai) {
        corr[ai] *= alpha;
        z01[ai] *= alpha;
        z23[ai] *= alpha;
      }
      l01 *= alpha;
      l23 *= alpha;
      m_run = mm;
    }
    const float c01 = k01 - m_run, c23 = k23 - m_run;
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pe[i] = fast_exp2(fmaf(sc[i], inv_kq, i < 2 ? c01 : c23));
    l01 += pe[0] + pe[1];
    l23 += pe[2] + pe[3];
    // ---- PV operand: pe * s as fp16 high / low parts
    f16x4 bp[NA];
#pragma unroll
    for (int ai = 0; ai < NA; ++ai) {
      _Float16 e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2v sz = as_h2(ld.vm[ai][i]);
        float sv = float(sz.x), zv = float(sz.y);
        if constexpr (PARTIAL) {
          const bool ok = 4 * qd + i < nvalid;
          sv = ok ? sv : 0.f;
          zv = ok ? zv : 0.f;
        }
        const float x = pe[i] * sv;
        if (i < 2)
          z01[ai] = fmaf(pe[i], zv, z01[ai]);
        else
          z23[ai] = fmaf(pe[i], zv, z23[ai]);
        const _Float16 hi = _Float16(x);
        const _Float16 lo = _Float16(x - float(hi));
        e[i] = lo_lane ? lo : hi;
        corr[ai] += float(e[i]);
      }
      bp[ai] = f16x4{e[0], e[1], e[2], e[3]};
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int ai = C::grp_of_rblock(r) / C::CG;
      acc[r] = mfma_v(ex.v(ld.vc[0], ld.vc[1], r), bp[ai], acc[r]);
    }
  };

  PageLoads<NA> cur, nxt;
  bool cur_ok = npw > 0 ? issue(0, cur) : false;
  for (int i = 0; i < npw; ++i) {
    bool nxt_ok = false;
    if (i + 1 < npw) nxt_ok = issue(i + 1, nxt);
    if (!cur_ok) {
      if (lane == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    } else {
      const int nvalid = min(PAGE, nh - PAGE * (j0 + wave + AW * i));
      if (nvalid == PAGE)
        page(cur, nvalid, std::false_type{});
      else
        page(cur, nvalid, std::true_type{});
    }
    cur = nxt;
    cur_ok = nxt_ok;
  }

  // ---- this wave's o[h][c], m[h], l[h] into LDS
  const float inv01 = fast_exp2(-k01), inv23 = fast_exp2(-k23);
  const float lt = quad_sum(fmaf(l01, inv01, l23 * inv23));
  float zacc[NA];
#pragma unroll
  for (int ai = 0; ai < NA; ++ai) {
    corr[ai] = quad_sum(corr[ai]);
    zacc[ai] = quad_sum(fmaf(z01[ai], inv01, z23[ai] * inv23));
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int g = C::grp_of_rblock(r);
    const int ai = g / C::CG;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float v = acc[r][ii] - corr[ai];
      v += row_ror<16 - GQA>(v);  // add the low-part column n + GQA
      if (part == 0 && ncol && cg == g % C::CG)
        o_lds[h * D + 16 * r + 4 * qd + ii] = fmaf(v, a.pv_unscale, zacc[ai]);
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

// Merge of one (request, KV head): LSE-combines the `used` partials of each
// query head of the group, rotates the history part back with R_V^T, adds
// the raw part (split 0) and normalises.  1024 threads: wave h computes head
// h's weights; then (head, channel, half of the splits) per thread.
constexpr int MERGE_THREADS = 1024;

template <int GQA>
__global__ void __launch_bounds__(MERGE_THREADS) merge_kernel(StepArgs a) {
  const int hk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const oscar_layer_cache &c = a.c;
  const int L = a.k_new ? a.len_before[b] + 1 : a.seq_lens[b];
  if (!valid_len(L, a.max_seq_len)) return;  // output zeroed by the prologue
  const int used = 1 + (n_hist_pages(L) + a.pages_per_split - 1) / a.pages_per_split;
  const int64_t head_stride = int64_t(1 + a.n_splits) * PART_STRIDE;
  const float *parts0 = a.parts + (int64_t(b) * a.n_q_heads + hk * GQA) * head_stride;
  __shared__ float w_lds[GQA][MAX_SPLITS + 1];
  __shared__ float lsum[GQA];
  __shared__ float rot[2][GQA][D];    // history part, two halves of the splits
  __shared__ float plain[GQA][D];
  __shared__ float back[8][GQA][D];   // R_V^T partial sums, 8 row groups
  if (wave < GQA) {
    const float *ph = parts0 + wave * head_stride;
    float m = -INFINITY;
    for (int s = lane; s < used; s += 64) m = fmaxf(m, ph[s * PART_STRIDE + D]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float l = 0.f;
    for (int s = lane; s < used; s += 64) {
      const float ms = ph[s * PART_STRIDE + D];
      const float w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - m);
      w_lds[wave][s] = w;
      l = fmaf(w, ph[s * PART_STRIDE + D + 1], l);
    }
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) lsum[wave] = l;
  }
  __syncthreads();
  for (int idx = tid; idx < 2 * GQA * D; idx += MERGE_THREADS) {
    const int hf = idx / (GQA * D), h = (idx / D) % GQA, ch = idx % D;
    const float *ph = parts0 + h * head_stride + ch;
    const int s0 = 1 + hf * ((used - 1 + 1) / 2), s1 = hf ? used : 1 + (used - 1 + 1) / 2;
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    int s = s0;
    for (; s + 3 < s1; s += 4) {
      o0 = fmaf(w_lds[h][s], ph[s * PART_STRIDE], o0);
      o1 = fmaf(w_lds[h][s + 1], ph[(s + 1) * PART_STRIDE], o1);
      o2 = fmaf(w_lds[h][s + 2], ph[(s + 2) * PART_STRIDE], o2);
      o3 = fmaf(w_lds[h][s + 3], ph[(s + 3) * PART_STRIDE], o3);
    }
    for (; s < s1; ++s) o0 = fmaf(w_lds[h][s], ph[s * PART_STRIDE], o0);
    rot[hf][h][ch] = (o0 + o1) + (o2 + o3);
    if (hf == 0) plain[h][ch] = w_lds[h][0] * ph[0];
  }
  __syncthreads();
  // (rot R_V^T)[h][c] = sum_i rot[h][i] R_V[c][i]; thread: c = tid % 128,
  // rows i in [16 g, 16 g + 16) with g = tid / 128
  {
    const int ch = tid & (D - 1), g = tid >> 7;
    const float *R = reinterpret_cast<const float *>(a.fv + FORM_R) + ch * D + 16 * g;
    f32x4 r[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) r[i4] = *reinterpret_cast<const f32x4 *>(R + 4 * i4);
    float acc[GQA];
#pragma unroll
    for (int h = 0; h < GQA; ++h) acc[h] = 0.f;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * g + 4 * i4 + e;
#pragma unroll
        for (int h = 0; h < GQA; ++h) acc[h] = fmaf(rot[0][h][i] + rot[1][h][i], r[i4][e], acc[h]);
      }
#pragma unroll
    for (int h = 0; h < GQA; ++h) back[g][h][ch] = acc[h];
  }
  __syncthreads();
  for (int idx = tid; idx < GQA * D; idx += MERGE_THREADS) {
    const int h = idx / D, ch = idx % D;
    float v = plain[h][ch];
#pragma unroll
    for (int g = 0; g < 8; ++g) v += back[g][h][ch];
    a.out[(int64_t(b) * a.n_q_heads + hk * GQA + h) * D + ch] = v / lsum[h];
  }
}

template <int GQA, int NG>
__global__ void __launch_bounds__(AW * 64) attend_kernel(StepArgs a) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const oscar_layer_cache &c = a.c;
  const int L = a.k_new ? a.len_before[b] + 1 : a.seq_lens[b];
  __shared__ float lds[AW * GQA * D + 2 * AW * GQA];
  __shared__ uint32_t frag_lds[FRAG_DW * 64];
  if (!valid_len(L, a.max_seq_len)) return;  // flagged (and out zeroed) by the prologue
  const int pages = n_hist_pages(L);
  const int used = 1 + (pages + a.pages_per_split - 1) / a.pages_per_split;
  if (split >= used) return;
  float *o_lds = lds;
  float *m_lds = lds + AW * GQA * D;
  float *l_lds = m_lds + AW * GQA;
  float *o_w = o_lds + wave * GQA * D;
  if (split == 0) {
    Bf16Wave<GQA> st;
    st.init(a.q + (int64_t(b) * a.n_q_heads + hk * GQA) * D, a.sm_scale, lane);
    for (int pg = wave; pg < BF16_PT; pg += AW) {
      const uint32_t valid = raw_valid_rows(L, pg);
      if (!valid) continue;
      const int page = c.bf16_pt[b * BF16_PT + pg];
      if (page < 0 || page >= c.n_bf16_pages) {
        if (lane == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
        continue;
      }
      const uint16_t *base = c.bf16 + (int64_t(page) * c.n_kv_heads + hk) * 2 * PAGE * D;
      typename Bf16Wave<GQA>::Loads ld;
      Bf16Wave<GQA>::issue(base, base + PAGE * D, ld, lane);
      st.compute(ld, valid, lane);
    }
    st.finish(o_w, m_lds + wave * GQA, l_lds + wave * GQA, lane);
  } else {
    const uint32_t *fr = a.frag + (int64_t(b) * c.n_kv_heads + hk) * FRAG_DW * 64;
    for (int e = tid; e < FRAG_DW * 64; e += AW * 64) frag_lds[e] = fr[e];
    __syncthreads();
    const int j0 = (split - 1) * a.pages_per_split;
    const int j1 = min(pages, j0 + a.pages_per_split);
    history_wave<GQA, NG>(a, b, hk, L, j0, j1, wave, lane, frag_lds, o_w, m_lds + wave * GQA,
                          l_lds + wave * GQA);
  }
  __syncthreads();
  const int64_t head_stride = int64_t(1 + a.n_splits) * PART_STRIDE;
  float *part0 = a.parts + (int64_t(b) * a.n_q_heads + hk * GQA) * head_stride + split * PART_STRIDE;
  combine_waves<GQA, AW>(o_lds, m_lds, l_lds, part0, head_stride, tid);
}

// ------------------------------------------------------------------ launch

template <int GQA, int NG>
static hipError_t launch_t(const StepArgs &a, int batch, int hkv, bool attend, hipStream_t s) {
  hipLaunchKernelGGL((prologue_kernel<GQA, NG>), dim3(hkv, batch), dim3(PRO_THREADS), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !attend) return e;
  hipLaunchKernelGGL((attend_kernel<GQA, NG>), dim3(1 + a.n_splits, hkv, batch), dim3(AW * 64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<GQA>), dim3(hkv, batch), dim3(MERGE_THREADS), 0, s, a);
  return hipGetLastError();
}

template <int GQA>
static hipError_t launch_g(const StepArgs &a, int G, int batch, int hkv, bool attend, hipStream_t s) {
  switch (G) {
    case 32: return launch_t<GQA, 4>(a, batch, hkv, attend, s);
    case 64: return launch_t<GQA, 2>(a, batch, hkv, attend, s);
    default: return launch_t<GQA, 1>(a, batch, hkv, attend, s);
  }
}

static float pv_scale_for(float clip_v) {
  // PV operand: p <= 2^LAZY_TH, s <= 2 clip / 3, 1/w <= 16; keep it under 2^15
  float k = 1.f;
  const float vmax = 8.f * 16.f * (2.f * clip_v / 3.f);
  while (vmax * k > 32768.f) k *= 0.5f;
  while (vmax * k * 2.f <= 32768.f && k < 65536.f) k *= 2.f;
  return k;
}

hipError_t launch_decode_step(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *k_new,
                              const uint16_t *v_new, const int32_t *len_before, const uint16_t *q,
                              int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                              float sm_scale, float *out, void *ws, hipStream_t s) {
  StepArgs a;
  a.c = c;
  a.fk = rk.forms;
  a.fv = rv.forms;
  a.clip_k = rk.clip;
  a.clip_v = rv.clip;
  a.k_new = k_new;
  a.v_new = v_new;
  a.len_before = len_before;
  a.q = q;
  a.seq_lens = seq_lens;
  a.n_q_heads = n_q_heads;
  a.max_seq_len = max_seq_len;
  a.sm_scale = sm_scale;
  a.out = out;
  a.frag = nullptr;
  a.parts = nullptr;
  a.pages_per_split = AW;
  a.n_splits = 0;
  a.pv_scale = pv_scale_for(rv.clip);
  a.pv_unscale = 1.f / a.pv_scale;
  a.ex_m4 = 0x03000300u;
  a.ex_m16 = 0x00C000C0u;
  a.ex_e = 0x3C003C00u;
  a.pk01 = std::log2(4.f * a.pv_scale);
  a.pk23 = std::log2(16.f * a.pv_scale);
  const bool attend = q != nullptr;
  if (attend) {
    const SplitPlan p = plan_int2_splits(batch, c.n_kv_heads, max_seq_len);
    a.pages_per_split = p.pages_per_split;
    a.n_splits = p.n_splits;
    uint8_t *w = static_cast<uint8_t *>(ws);
    a.frag = reinterpret_cast<uint32_t *>(w);
    a.parts = reinterpret_cast<float *>(w + frag_bytes(batch, c.n_kv_heads));
  }
  const int gqa = attend ? n_q_heads / c.n_kv_heads : 1;
  switch (gqa) {
    case 1: return launch_g<1>(a, c.group, batch, c.n_kv_heads, attend, s);
    case 2: return launch_g<2>(a, c.group, batch, c.n_kv_heads, attend, s);
    case 4: return launch_g<4>(a, c.group, batch, c.n_kv_heads, attend, s);
    case 8: return launch_g<8>(a, c.group, batch, c.n_kv_heads, attend, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_int2(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q,
                              int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                              float sm_scale, float *out, void *ws, hipStream_t s) {
  return launch_decode_step(c, rk, rv, nullptr, nullptr, nullptr, q, n_q_heads, seq_lens, batch, max_seq_len,
                            sm_scale, out, ws, s);
}

}  // namespace oscar
