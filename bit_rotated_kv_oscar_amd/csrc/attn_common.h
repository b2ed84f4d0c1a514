// Device helpers shared by the decode kernels: matrix-core operand types,
// DPP / cross-lane reductions, the 2-bit code expansion, and one wave's pass
// over a BF16 page.
#pragma once

#include "kernels.h"

namespace oscar {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
// The running max of a softmax is raised only when a score exceeds it by more
// than this (log2 units), so probabilities stay <= 2^LAZY_TH; nearly every
// page then skips the rescale of the accumulators.
constexpr float LAZY_TH = 8.0f;
constexpr int PART_STRIDE = D + 2;  // partial: o[128], m, l

// lane l receives the value of lane l - N (mod 16) of its row of 16
template <int N>
__device__ inline float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

// DPP quad_perm: lane l receives lane (l & ~3) | sel[l & 3] (XOR1: 1,0,3,2;
// XOR2: 2,3,0,1)
template <int CTRL>
__device__ inline float quad_perm(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int QP_XOR1 = 0xB1, QP_XOR2 = 0x4E;

// Sum over the aligned group of 8 lanes; the total is in lanes with
// (l & 7) >= 4 (others hold a mix of two groups).
__device__ inline float oct_sum(float v) {
  v += quad_perm<QP_XOR1>(v);
  v += quad_perm<QP_XOR2>(v);
  return v + row_ror<4>(v);
}

// Every lane of a row of 16 receives the row's sum / max.
__device__ inline float row_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  return v + row_ror<1>(v);
}
__device__ inline float row_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
__device__ inline float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Whole-wave sum / max, the same in every lane (row reductions by DPP, then
// four lane reads: no LDS round trips)
__device__ inline float wave_sum(float v) {
  v = row_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ inline float wave_max(float v) {
  v = row_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ inline float wave_min(float v) {
  v = fminf(v, row_ror<8>(v));
  v = fminf(v, row_ror<4>(v));
  v = fminf(v, row_ror<2>(v));
  v = fminf(v, row_ror<1>(v));
  return fminf(fminf(lane_value(v, 0), lane_value(v, 16)), fminf(lane_value(v, 32), lane_value(v, 48)));
}
// Min / max over aligned segments of SEG = 32 or 64 lanes, the same in every
// lane of the segment.
template <int SEG>
__device__ inline float seg_min(float v, int lane) {
  static_assert(SEG == 32 || SEG == 64, "segment of 32 or 64 lanes");
  v = fminf(v, row_ror<8>(v));
  v = fminf(v, row_ror<4>(v));
  v = fminf(v, row_ror<2>(v));
  v = fminf(v, row_ror<1>(v));
  const float r01 = fminf(lane_value(v, 0), lane_value(v, 16)), r23 = fminf(lane_value(v, 32), lane_value(v, 48));
  if constexpr (SEG == 64) return fminf(r01, r23);
  return lane < 32 ? r01 : r23;
}
template <int SEG>
__device__ inline float seg_max(float v, int lane) {
  static_assert(SEG == 32 || SEG == 64, "segment of 32 or 64 lanes");
  v = row_max(v);
  const float r01 = fmaxf(lane_value(v, 0), lane_value(v, 16)), r23 = fmaxf(lane_value(v, 32), lane_value(v, 48));
  if constexpr (SEG == 64) return fmaxf(r01, r23);
  return lane < 32 ? r01 : r23;
}
// Sum over aligned segments of SEG = 32 or 64 lanes, the same in every lane
// of the segment.
template <int SEG>
__device__ inline float seg_sum(float v, int lane) {
  static_assert(SEG == 32 || SEG == 64, "segment of 32 or 64 lanes");
  v = row_sum(v);
  const float r01 = lane_value(v, 0) + lane_value(v, 16), r23 = lane_value(v, 32) + lane_value(v, 48);
  if constexpr (SEG == 64) return r01 + r23;
  return lane < 32 ? r01 : r23;
}

__device__ inline float quad_sum(float v) {  // sum over lanes l, l^16, l^32, l^48
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ inline float quad_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
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

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ code expansion
// A code dword expands into fp16 pairs 1 + c/4 (mask 0x0300, slot pairs at
// bits 8-9 / 24-25) and 1 + c/16 (mask 0x00C0, bits 6-7 / 22-23) after one of
// four shifts (none, >>4, <<4, rotate right 8).  The constant 1 and the 1/4,
// 1/16 weights are undone by the operand on the other side of the product.
__device__ inline uint32_t rotr8(uint32_t x) { return __builtin_amdgcn_alignbit(x, x, 8); }

__device__ inline f16x8 as_f16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(f16x8, u);
}
__device__ inline f16x4 as_f16x4(uint32_t a, uint32_t b) {
  u32x2 u = {a, b};
  return __builtin_bit_cast(f16x4, u);
}

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

// INT4 codes as fp16 1 + c/16: a nibble moved to mantissa bits 6-9 (and
// 22-25 for the high half) under the exponent of 1.0.  Pair p of a dword
// holds nibbles p and p + 4, so the four pairs of a K dword are channels
// 0..7 of its block in order, and pairs 0, 1 (2, 3) of a V dword are rows
// 0..3 of its first (second) channel.
struct Expander4 {
  uint32_t m, e;  // 0x03C003C0, 0x3C003C00
  __device__ uint32_t pair(uint32_t x, int p) const {
    const uint32_t y = p == 0 ? (x << 6) : p == 1 ? (x << 2) : p == 2 ? (x >> 2) : (x >> 6);
    return and_or(y, m, e);
  }
  __device__ f16x8 k(uint32_t x) const { return as_f16x8(pair(x, 0), pair(x, 1), pair(x, 2), pair(x, 3)); }
  __device__ f16x4 v(uint32_t x, int h) const { return as_f16x4(pair(x, 2 * h), pair(x, 2 * h + 1)); }
};

__device__ inline f32x4 mfma_k(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_v(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ inline float lo_f16(uint32_t w) {
  return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xFFFFu)));
}
__device__ inline float hi_f16(uint32_t w) {
  return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16)));
}
__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------ BF16 pages
// One wave's online-softmax state over BF16 pages.  Scores use the 16x16x32
// bf16 matrix core (lane (t = l%16, quad q = l/16) supplies K row t, channels
// 32k+8q..+7; B holds the query heads in columns, bf16 exactly as given).
// Probabilities go to the PV lanes by shuffles; PV runs on the vector ALUs
// with lane (c = l%16, r = l/16) owning channels 8c..8c+7 and, per page, rows
// 4r..4r+3 (partial sums reduced over r once at the end).
template <int GQA>
struct Bf16Wave {
  bf16x8 bq[4];
  float m_run, l_run;  // of head (l%16) in lanes with l%16 < GQA
  float acc[GQA][8];
  float scale;         // sm_scale * log2(e)

  __device__ void init(const uint16_t *q_heads /* [GQA][128] bf16 */, float sm_scale, int lane) {
    const int n = lane & 15, qd = lane >> 4;
    for (int k = 0; k < 4; ++k) {
      u32x4 u = {0, 0, 0, 0};
      if (n < GQA) u = *reinterpret_cast<const u32x4 *>(q_heads + n * D + 32 * k + 8 * qd);
      bq[k] = __builtin_bit_cast(bf16x8, u);
    }
    m_run = -INFINITY;
    l_run = 0.f;
    for (int h = 0; h < GQA; ++h)
      for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
    scale = sm_scale * LOG2E;
  }

  struct Loads {
    u32x4 kf[4], vf[4];
  };

  // Issues the loads of one page: kp, vp = its K and V rows (16 x 128 bf16).
  __device__ static void issue(const uint16_t *kp, const uint16_t *vp, Loads &ld, int lane) {
    const int n = lane & 15, qd = lane >> 4;
    for (int k = 0; k < 4; ++k) ld.kf[k] = *reinterpret_cast<const u32x4 *>(kp + n * D + 32 * k + 8 * qd);
    for (int i = 0; i < 4; ++i) ld.vf[i] = *reinterpret_cast<const u32x4 *>(vp + (4 * qd + i) * D + 8 * n);
  }

  // As above, with row `row` of the page taken from krow / vrow (128 bf16 each).
  __device__ static void issue(const uint16_t *kp, const uint16_t *vp, Loads &ld, int lane, int row,
                               const uint16_t *krow, const uint16_t *vrow) {
    const int n = lane & 15, qd = lane >> 4;
    const uint16_t *kr = n == row ? krow : kp + n * D;
    for (int k = 0; k < 4; ++k) ld.kf[k] = *reinterpret_cast<const u32x4 *>(kr + 32 * k + 8 * qd);
    for (int i = 0; i < 4; ++i) {
      const uint16_t *vr = (4 * qd + i) == row ? vrow : vp + (4 * qd + i) * D;
      ld.vf[i] = *reinterpret_cast<const u32x4 *>(vr + 8 * n);
    }
  }

  // Attends over one loaded page; rows whose bit in `valid` is clear are
  // ignored (their bits may be anything, even NaN).
  __device__ void compute(const Loads &ld, uint32_t valid, int lane) {
    const int qd = lane >> 4;
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < 4; ++k)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ld.kf[k]), bq[k], d, 0, 0, 0);
    float sc[4];
    float mx = -INFINITY;
    for (int i = 0; i < 4; ++i) {
      const bool ok = (valid >> (4 * qd + i)) & 1u;
      sc[i] = ok ? d[i] * scale : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    if (__any(mx > m_run + LAZY_TH)) {
      const float mm = quad_max(fmaxf(mx, m_run));
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mm);
      l_run *= alpha;
      m_run = mm;
      for (int h = 0; h < GQA; ++h) {
        const float ah = __shfl(alpha, (lane & 48) | h);
        for (int j = 0; j < 8; ++j) acc[h][j] *= ah;
      }
    }
    float p[4];
    for (int i = 0; i < 4; ++i) {
      p[i] = (sc[i] == -INFINITY) ? 0.f : fast_exp2(sc[i] - m_run);
      l_run += p[i];
    }
    for (int i = 0; i < 4; ++i) {
      const bool ok = (valid >> (4 * qd + i)) & 1u;
      float v[8];
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = ok ? bf16lo(ld.vf[i][j]) : 0.f;
        v[2 * j + 1] = ok ? bf16hi(ld.vf[i][j]) : 0.f;
      }
      for (int h = 0; h < GQA; ++h) {
        const float ph = __shfl(p[i], (lane & 48) | h);
        for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(ph, v[j], acc[h][j]);
      }
    }
  }

  // Writes o[h][c] (unnormalised), m[h], l[h] of this wave into LDS.
  __device__ void finish(float *o, float *m, float *l, int lane) {
    const int n = lane & 15, qd = lane >> 4;
    const float lt = quad_sum(l_run);
    for (int h = 0; h < GQA; ++h)
      for (int j = 0; j < 8; ++j) {
        const float s = quad_sum(acc[h][j]);
        if (qd == 0) o[h * D + 8 * n + j] = s;
      }
    if (qd == 0 && n < GQA) {
      m[n] = m_run;
      l[n] = lt;
    }
  }
};

// Stores of values that another workgroup, possibly on another XCD, reads
// in the same kernel: agent-scope atomic stores, which go through the XCD's
// L2 to memory (the L2 caches of the XCDs are not coherent with each other).
__device__ inline void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_agent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ split merge
constexpr int MAX_MERGE_SPLITS = 256;  // partials per query head one merge combines
constexpr int MERGE_WINDOW = 32;       // slots per head the merge loads without bounds checks
constexpr int COUNTER_STRIDE = 64;     // uint32 words per merge counter (one 256-byte line)

// Merge of one (request, KV head), run inside a split-K decode kernel by
// the workgroup (NT threads) that finishes last: LSE-combines the `used`
// partials (o[128], m, l; PART_STRIDE floats apart, head_stride apart per
// query head, at least MERGE_WINDOW slots per head) of each query head of the
// group, normalises, and writes out0 [GQA][128].  Built for latency: thread (h, c)
// issues the loads of all its partial values and the (m, l) pairs at once,
// so the workgroup waits on memory about once.  The partials of other
// workgroups are read with agent-scope loads (they may sit in the L2 of
// another XCD until written through).
template <int GQA>
struct MergeWork {
  float w[GQA][MAX_MERGE_SPLITS];  // m, then the weight of each split (0 past `used`)
  float l[GQA][MAX_MERGE_SPLITS];
  float lsum[GQA];
};

// partials per (head, channel) a merging thread holds in registers at a time
template <int GQA>
constexpr int merge_ch() { return GQA >= 8 ? 16 : 32; }

template <int GQA, int NT>
__device__ void merge_partials(const float *parts0, int64_t head_stride, int used, float *out0, int tid,
                               MergeWork<GQA> &mw) {
  constexpr int KH = (GQA * D + NT - 1) / NT;  // (head, channel) pairs per thread
  constexpr int MCH = merge_ch<GQA>();
  static_assert(MCH <= MERGE_WINDOW && MCH <= MAX_MERGE_SPLITS, "the first register window fits");

  // ---- loads, all issued before any use: partial values of splits
  // 0..MCH-1 (every head has at least MCH slots, so these loads need no
  // bounds; slots >= used are never summed), then the (m, l) pairs
  float ov[KH][MCH];
#pragma unroll
  for (int k = 0; k < KH; ++k) {
    const int idx = tid + NT * k, h = idx / D, c = idx % D;
    const float *ph = parts0 + (h < GQA ? h : 0) * head_stride + c;
#pragma unroll
    for (int j = 0; j < MCH; ++j) ov[k][j] = load_agent(ph + j * PART_STRIDE);
  }
  for (int e = tid; e < GQA * used; e += NT) {
    const int hh = e / used, sp = e % used;
    const float *pm = parts0 + hh * head_stride + sp * PART_STRIDE + D;
    mw.w[hh][sp] = load_agent(pm);
    mw.l[hh][sp] = load_agent(pm + 1);
  }
  __syncthreads();
  // ---- per head: max over splits, split weights, total l (wave hh; DPP
  // reductions)
  {
    const int wave = wave_id(), lane = tid & 63;
    const int nw = used > MCH ? used : MCH;
    for (int hh = wave; hh < GQA; hh += NT / 64) {
      float m = -INFINITY;
      for (int sp = lane; sp < used; sp += 64) m = fmaxf(m, mw.w[hh][sp]);
      m = wave_max(m);
      float l = 0.f;
      for (int sp = lane; sp < nw; sp += 64) {
        float w = 0.f;
        if (sp < used) {
          const float ms = mw.w[hh][sp];
          w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - m);
          l = fmaf(w, mw.l[hh][sp], l);
        }
        mw.w[hh][sp] = w;
      }
      l = wave_sum(l);
      if (lane == 0) mw.lsum[hh] = l;
    }
  }
  __syncthreads();
  // ---- output channel c of head h
#pragma unroll
  for (int k = 0; k < KH; ++k) {
    const int idx = tid + NT * k, h = idx / D, c = idx % D;
    if (h < GQA) {
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int j = 0; j < MCH; ++j) {
        const float t = fmaf(mw.w[h][j], ov[k][j], j & 1 ? acc1 : acc0);
        if (j & 1)
          acc1 = (j < used) ? t : acc1;
        else
          acc0 = (j < used) ? t : acc0;
      }
      // the first window is summed here, before the later windows' loads
      asm volatile("" : "+v"(acc0), "+v"(acc1));
      const float *ph = parts0 + h * head_stride + c;
      for (int s0 = MCH; s0 < used; s0 += MCH) {
        float o2[MCH];
#pragma unroll
        for (int j = 0; j < MCH; ++j) o2[j] = (s0 + j < used) ? load_agent(ph + (s0 + j) * PART_STRIDE) : 0.f;
#pragma unroll
        for (int j = 0; j < MCH; ++j) {
          const float w = (s0 + j < used) ? mw.w[h][s0 + j] : 0.f;
          acc0 = fmaf(w, o2[j], acc0);
        }
      }
      out0[h * D + c] = (acc0 + acc1) / mw.lsum[h];
    }
  }
}

// Combines the NW per-wave states in LDS (o [NW][GQA][128], m, l [NW][GQA])
// and writes one unnormalised partial (o[128], m, l) per query head
// (AGENT: with agent-scope stores).  With xm, one more token joins: value
// xo[128] (every head), score xm[h] (log2 units, finite).
template <int GQA, int NW, bool AGENT = false>
__device__ inline void combine_waves(const float *o_lds, const float *m_lds, const float *l_lds,
                                     float *part0, int64_t head_stride, int tid, int o_wave_stride = GQA * D,
                                     const float *xo = nullptr, const float *xm = nullptr) {
  for (int idx = tid; idx < GQA * D; idx += NW * 64) {
    const int h = idx / D, c = idx % D;
    float mst = xm ? xm[h] : -INFINITY;
    for (int w = 0; w < NW; ++w) mst = fmaxf(mst, m_lds[w * GQA + h]);
    float o = 0.f, l = 0.f;
    if (xm) {
      const float e = fast_exp2(xm[h] - mst);
      o = e * xo[c];
      l = e;
    }
    for (int w = 0; w < NW; ++w) {
      const float mw = m_lds[w * GQA + h];
      const float e = (mw == -INFINITY) ? 0.f : fast_exp2(mw - mst);
      o = fmaf(e, o_lds[w * o_wave_stride + h * D + c], o);
      l = fmaf(e, l_lds[w * GQA + h], l);
    }
    float *part = part0 + h * head_stride;
    if constexpr (AGENT) {
      store_agent(part + c, o);
      if (c == 0) {
        store_agent(part + D, mst);
        store_agent(part + D + 1, l);
      }
    } else {
      part[c] = o;
      if (c == 0) {
        part[D] = mst;
        part[D + 1] = l;
      }
    }
  }
}

}  // namespace oscar
