// Fused KV write: rotate, clip, INT2- (or INT4-) pack and page-store history
// tokens; store sink / recent tokens raw.  OSCAR online phase (gist.science nl/fr technical
// summaries, section 2.2.B: history kept as INT2 after the fixed rotation and
// clipping, sink and recent tokens in BF16; arXiv:2605.17757 v2 abstract:
// fused write kernel over a paged cache).
//
// Two launches per call, in stream order:
//   1. write_hist_kernel: one workgroup per (request, touched history page,
//      K|V, up to 8 KV heads).  It gathers the 16 rows of the page that
//      enter history in this call -- new tokens, or ring tokens pushed out
//      of the recent window -- rotates them on the matrix cores, clips,
//      computes per-group fp16 scale / zero and codes, and stores codes and
//      meta in the documented layout (read-modify-write for rows already
//      present).
//   2. write_raw_kernel: stores new sink / recent tokens raw, after (1) has
//      read any ring slot it overwrites.
#include "kernels.h"

namespace oscar {

struct WriteArgs {
  oscar_layer_cache c;
  const uint8_t *forms[2];
  float clip[2];
  int64_t fstride[2];              // bytes between KV heads' forms (0: one rotation for the layer)
  float hclip[2][MAX_HEAD_ROT];    // per-head clips (fstride != 0)
  const uint16_t *src[2];  // k_new, v_new
  const int32_t *cu_new;
  const int32_t *len_before;
  int64_t total_tokens;
  int max_new;
};

// Request b's rows cu_new[b]..cu_new[b+1]-1 must lie in [0, total_tokens) and
// number at most max_new (the grid covers no more); otherwise the request is
// skipped and flagged.
// The values are read into scalars, so the checks and everything that
// follows from them stay uniform branches.
__device__ inline bool request_ok(const WriteArgs &a, int b, int &L0, int &n) {
  const int c0 = __builtin_amdgcn_readfirstlane(a.cu_new[b]);
  const int c1 = __builtin_amdgcn_readfirstlane(a.cu_new[b + 1]);
  L0 = __builtin_amdgcn_readfirstlane(a.len_before[b]);
  n = c1 - c0;
  return c0 >= 0 && c1 >= c0 && int64_t(c1) <= a.total_tokens && n <= a.max_new && L0 >= 0 &&
         int64_t(L0) + n < (int64_t(1) << 30);
}

constexpr int WHC = 4;   // KV heads per write workgroup (one rotation for the layer)
constexpr int WPP = 16;  // history pages per write workgroup (the R pieces stay in registers)
// LDS bytes per staged token row (all HC heads of a workgroup; padded).  With
// a rotation per KV head a workgroup takes one head (HC = 1): its R pieces
// are the ones in registers.
template <int HC>
constexpr int xstr() { return HC * D * 2 + 16; }

typedef _Float16 f16x8w __attribute__((ext_vector_type(8)));
typedef float f32x4w __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4w __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2w __attribute__((ext_vector_type(2)));

// Minimum / maximum over the four lanes l, l^16, l^32, l^48 (one token of
// the transposed product), in every one of them: row swaps between lanes of
// registers, no LDS round trip.
__device__ inline float lanes4_min(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float lanes4_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Eight bf16 values (four dwords) as eight fp16 values: exact for
// 2^-14 <= |x| <= 65504; below, within 2^-24; beyond, saturated to 65504
// (round toward zero).
__device__ inline u32x4w bf16x8_to_f16x8(u32x4w u) {
  u32x4w r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(u[i] << 16), __uint_as_float(u[i] & 0xFFFF0000u));
    r[i] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

// One code dword of the documented layout from 16 code bytes (code k in the
// low two bits of byte k % 4 of w[k / 4]; code k goes to slot k / 2, low
// half for even k, high half for odd k).  The slot bit offsets fall into
// four classes by their offset within a byte (0, 2, 4, 6); each class is one
// byte permutation, shifted into place.
__device__ inline uint32_t pack16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const uint32_t p0 = __builtin_amdgcn_perm(w0, w3, 0x05000401u);
  const uint32_t p2 = __builtin_amdgcn_perm(w1, w2, 0x07030602u);
  const uint32_t p4 = __builtin_amdgcn_perm(w1, w2, 0x05010400u);
  const uint32_t p6 = __builtin_amdgcn_perm(w0, w3, 0x03070206u);
  return p0 | (p2 << 2) | (p4 << 4) | (p6 << 6);
}

// One INT4 code dword from eight code bytes x0 (codes a0..a3), x1 (b0..b3):
// nibbles 0..7 = a0, a2, b0, b2, a1, a3, b1, b3.  For K, x0 / x1 are channels
// j = 0..3 / 4..7 of a token (nibble e then holds channel 2 (e % 4) + e / 4);
// for V, rows 0..3 of channel 16 (2d) + m / 16 (2d + 1) + m.  x | x >> 12
// puts a0 | a2 << 4 in byte 0 and a1 | a3 << 4 in byte 1 (codes < 16).
__device__ inline uint32_t pack8(uint32_t x0, uint32_t x1) {
  const uint32_t e0 = x0 | (x0 >> 12), e1 = x1 | (x1 >> 12);
  return __builtin_amdgcn_perm(e1, e0, 0x05010400u);
}

// K code rows in LDS: 136 bytes apart (34 dwords), so the 16 tokens of a
// row-group write and read distinct banks
constexpr int KROW = D + 8;

template <int G, int HC>
struct WriteShared {
  uint8_t xs[PAGE * xstr<HC>()];            // the page's rows, all heads of the chunk (bf16)
  uint8_t codes[2][HC][PAGE * KROW];        // per buffer -- K: [token][channel] (rows KROW bytes apart); V: [channel][token]
  float pmin[HC][PAGE][4], pmax[HC][PAGE][4];  // per wave (groups wider than a wave)
  float sz[2][HC][D / G][PAGE][2];          // per buffer: (scale, zero) after fp16 rounding
  int bad[2][4];                            // per page parity: a wave met a bad ring page id
};

// Where the token at position p (uniform) comes from: the ring (it leaves
// the recent window now) or the new rows (src: rows of head h0, starting at
// the request's first new row).  Sets row/stride (elements between heads) or
// leaves row null (inactive); bad: its ring page id is out of range.  ids:
// lane 16 + i holds bf16_pt[b][i] (the request's BF16 page ids, loaded once).
__device__ inline void token_source(const WriteArgs &a, int ids, int tensor, int h0, int L0, int hlo, int hhi,
                                    int p, const uint16_t *src, const uint16_t *&row, int &stride, bool &bad) {
  const oscar_layer_cache &c = a.c;
  const int hkv = c.n_kv_heads;
  row = nullptr;
  stride = 0;
  bad = false;
  if (p < hlo || p >= hhi) return;
  if (p >= L0) {
    row = src + int64_t(p - L0) * hkv * D;
    stride = D;
  } else {
    const int slot = p % N_RECENT;
    const int bp = __builtin_amdgcn_readlane(ids, 16 + 1 + slot / PAGE);
    if (bp >= 0 && bp < c.n_bf16_pages) {
      row = c.bf16 + ((int64_t(bp) * hkv + h0) * 2 + tensor) * (PAGE * D) + (slot % PAGE) * D;
      stride = 2 * PAGE * D;
    } else {
      bad = true;
    }
  }
}

// One workgroup (4 waves) per (request, WPP consecutive history pages, K|V,
// up to HC KV heads).  Per page: the rows that enter history in this call
// -- new tokens, or ring tokens pushed out of the recent window -- are staged
// in LDS for all heads of the chunk as fp16 (exact in fp16's normal range),
// rotated on the matrix cores as 2^11 Y = X (2^11 R_hi) + X R_lo with
// R_hi = fp16(R) and R_lo = fp16(2^11 (R - R_hi)), both products summed in
// one fp32 accumulator (the small ones first), so the error stays within the
// fp32 dot-product bound.  Wave w computes output channels 32w .. 32w+31 of
// every head; then clip, per-(token, group) fp16 zero = min and scale =
// (max - min)/3 (reductions across the lanes of a token, then across the
// waves of a group wider than 32), codes, and the packed store in the
// documented layout.
//
// Pipeline: page j's rows are staged from registers loaded during page j-1;
// page j+1's loads are issued right after staging, then page j-1's codes and
// meta (kept in the other LDS buffer) are stored, then page j is computed.
// The next wait for loads comes at page j+1's staging, a whole page later.
// All page ids of the workgroup are loaded once, into lanes of one register.
template <int G, int TENSOR, int BITS, int HC>
__device__ __forceinline__ void write_hist_body(const WriteArgs &a, WriteShared<G, HC> &sh) {
  constexpr int XSTR = xstr<HC>();
  constexpr int NG = D / G, WPG = G / 32;
  constexpr int LEVELS = (1 << BITS) - 1;     // highest code
  constexpr uint32_t CMASK = 0x01010101u * LEVELS;  // one code per byte
  // workgroup and work-item ids through the builtins: in an inlined body,
  // blockIdx / threadIdx may become calls that return vector registers
  const int bx = __builtin_amdgcn_workgroup_id_x(), by = __builtin_amdgcn_workgroup_id_y();
  const int b = __builtin_amdgcn_workgroup_id_z();
  constexpr int tensor = TENSOR;  // 0: K, 1: V (the low bit of blockIdx.y)
  const int hc = by >> 1;
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const oscar_layer_cache &c = a.c;
  const int hkv = c.n_kv_heads;
  const int h0 = hc * HC;
  if (h0 >= hkv) return;
  const int nh = min(HC, hkv - h0);

  int L0, n;
  if (!request_ok(a, b, L0, n)) {
    if (tid == 0 && bx == 0 && by == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  const int L = L0 + n;
  const int hlo = max(N_SINK, L0 - N_RECENT);  // first position entering history
  const int hhi = L - N_RECENT;                 // one past the last
  if (hhi <= hlo) return;
  const int jfirst = (hlo - N_SINK) / PAGE + bx * WPP;
  if (N_SINK + PAGE * jfirst >= hhi) return;
  const int jend = min((hhi - N_SINK + PAGE - 1) / PAGE, jfirst + WPP);
  // the clip (the chunk's head's own with a rotation per head) in the
  // accumulators' 2^11 scale
  const float clip_s = (a.fstride[tensor] ? a.hclip[tensor][h0] : a.clip[tensor]) * 2048.0f;
  const int r_a = lane & 15, qd = lane >> 4;  // MFMA: token row (A) / column (B, D); k sub-block / row group

  // page ids: lane i < WPP holds hist_pt[b][jfirst + i] (-1 past the table),
  // lane 16 + i holds bf16_pt[b][i]
  static_assert(WPP <= 16 && 16 + BF16_PT <= 64, "page ids fit the lanes of one register");
  int ids = -1;
  if (lane < WPP) {
    const int j = jfirst + lane;
    if (j < jend && j < c.hist_pt_stride) ids = c.hist_pt[int64_t(b) * c.hist_pt_stride + j];
  } else if (lane >= 16 && lane < 16 + BF16_PT) {
    ids = c.bf16_pt[b * BF16_PT + lane - 16];
  }

  // ---- the next page's rows, into registers: thread piece k covers token
  // wave + 4k, head (lane / 16), bytes 16 (lane % 16) .. of its row.  Each
  // row is read through a buffer resource whose size covers exactly the
  // chunk's heads of that row (none when the position has no row): lanes
  // past it read zeros, with no select and no wait after the loads.
  u32x4w xr[4];
  bool bad_next = false;
  // the request's new rows of head h0 (a uniform base: scalar address math)
  const uint16_t *src0 = a.src[tensor] + (int64_t(__builtin_amdgcn_readfirstlane(a.cu_new[b])) * hkv + h0) * D;
  // lane byte offsets in a new row (heads D elements apart) and in a ring
  // row (heads 2 PAGE D elements apart)
  const uint32_t off_new = uint32_t((lane >> 4) * (D * 2) + 16 * (lane & 15));
  const uint32_t off_ring = uint32_t((lane >> 4) * (2 * PAGE * D * 2) + 16 * (lane & 15));
  auto load_page = [&](int j) {
    const int pos0 = N_SINK + PAGE * j;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = __builtin_amdgcn_readfirstlane(pos0 + wave + 4 * k);
      const uint16_t *row;
      int stride;
      bool bd;
      token_source(a, ids, tensor, h0, L0, hlo, hhi, p, src0, row, stride, bd);
      bad |= bd;
      const bool ring = stride != D;
      const int nrec = row == nullptr ? 0 : (nh - 1) * stride * 2 + D * 2;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(row ? row : src0), 0, nrec, 0x00020000);
      xr[k] = __builtin_bit_cast(u32x4w, __builtin_amdgcn_raw_buffer_load_b128(rs, ring ? off_ring : off_new, 0, 0));
    }
    bad_next = bad;
  };
  load_page(jfirst);

  // A operands: 2^11 times the fp16 high part and the 2^11-scaled fp16 low
  // part of R (both exact scalings) for this wave's two tiles of output
  // channels; lane l holds R[i][j] for j = 32 wave + 16 ct + l%16,
  // i = 32 kk + 8 (l/16) .. + 7.  The products then land in one accumulator
  // as 2^11 y.
  f16x8w rh[2][4], rl[2][4];
  {
    const uint8_t *F = a.forms[tensor] + h0 * a.fstride[tensor];
    const uint16_t *RH = reinterpret_cast<const uint16_t *>(F + FORM_RT_HI);
    const uint16_t *RL = reinterpret_cast<const uint16_t *>(F + FORM_RT_LO);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int jj = 32 * wave + 16 * ct + r_a, ii = 32 * kk + 8 * qd;
        rh[ct][kk] = __builtin_bit_cast(f16x8w, *reinterpret_cast<const u32x4w *>(RH + jj * D + ii)) *
                     (_Float16)2048.0f;
        rl[ct][kk] = __builtin_bit_cast(f16x8w, *reinterpret_cast<const u32x4w *>(RL + jj * D + ii));
      }
  }

  // ---- packed store of a computed page (codes and meta in LDS buffer buf):
  // the code dwords of each head (INT2: 128, one per thread; INT4: 256, two
  // per thread), then the meta entries.  INT2 K dword (token t, q, d):
  // channels 64d + 8q .. +7 and 64d + 32 + 8q .. +7 of token t; V dword
  // (q, m, d): tokens 4q .. 4q+3 of channels 16 (4d + r) + m, r < 4.  INT4 K
  // dword (t, q, i): channels 32i + 8q .. +7 of token t; V dword (q, m, i):
  // tokens 4q .. 4q+3 of channels 16 (2i) + m and 16 (2i + 1) + m.  Rows
  // below hlo are already in history and are kept (read-modify-write); rows
  // at or past hhi are not yet and may be overwritten.
  const int hbb = hist_block_bytes(G, BITS);
  // Heads are wave-uniform (waves 2i, 2i+1 take head 2k + i of the codes,
  // wave w head w of the meta), so block addresses stay scalar.
  auto store_page = [&](int pid, int pos0, int buf) {
    for (int hb = 0; hb < nh; hb += 2) {
      const int hh = hb + (wave >> 1);
      if (hh >= nh) break;
      const int w = tid & 127;
      const int ln = w >> 1, d = w & 1, lq = ln >> 4, la = ln & 15;
      uint8_t *blk = c.hist + (int64_t(pid) * hkv + h0 + hh) * hbb;
      if constexpr (BITS == 4) {
        // dwords 4 ln + 2 d and 4 ln + 2 d + 1 of the head's code area
        if constexpr (tensor == 0) {
          const int t = la, p = pos0 + t;
          if (p < hlo || p >= hhi) continue;
          const uint8_t *src = &sh.codes[buf][hh][t * KROW + 64 * d + 8 * lq];
          const u32x2w x0 = *reinterpret_cast<const u32x2w *>(src);
          const u32x2w x1 = *reinterpret_cast<const u32x2w *>(src + 32);
          reinterpret_cast<u32x2w *>(blk + k_codes_off(G, 4))[w] = u32x2w{pack8(x0[0], x0[1]), pack8(x1[0], x1[1])};
        } else {
          uint32_t keep = 0, on = 0;  // code bytes of kept / written tokens 4lq + byte
#pragma unroll
          for (int by = 0; by < 4; ++by) {
            const int p = pos0 + 4 * lq + by;
            if (p < hlo) keep |= 0x0Fu << (8 * by);
            else if (p < hhi) on |= 0x0Fu << (8 * by);
          }
          if (!on) continue;
          uint32_t word[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int i = 2 * d + s2;
            const uint32_t xa =
                *reinterpret_cast<const uint32_t *>(&sh.codes[buf][hh][(16 * (2 * i) + la) * PAGE + 4 * lq]) & on;
            const uint32_t xb =
                *reinterpret_cast<const uint32_t *>(&sh.codes[buf][hh][(16 * (2 * i + 1) + la) * PAGE + 4 * lq]) & on;
            word[s2] = pack8(xa, xb);
          }
          u32x2w *dst = reinterpret_cast<u32x2w *>(blk + v_codes_off(G, 4)) + w;
          if (keep) {
            const uint32_t km = pack8(keep, keep);
            const u32x2w old = *dst;
            *dst = u32x2w{(old[0] & km) | word[0], (old[1] & km) | word[1]};
          } else {
            *dst = u32x2w{word[0], word[1]};
          }
        }
      } else if constexpr (tensor == 0) {
        const int t = la, p = pos0 + t;
        if (p < hlo || p >= hhi) continue;
        const uint8_t *src = &sh.codes[buf][hh][t * KROW + 64 * d + 8 * lq];
        const u32x2w x0 = *reinterpret_cast<const u32x2w *>(src);
        const u32x2w x1 = *reinterpret_cast<const u32x2w *>(src + 32);
        reinterpret_cast<uint32_t *>(blk + k_codes_off(G))[w] = pack16(x0[0], x0[1], x1[0], x1[1]);
      } else {
        uint32_t keep = 0, on = 0;  // bytes of kept / written tokens 4lq + byte
#pragma unroll
        for (int by = 0; by < 4; ++by) {
          const int p = pos0 + 4 * lq + by;
          if (p < hlo) keep |= 0x03u << (8 * by);
          else if (p < hhi) on |= 0x03u << (8 * by);
        }
        if (!on) continue;
        uint32_t x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          x[r] = *reinterpret_cast<const uint32_t *>(&sh.codes[buf][hh][(16 * (4 * d + r) + la) * PAGE + 4 * lq]) & on;
        const uint32_t word = pack16(x[0], x[1], x[2], x[3]);
        uint32_t *dst = reinterpret_cast<uint32_t *>(blk + v_codes_off(G)) + w;
        if (keep) {
          const uint32_t km = pack16(keep, keep, keep, keep);
          *dst = (*dst & km) | word;
        } else {
          *dst = word;
        }
      }
    }
    if (wave < nh && lane < PAGE * NG) {
      const int hh = wave, t = lane / NG, gg = lane % NG;
      const int p = pos0 + t;
      if (p >= hlo && p < hhi) {
        uint8_t *blk = c.hist + (int64_t(pid) * hkv + h0 + hh) * hbb;
        __half2 *meta = reinterpret_cast<__half2 *>(blk + (tensor ? v_meta_off(G, BITS) : k_meta_off(G, BITS)));
        meta[PAGE * gg + t] =
            __halves2half2(__float2half_rn(sh.sz[buf][hh][gg][t][0]), __float2half_rn(sh.sz[buf][hh][gg][t][1]));
      }
    }
  };

  int prev_pid = -1, prev_pos0 = 0, buf = 0;
  for (int jv = jfirst; jv < jend; ++jv) {
    const int j = __builtin_amdgcn_readfirstlane(jv);  // uniform (kept scalar)
    const int pos0 = N_SINK + PAGE * j;
    // ---- stage this page's rows (the previous page's barrier freed xs)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = wave + 4 * k, hh = lane >> 4, c16 = lane & 15;
      const u32x4w v = bf16x8_to_f16x8(xr[k]);
      if (hh < HC) *reinterpret_cast<u32x4w *>(sh.xs + t * XSTR + hh * (D * 2) + 16 * c16) = v;
    }
    if (lane == 0) sh.bad[j & 1][wave] = __ballot(bad_next) != 0;
    __syncthreads();
    const bool page_bad =
        __builtin_amdgcn_readfirstlane(sh.bad[j & 1][0] | sh.bad[j & 1][1] | sh.bad[j & 1][2] | sh.bad[j & 1][3]) != 0;
    if (j + 1 < jend) load_page(j + 1);  // in flight during this page
    if (prev_pid >= 0) store_page(prev_pid, prev_pos0, buf ^ 1);
    const int pid = __builtin_amdgcn_readlane(ids, j - jfirst);
    const bool skip = page_bad || pid < 0 || pid >= c.n_hist_pages;  // uniform
    if (skip) {
      if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    } else {
      // ---- rotate, clip, per-(token, wave) min / max; then scale, zero and
      // codes (at once when a group is the wave's 32 channels, else after
      // the waves of each group have combined their partials through LDS).
      // The product is taken transposed, Y^T = R^T X^T (A: rows of R^T, B:
      // the staged rows), so that lane (n = l%16, qd = l/16) holds token n,
      // channels 32 wave + 16 ct + 4 qd + i: the per-token work runs once
      // per lane, and a token's 32 channels of the wave are in the four
      // lanes n + 16 qd.
      const int g = (32 * wave) / G;
      const int tok = r_a;
      // byte selectors of the quad transpose: first swap 2-byte halves with
      // lane ^ 2, then single bytes with lane ^ 1 (perm: bytes 0-3 own, 4-7
      // the partner's)
      const uint32_t selA = (tok & 2) ? 0x03020706u : 0x05040100u;
      const uint32_t selB = (tok & 1) ? 0x03070105u : 0x06020400u;
      float szv[HC][2];  // (scale, zero) of each head's group; stored after the heads
      auto products = [&](int hh, f32x4w (&acc2)[2]) {
        f16x8w xb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          xb[kk] = __builtin_bit_cast(
              f16x8w, *reinterpret_cast<const u32x4w *>(sh.xs + tok * XSTR + hh * (D * 2) + 2 * (32 * kk + 8 * qd)));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          // fp16 x fp16 products are exact in fp32; the small low-part
          // products are summed first, so the accumulator's rounding stays
          // within the fp32 dot-product bound of the high part's sum, and R
          // is carried to 2^-22 relative
          f32x4w acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(rl[ct][kk], xb[kk], acc, 0, 0, 0);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(rh[ct][kk], xb[kk], acc, 0, 0, 0);
          acc2[ct] = acc;
        }
      };
      auto finish = [&](const f32x4w (&acc2)[2], f32x4w (&yc)[2], float &lo, float &hi) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) yc[ct][i] = __builtin_amdgcn_fmed3f(acc2[ct][i], -clip_s, clip_s);
        lo = fminf(fminf(fminf(yc[0][0], yc[0][1]), fminf(yc[0][2], yc[0][3])),
                   fminf(fminf(yc[1][0], yc[1][1]), fminf(yc[1][2], yc[1][3])));
        hi = fmaxf(fmaxf(fmaxf(yc[0][0], yc[0][1]), fmaxf(yc[0][2], yc[0][3])),
                   fmaxf(fmaxf(yc[1][0], yc[1][1]), fmaxf(yc[1][2], yc[1][3])));
        lo = lanes4_min(lo) * (1.0f / 2048.0f);
        hi = lanes4_max(hi) * (1.0f / 2048.0f);
      };
      auto quantise = [&](int hh, const f32x4w (&yc)[2], float lo, float hi) {
        // (max - min) / LEVELS by a product with fp32(1 / LEVELS) and the
        // code step by a hardware reciprocal: each within three fp32 ulps,
        // far inside the error bound of the rotated values they come from
        const float sq = __half2float(__float2half_rn((hi - lo) * (1.0f / float(LEVELS))));
        const float zq = __half2float(__float2half_rn(lo));
        szv[hh][0] = sq;
        szv[hh][1] = zq;
        // scale and zero in the accumulators' 2^11 scale (exact)
        const float ss = sq * 2048.0f, zs = zq * 2048.0f;
        const float inv = sq > 0.f ? __builtin_amdgcn_rcpf(ss) : 0.f;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          // step t = (x - z) / s: x - z is exact for exactly representable
          // inputs, and one residual correction of the reciprocal product
          // makes t exact whenever the true quotient is a float, so a value
          // exactly halfway between two levels rounds like the fp64 rule
          // (x - z = 1.5 s happens with unrotated bf16 inputs).  Then code =
          // round-half-even of the clamped step: adding 1.5 * 2^23 rounds to
          // an integer (ulp 1) and leaves it in the low byte.
          uint32_t cd[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float d = yc[ct][i] - zs;
            const float t0 = d * inv;
            const float t = fmaf(fmaf(-t0, ss, d), inv, t0);
            cd[i] = __float_as_uint(__builtin_amdgcn_fmed3f(t, 0.f, float(LEVELS)) + 12582912.0f);
          }
          const int ch = 32 * wave + 16 * ct + 4 * qd;
          // the four codes (channels ch .. ch+3 of the lane's token) as bytes
          const uint32_t pk = __builtin_amdgcn_perm(__builtin_amdgcn_perm(cd[3], cd[2], 0x0c0c0400u),
                                                    __builtin_amdgcn_perm(cd[1], cd[0], 0x0c0c0400u), 0x05040100u);
          if constexpr (tensor == 0) {
            *reinterpret_cast<uint32_t *>(&sh.codes[buf][hh][tok * KROW + ch]) = pk;
          } else {
            // 4 x 4 byte transpose within each quad of lanes (tokens 4q ..
            // 4q+3): afterwards lane 4q + r holds channel ch + r of the
            // quad's four tokens, one dword of the [channel][token] layout
            const uint32_t xa = uint32_t(__builtin_amdgcn_mov_dpp(int(pk), 0x4E, 0xF, 0xF, false));  // lane ^ 2
            const uint32_t pa = __builtin_amdgcn_perm(xa, pk, selA);
            const uint32_t xb = uint32_t(__builtin_amdgcn_mov_dpp(int(pa), 0xB1, 0xF, 0xF, false));  // lane ^ 1
            const uint32_t pb = __builtin_amdgcn_perm(xb, pa, selB);
            *reinterpret_cast<uint32_t *>(&sh.codes[buf][hh][(ch + (tok & 3)) * PAGE + (tok & ~3)]) = pb;
          }
        }
      };
      if constexpr (WPG == 1) {
        // the next head's products are issued before this head's vector
        // work, so the matrix cores run while the lanes quantise
        f32x4w acc_cur[2], acc_next[2];
        products(0, acc_cur);
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          if (hh + 1 < HC) products(hh + 1, acc_next);
          f32x4w yc[2];
          float lo, hi;
          finish(acc_cur, yc, lo, hi);
          quantise(hh, yc, lo, hi);
          if (hh + 1 < HC) {
            acc_cur[0] = acc_next[0];
            acc_cur[1] = acc_next[1];
            // spread the next head's sixteen products over this head's
            // vector instructions
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
          }
        }
      } else {
        f32x4w yc[HC][2];
        float lo[HC], hi[HC];
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          f32x4w acc2[2];
          products(hh, acc2);
          finish(acc2, yc[hh], lo[hh], hi[hh]);
          if (qd == 0) {
            sh.pmin[hh][tok][wave] = lo[hh];
            sh.pmax[hh][tok][wave] = hi[hh];
          }
        }
        __syncthreads();
        const int w0 = (wave / WPG) * WPG;
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          float l2 = sh.pmin[hh][tok][w0], h2 = sh.pmax[hh][tok][w0];
#pragma unroll
          for (int w = 1; w < WPG; ++w) {
            l2 = fminf(l2, sh.pmin[hh][tok][w0 + w]);
            h2 = fmaxf(h2, sh.pmax[hh][tok][w0 + w]);
          }
          quantise(hh, yc[hh], l2, h2);
        }
      }
      if (qd == 0 && wave % WPG == 0) {
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          sh.sz[buf][hh][g][tok][0] = szv[hh][0];
          sh.sz[buf][hh][g][tok][1] = szv[hh][1];
        }
      }
    }
    // this page's codes are complete and nobody reads xs any more
    __syncthreads();
    prev_pid = skip ? -1 : pid;
    prev_pos0 = pos0;
    if (!skip) buf ^= 1;
  }
  if (prev_pid >= 0) store_page(prev_pid, prev_pos0, buf ^ 1);
}

// G = 32 fits three waves per SIMD without spills (one group per wave: no
// min / max partials held across a barrier); wider groups keep two.
// K and V workgroups (the low bit of blockIdx.y) run separate instances of
// the body, so the tensor's branches are resolved at compile time.
template <int G, int BITS, int HC>
__global__ void __launch_bounds__(256) write_hist_kernel(WriteArgs a) {
  __shared__ __attribute__((aligned(16))) WriteShared<G, HC> sh;
  if (__builtin_amdgcn_workgroup_id_y() & 1)
    write_hist_body<G, 1, BITS, HC>(a, sh);
  else
    write_hist_body<G, 0, BITS, HC>(a, sh);
}
template <int BITS, int HC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) write_hist_kernel_g32(WriteArgs a) {
  __shared__ __attribute__((aligned(16))) WriteShared<32, HC> sh;
  if (__builtin_amdgcn_workgroup_id_y() & 1)
    write_hist_body<32, 1, BITS, HC>(a, sh);
  else
    write_hist_body<32, 0, BITS, HC>(a, sh);
}

// New tokens that land in the sink or the recent ring: raw bf16 copies.
// Block x < 16 takes sink position x, block x >= 16 takes position
// L - 128 + (x - 16) of the recent window; positions outside this call's new
// tokens are skipped.
__global__ void __launch_bounds__(256) write_raw_kernel(WriteArgs a) {
  const int b = blockIdx.y;
  const int x = blockIdx.x;
  const oscar_layer_cache &c = a.c;
  int L0, n;
  if (!request_ok(a, b, L0, n)) return;  // flagged by write_hist_kernel
  const int L = L0 + n;
  int p, page, row;
  if (x < N_SINK) {
    p = x;
    if (p < L0 || p >= L) return;
    page = c.bf16_pt[b * BF16_PT];
    row = p;
  } else {
    p = L - N_RECENT + (x - N_SINK);
    if (p < L0 || p < N_SINK || p >= L) return;
    const int slot = p % N_RECENT;
    page = c.bf16_pt[b * BF16_PT + 1 + slot / PAGE];
    row = slot % PAGE;
  }
  if (page < 0 || page >= c.n_bf16_pages) {
    if (threadIdx.x == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    return;
  }
  const int hkv = c.n_kv_heads;
  const int64_t src_row = a.cu_new[b] + (p - L0);
  for (int e = threadIdx.x; e < hkv * 2 * D; e += 256) {
    const int h = e / (2 * D), tensor = (e / D) & 1, ch = e % D;
    c.bf16[((int64_t(page) * hkv + h) * 2 + tensor) * (PAGE * D) + row * D + ch] =
        a.src[tensor][(src_row * hkv + h) * D + ch];
  }
}

hipError_t launch_write_kv(const oscar_layer_cache &c, RotArg rk, RotArg rv,
                           const uint16_t *k_new, const uint16_t *v_new, const int32_t *cu_new,
                           const int32_t *len_before, int batch, int64_t total_tokens, int max_new,
                           hipStream_t s) {
  WriteArgs a;
  a.c = c;
  a.forms[0] = rk.forms;
  a.forms[1] = rv.forms;
  a.clip[0] = rk.clip;
  a.clip[1] = rv.clip;
  a.fstride[0] = rk.stride;
  a.fstride[1] = rv.stride;
  for (int h = 0; h < MAX_HEAD_ROT; ++h) {
    a.hclip[0][h] = rk.head_clip[h];
    a.hclip[1][h] = rv.head_clip[h];
  }
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.cu_new = cu_new;
  a.len_before = len_before;
  a.total_tokens = total_tokens;
  a.max_new = max_new;
  // history positions entering in one call span at most max_new + 16 rows;
  // a rotation per KV head: one head per workgroup
  const bool per_head = rk.stride != 0 || rv.stride != 0;
  const int hc = per_head ? 1 : WHC;
  const int tiles = (max_new + PAGE - 1) / PAGE + 2;
  const dim3 grid((tiles + WPP - 1) / WPP, 2 * ((c.n_kv_heads + hc - 1) / hc), batch);
  const KernelEvents ev = take_profile_events();
  const bool int4 = cache_bits(c) == 4;
  auto go = [&](auto kern) { hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, s, ev.before, ev.after, 0, a); };
  auto pick = [&](auto hc_tag) {
    constexpr int H = decltype(hc_tag)::value;
    switch (c.group) {
      case 32: int4 ? go(write_hist_kernel_g32<4, H>) : go(write_hist_kernel_g32<2, H>); break;
      case 64: int4 ? go(write_hist_kernel<64, 4, H>) : go(write_hist_kernel<64, 2, H>); break;
      default: int4 ? go(write_hist_kernel<128, 4, H>) : go(write_hist_kernel<128, 2, H>); break;
    }
  };
  if (per_head)
    pick(std::integral_constant<int, 1>{});
  else
    pick(std::integral_constant<int, WHC>{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(write_raw_kernel, dim3(N_SINK + N_RECENT, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
