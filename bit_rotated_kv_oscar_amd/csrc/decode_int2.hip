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
// history part of the output is rotated back by R_V^T once per partial sum
// over a split of pages (or once per (request, query head) when a separate
// merge kernel combines the splits).  Per-group scale s and zero z are
// factored out of both
// contractions so the matrix cores see the 2-bit codes as exact fp16 values:
//   score_t = sum_g s_tg (q_g . c_tg) + z_tg sum_{i in g} q_i
//   o       = sum_g [ sum_t (p_t s_tg) c_tg ] + sum_t p_t z_tg
//
// The attend kernel runs one workgroup of 8 waves per (request, KV head,
// split):
//     split 0 attends over the raw BF16 sink + recent pages (a token being
//     appended is read from k_new / v_new); splits s >= 1 over history pages
//     (wave w takes every 8th page of the split; its first 64 page ids are
//     loaded at entry with the other loads that need no request length;
//     pages are copied straight into a per-wave LDS ring 4 pages ahead of
//     the one being computed).  While the first pages fly, each history
//     workgroup computes q_rot = q R_K * sm_scale * log2(e) for the query
//     heads of its group and lays it out as the A operand of the score
//     MFMAs (fp16 high + low parts, scale groups in separate rows).  On an
//     append whose token at position L-128 leaves the recent window (L >=
//     144), the raw workgroup rotates, clips and quantises that token into
//     history, stores the new token in its ring row, and attends the token
//     itself (dequantised, rotated back); the history workgroups leave its
//     row out.  Each workgroup writes an unnormalised partial (o[128], m, l)
//     per query head.
//   Merging the partials (LSE-combine, normalise, fp32 out) takes one of two
//   forms.  When all workgroups run in one round (small batches), the
//   attend kernel merges: history workgroups rotate their partial back with
//   R_V^T before storing it, and the last workgroup of a (request, KV head)
//   to finish, counted by an atomic counter in the workspace, combines them.
//   The L2 caches of the eight XCDs are not coherent with each other, and a
//   device-scope release fence writes back the whole L2, so the partials
//   travel by agent-scope stores and loads instead (they bypass the
//   non-coherent L2 state): a workgroup's stores complete before its count,
//   and the last workgroup's loads start after it.  Otherwise a merge kernel
//   (one block per (request, KV head)) combines the partials after the
//   attend kernel, rotating the history part back once.
#include <cmath>
#include <mutex>
#include <type_traits>

#include "attn_common.h"

namespace oscar {

constexpr int AW = 8;                // waves per attend workgroup
constexpr int MAX_SPLITS = 255;      // history splits per (request, KV head)

// Row layout of the score product for a GQA group of GQA query heads and NG
// scale groups.  The A operand (16 rows) holds q' = q R_K: row r of chain ch
// is J hl + 2 g + part (J = 2 NG rows per head): head HC ch + hl, scale group
// g, part 0/1 = fp16 high part / low part x 2^11 (zero outside group g).
// Lane (t = l%16, qd = l/16) of the result holds rows 4qd..4qd+3 for token t:
// the two parts of row pairs 2qd and 2qd+1, pair P being (head P / NG,
// group P % NG), so it forms its head's score for token t by itself (for
// NG = 4 a head spans lanes l and l^16).
template <int GQA, int NG>
struct Rows {
  static constexpr int G = D / NG;
  static constexpr int J = 2 * NG;
  static constexpr int HC = 16 / J;                // heads per chain
  static constexpr int NCH = (GQA + HC - 1) / HC;  // chains
  static constexpr int SPL = NG == 1 ? 2 : 1;      // scores per lane and chain
  // per-lane dwords of the fragment block
  static constexpr int FR_A = 0;                   // 16 per chain: A operand
  static constexpr int FR_INIT = 16 * NCH;         // 4 per chain: accumulator start (rows 4qd + i)
  static constexpr int FR_Q = FR_INIT + 4 * NCH;   // 2 per chain: kq * group sum of q' of pairs 2qd, 2qd+1
  static constexpr int FR_INVKQ = FR_Q + 2 * NCH;  // 1: 1 / kq
  static constexpr int FR_DW = FR_INVKQ + 1;
  // head of score slot s of lane group qd (chain-local)
  __device__ static constexpr int slot_head(int qd, int s) { return NG == 1 ? 2 * qd + s : (2 * qd) / NG; }
  // chain-local head and group of pair k of lane group qd
  __device__ static constexpr int pair_head(int qd, int k) { return (2 * qd + k) / NG; }
  __device__ static constexpr int pair_group(int qd, int k) { return (2 * qd + k) % NG; }
  // score slot holding pair k
  __device__ static constexpr int pair_slot(int k) { return NG == 1 ? k : 0; }
  // where head h's scores live: chain, lane group (for NG = 4 the first of
  // the two), slot
  __device__ static constexpr int head_chain(int h) { return h / HC; }
  __device__ static constexpr int head_qd(int h) { return NG == 1 ? (h % HC) / 2 : NG == 2 ? h % HC : 2 * (h % HC); }
  __device__ static constexpr int head_slot(int h) { return NG == 1 ? (h % HC) % 2 : 0; }
};

// INT2 with one or two scale groups per head (F4 below): the score product
// runs on the fp8 x fp4 matrix core instead (16x16x128, one instruction per
// 16 rows over all 128 channels).  The stored 2-bit codes become fp4 (e2m1)
// values c/2 by masking alone (nibble 00cc), and q' goes in as four fp8
// (e4m3) parts whose sum carries it to 2^-16 of its group's largest value,
// each part scaled back by the product's per-row power-of-two scale.  Per
// chain two products: product j row 4qd + p is part p of pair (2qd + j) of
// that chain (head and group as above), so lane (t, qd) again holds the
// whole score of its pairs for token t.
// Both plans (with the one-round plan's two-wave register budget the
// batch-1 kernel gains 2.5 % from it; FUSED is kept as a parameter for
// the choice).
template <int BITS, int NG, bool FUSED>
constexpr bool f4_scores() { return BITS == 2 && NG <= 2; }

// Channel of the K code in nibble s of fp4 operand lane group gB, once the
// lane's two code dwords are spread to nibbles (register v = s / 8 is dword
// v / 2 masked with 0x33333333 after a right shift by 2 (v % 2)): the code
// at bit pos of dword d is slot u of the code slot tables (low slot for
// even channels, high for odd), channel 32 (2d + u / 4) + 8 gB + 2 (u % 4)
// (+ 1 when high).
__device__ inline int f4_channel(int gB, int s) {
  const int v = s >> 3, pos = 4 * (s & 7) + 2 * (v & 1), hp = pos >> 1;
  const int u = int((0xE9832Eu >> (3 * (hp & 7))) & 7u);  // slots 6 5 4 1 0 3 2 7 at bits 0 2 4 .. 14 (mod 16)
  const int par = (hp >= 8) != ((hp & 7) == 0);
  return 32 * (2 * (v >> 1) + (u >> 2)) + 8 * gB + 2 * (u & 3) + par;
}

// 2^n for -126 <= n <= 127, exactly
__device__ inline float pow2i(int n) { return __uint_as_float(uint32_t(127 + n) << 23); }

// fp8 e4m3 (bias 7, subnormal step 2^-9) round-to-nearest-even of t,
// |t| < 448: the byte, and its value in val
__device__ inline uint32_t fp8_rne(float t, float &val) {
  const float a = fabsf(t);
  const int e = max(int((__float_as_uint(a) >> 23) & 255u) - 127, -6);  // floor(log2 a), at least -6
  const float q = rintf(a * pow2i(3 - e));                                // 0 .. 16
  val = copysignf(q * pow2i(e - 3), t);
  return (t < 0.f && q > 0.f ? 0x80u : 0u) | uint32_t(((e + 7) << 3) + int(q) - 8);
}

// The four fp8 part bytes of y (byte p = part p) for a group whose largest
// |y| has exponent E: part 0 is y 2^(7-E) rounded (below 256 in magnitude),
// each later part the remainder times 16 rounded (below 128)
__device__ inline uint32_t fp8_parts(float y, int E) {
  float t = y * pow2i(7 - E), val;
  uint32_t w = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    w |= fp8_rne(t, val) << (8 * p);
    t = (t - val) * 16.f;
  }
  return w;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
// the 32 fp8 bytes of an F4 A operand, held as two f16x8 fragment registers
__device__ inline i32x8 f4_operand(f16x8 lo, f16x8 hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
}

// Compute units of the current device (256 on MI355X; 256 when it cannot
// be queried, e.g. while sizing a workspace on a host without a GPU).
int64_t device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0)
    return n;
  return 256;
}

SplitPlan plan_int2_splits(int batch, int n_kv_heads, int max_seq_len) {
  const int pages = n_hist_pages(max_seq_len);
  SplitPlan p;
  if (pages == 0) {  // the raw workgroup alone: it merges its own partial
    p.pages_per_split = AW;
    p.n_splits = 0;
    p.fused = true;
    return p;
  }
  // One round of attend workgroups, one per CU (measured faster
  // at batch 1 than two per CU: each workgroup's fixed work, the q fragment
  // and the epilogue, is paid half as often and the merge reads half the
  // partials).  When every unit (request, KV head) fits in that round with
  // at least one history split, spread each unit's pages over as many splits
  // as it holds (its raw workgroup included); otherwise use splits of 64
  // pages per wave (measured with the split index slowest in the grid: at
  // batch 64 / 28 x 100K, 24, 32 and 48 pages lose 8 / 26, 4 / 15 and 1 / 4 %
  // to 64 in per-workgroup fixed work, 96 and 128 lose 4-13 % to the last
  // round's imbalance).
  // In the one-round case the last workgroup of each unit merges inside the
  // attend kernel (measured: ~2.5 us less per call at batch 1); with several
  // rounds, the election and the merge hold workgroup slots that other units
  // need, and a separate merge kernel is faster (~6 % at batch 64).
  const int64_t units = int64_t(batch) * n_kv_heads;
  const int64_t slots = device_cus();
  int64_t pps;
  if (slots - units >= units) {
    const int64_t per_unit = (slots - units) / units;
    pps = (pages + per_unit - 1) / per_unit;
    p.fused = true;
  } else {
    pps = 64 * AW;
  }
  if (pps < AW) pps = AW;
  const int64_t min_pps = (pages + MAX_SPLITS - 1) / MAX_SPLITS;  // bounds the merge's LDS
  if (pps < min_pps) pps = min_pps;
  p.pages_per_split = int(pps);
  p.n_splits = int((pages + pps - 1) / pps);
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Partial slots per query head: one per split (raw + history), and at least
// the merge's first register window, which it loads without bounds checks.
static_assert(MAX_SPLITS + 1 <= MAX_MERGE_SPLITS, "the merge holds every split's weight");
static int part_slots(const SplitPlan &p) { return 1 + (p.n_splits > MERGE_WINDOW ? p.n_splits : MERGE_WINDOW); }

// Workspace: the partials, then one merge counter per (request, KV head),
// each on a 256-byte line of its own (COUNTER_STRIDE words: atomics on one
// line serialise)
static size_t parts_bytes(int batch, int n_q_heads, const SplitPlan &p) {
  return align256(size_t(batch) * n_q_heads * part_slots(p) * PART_STRIDE * sizeof(float));
}

size_t decode_int2_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  const SplitPlan p = plan_int2_splits(batch, n_kv_heads, max_seq_len);
  return parts_bytes(batch, n_q_heads, p) + size_t(batch) * n_kv_heads * COUNTER_STRIDE * sizeof(uint32_t);
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
  uint32_t ex_mn;                 // INT4 expansion mask 0x03C003C0
  float *parts;                   // [B][Hq][part_slots][PART_STRIDE]
  int part_slots;                 // partials per query head: 1 + max(n_splits, merge window)
  uint32_t *counters;             // [B][Hkv][COUNTER_STRIDE]: word 0 = workgroups done (zero between calls)
  float *out;                     // [B][Hq][128]
  // per-KV-head rotations (last, so the fields above keep their offsets)
  int64_t fstride_k, fstride_v;   // bytes between KV heads' forms (0: one rotation for the layer)
  float hclip_k[MAX_HEAD_ROT], hclip_v[MAX_HEAD_ROT];  // per-head clips (fstride != 0)
};

__device__ inline bool valid_len(int L, int max_len) { return L >= 1 && L <= max_len; }

// KV head hk's rotation forms and clips.  PH (a rotation per KV head) is a
// template parameter: the per-layer instances read neither the strides nor
// the head clips, and compile as they would without them.
template <bool PH>
__device__ inline const uint8_t *forms_k(const StepArgs &a, int hk) { return PH ? a.fk + hk * a.fstride_k : a.fk; }
template <bool PH>
__device__ inline const uint8_t *forms_v(const StepArgs &a, int hk) { return PH ? a.fv + hk * a.fstride_v : a.fv; }
template <bool PH>
__device__ inline float head_clip_k(const StepArgs &a, int hk) {
  return (PH && a.fstride_k) ? a.hclip_k[hk] : a.clip_k;
}
template <bool PH>
__device__ inline float head_clip_v(const StepArgs &a, int hk) {
  return (PH && a.fstride_v) ? a.hclip_v[hk] : a.clip_v;
}

// ------------------------------------------------------------------ q and append

// LDS work area of the q fragment build.
template <int GQA, int NG>
struct QWork {
  static constexpr int SEG = (D / NG) < 64 ? (D / NG) : 64;  // channels per wave-level partial sum
  float x[GQA][D];  // q heads
  float y[GQA][D];  // rotated
  _Float16 qa[2][GQA][D];
  float gpart[3][GQA][D / SEG];
  float red[AW];
};

// Where the new token of an append goes and which token leaves the window.
struct AppendPlan {
  int L0;          // position of the new token
  int raw_page;    // BF16 page id of its row (-1 if bad)
  int raw_row;     // row in that page
  int raw_pg;      // index of that page in the request's BF16 table (0 sink, 1..8 ring)
  bool evict;      // position L0 - 128 moves into history (L0 >= 144)
  int evict_j;     // its history page index (= last history page)
  int evict_row;   // its row
};

// bpt_lane: entry min(lane, 8) of the request's BF16 page table (loaded by
// the caller before the length is known)
__device__ inline AppendPlan plan_append(const StepArgs &a, int len_before, int bpt_lane) {
  AppendPlan p;
  const oscar_layer_cache &c = a.c;
  p.L0 = len_before;
  if (p.L0 < N_SINK) {
    p.raw_pg = 0;
    p.raw_row = p.L0;
  } else {
    const int slot = p.L0 % N_RECENT;
    p.raw_pg = 1 + slot / PAGE;
    p.raw_row = slot % PAGE;
  }
  const int page = __builtin_amdgcn_readlane(bpt_lane, p.raw_pg);
  p.raw_page = (page >= 0 && page < c.n_bf16_pages) ? page : -1;
  p.evict = p.L0 >= N_RAW;
  const int h = p.L0 - N_RAW;  // history index of position L0 - 128
  p.evict_j = p.evict ? h / PAGE : -1;
  p.evict_row = p.evict ? h % PAGE : 0;
  return p;
}

// LDS work area of the token that leaves the recent window.
struct EvictWork {
  float x[2][D];      // its K and V (plain basis)
  float y[2][D];      // rotated
  float d[2][D];      // dequantised (rotated basis)
  float u[2][D];      // dequantised, rotated back to the plain basis
  float mm[2][2][2];  // groups of 128 channels: per vector and wave, min and max
  float sz[2][8];     // per vector and group: s, z
  uint8_t codes[2][D];
  float sc[8];        // its score per query head (log2 units)
};

// Append, raw workgroup: the token at position L0 - 128 leaves the recent
// window (OSCAR write path, gist.science technical summaries section 2.2:
// rotate, clip, quantise per group into the paged INT2 -- or INT4 --
// history).  Its K and
// V are read from their ring row and rotated by R_K / R_V, clipped and
// quantised (G channels per group), and its row of history block `blk` (null:
// bad page id) is written: the K codes and the meta are dwords of its own; the
// V codes share dwords with three other tokens (read-modify-write).  The new
// token then takes the ring row.  The attention takes this token from here,
// dequantised and rotated back (e.u; q.k is the same in either basis) with its
// score per query head (e.sc): the history workgroups leave its row out,
// since their copy of the page may predate this write.  Workgroup-wide.
template <int GQA, int G, int BITS, bool PH>
__device__ void evict_token(const StepArgs &a, int b, int hk, int tid, int wave, const AppendPlan &ap, uint8_t *blk,
                            EvictWork &e) {
  constexpr int LEVELS = (1 << BITS) - 1;
  const oscar_layer_cache &c = a.c;
  const int hkv = c.n_kv_heads, lane = tid & 63;
  const int jr = tid >> 3, qq = tid & 7;  // rows jr, jr + 64; inputs 32k + 4qq .. + 3
  // ---- loads: ring row and new token (threads < 256: K channel tid, V
  // channel tid - 128), R^T rows of R_K and R_V, the query heads
  const int v = (tid >> 7) & 1, ch = tid & (D - 1);
  uint16_t *ring = c.bf16 + ((int64_t(ap.raw_page) * hkv + hk) * 2 + v) * (PAGE * D) + ap.raw_row * D + ch;
  const uint16_t *nw = (v ? a.v_new : a.k_new) + (int64_t(b) * hkv + hk) * D + ch;
  uint16_t old_kv = 0, new_kv = 0;
  if (tid < 2 * D) {
    old_kv = *ring;
    new_kv = *nw;
  }
  f32x4 rf[2][8];
#pragma unroll
  for (int vec = 0; vec < 2; ++vec) {
    const float *RT = reinterpret_cast<const float *>((vec ? forms_v<PH>(a, hk) : forms_k<PH>(a, hk)) + FORM_RT) + jr * D + 4 * qq;
#pragma unroll
    for (int k = 0; k < 8; ++k) rf[vec][k] = *reinterpret_cast<const f32x4 *>(RT + (k >> 2) * 64 * D + 32 * (k & 3));
  }
  float q0 = 0.f, q1 = 0.f;
  if (wave < GQA) {
    const uint16_t *qh = a.q + (int64_t(b) * a.n_q_heads + hk * GQA + wave) * D;
    q0 = bf16_to_f32(qh[lane]);
    q1 = bf16_to_f32(qh[lane + 64]);
  }
  if (tid < 2 * D) {
    e.x[v][ch] = bf16_to_f32(old_kv);
    *ring = new_kv;  // the old value is read: the new token takes the row
  }
  __syncthreads();
  // ---- rotate: y[j] = sum_i x[i] R[i][j]; the eight lanes of a row combine
  // by DPP, the sum lands in lanes qq >= 4
  {
    float y0[2] = {0.f, 0.f}, y1[2] = {0.f, 0.f};
#pragma unroll
    for (int vec = 0; vec < 2; ++vec)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 xi = *reinterpret_cast<const f32x4 *>(&e.x[vec][32 * k + 4 * qq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y0[vec] = fmaf(xi[i], rf[vec][k][i], y0[vec]);
          y1[vec] = fmaf(xi[i], rf[vec][4 + k][i], y1[vec]);
        }
      }
#pragma unroll
    for (int vec = 0; vec < 2; ++vec) {
      y0[vec] = oct_sum(y0[vec]);
      y1[vec] = oct_sum(y1[vec]);
      if (qq == 4) {
        e.y[vec][jr] = y0[vec];
        e.y[vec][jr + 64] = y1[vec];
      }
    }
  }
  // rows of R_K and R_V for the way back, in flight during the quantisation
  f32x4 rb[2][8];
#pragma unroll
  for (int vec = 0; vec < 2; ++vec) {
    const float *Rr = reinterpret_cast<const float *>((vec ? forms_v<PH>(a, hk) : forms_k<PH>(a, hk)) + FORM_R) + jr * D + 4 * qq;
#pragma unroll
    for (int k = 0; k < 8; ++k) rb[vec][k] = *reinterpret_cast<const f32x4 *>(Rr + (k >> 2) * 64 * D + 32 * (k & 3));
  }
  __syncthreads();
  // ---- clip and quantise: group min / max over G consecutive channels (all
  // threads take part; threads >= 256 repeat the work of threads < 256)
  const float clip = v ? head_clip_v<PH>(a, hk) : head_clip_k<PH>(a, hk);
  const float xc = fminf(fmaxf(e.y[v][ch], -clip), clip);
  float lo, hi;
  if constexpr (G == 128) {
    lo = wave_min(xc);
    hi = wave_max(xc);
    if (lane == 0 && tid < 2 * D) {
      e.mm[v][wave & 1][0] = lo;
      e.mm[v][wave & 1][1] = hi;
    }
    __syncthreads();
    lo = fminf(e.mm[v][0][0], e.mm[v][1][0]);
    hi = fmaxf(e.mm[v][0][1], e.mm[v][1][1]);
  } else {
    lo = seg_min<G>(xc, lane);
    hi = seg_max<G>(xc, lane);
  }
  const float sq = __half2float(__float2half_rn((hi - lo) / float(LEVELS)));
  const float zq = __half2float(__float2half_rn(lo));
  const int code = sq > 0.f ? min(LEVELS, max(0, int(rintf((xc - zq) / sq)))) : 0;
  if (tid < 2 * D) {
    e.codes[v][ch] = uint8_t(code);
    e.d[v][ch] = fmaf(sq, float(code), zq);
    if (ch % G == 0) {
      e.sz[v][2 * (ch / G)] = sq;
      e.sz[v][2 * (ch / G) + 1] = zq;
    }
  }
  __syncthreads();
  // ---- the row in history (layouts of the code dwords: include/oscar.h)
  if (blk && BITS == 4) {
    const int row = ap.evict_row;
    if (tid < 16) {
      // K: dwords i of lanes 16q + row hold channels 32i + 8q + j of token
      // `row`, channel offset j = 2 (e % 4) + e / 4 in nibble e
      const int q = tid >> 2, i = tid & 3;
      uint32_t w = 0;
      for (int ee = 0; ee < 8; ++ee) w |= uint32_t(e.codes[0][32 * i + 8 * q + 2 * (ee % 4) + ee / 4]) << (4 * ee);
      *reinterpret_cast<uint32_t *>(blk + k_codes_off(G, 4) + 4 * (4 * (16 * q + row) + i)) = w;
    } else if (tid >= 64 && tid < 128) {
      // V: token `row` (quad q = row / 4, k = row % 4) is nibble e0 (channel
      // 16 (2d) + m) and e0 + 2 (channel 16 (2d + 1) + m) of dword d of lane
      // 16 q + m, with k = 2 (e0 % 2) + e0 / 4
      const int t = tid - 64, m = t & 15, d = t >> 4, q = row >> 2, k = row & 3;
      const int e0 = (k & 1) * 4 + (k >> 1);
      const uint32_t w = (uint32_t(e.codes[1][16 * (2 * d) + m]) << (4 * e0)) |
                         (uint32_t(e.codes[1][16 * (2 * d + 1) + m]) << (4 * (e0 + 2)));
      const uint32_t mask = (0xFu << (4 * e0)) | (0xFu << (4 * (e0 + 2)));
      uint32_t *p = reinterpret_cast<uint32_t *>(blk + v_codes_off(G, 4) + 4 * (4 * (16 * q + m) + d));
      *p = (*p & ~mask) | w;
    } else if (tid >= 128 && tid < 128 + 2 * (D / G)) {
      const int vec = (tid - 128) / (D / G), g = (tid - 128) % (D / G);
      const uint32_t w = uint32_t(__half_as_ushort(__float2half_rn(e.sz[vec][2 * g]))) |
                         (uint32_t(__half_as_ushort(__float2half_rn(e.sz[vec][2 * g + 1]))) << 16);
      *reinterpret_cast<uint32_t *>(blk + (vec ? v_meta_off(G, 4) : k_meta_off(G, 4)) + 4 * (PAGE * g + row)) = w;
    }
  } else if (blk) {
    const int row = ap.evict_row;
    if (tid < 8) {
      // K: the 8 dwords of token `row` (lanes 16q + row, halves d)
      const int q = tid >> 1, d = tid & 1;
      uint32_t w = 0;
      for (int u = 0; u < 8; ++u) {
        const int c0 = 32 * (2 * d + u / 4) + 8 * q + 2 * (u % 4);
        w |= uint32_t(e.codes[0][c0]) << slot_lo(u);
        w |= uint32_t(e.codes[0][c0 + 1]) << slot_hi(u);
      }
      *reinterpret_cast<uint32_t *>(blk + k_codes_off(G) + 4 * (2 * (16 * q + row) + d)) = w;
    } else if (tid >= 64 && tid < 96) {
      // V: 4 codes of token `row` in each of 32 dwords (lanes 16 (row/4) + m, halves d)
      const int t = tid - 64, m = t & 15, d = t >> 4, q = row >> 2, jj = (row & 3) >> 1;
      uint32_t w = 0, mask = 0;
      for (int rr = 0; rr < 4; ++rr) {
        const int u = 2 * rr + jj;
        const int bit = (row & 1) ? slot_hi(u) : slot_lo(u);
        w |= uint32_t(e.codes[1][16 * (4 * d + rr) + m]) << bit;
        mask |= 3u << bit;
      }
      uint32_t *p = reinterpret_cast<uint32_t *>(blk + v_codes_off(G) + 4 * (2 * (16 * q + m) + d));
      *p = (*p & ~mask) | w;
    } else if (tid >= 128 && tid < 128 + 2 * (D / G)) {
      // meta: (s, z) as fp16 per vector and group
      const int vec = (tid - 128) / (D / G), g = (tid - 128) % (D / G);
      const uint32_t w = uint32_t(__half_as_ushort(__float2half_rn(e.sz[vec][2 * g]))) |
                         (uint32_t(__half_as_ushort(__float2half_rn(e.sz[vec][2 * g + 1]))) << 16);
      *reinterpret_cast<uint32_t *>(blk + (vec ? v_meta_off(G) : k_meta_off(G)) + 4 * (PAGE * g + row)) = w;
    }
  }
  // ---- back to the plain basis: u[i] = sum_j d[j] R[i][j]
  {
    float u0[2] = {0.f, 0.f}, u1[2] = {0.f, 0.f};
#pragma unroll
    for (int vec = 0; vec < 2; ++vec)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 di = *reinterpret_cast<const f32x4 *>(&e.d[vec][32 * k + 4 * qq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u0[vec] = fmaf(di[i], rb[vec][k][i], u0[vec]);
          u1[vec] = fmaf(di[i], rb[vec][4 + k][i], u1[vec]);
        }
      }
#pragma unroll
    for (int vec = 0; vec < 2; ++vec) {
      u0[vec] = oct_sum(u0[vec]);
      u1[vec] = oct_sum(u1[vec]);
      if (qq == 4) {
        e.u[vec][jr] = u0[vec];
        e.u[vec][jr + 64] = u1[vec];
      }
    }
  }
  __syncthreads();
  // ---- its score per query head (wave h < GQA)
  if (wave < GQA) {
    const float sc = wave_sum(fmaf(q0, e.u[0][lane], q1 * e.u[0][lane + 64])) * (a.sm_scale * LOG2E);
    if (lane == 0) e.sc[wave] = sc;
  }
  __syncthreads();
}

// Global loads of the q fragment build, held in registers.  They are
// issued with the other loads that need no request length, ahead of the
// first page loads: the compiler waits for a load by counting the memory
// instructions issued after it, so the build then starts without waiting
// for any page.
template <int GQA>
struct QLoads {
  static constexpr int NQ = (GQA * D + AW * 64 - 1) / (AW * 64);
  f32x4 rk[8];     // R^T rows jr and jr + 64 of R_K, inputs 32k + 4qq .. + 3
  uint16_t q[NQ];  // query elements tid + 512 i of the group
};

// Every load is issued on every path (`hist` false: every lane re-reads one
// line of R_K), so the compiler can count exactly how many loads its waits
// may leave in flight.
template <int GQA, bool PH>
__device__ inline void build_q_issue(const StepArgs &a, int b, int hk, int tid, bool hist, QLoads<GQA> &ql) {
  constexpr int NT = AW * 64;
  // eight consecutive lanes read one 128-byte line of a row
  const int jr = tid >> 3, qq = tid & 7;
  const float *RT = reinterpret_cast<const float *>(forms_k<PH>(a, hk) + FORM_RT) + (hist ? jr * D : 0) + 4 * qq;
  const int s_hi = hist ? 64 * D : 0, s_k = hist ? 32 : 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ql.rk[k] = *reinterpret_cast<const f32x4 *>(RT + (k >> 2) * s_hi + s_k * (k & 3));
  const uint16_t *qg = a.q + (int64_t(b) * a.n_q_heads + hk * GQA) * D;
#pragma unroll
  for (int i = 0; i < QLoads<GQA>::NQ; ++i) ql.q[i] = qg[min(tid + NT * i, GQA * D - 1)];
}

// Workgroup-wide, from the loads above: q' = q R_K and the A-operand
// fragment block of the score product in frag_lds (layout of Rows).
template <int GQA, int NG, int BITS, bool F4>
__device__ __forceinline__ void build_q(const StepArgs &a, int tid, QWork<GQA, NG> &w, uint32_t *frag_lds, const QLoads<GQA> &ql) {
  using R = Rows<GQA, NG>;
  constexpr int G = R::G, SEG = QWork<GQA, NG>::SEG, NT = AW * 64;
  const int jr = tid >> 3, qq = tid & 7;
  const f32x4(&rk)[8] = ql.rk;
#pragma unroll
  for (int i = 0; i < QLoads<GQA>::NQ; ++i) {
    const int e = tid + NT * i;
    if (e < GQA * D) w.x[e / D][e % D] = bf16_to_f32(ql.q[i]);
  }
  __syncthreads();
  // rotations: thread (jr, qq) sums 16 inputs of rows jr and jr + 64, the
  // eight lanes of a row combine by DPP (the sum lands in lanes qq >= 4);
  // the largest |q'| is tracked on the way
  const bool wr = qq == 4;
  float amax = 0.f;
  {
    float a0[GQA], a1[GQA];
#pragma unroll
    for (int v = 0; v < GQA; ++v) {
      a0[v] = a1[v] = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 xi = *reinterpret_cast<const f32x4 *>(&w.x[v][32 * k + 4 * qq]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0[v] = fmaf(xi[e], rk[k][e], a0[v]);
          a1[v] = fmaf(xi[e], rk[4 + k][e], a1[v]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < GQA; ++v) {
      a0[v] = oct_sum(a0[v]);
      a1[v] = oct_sum(a1[v]);
      if (wr) {
        w.y[v][jr] = a0[v];
        w.y[v][jr + 64] = a1[v];
        amax = fmaxf(amax, fmaxf(fabsf(a0[v]), fabsf(a1[v])));
      }
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) w.red[tid >> 6] = amax;
  __syncthreads();
  // ---------------- the fragment block
  const float sc = a.sm_scale * LOG2E;
  float gmax = 0.f;
#pragma unroll
  for (int i = 0; i < AW; ++i) gmax = fmaxf(gmax, w.red[i]);
  gmax *= sc;
  float kq = 1.f;  // keeps |q' * 16 * kq| <= 2^14 (fp16 operands)
  if constexpr (!F4)
    while (gmax * 16.f * kq > 16384.f) kq *= 0.5f;
  // A operand values q' * w_c * kq as fp16 high part and low part x 2^11
  // (w_c, the weight that the K code expansion puts on channel c: INT2 4 or
  // 16, INT4 16 on every channel),
  // and their sums over each scale group by wave reductions: a wave covers
  // 64 consecutive channels of one head (uniform loop bounds)
  if constexpr (F4)  // the A operand and scale bytes are scattered into place below
    for (int i = tid; i < R::FR_Q * 64; i += NT) frag_lds[R::FR_A * 64 + i] = 0u;
  for (int e0 = 0; e0 < GQA * D; e0 += NT) {
    const int e = e0 + tid;
    const bool in = e < GQA * D;
    const int h = in ? e / D : 0, ch = e % D;
    float vh = 0.f, vl = 0.f, vq = 0.f;
    if (in) {
      const float y = w.y[h][ch] * sc;
      if constexpr (!F4) {
        const float x = y * ((BITS == 2 && (ch & 3) < 2) ? 4.f : 16.f) * kq;
        const _Float16 hi = _Float16(x), lo = _Float16((x - float(hi)) * 2048.f);
        w.qa[0][h][ch] = hi;
        w.qa[1][h][ch] = lo;
        vh = float(hi);
        vl = float(lo);
      }
      vq = y * kq;
    }
    if constexpr (!F4) {
      vh = seg_sum<SEG>(vh, tid & 63);
      vl = seg_sum<SEG>(vl, tid & 63);
    }
    vq = seg_sum<SEG>(vq, tid & 63);
    if (in && ch % SEG == 0) {
      w.gpart[0][h][ch / SEG] = vh;
      w.gpart[1][h][ch / SEG] = vl;
      w.gpart[2][h][ch / SEG] = vq;
    }
  }
  __syncthreads();
  auto gsum = [&](int which, int h, int g) {
    float sum = 0.f;
    for (int k = 0; k < G / SEG; ++k) sum += w.gpart[which][h][g * (G / SEG) + k];
    return sum;
  };
  if constexpr (F4) {
    // Thread (h, b, s) takes K = 32 b + s: the channel c whose code is
    // nibble s of fp4 lane group b, and the fp8 slot of that K.  A row's
    // E8M0 scale from lane group b applies to K block b (K = 32 b .. 32 b +
    // 31, read off the hardware), so each block of each row gets its own
    // exponent E (of its group's largest |y| in the block; the block's 32
    // K are 32 consecutive lanes here): its four fp8 part bytes and the
    // block's scales go straight into the fragment.
    uint8_t *fb = reinterpret_cast<uint8_t *>(frag_lds);
    for (int e = tid; e < GQA * D; e += NT) {
      const int h = e / D, K = e % D, b = K >> 5;
      const int c = f4_channel(b, K & 31), g = c / G;
      const float y = w.y[h][c] * sc;
      int E = 0;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const float mx = seg_max<32>(g == gg ? fabsf(y) : 0.f, tid & 63);
        const int Eg = int((__float_as_uint(mx) >> 23) & 255u) - 127;  // mx < 2^(Eg+1)
        if (gg == g) E = Eg;
        // pair P of chain ch: row 4 (P / 2) + part of product P % 2
        const int P = NG == 1 ? h % R::HC : 2 * (h % R::HC) + gg, ch = h / R::HC;
        if ((K & 31) == 0 && Eg > -90)
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
            fb[4 * ((R::FR_INIT + 4 * ch) * 64 + 16 * b + 4 * (P >> 1) + pp) + (P & 1)] = uint8_t(127 + Eg - 7 - 4 * pp);
      }
      if (E <= -90) continue;  // zero (or negligible) block: zero parts
      const uint32_t parts = fp8_parts(y, E);
      const int P = NG == 1 ? h % R::HC : 2 * (h % R::HC) + g, ch = h / R::HC;
      // fp8 slot of K: lane group gA, byte sA (K = 16 gA + sA, or 64 + 16 gA + sA - 16)
      const int gA = (K & 63) >> 4, sA = (K & 15) + (K >= 64 ? 16 : 0);
      const int dw = R::FR_A + 16 * ch + 8 * (P & 1) + (sA >> 2);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) fb[4 * (dw * 64 + 16 * gA + 4 * (P >> 1) + pp) + (sA & 3)] = uint8_t(parts >> (8 * pp));
    }
  }
  for (int idx = tid; idx < R::FR_DW * 64; idx += NT) {
    const int d = idx / 64, lane = idx % 64, r = lane & 15, qd = lane >> 4;
    uint32_t fw;
    if constexpr (F4) {
      // (product j of chain ch, row r = 4 qr + part): pair 2 qr + j
      const int qr = r >> 2, part = r & 3;
      if (d < R::FR_INIT) {
        continue;  // the A operand, scattered above
      } else if (d < R::FR_Q) {
        continue;  // the E8M0 scales, written above
      } else if (d < R::FR_INVKQ) {
        const int ch = (d - R::FR_Q) / 2, k = (d - R::FR_Q) % 2;
        const int h = R::HC * ch + R::pair_head(qd, k), g = R::pair_group(qd, k);
        fw = __float_as_uint(h < GQA ? gsum(2, h, g) : 0.f);
      } else {
        fw = __float_as_uint(1.f);
      }
      frag_lds[idx] = fw;
      continue;
    }
    if (d < R::FR_INIT) {
      // A operand: row r of chain ch, k-block kb, dword v (channels c0, c0+1)
      const int ch = d / 16, kb = (d % 16) / 4, v = d % 4;
      const int h = R::HC * ch + r / R::J, g = (r % R::J) / 2, part = r & 1;
      const int c0 = 32 * kb + 8 * qd + 2 * v;
      auto bits = [&](int cc) -> uint32_t {
        return (h < GQA && cc / G == g) ? uint32_t(__builtin_bit_cast(uint16_t, w.qa[part][h][cc])) : 0u;
      };
      fw = bits(c0) | (bits(c0 + 1) << 16);
    } else if (d < R::FR_Q) {
      // the expanded codes are 1 + c / w_c: each row starts at minus its sum
      const int ch = (d - R::FR_INIT) / 4, i = (d - R::FR_INIT) % 4;
      const int rr = 4 * qd + i;
      const int h = R::HC * ch + rr / R::J, g = (rr % R::J) / 2, part = rr & 1;
      fw = __float_as_uint(h < GQA ? -gsum(part, h, g) : 0.f);
    } else if (d < R::FR_INVKQ) {
      const int ch = (d - R::FR_Q) / 2, k = (d - R::FR_Q) % 2;
      const int h = R::HC * ch + R::pair_head(qd, k), g = R::pair_group(qd, k);
      fw = __float_as_uint(h < GQA ? gsum(2, h, g) : 0.f);
    } else {
      fw = __float_as_uint(1.f / kq);
    }
    frag_lds[idx] = fw;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ attend

// History pages reach LDS by direct buffer->LDS copies (buffer_load ... lds):
// several pages per wave in flight without holding registers.  One INT2
// page block is 1024 + 128 NG bytes: one 16-byte-per-lane copy of the first
// 1 KB, one of the rest on the first 8 NG lanes (INT4: two copies of 1 KB,
// then the rest).  The compiler does not order LDS reads after these copies,
// so the page loop waits for them itself (vmcnt counts per instruction;
// loads complete in issue order).
// Pages in flight per wave (the ring's depth): 4 INT2 pages; INT4 blocks
// are 1.7-1.9 times larger, and three of them hold more bytes than four INT2
// pages while two workgroups' rings still fit a CU's LDS.  (A ring of 8 INT2
// pages, every page of a batch-1 wave requested at once, measured slower:
// 18.5 against 17.3 us per layer at 32K.)  Up to 3 pages are loaded through
// registers before the q build, the rest by direct copies after it.
template <int BITS>
constexpr int depth_of() { return BITS == 2 ? 4 : 3; }

// Copies of one page block (wave-uniform address, `bytes` long) through a
// buffer resource built in scalar registers: each copy takes the lane's
// 32-bit offset, with no 64-bit address arithmetic per lane
__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t *p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a)), hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((uint64_t(hi) << 32) | lo), 0, bytes, 0x00020000);
}
__device__ inline void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, off, 0, 0, 0);
}

template <int N>
__device__ inline void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most `pages` page copies (IPP instructions each) are pending,
// with EXTRA younger loads issued after the last page copy
template <int IPP, int P, int EXTRA = 0>
__device__ inline void wait_pages(int pages) {
  static_assert(IPP * P + EXTRA <= 63, "vmcnt range");
  if constexpr (P == 0) {
    wait_vmem<EXTRA>();
  } else {
    if (pages >= P)
      wait_vmem<IPP * P + EXTRA>();
    else
      wait_pages<IPP, P - 1, EXTRA>(pages);
  }
}

// Orders this wave's LDS accesses around an exchange between its lanes: the
// LDS unit runs one wave's instructions in order, so keeping the compiler
// from moving loads and stores across this point is enough.
__device__ inline void lds_order() { asm volatile("" ::: "memory"); }

// LDS byte address of a pointer into __shared__ memory
__device__ inline uint32_t lds_addr(const void *p) {
  return uint32_t(uintptr_t((const __attribute__((address_space(3))) void *)p));
}

// One page's operands out of its ring slot.  Plain ds_read instructions in
// one asm block that also waits for them: loads the compiler sees would each
// get a wait for every LDS copy in flight, the prefetched pages included.
// kc/vc: K/V code dwords of the lane; km/vm: K/V meta of (token, pair 0/1).
template <int VCODE, int KMETA, int VMETA, int POFF, int SOFF = 0>
struct RingRead {
  u32x2 kc, vc;
  uint32_t km0, km1, vm0, vm1;
  template <int NG>
  __device__ void load(uint32_t a_code, uint32_t a_meta) {
    if constexpr (NG == 1) {
      asm volatile(
          "ds_read_b64 %0, %4 offset:%9\n\t"
          "ds_read_b64 %1, %4 offset:%6\n\t"
          "ds_read_b32 %2, %5 offset:%7\n\t"
          "ds_read_b32 %3, %5 offset:%8\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc), "=&v"(vc), "=&v"(km0), "=&v"(vm0)
          : "v"(a_code), "v"(a_meta), "n"(VCODE + SOFF), "n"(KMETA + SOFF), "n"(VMETA + SOFF), "n"(SOFF)
          : "memory");
      km1 = km0;
      vm1 = vm0;
    } else {
      asm volatile(
          "ds_read_b64 %0, %6 offset:%13\n\t"
          "ds_read_b64 %1, %6 offset:%8\n\t"
          "ds_read_b32 %2, %7 offset:%9\n\t"
          "ds_read_b32 %3, %7 offset:%10\n\t"
          "ds_read_b32 %4, %7 offset:%11\n\t"
          "ds_read_b32 %5, %7 offset:%12\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc), "=&v"(vc), "=&v"(km0), "=&v"(km1), "=&v"(vm0), "=&v"(vm1)
          : "v"(a_code), "v"(a_meta), "n"(VCODE + SOFF), "n"(KMETA + SOFF), "n"(KMETA + POFF + SOFF),
            "n"(VMETA + SOFF), "n"(VMETA + POFF + SOFF), "n"(SOFF)
          : "memory");
    }
  }
};

// The same for INT4 pages: 16 code bytes per lane and tensor.
template <int VCODE, int KMETA, int VMETA, int POFF, int SOFF = 0>
struct RingRead4 {
  u32x4 kc, vc;
  uint32_t km0, km1, vm0, vm1;
  template <int NG>
  __device__ void load(uint32_t a_code, uint32_t a_meta) {
    if constexpr (NG == 1) {
      asm volatile(
          "ds_read_b128 %0, %4 offset:%9\n\t"
          "ds_read_b128 %1, %4 offset:%6\n\t"
          "ds_read_b32 %2, %5 offset:%7\n\t"
          "ds_read_b32 %3, %5 offset:%8\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc), "=&v"(vc), "=&v"(km0), "=&v"(vm0)
          : "v"(a_code), "v"(a_meta), "n"(VCODE + SOFF), "n"(KMETA + SOFF), "n"(VMETA + SOFF), "n"(SOFF)
          : "memory");
      km1 = km0;
      vm1 = vm0;
    } else {
      asm volatile(
          "ds_read_b128 %0, %6 offset:%13\n\t"
          "ds_read_b128 %1, %6 offset:%8\n\t"
          "ds_read_b32 %2, %7 offset:%9\n\t"
          "ds_read_b32 %3, %7 offset:%10\n\t"
          "ds_read_b32 %4, %7 offset:%11\n\t"
          "ds_read_b32 %5, %7 offset:%12\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc), "=&v"(vc), "=&v"(km0), "=&v"(km1), "=&v"(vm0), "=&v"(vm1)
          : "v"(a_code), "v"(a_meta), "n"(VCODE + SOFF), "n"(KMETA + SOFF), "n"(KMETA + POFF + SOFF),
            "n"(VMETA + SOFF), "n"(VMETA + POFF + SOFF), "n"(SOFF)
          : "memory");
    }
  }
};

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ inline h2v as_h2(uint32_t w) { return __builtin_bit_cast(h2v, w); }

// x[ch][sl] of lane src (a byte address, 4 * lane) where (ch, sl) is this
// lane's (chain, slot) pair; ds_bpermute moves registers between lanes
// without touching memory.
template <int NCH, int SPL>
__device__ inline float gather(const float (&x)[NCH][SPL], int src, int my_ch, int my_sl) {
  float v = 0.f;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int sl = 0; sl < SPL; ++sl) {
      const float y = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x[ch][sl])));
      if constexpr (NCH * SPL == 1)
        v = y;
      else
        v = (ch == my_ch && sl == my_sl) ? y : v;
    }
  return v;
}

// x[ch] of lane src (a byte address, 4 * lane), ch being this lane's chain.
template <int NCH>
__device__ inline uint32_t gather_u32(const uint32_t (&x)[NCH], int src, int my_ch) {
  uint32_t v = 0;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const uint32_t y = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(x[ch])));
    v = (NCH == 1 || ch == my_ch) ? y : v;
  }
  return v;
}

// Halves of two dwords: (lo(a), lo(b)) or (hi(a), hi(b)) as one dword
constexpr uint32_t PERM_LO = 0x05040100u, PERM_HI = 0x07060302u;
__device__ inline uint32_t halves(uint32_t a, uint32_t b, uint32_t sel) { return __builtin_amdgcn_perm(b, a, sel); }

// One wave over its history pages j = j0 + wave + AW*i, i < npw.
//
// Scores: D[r][t] = init_r + sum_c A[r][c] (1 + code_tc / w_c) over the four
// 32-channel blocks (A: the q fragment, rows as in Rows; B: the exactly
// expanded K codes, token t = column).  Lane (t, qd) turns its four rows into
// score(h, t) = sum_g s_tg (D_hi + 2^-11 D_lo) + z_tg kq sum_{c in g} q'_c,
// in kq units, and keeps m, l and the z sums of its head(s) for token t.
// Probabilities leave the lane as pw = p w_t 2^kpv (w_t = 4 for tokens
// 4q, 4q+1 and 16 for 4q+2, 4q+3, the weights of the V code expansion;
// 2^kpv keeps the fp16 operand in range), folded into the exponent.
// PV: lane (n, tq) takes pw of head n for tokens 4tq..4tq+3 from LDS and
// forms B_g = fp16(pw s_tg) for each scale group g; acc[r] += Vexp_r B_g(r)
// with Vexp = 1 + code/w_t, and cacc[g] += 1 B_g, whose rows all equal the
// column sums of B_g: acc - cacc is then exactly sum_t B code / w_t.
// LATE (N_LATE > 0): late() issues N_LATE loads into registers once the
// wave has issued its last page copy (the fast page path); the waits of the
// remaining pages count them.  Returns whether late() was called.
template <int GQA, int NG, int BITS, int DP, bool F4, int N_LATE, int RP, class Prep, class Late>
__device__ bool history_wave(const StepArgs &a, int b, int hk, int nh, int j0, int j1, int wave, int lane,
                             int pid_pre, Prep &&prep, Late &&late, const uint32_t *frag_lds, uint8_t *ring,
                             float *zs, float *o_lds, float *m_lds, float *l_lds) {
  bool late_done = false;
  using R = Rows<GQA, NG>;
  constexpr int NCH = R::NCH, SPL = R::SPL, G = R::G, HC = R::HC;
  constexpr int SB = hist_block_bytes(G, BITS);
  constexpr int kmeta = k_meta_off(G, BITS), vcode = v_codes_off(G, BITS), vmeta = v_meta_off(G, BITS);
  // a block is HB = 2 code areas' worth of bytes (1 or 2 KB) copied 1 KB
  // per instruction, then 128 NG bytes of tail: IPP copy instructions per page
  constexpr int HB = 2 * code_area_bytes(BITS), NHB = HB / 1024, IPP = NHB + 1;
  constexpr int RPB = DP - 1 < RP ? DP - 1 : RP;  // pages loaded through registers
  const oscar_layer_cache &c = a.c;
  const int t = lane & 15, qd = lane >> 4;  // score side: token, lane group
  const int hp = t % GQA;                   // PV side: head of column n = l%16 (tq = qd)
  // PV side: lanes and registers holding head hp's scores for tokens 4qd + i
  const int src_ch = R::head_chain(hp), src_sl = R::head_slot(hp);
  const int src0 = 4 * (16 * R::head_qd(hp) + 4 * qd);
  const int npw = j1 > j0 + wave ? (j1 - j0 - wave + AW - 1) / AW : 0;

  // the q fragment (filled from LDS once the first page copies are issued)
  f16x8 aq[NCH][4];
  f32x4 dinit[NCH];
  float qz[NCH][2];
  float inv_kq = 1.f, kq = 1.f;
  const bool w16 = BITS == 4 || (t & 3) >= 2;
  const float lw_t = w16 ? a.pk23 : a.pk01;  // log2(w_t 2^kpv)
  const float inv_w = w16 ? 0.0625f : 0.25f;
  // K/V meta dword of (token t, group of pair 0); pair 1 sits 16 dwords on
  // (next group), or on the same dword when NG = 1
  const int moff = 4 * (16 * R::pair_group(qd, 0) + t);
  constexpr int POFF = NG == 1 ? 0 : 64;
  Expander ex;
  ex.m4 = a.ex_m4;
  ex.m16 = a.ex_m16;
  ex.e = a.ex_e;
  // keep the exponent pattern in a VGPR (the mask stays in an SGPR): then one
  // v_and_or_b32 per expanded register.  The empty asm emits no instruction.
  asm volatile("" : "+v"(ex.e));
  Expander4 ex4;
  ex4.m = a.ex_mn;
  ex4.e = ex.e;
  const f16x4 ones = as_f16x4(0x3C003C00u, 0x3C003C00u);

  bool started = false;  // wave-uniform: a max has been set
  float m_run[NCH][SPL], thr[NCH][SPL], cl[NCH][SPL], lw[NCH][SPL], zw[NCH][2];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int sl = 0; sl < SPL; ++sl) {
      m_run[ch][sl] = -INFINITY;
      thr[ch][sl] = -INFINITY;
      cl[ch][sl] = 0.f;
      lw[ch][sl] = 0.f;
    }
    zw[ch][0] = zw[ch][1] = 0.f;
  }
  f32x4 acc[8], cacc[NG];  // zeroed once the prologue is done (register pressure)

  // page ids of pages 64k + lane, loaded per chunk of 64 (the first chunk by
  // the caller; lanes past the wave's pages hold ids that are never used)
  const int32_t *pt = c.hist_pt + int64_t(b) * c.hist_pt_stride + j0 + wave;
  int my_pid = -1;

  // copy page i into ring slot sl; a bad page id copies page 0 instead (the
  // page is skipped), so every page costs the same two copy instructions
  uint32_t ok_slots = 0;
  const uint32_t lane16 = 16u * uint32_t(lane);
  constexpr int N2 = (SB - HB) / 16;  // lanes of the tail copy
  static_assert((N2 & (N2 - 1)) == 0 && N2 <= 64, "second copy part: a power of two of lanes");
  auto page_block = [&](int i, int sl) {
    if ((i & 63) == 0 && i > 0) {
      my_pid = (i + lane < npw) ? pt[int64_t(AW) * (i + lane)] : -1;
      // take the wait for this load here, once per 64 pages: otherwise the
      // compiler cannot tell on later pages that it has landed and waits for
      // every copy in flight before each readlane
      asm volatile("" : "+v"(my_pid));
    }
    int pid = __builtin_amdgcn_readlane(my_pid, i & 63);
    const bool ok = pid >= 0 && pid < c.n_hist_pages;
    pid = ok ? pid : 0;
    ok_slots = ok ? (ok_slots | (1u << sl)) : (ok_slots & ~(1u << sl));
    return c.hist + (int64_t(pid) * c.n_kv_heads + hk) * SB;
  };
  auto issue = [&](int i, int sl) {
    const auto rs = block_rsrc(page_block(i, sl), SB);
    uint8_t *dst = ring + sl * SB;
#pragma unroll
    for (int k = 0; k < NHB; ++k) lds_copy16(rs, 1024u * k + lane16, dst + 1024 * k);
    if (lane < N2) lds_copy16(rs, uint32_t(HB) + lane16, dst + HB);
  };
  // the first DEPTH - 1 pages go through registers: no copy into LDS is in
  // flight while the workgroup builds the q fragment (the compiler would
  // wait for every such copy before the build's first LDS access).  A page
  // is 16 bytes per lane, then its last SB - 1024 bytes as one or two dwords
  // per lane.  Both loads are issued in every lane and on every path (lanes
  // past the tail re-read it; with no pages the rotation forms stand in), so
  // the compiler's waits count them exactly.
  typedef typename std::conditional<(SB - HB > 256), u32x2, uint32_t>::type Tail;
  constexpr int TB = sizeof(Tail), NT2 = (SB - HB) / TB;  // tail lanes
  static_assert((NT2 & (NT2 - 1)) == 0 && NT2 <= 64, "tail: a power of two of lanes");
  typedef const __attribute__((address_space(1))) u32x4 *gp4;
  typedef const __attribute__((address_space(1))) Tail *gpt;
  u32x4 preg[RPB][NHB];
  Tail ptail[RPB];
  auto issue_reg = [&](int i, bool on) {
    const uint8_t *blk = on ? page_block(i, i) : a.fk;
#pragma unroll
    for (int k = 0; k < NHB; ++k) preg[i][k] = *(gp4)(blk + 1024u * k + lane16);
    ptail[i] = *(gpt)(blk + uint32_t(HB) + TB * uint32_t(lane & (NT2 - 1)));
  };

  // one page from the ring; PARTIAL: rows >= nvalid are absent (any bits)
  // soff_tag: a ring slot's byte offset known at compile time (the unrolled
  // loop: immediate offsets of the ring reads), else 0 with src at the slot
  auto page = [&](const uint8_t *src, int nvalid, auto partial_tag, auto soff_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    constexpr int SOFF = decltype(soff_tag)::value;
    const uint32_t base = lds_addr(src);
    typedef typename std::conditional<BITS == 2, RingRead<vcode, kmeta, vmeta, POFF, SOFF>,
                                      RingRead4<vcode, kmeta, vmeta, POFF, SOFF>>::type Rd;
    Rd rd;
    rd.template load<NG>(base + (BITS == 2 ? 8 : 16) * lane, base + moff);
    const auto kc = rd.kc, vc = rd.vc;
    const h2v km0 = as_h2(rd.km0), km1 = as_h2(rd.km1);
    const h2v vm0 = as_h2(rd.vm0), vm1 = as_h2(rd.vm1);
    const bool tok_ok = !PARTIAL || t < nvalid;
    // ---- scores (kq units)
    f16x8 kx[4];
    i32x8 k4;  // F4: the codes as fp4 c/2, nibbles of the spread dwords
    if constexpr (F4) {
      const uint32_t M = 0x33333333u;
      k4 = i32x8{int(kc[0] & M), int((kc[0] >> 2) & M), int(kc[1] & M), int((kc[1] >> 2) & M), 0, 0, 0, 0};
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if constexpr (BITS == 2)
          kx[kb] = ex.k(kc[0], kc[1], kb);
        else
          kx[kb] = ex4.k(kc[kb]);
      }
    }
    float S[NCH][SPL];
    bool up = false;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      float d0, d1;
      if constexpr (F4) {
        // the four parts of the lane's pairs (2qd, 2qd + 1), each product's
        // rows scaled by their own power of two (byte j of the chain's scale
        // dword); the fp4 operand scaled by 2 (c/2 -> c)
        const int scl = int(__float_as_uint(dinit[ch][0]));
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        const f32x4 e0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            f4_operand(aq[ch][0], aq[ch][1]), k4, z4, 0, 4, 0, scl, 0, 128);
        const f32x4 e1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            f4_operand(aq[ch][2], aq[ch][3]), k4, z4, 0, 4, 1, scl, 0, 128);
        d0 = (e0[0] + e0[1]) + (e0[2] + e0[3]);
        d1 = (e1[0] + e1[1]) + (e1[2] + e1[3]);
      } else {
        f32x4 d = dinit[ch];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) d = mfma_k(aq[ch][kb], kx[kb], d);
        // s_g (d_hi + 2^-11 d_lo) + z_g qz_g per pair, as mixed-precision
        // FMAs on the packed meta (fp16 operands taken as they are)
        d0 = fmaf(d[1], 0x1p-11f, d[0]);
        d1 = fmaf(d[3], 0x1p-11f, d[2]);
      }
      if constexpr (NG == 1) {
        S[ch][0] = fmaf(float(km0.x), d0, fmaf(float(km0.y), qz[ch][0], 0.f));
        S[ch][1] = fmaf(float(km1.x), d1, fmaf(float(km1.y), qz[ch][1], 0.f));
      } else {
        const float z = fmaf(float(km1.y), qz[ch][1], fmaf(float(km0.y), qz[ch][0], 0.f));
        float sv = fmaf(float(km1.x), d1, fmaf(float(km0.x), d0, z));
        if constexpr (NG == 4) sv += __shfl_xor(sv, 16);
        S[ch][0] = sv;
      }
#pragma unroll
      for (int sl = 0; sl < SPL; ++sl) {
        if constexpr (PARTIAL) S[ch][sl] = tok_ok ? S[ch][sl] : -INFINITY;
        up |= S[ch][sl] > thr[ch][sl];
      }
    }
    // ---- online softmax: the running max moves only when a score passes it
    // by more than LAZY_TH (log2 units); then every lane of the head's row
    // takes the row max
    if (__any(up)) {
      // the first rescale only sets the max: nothing has been accumulated
      const bool scale = started;
      started = true;
      float alpha[NCH][SPL];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int sl = 0; sl < SPL; ++sl) {
          float mx = fmaxf(S[ch][sl] * inv_kq, m_run[ch][sl]);
          mx = fmaxf(mx, row_ror<8>(mx));
          mx = fmaxf(mx, row_ror<4>(mx));
          mx = fmaxf(mx, row_ror<2>(mx));
          mx = fmaxf(mx, row_ror<1>(mx));
          const float al = m_run[ch][sl] == -INFINITY ? 0.f : fast_exp2(m_run[ch][sl] - mx);
          alpha[ch][sl] = al;
          m_run[ch][sl] = mx;
          thr[ch][sl] = (mx + LAZY_TH) * kq;
          cl[ch][sl] = lw_t - mx;
          if (scale) {
            lw[ch][sl] *= al;
#pragma unroll
            for (int k = 0; k < 2; ++k)
              if (R::pair_slot(k) == sl) zw[ch][k] *= al;
          }
        }
      if (scale) {
        const float al = gather(alpha, src0, src_ch, src_sl);
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] *= al;
#pragma unroll
        for (int g = 0; g < NG; ++g) cacc[g] *= al;
      }
    }
    float pw[NCH][SPL];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
      for (int sl = 0; sl < SPL; ++sl) {
        pw[ch][sl] = fast_exp2(fmaf(S[ch][sl], inv_kq, cl[ch][sl]));
        lw[ch][sl] += pw[ch][sl];
      }
      float z0 = float(vm0.y), z1 = float(vm1.y);
      if constexpr (PARTIAL) {
        z0 = tok_ok ? z0 : 0.f;
        z1 = tok_ok ? z1 : 0.f;
      }
      zw[ch][0] = fmaf(pw[ch][R::pair_slot(0)], z0, zw[ch][0]);
      zw[ch][1] = fmaf(pw[ch][R::pair_slot(1)], z1, zw[ch][1]);
    }
    // ---- PV operands, formed where the probabilities are: fp16(pw s_tg) of
    // the lane's two scale groups (NG >= 2: pair 0, pair 1) or of its two
    // heads (NG = 1) in one dword
    uint32_t ps[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      // each half one mixed-precision FMA (fp16 scale in, fp16 product out)
      _Float16 x0, x1;
      if constexpr (NG == 1) {
        x0 = _Float16(fmaf(pw[ch][0], float(vm0.x), 0.f));
        x1 = _Float16(fmaf(pw[ch][1], float(vm0.x), 0.f));
      } else {
        x0 = _Float16(fmaf(pw[ch][0], float(vm0.x), 0.f));
        x1 = _Float16(fmaf(pw[ch][0], float(vm1.x), 0.f));
      }
      if constexpr (PARTIAL) {  // absent rows: their meta may be anything
        x0 = tok_ok ? x0 : _Float16(0.f);
        x1 = tok_ok ? x1 : _Float16(0.f);
      }
      const h2v hv = {x0, x1};
      ps[ch] = __builtin_bit_cast(uint32_t, hv);
    }
    // lane (n, tq) = head hp, tokens 4tq..4tq+3: B_g from the dwords of its
    // head's lanes (NG = 4: groups 0, 1 in the first lane group, 2, 3 in the
    // next)
    f16x4 bp[NG];
    {
      constexpr int ND = NG == 4 ? 8 : 4;
      uint32_t dw[ND];
#pragma unroll
      for (int i = 0; i < ND; ++i) dw[i] = gather_u32<NCH>(ps, src0 + 4 * (i & 3) + 64 * (i >> 2), src_ch);
      if constexpr (NG == 1) {
        const uint32_t sel = src_sl ? PERM_HI : PERM_LO;
        bp[0] = __builtin_bit_cast(f16x4, u32x2{halves(dw[0], dw[1], sel), halves(dw[2], dw[3], sel)});
      } else {
#pragma unroll
        for (int gp = 0; gp < NG / 2; ++gp) {
          const uint32_t *d = dw + 4 * gp;
          bp[2 * gp] = __builtin_bit_cast(f16x4, u32x2{halves(d[0], d[1], PERM_LO), halves(d[2], d[3], PERM_LO)});
          bp[2 * gp + 1] = __builtin_bit_cast(f16x4, u32x2{halves(d[0], d[1], PERM_HI), halves(d[2], d[3], PERM_HI)});
        }
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) cacc[g] = mfma_v(ones, bp[g], cacc[g]);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (BITS == 2)
        acc[r] = mfma_v(ex.v(vc[0], vc[1], r), bp[(16 * r) / G], acc[r]);
      else
        acc[r] = mfma_v(ex4.v(vc[r >> 1], r & 1), bp[(16 * r) / G], acc[r]);
    }
  };

  auto step = [&](int i, auto partial_tag) {
    if (i + DP - 1 < npw) issue(i + DP - 1, (i + DP - 1) % DP);
    wait_pages<IPP, DP - 1>(min(DP - 1, npw - 1 - i));
    const int sl = i % DP;
    // tested as a per-lane value (the same in every lane): as a scalar branch
    // the compiler copies the accumulators at its merge point every page
    uint32_t okv = ok_slots;
    asm volatile("" : "+v"(okv));
    if (!((okv >> sl) & 1u)) {
      if (lane == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    } else {
      page(ring + sl * SB, nh - PAGE * (j0 + wave + AW * i), partial_tag, std::integral_constant<int, 0>{});
    }
  };

  // the common case: every page id of the wave in its first chunk and in
  // range (checked once), so no per-page checks or bookkeeping
  auto issue_fast = [&](int i, int sl) {
    const int pid = __builtin_amdgcn_readlane(my_pid, i);
    const auto rs = block_rsrc(c.hist + (int64_t(pid) * c.n_kv_heads + hk) * SB, SB);
    uint8_t *dst = ring + sl * SB;
#pragma unroll
    for (int k = 0; k < NHB; ++k) lds_copy16(rs, 1024u * k + lane16, dst + 1024 * k);
    if (lane < N2) lds_copy16(rs, uint32_t(HB) + lane16, dst + HB);
  };
  auto step_fast = [&](int i, auto partial_tag) {
    if (i + DP - 1 < npw) issue_fast(i + DP - 1, (i + DP - 1) % DP);
    wait_pages<IPP, DP - 1>(min(DP - 1, npw - 1 - i));
    page(ring + (i % DP) * SB, nh - PAGE * (j0 + wave + AW * i), partial_tag, std::integral_constant<int, 0>{});
  };
  // page i known to sit in ring slot S (i % DP == S)
  auto step_slot = [&](int i, auto slot_tag) {
    constexpr int S = decltype(slot_tag)::value;
    if (i + DP - 1 < npw) issue_fast(i + DP - 1, (S + DP - 1) % DP);
    wait_pages<IPP, DP - 1>(min(DP - 1, npw - 1 - i));
    page(ring, nh - PAGE * (j0 + wave + AW * i), std::false_type{}, std::integral_constant<int, S * SB>{});
  };

  // the page ids (loaded by the caller, with the loads of the q fragment
  // build), then the first pages; the build (workgroup-wide: the q fragment
  // into frag_lds, and the append) runs while the pages fly
  const bool any_pages = npw > 0 && c.n_hist_pages >= 1;
  my_pid = pid_pre;
  asm volatile("" : "+v"(my_pid));
#pragma unroll
  for (int i = 0; i < RPB; ++i) issue_reg(i, any_pages);
  prep();
  // stored on every path, used or not: a load still in flight into a
  // register at the loop entry would make the compiler wait for every load
  // in flight (the prefetched pages) wherever the loop reuses that register
#pragma unroll
  for (int i = 0; i < RPB; ++i) {
#pragma unroll
    for (int k = 0; k < NHB; ++k) *reinterpret_cast<u32x4 *>(ring + i * SB + 1024u * k + lane16) = preg[i][k];
    if (lane < NT2) *reinterpret_cast<Tail *>(ring + i * SB + uint32_t(HB) + TB * lane) = ptail[i];
  }
  // the rest of the ring fills by direct copies from here
  if (any_pages)
    for (int i = RPB; i < DP - 1 && i < npw; ++i) issue(i, i);
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < NG; ++g) cacc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t *f = frag_lds + (R::FR_A + 16 * ch + 4 * kb) * 64 + lane;
      aq[ch][kb] = as_f16x8(f[0], f[64], f[128], f[192]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dinit[ch][i] = __uint_as_float(frag_lds[(R::FR_INIT + 4 * ch + i) * 64 + lane]);
    qz[ch][0] = __uint_as_float(frag_lds[(R::FR_Q + 2 * ch) * 64 + lane]);
    qz[ch][1] = __uint_as_float(frag_lds[(R::FR_Q + 2 * ch + 1) * 64 + lane]);
  }
  inv_kq = __uint_as_float(frag_lds[R::FR_INVKQ * 64 + lane]);
  kq = 1.f / inv_kq;

  if (npw > 0 && !any_pages) {
    if (lane == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
  } else if (npw > 0) {
    // only the last history page of the request can be partial; it is the
    // last page of whichever wave holds it
    const bool last_partial = (nh % PAGE) != 0 && j0 + wave + AW * (npw - 1) == (nh - 1) / PAGE;
    const int nfull = npw - (last_partial ? 1 : 0);
    const bool fast = npw <= 64 && __ballot(lane < npw && !(my_pid >= 0 && my_pid < c.n_hist_pages)) == 0;
    if (fast) {
      // the fp4-score instances with 8 or more score rows per lane group:
      // DP pages per trip, each ring slot's reads at immediate offsets
      // (smaller instances would spill)
      constexpr bool UNR = F4 && GQA * NG >= 8;
      static_assert(DP == 3 || DP == 4, "ring depth");
      int i = 0;
      if constexpr (UNR) {
        for (; i + DP <= nfull; i += DP) {
          step_slot(i, std::integral_constant<int, 0>{});
          step_slot(i + 1, std::integral_constant<int, 1>{});
          step_slot(i + 2, std::integral_constant<int, 2>{});
          if constexpr (DP == 4) step_slot(i + 3, std::integral_constant<int, 3>{});
        }
      }
      if constexpr (N_LATE > 0) {
        // the late loads go out once the wave has issued its last page copy
        // and finished the unrolled trips (stopping the trips earlier, so
        // that the loads fly during more pages, measured 1 % slower at
        // batch 1); the waits of the pages left count them
        const int i0 = max(0, npw - DP + 1);
        for (; i < i0; ++i) step_fast(i, std::false_type{});
        late();
        late_done = true;
        auto step_late = [&](int ii, auto partial_tag) {
          wait_pages<IPP, DP - 1, N_LATE>(min(DP - 1, npw - 1 - ii));
          page(ring + (ii % DP) * SB, nh - PAGE * (j0 + wave + AW * ii), partial_tag, std::integral_constant<int, 0>{});
        };
        for (; i < nfull; ++i) step_late(i, std::false_type{});
        if (last_partial) step_late(npw - 1, std::true_type{});
      } else {
        for (; i < nfull; ++i) step_fast(i, std::false_type{});
        if (last_partial) step_fast(npw - 1, std::true_type{});
      }
    } else {
      for (int i = 0; i < nfull; ++i) step(i, std::false_type{});
      if (last_partial) step(npw - 1, std::true_type{});
    }
  }

  // ---- this wave's o[h][c], m[h], l[h] into LDS
  float zsum[NCH][2];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int sl = 0; sl < SPL; ++sl) {
      float l = lw[ch][sl] * inv_w;
      l += row_ror<8>(l);
      l += row_ror<4>(l);
      l += row_ror<2>(l);
      l += row_ror<1>(l);
      const int h = HC * ch + R::slot_head(qd, sl);
      if (t == 0 && h < GQA && ((NG != 4) || (qd & 1) == 0)) {
        m_lds[h] = m_run[ch][sl];
        l_lds[h] = l * a.pv_unscale;
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float z = zw[ch][k] * inv_w;
      z += row_ror<8>(z);
      z += row_ror<4>(z);
      z += row_ror<2>(z);
      z += row_ror<1>(z);
      zsum[ch][k] = z;
    }
  }
  lds_order();
  // z sums per (head, group) through LDS
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int h = HC * ch + R::pair_head(qd, k), g = R::pair_group(qd, k);
      if (t == 0 && h < GQA) zs[h * NG + g] = zsum[ch][k];
    }
  lds_order();
  if (t < GQA) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int g = (16 * r) / G;
      const float zg = zs[t * NG + g];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o_lds[t * D + 16 * r + 4 * qd + i] = (acc[r][i] - cacc[g][i] + zg) * a.pv_unscale;
    }
  }
  return late_done;
}

// R_V rows of a workgroup thread for the way back to the plain basis: rows
// cr + 64 m (m < 2), inputs 32 k + 4 qq .. + 3 (cr = tid / 8, qq = tid % 8);
// eight lanes per row read 128 contiguous bytes.
struct RvRows {
  static constexpr int N_LOADS = 8;  // load instructions of load()
  f32x4 r[8];
  __device__ void load(const uint8_t *fv, int tid) {
    const float *Rc = reinterpret_cast<const float *>(fv + FORM_R) + (tid >> 3) * D + 4 * (tid & 7);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int k = 0; k < 4; ++k) r[4 * m + k] = *reinterpret_cast<const f32x4 *>(Rc + m * 64 * D + 32 * k);
  }
};
static_assert(AW * 64 == 512, "R_V rows: 128 rows x 8 lanes over the workgroup");

// History workgroups: combines the per-wave states like combine_waves and
// brings the partial back to the plain basis before it is stored,
// o_plain[h][c] = sum_i o_rot[h][i] R_V[c][i] (linear, so the merge's
// weighted sum may follow), through rot[GQA][D] in LDS.  Agent-scope stores.
template <int GQA>
__device__ void combine_rotate(const float *o_lds, const float *m_lds, const float *l_lds, float *part0,
                               int64_t head_stride, int tid, int o_wave_stride, const RvRows &rv,
                               float (*rot)[D]) {
  for (int idx = tid; idx < GQA * D; idx += AW * 64) {
    const int h = idx / D, c = idx % D;
    float mst = -INFINITY;
    for (int w = 0; w < AW; ++w) mst = fmaxf(mst, m_lds[w * GQA + h]);
    float o = 0.f, l = 0.f;
    for (int w = 0; w < AW; ++w) {
      const float mw = m_lds[w * GQA + h];
      const float e = (mw == -INFINITY) ? 0.f : fast_exp2(mw - mst);
      o = fmaf(e, o_lds[w * o_wave_stride + h * D + c], o);
      l = fmaf(e, l_lds[w * GQA + h], l);
    }
    rot[h][c] = o;
    if (c == 0) {
      store_agent(part0 + h * head_stride + D, mst);
      store_agent(part0 + h * head_stride + D + 1, l);
    }
  }
  __syncthreads();
  // the eight lanes of a row combine by DPP (the sum lands in lanes qq >= 4)
  const int cr = tid >> 3, qq = tid & 7;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int cc = cr + 64 * m;
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 r = *reinterpret_cast<const f32x4 *>(&rot[hh][32 * k + 4 * qq]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(r[e], rv.r[4 * m + k][e], acc);
      }
      acc = oct_sum(acc);
      if (qq == 4) store_agent(part0 + hh * head_stride + cc, acc);
    }
  }
}

// Merge of one (request, KV head) inside the attend kernel (the partials
// are all in the plain basis: the history workgroups rotated theirs back).
template <int GQA>
__device__ void merge_unit(const StepArgs &a, int b, int hk, int used, int tid, MergeWork<GQA> &mw) {
  const int64_t head_stride = int64_t(a.part_slots) * PART_STRIDE;
  const float *parts0 = a.parts + (int64_t(b) * a.n_q_heads + hk * GQA) * head_stride;
  merge_partials<GQA, AW * 64>(parts0, head_stride, used, a.out + (int64_t(b) * a.n_q_heads + hk * GQA) * D, tid,
                               mw);
}

// Separate merge kernel (large batches, where the attend workgroups run in
// several rounds and the in-kernel election costs more than a launch): one
// block per (request, KV head) LSE-combines the `used` partials of each
// query head of the group, rotates the history part back with R_V^T, adds
// the raw part (split 0) and normalises.  Built for latency: thread (h, c)
// issues the loads of all its partial values, the (m, l) pairs and its slice
// of R_V at once, so the kernel waits on memory about once.
template <int GQA>
constexpr int merge_threads() { return D * (GQA < 2 ? 2 : GQA); }

template <int GQA, bool PH>
__global__ void __launch_bounds__(merge_threads<GQA>()) merge_kernel(StepArgs a) {
  constexpr int NT = merge_threads<GQA>(), MCH = merge_ch<GQA>();
  const int hk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int h = tid / D, c = tid % D;  // (query head of the group, channel); h may be >= GQA
  const int L = a.k_new ? a.len_before[b] + 1 : a.seq_lens[b];
  if (!valid_len(L, a.max_seq_len)) return;  // output zeroed by the attend kernel
  const int used = 1 + (n_hist_pages(L) + a.pages_per_split - 1) / a.pages_per_split;
  const int64_t head_stride = int64_t(a.part_slots) * PART_STRIDE;
  const float *parts0 = a.parts + (int64_t(b) * a.n_q_heads + hk * GQA) * head_stride;
  __shared__ float w_lds[GQA][MAX_SPLITS + 1];  // m, then the weight of each split
  __shared__ float l_lds[GQA][MAX_SPLITS + 1];
  __shared__ float lsum[GQA];
  __shared__ __attribute__((aligned(16))) float rot[GQA][D];
  __shared__ float back[GQA][D];

  // ---- loads, all issued before any use
  // R_V rows cr + 64 m (m < NR), inputs 16 k + 2 qq .. ; eight lanes per row
  // read 128 contiguous bytes
  constexpr int NR = 1024 / NT;  // rows per thread: 128 rows x 8 lanes over NT threads
  const int cr = tid >> 3, qq = tid & 7;
  const float *Rc = reinterpret_cast<const float *>(forms_v<PH>(a, hk) + FORM_R) + cr * D + 4 * qq;
  f32x4 rv[4 * NR];
#pragma unroll
  for (int m = 0; m < NR; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      rv[4 * m + k] = *reinterpret_cast<const f32x4 *>(Rc + m * (NT / 8) * D + 32 * k);
  const bool own = h < GQA;
  const float *ph = parts0 + (own ? h : 0) * head_stride + c;
  float ov[MCH];
#pragma unroll
  for (int j = 0; j < MCH; ++j) ov[j] = (own && 1 + j < used) ? ph[(1 + j) * PART_STRIDE] : 0.f;
  const float o_raw = own ? ph[0] : 0.f;
  for (int e = tid; e < GQA * used; e += NT) {
    const int hh = e / used, sp = e % used;
    const float *pm = parts0 + hh * head_stride + sp * PART_STRIDE + D;
    w_lds[hh][sp] = pm[0];
    l_lds[hh][sp] = pm[1];
  }
  __syncthreads();
  // ---- per head: max over splits, split weights, total l (wave hh; DPP
  // reductions)
  {
    const int wave = wave_id(), lane = tid & 63;
    for (int hh = wave; hh < GQA; hh += NT / 64) {
      float m = -INFINITY;
      for (int sp = lane; sp < used; sp += 64) m = fmaxf(m, w_lds[hh][sp]);
      m = wave_max(m);
      float l = 0.f;
      for (int sp = lane; sp < used; sp += 64) {
        const float ms = w_lds[hh][sp];
        const float w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - m);
        w_lds[hh][sp] = w;
        l = fmaf(w, l_lds[hh][sp], l);
      }
      l = wave_sum(l);
      if (lane == 0) lsum[hh] = l;
    }
  }
  __syncthreads();
  // ---- history part of head h, channel c (rotated basis)
  float raw = 0.f;
  if (own) {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int j = 0; j < MCH; ++j) {
      const float w = (1 + j < used) ? w_lds[h][1 + j] : 0.f;
      if (j & 1)
        acc1 = fmaf(w, ov[j], acc1);
      else
        acc0 = fmaf(w, ov[j], acc0);
    }
    for (int s0 = 1 + MCH; s0 < used; s0 += MCH) {
      float o2[MCH];
#pragma unroll
      for (int j = 0; j < MCH; ++j) o2[j] = (s0 + j < used) ? ph[(s0 + j) * PART_STRIDE] : 0.f;
#pragma unroll
      for (int j = 0; j < MCH; ++j) {
        const float w = (s0 + j < used) ? w_lds[h][s0 + j] : 0.f;
        acc0 = fmaf(w, o2[j], acc0);
      }
    }
    rot[h][c] = acc0 + acc1;
    raw = w_lds[h][0] * o_raw;
  }
  __syncthreads();
  // ---- (rot R_V^T)[hh][c] = sum_i rot[hh][i] R_V[c][i]: the eight lanes of
  // a row combine by DPP (the sum lands in lanes qq >= 4)
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int cc = cr + m * (NT / 8);
    float acc[GQA];
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      acc[hh] = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 r = *reinterpret_cast<const f32x4 *>(&rot[hh][32 * k + 4 * qq]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[hh] = fmaf(r[e], rv[4 * m + k][e], acc[hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      acc[hh] = oct_sum(acc[hh]);
      if (qq == 4) back[hh][cc] = acc[hh];
    }
  }
  __syncthreads();
  if (own) a.out[(int64_t(b) * a.n_q_heads + hk * GQA + h) * D + c] = (raw + back[h][c]) / lsum[h];
}

// Waves per SIMD the register budget is set for: 4 (two workgroups per CU,
// at most 128 registers) where the page loop fits, else whatever it needs;
// the one-round plan runs one workgroup per CU (two waves per SIMD), and
// its waves hold the R_V rows through their last pages.
template <int GQA, int NG, bool FUSED>
constexpr int attend_waves() { return (GQA <= 4 && NG <= 2) ? (FUSED ? 2 : 4) : 1; }

template <int GQA, int NG, bool FUSED, int BITS, bool PH>
__global__ void __launch_bounds__(AW * 64) __attribute__((amdgpu_waves_per_eu(attend_waves<GQA, NG, FUSED>())))
attend_kernel(StepArgs a) {
  // several rounds: the split index varies slowest, so every unit's first
  // splits are dispatched before any unit's (shorter) last one, and the
  // final round holds the short work; one round: splits of a unit together
  const int split = FUSED ? blockIdx.x : blockIdx.z;
  const int hk = FUSED ? blockIdx.y : blockIdx.x, b = FUSED ? blockIdx.z : blockIdx.y;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const oscar_layer_cache &c = a.c;
  const bool append = a.k_new != nullptr;
  // loads that need no request length, issued together: the length, the
  // request's BF16 page table, the first 64 page ids of each wave (history
  // splits) and the loads of the q fragment build
  const int L0 = append ? a.len_before[b] : a.seq_lens[b];
  const int bpt_lane = c.bf16_pt[b * BF16_PT + min(lane, BF16_PT - 1)];
  const int j0 = (split - 1) * a.pages_per_split;
  int pid_pre;
  {
    const int jend = min(c.hist_pt_stride, j0 + a.pages_per_split);
    const int j = max(0, min(j0 + wave + AW * lane, jend - 1));
    pid_pre = c.hist_pt[int64_t(b) * c.hist_pt_stride + j];
  }
  QLoads<GQA> ql;
  build_q_issue<GQA, PH>(a, b, hk, tid, split > 0, ql);
  // keeps these loads ahead of the length checks below (otherwise the
  // compiler sinks them past the early exits, behind the wait for L0)
  asm volatile("" ::: "memory");
  const int L = append ? L0 + 1 : L0;
  // per wave: its page ring, reused for its o[GQA][128] once the pages are done
  constexpr int SB = hist_block_bytes(D / NG, BITS);
  constexpr int DPK = depth_of<BITS>();
  constexpr int WREG = DPK * SB > GQA * D * 4 ? DPK * SB : GQA * D * 4;
  __shared__ __attribute__((aligned(16))) uint8_t wave_lds[AW * WREG];
  __shared__ float ml_lds[2 * AW * GQA];
  __shared__ float zs_lds[AW * GQA * NG];  // per wave: z sums per (head, group)
  __shared__ uint32_t frag_lds[Rows<GQA, NG>::FR_DW * 64];
  __shared__ __attribute__((aligned(16))) union {
    QWork<GQA, NG> q;  // history workgroups
    EvictWork e;       // the raw workgroup of an append
  } work;
  if (!valid_len(L, a.max_seq_len)) {
    // the request is skipped: flag it once, zero its output
    if (split == 0) {
      if (tid == 0 && hk == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
      for (int e = tid; e < GQA * D; e += AW * 64) a.out[(int64_t(b) * a.n_q_heads + hk * GQA) * D + e] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);  // the loads above land before the wave ends
    return;
  }
  const int pages = n_hist_pages(L);
  const int used = 1 + (pages + a.pages_per_split - 1) / a.pages_per_split;
  if (split >= used) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  float *o_lds = reinterpret_cast<float *>(wave_lds);
  float *m_lds = ml_lds;
  float *l_lds = m_lds + AW * GQA;
  float *o_w = o_lds + wave * (WREG / 4);
  bool extra = false;  // the raw workgroup attends the token leaving the window
  RvRows rv;             // history workgroups of the one-round plan: R_V rows
  bool rv_loaded = false;
  if (split == 0) {
    AppendPlan ap{};
    if (append) ap = plan_append(a, L0, bpt_lane);
    // raw BF16 sink + recent pages; an appended token is read from k_new /
    // v_new (its slot may still hold the token that leaves the window)
    const uint16_t *kn = append ? a.k_new + (int64_t(b) * c.n_kv_heads + hk) * D : nullptr;
    const uint16_t *vn = append ? a.v_new + (int64_t(b) * c.n_kv_heads + hk) * D : nullptr;
    if (append && ap.raw_page < 0 && tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    if (append && !ap.evict && ap.raw_page >= 0) {
      // nothing leaves the window: store the new token in its row now
      uint16_t *rk_ = c.bf16 + ((int64_t(ap.raw_page) * c.n_kv_heads + hk) * 2) * (PAGE * D) + ap.raw_row * D;
      if (tid < D) rk_[tid] = kn[tid];
      else if (tid < 2 * D) rk_[PAGE * D + tid - D] = vn[tid - D];
    }
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
      if (append && pg == ap.raw_pg)
        Bf16Wave<GQA>::issue(base, base + PAGE * D, ld, lane, ap.raw_row, kn, vn);
      else
        Bf16Wave<GQA>::issue(base, base + PAGE * D, ld, lane);
      st.compute(ld, valid, lane);
    }
    st.finish(o_w, m_lds + wave * GQA, l_lds + wave * GQA, lane);
    if (append && ap.evict && ap.raw_page >= 0) {
      const int pid = c.hist_pt[int64_t(b) * c.hist_pt_stride + ap.evict_j];
      uint8_t *blk = nullptr;
      if (pid >= 0 && pid < c.n_hist_pages)
        blk = c.hist + (int64_t(pid) * c.n_kv_heads + hk) * hist_block_bytes(D / NG, BITS);
      else if (tid == 0)
        flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
      evict_token<GQA, D / NG, BITS, PH>(a, b, hk, tid, wave, ap, blk, work.e);
      extra = true;
    }
  } else {
    // the newest history token has just left the recent window in an
    // append: the raw workgroup attends it
    const int nh = n_hist_tokens(L) - (append && L0 >= N_RAW ? 1 : 0);
    const int j1 = min((nh + PAGE - 1) / PAGE, j0 + a.pages_per_split);
    constexpr bool F4 = f4_scores<BITS, NG, FUSED>();
    auto prep = [&] { build_q<GQA, NG, BITS, F4>(a, tid, work.q, frag_lds, ql); };
    // one round: the R_V rows for the partial's way back are loaded inside
    // the page loop, behind the wave's last page copies (not at GQA 8 with
    // four scale groups, whose registers are full already)
    auto late = [&] {
      asm volatile("" ::: "memory");
      rv.load(forms_v<PH>(a, hk), tid);
      asm volatile("" ::: "memory");
    };
    // every wave of the workgroup calls this (it holds workgroup barriers)
    // pages per wave loaded through registers before the q build: 3, or 2 in
    // the one-round plan (its 64 KB of R_K per workgroup lands sooner; A/B:
    // batch-1 step -0.6 %, batch 64 +1 % with 2)
    rv_loaded = history_wave<GQA, NG, BITS, DPK, F4, (FUSED && GQA * NG <= 16) ? RvRows::N_LOADS : 0, FUSED ? 2 : 3>(
        a, b, hk, nh, j0, j1, wave, lane, pid_pre, prep, late, frag_lds, wave_lds + wave * WREG,
        zs_lds + wave * GQA * NG, o_w, m_lds + wave * GQA, l_lds + wave * GQA);
  }
  const int64_t head_stride = int64_t(a.part_slots) * PART_STRIDE;
  float *part0 = a.parts + (int64_t(b) * a.n_q_heads + hk * GQA) * head_stride + split * PART_STRIDE;
  if constexpr (!FUSED) {
    // partials for the merge kernel
    __syncthreads();
    if (extra)
      combine_waves<GQA, AW>(o_lds, m_lds, l_lds, part0, head_stride, tid, WREG / 4, work.e.u[1], work.e.sc);
    else
      combine_waves<GQA, AW>(o_lds, m_lds, l_lds, part0, head_stride, tid, WREG / 4);
  } else {
    // R_V rows for the history partial's way back, unless the page loop
    // loaded them already (in flight during the barrier)
    if (split > 0 && !rv_loaded) rv.load(forms_v<PH>(a, hk), tid);
    __syncthreads();
    if (split > 0)
      combine_rotate<GQA>(o_lds, m_lds, l_lds, part0, head_stride, tid, WREG / 4, rv, work.q.y);
    else if (extra)
      combine_waves<GQA, AW, true>(o_lds, m_lds, l_lds, part0, head_stride, tid, WREG / 4, work.e.u[1],
                                   work.e.sc);
    else
      combine_waves<GQA, AW, true>(o_lds, m_lds, l_lds, part0, head_stride, tid, WREG / 4);
    // ---- the last workgroup of (b, hk) to finish merges.  Its partial
    // stores have completed (agent scope: in memory, past this XCD's L2)
    // before the counter counts the workgroup in; the last one reads every
    // partial with agent-scope loads and leaves the counter at zero for the
    // next call.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (used > 1) {
      __shared__ int last;
      if (tid == 0) {
        uint32_t *cnt = a.counters + COUNTER_STRIDE * (b * c.n_kv_heads + hk);
        const uint32_t done = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = done == uint32_t(used - 1);
        if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (!last) return;
    }
    static_assert(sizeof(MergeWork<GQA>) <= sizeof(wave_lds), "merge work area fits the page rings");
    merge_unit<GQA>(a, b, hk, used, tid, *reinterpret_cast<MergeWork<GQA> *>(wave_lds));
  }
}

// ------------------------------------------------------------------ launch

template <int GQA, int NG, int BITS>
static hipError_t launch_t(const StepArgs &a, bool fused, int batch, int hkv, hipStream_t s) {
  const KernelEvents ev = take_profile_events();
  const dim3 grid = fused ? dim3(1 + a.n_splits, hkv, batch) : dim3(hkv, batch, 1 + a.n_splits);
  auto go = [&](auto ph_tag) -> hipError_t {
    constexpr bool PH = decltype(ph_tag)::value;
    if (fused) {
      hipExtLaunchKernelGGL((attend_kernel<GQA, NG, true, BITS, PH>), grid, dim3(AW * 64), 0, s, ev.before, ev.after,
                            0, a);
      return hipGetLastError();
    }
    hipExtLaunchKernelGGL((attend_kernel<GQA, NG, false, BITS, PH>), grid, dim3(AW * 64), 0, s, ev.before, ev.after,
                          0, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((merge_kernel<GQA, PH>), dim3(hkv, batch), dim3(merge_threads<GQA>()), 0, s, a);
    return hipGetLastError();
  };
  // a rotation per KV head (either tensor) runs the instances that index them
  return (a.fstride_k || a.fstride_v) ? go(std::true_type{}) : go(std::false_type{});
}

template <int GQA, int BITS>
static hipError_t launch_gb(const StepArgs &a, bool fused, int G, int batch, int hkv, hipStream_t s) {
  switch (G) {
    case 32: return launch_t<GQA, 4, BITS>(a, fused, batch, hkv, s);
    case 64: return launch_t<GQA, 2, BITS>(a, fused, batch, hkv, s);
    default: return launch_t<GQA, 1, BITS>(a, fused, batch, hkv, s);
  }
}

template <int GQA>
static hipError_t launch_g(const StepArgs &a, bool fused, int G, int batch, int hkv, hipStream_t s) {
  return cache_bits(a.c) == 4 ? launch_gb<GQA, 4>(a, fused, G, batch, hkv, s)
                              : launch_gb<GQA, 2>(a, fused, G, batch, hkv, s);
}

static float pv_scale_for(float clip_v) {
  // PV operand: p <= 2^LAZY_TH, s <= 2 clip / 3, 1/w <= 16; keep it under 2^15
  float k = 1.f;
  const float vmax = exp2f(LAZY_TH) * 16.f * (2.f * clip_v / 3.f);
  while (vmax * k > 32768.f) k *= 0.5f;
  while (vmax * k * 2.f <= 32768.f && k < 65536.f) k *= 2.f;
  return k;
}

hipError_t launch_decode_step(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *k_new,
                              const uint16_t *v_new, const int32_t *len_before, const uint16_t *q,
                              int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                              float sm_scale, float *out, void *ws, hipStream_t s, uint32_t *counters) {
  StepArgs a;
  a.c = c;
  a.fk = rk.forms;
  a.fv = rv.forms;
  a.clip_k = rk.clip;
  a.clip_v = rv.clip;  // with a rotation per head, the largest head clip (bounds the PV operand)
  a.fstride_k = rk.stride;
  a.fstride_v = rv.stride;
  for (int h = 0; h < MAX_HEAD_ROT; ++h) {
    a.hclip_k[h] = rk.head_clip[h];
    a.hclip_v[h] = rv.head_clip[h];
  }
  a.k_new = k_new;
  a.v_new = v_new;
  a.len_before = len_before;
  a.q = q;
  a.seq_lens = seq_lens;
  a.n_q_heads = n_q_heads;
  a.max_seq_len = max_seq_len;
  a.sm_scale = sm_scale;
  a.out = out;
  a.pv_scale = pv_scale_for(rv.clip);
  a.pv_unscale = 1.f / a.pv_scale;
  a.ex_m4 = 0x03000300u;
  a.ex_m16 = 0x00C000C0u;
  a.ex_e = 0x3C003C00u;
  a.ex_mn = 0x03C003C0u;
  a.pk01 = std::log2(4.f * a.pv_scale);
  a.pk23 = std::log2(16.f * a.pv_scale);
  const SplitPlan p = plan_int2_splits(batch, c.n_kv_heads, max_seq_len);
  a.pages_per_split = p.pages_per_split;
  a.n_splits = p.n_splits;
  a.parts = static_cast<float *>(ws);
  a.part_slots = part_slots(p);
  a.counters = counters ? counters
                        : reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + parts_bytes(batch, n_q_heads, p));
  switch (n_q_heads / c.n_kv_heads) {
    case 1: return launch_g<1>(a, p.fused, c.group, batch, c.n_kv_heads, s);
    case 2: return launch_g<2>(a, p.fused, c.group, batch, c.n_kv_heads, s);
    case 4: return launch_g<4>(a, p.fused, c.group, batch, c.n_kv_heads, s);
    case 8: return launch_g<8>(a, p.fused, c.group, batch, c.n_kv_heads, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ scratch
// Decode without a caller workspace (oscar_decode_attn_noalloc): the partials
// and the merge counters live in this file-scope device array, one copy per
// GPU.  Host code never passes the array's name to a kernel (on the host it
// is a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept.  Layout: the counters first (a fixed region, cleared by a fill
// kernel when the address is first taken; every completed call leaves them
// at zero again, whatever its shape), then the partials.
constexpr size_t SCRATCH_COUNTERS = size_t(NOALLOC_MAX_UNITS) * COUNTER_STRIDE * sizeof(uint32_t);
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];
static_assert(SCRATCH_COUNTERS % 256 == 0 && SCRATCH_COUNTERS < NOALLOC_SCRATCH_BYTES, "scratch layout");

__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t *p, int64_t n, uint32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = v;
}

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};
}  // namespace

// The device address of this GPU's scratch array (set up on first use on the
// device, counters cleared on stream s).
static hipError_t scratch_address(hipStream_t s, uint8_t **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    const int64_t n = int64_t(SCRATCH_COUNTERS / sizeof(uint32_t));
    hipLaunchKernelGGL(fill_u32_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint32_t *>(ptr), n, 0u);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<uint8_t *>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t decode_int2_parts_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  return parts_bytes(batch, n_q_heads, plan_int2_splits(batch, n_kv_heads, max_seq_len));
}

hipError_t launch_decode_int2_noalloc(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q,
                                      int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                                      float sm_scale, float *out, hipStream_t s) {
  uint8_t *base = nullptr;
  hipError_t e = scratch_address(s, &base);
  if (e != hipSuccess) return e;
  return launch_decode_step(c, rk, rv, nullptr, nullptr, nullptr, q, n_q_heads, seq_lens, batch, max_seq_len,
                            sm_scale, out, base + SCRATCH_COUNTERS, s, reinterpret_cast<uint32_t *>(base));
}

hipError_t launch_decode_int2(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q,
                              int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                              float sm_scale, float *out, void *ws, hipStream_t s) {
  return launch_decode_step(c, rk, rv, nullptr, nullptr, nullptr, q, n_q_heads, seq_lens, batch, max_seq_len,
                            sm_scale, out, ws, s);
}

}  // namespace oscar
