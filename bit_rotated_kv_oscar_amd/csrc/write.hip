// Fused KV write: rotate, clip, INT2-pack and page-store history tokens; store
// sink / recent tokens raw.  OSCAR online phase (gist.science nl/fr technical
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
  const uint16_t *src[2];  // k_new, v_new
  const int32_t *cu_new;
  const int32_t *len_before;
  int64_t total_tokens;
  int max_new;
};

// Request b's rows cu_new[b]..cu_new[b+1]-1 must lie in [0, total_tokens) and
// number at most max_new (the grid covers no more); otherwise the request is
// skipped and flagged.
__device__ inline bool request_ok(const WriteArgs &a, int b, int &L0, int &n) {
  const int c0 = a.cu_new[b], c1 = a.cu_new[b + 1];
  L0 = a.len_before[b];
  n = c1 - c0;
  return c0 >= 0 && c1 >= c0 && int64_t(c1) <= a.total_tokens && n <= a.max_new && L0 >= 0 &&
         int64_t(L0) + n < (int64_t(1) << 30);
}

constexpr int WHC = 8;  // KV heads per write workgroup

typedef __bf16 bf16x8w __attribute__((ext_vector_type(8)));
typedef float f32x4w __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4w __attribute__((ext_vector_type(4)));

// One workgroup (4 waves) per (request, touched history page, K|V, chunk of
// up to 8 KV heads).  The page's 16 rows that enter history in this call --
// new tokens, or ring tokens pushed out of the recent window -- are rotated
// on the matrix cores: Y = X R with X the bf16 rows (exact) and R split into
// three bf16 pieces (b1 + b2 + b3 = R to 2^-24), each piece accumulated in
// its own fp32 accumulator and added at the end (small pieces last), so the
// error stays within the fp32 dot-product bound.  Wave w computes output
// channels 32w .. 32w+31 (two 16-column tiles) for every head of the chunk;
// then clip, per-(token, group) fp16 zero = min and scale = (max - min)/3
// (group min / max by row reductions across the 16 lanes of a tile row,
// then across the waves of a group), codes, and the packed store in the
// documented layout (read-modify-write for rows already present).
constexpr int WPP = 8;  // history pages per write workgroup (the R pieces stay in registers)

// value of lane (l - N) mod 16 within each row of 16 lanes (DPP row_ror)
template <int N>
__device__ inline float row_rot(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

template <int G>
struct WriteShared {
  const uint16_t *tok_ptr[PAGE];  // row of head h0 (or null: inactive)
  int tok_stride[PAGE];           // elements between heads
  int active_s[PAGE];
  int bad;
  const uint16_t *any_row;  // a valid row for loads whose result is discarded
  float pmin[WHC][PAGE][4], pmax[WHC][PAGE][4];
  float sz[WHC][PAGE][D / G][2];
  uint8_t codes[WHC][PAGE][D];
};

template <int G>
__device__ void write_page(const WriteArgs &a, int b, int tensor, int h0, int nh, int L0, int hlo, int hhi,
                           int pos0, int pid, float clip, const bf16x8w (&rb)[2][4][3], WriteShared<G> &sh,
                           int tid, int wave, int lane);

template <int G>
__global__ void __launch_bounds__(256) write_hist_kernel(WriteArgs a) {
  const int b = blockIdx.z;
  const int tensor = blockIdx.y & 1, hc = blockIdx.y >> 1;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const oscar_layer_cache &c = a.c;
  const int hkv = c.n_kv_heads;
  const int h0 = hc * WHC;
  if (h0 >= hkv) return;
  const int nh = min(WHC, hkv - h0);

  int L0, n;
  if (!request_ok(a, b, L0, n)) {
    if (tid == 0 && blockIdx.x == 0 && blockIdx.y == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  const int L = L0 + n;
  const int hlo = max(N_SINK, L0 - N_RECENT);  // first position entering history
  const int hhi = L - N_RECENT;                 // one past the last
  if (hhi <= hlo) return;
  const int jfirst = (hlo - N_SINK) / PAGE + blockIdx.x * WPP;
  if (N_SINK + PAGE * jfirst >= hhi) return;
  __shared__ WriteShared<G> sh;
  // B operands: R pieces for this wave's two column tiles; lane l holds
  // R[i][j] for j = 32 wave + 16 ct + l%16, i = 32 kk + 8 (l/16) .. + 7
  bf16x8w rb[2][4][3];
  {
    const uint16_t *RB = reinterpret_cast<const uint16_t *>(a.forms[tensor] + FORM_RT_B);
    const int qd = lane >> 4, nn = lane & 15;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
          const int jj = 32 * wave + 16 * ct + nn, ii = 32 * kk + 8 * qd;
          const u32x4w u = *reinterpret_cast<const u32x4w *>(RB + pc * D * D + jj * D + ii);
          rb[ct][kk][pc] = __builtin_bit_cast(bf16x8w, u);
        }
  }
  const float clip = a.clip[tensor];
  for (int jj = 0; jj < WPP; ++jj) {
    const int j = jfirst + jj;
    const int pos0 = N_SINK + PAGE * j;
    if (pos0 >= hhi) break;  // uniform
    if (j >= c.hist_pt_stride) {
      if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
      break;
    }
    const int pid = c.hist_pt[int64_t(b) * c.hist_pt_stride + j];
    if (pid < 0 || pid >= c.n_hist_pages) {
      if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
      continue;
    }
    write_page<G>(a, b, tensor, h0, nh, L0, hlo, hhi, pos0, pid, clip, rb, sh, tid, wave, lane);
  }
}

// One history page of the chunk's heads (all threads of the workgroup).
template <int G>
__device__ void write_page(const WriteArgs &a, int b, int tensor, int h0, int nh, int L0, int hlo, int hhi,
                           int pos0, int pid, float clip, const bf16x8w (&rb)[2][4][3], WriteShared<G> &sh,
                           int tid, int wave, int lane) {
  constexpr int NG = D / G, WPG = G / 32;
  const oscar_layer_cache &c = a.c;
  const int hkv = c.n_kv_heads;
  auto &tok_ptr = sh.tok_ptr;
  auto &tok_stride = sh.tok_stride;
  auto &active_s = sh.active_s;
  auto &pmin = sh.pmin;
  auto &pmax = sh.pmax;
  auto &sz = sh.sz;
  auto &codes = sh.codes;
  __syncthreads();  // the previous page is done with the shared arrays
  if (tid < PAGE) {
    const int p = pos0 + tid;
    const bool act = p >= hlo && p < hhi;
    const uint16_t *row = nullptr;
    int stride = 0;
    int is_bad = 0;
    if (act) {
      if (p < L0) {  // leaves the ring now
        const int slot = p % N_RECENT;
        const int bp = c.bf16_pt[b * BF16_PT + 1 + slot / PAGE];
        if (bp >= 0 && bp < c.n_bf16_pages) {
          row = c.bf16 + ((int64_t(bp) * hkv + h0) * 2 + tensor) * (PAGE * D) + (slot % PAGE) * D;
          stride = 2 * PAGE * D;
        } else {
          is_bad = 1;
        }
      } else {
        const int64_t src_row = a.cu_new[b] + (p - L0);
        row = a.src[tensor] + (src_row * hkv + h0) * D;
        stride = D;
      }
    }
    tok_ptr[tid] = row;
    tok_stride[tid] = stride;
    active_s[tid] = act;
    // any bad row makes the whole page bad (flagged, nothing written)
    const uint64_t any_bad = __ballot(is_bad);
    const uint64_t on = __ballot(row != nullptr);
    if (tid == 0) sh.bad = any_bad != 0;
    if (on && tid == __builtin_ctzll(on)) sh.any_row = row;
  }
  __syncthreads();
  if (sh.bad) {
    if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    return;
  }
  const int r_a = lane & 15, qd = lane >> 4;  // A operand: row (token), k sub-block
  const uint16_t *my_row = tok_ptr[r_a];
  const int my_stride = tok_stride[r_a];
  const int g = (32 * wave) / G;  // scale group of this wave's channels
  // rows of head hh (A operand), loaded one head ahead; an inactive row (or
  // a head past the chunk) reads row 0 of the page's first active token and
  // is zeroed after the load, so the loads carry no branch.  The pointers
  // come back from LDS, so they are cast to the global address space: flat
  // loads would also count against the LDS wait counter.
  typedef const __attribute__((address_space(1))) u32x4w *gptr;
  const bool row_on = my_row != nullptr;
  const uint16_t *safe_row = row_on ? my_row : sh.any_row;
  auto load_x = [&](int hh, u32x4w (&u)[4]) {
    const bool on = row_on && hh < nh;
    const uint16_t *rp = safe_row + (on ? int64_t(hh) * my_stride : 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4w v = *(gptr)(rp + 32 * kk + 8 * qd);
      u[kk] = on ? v : u32x4w{0u, 0u, 0u, 0u};
    }
  };
  u32x4w xn[4];
  load_x(0, xn);
  for (int hh = 0; hh < nh; ++hh) {
    bf16x8w xa[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xa[kk] = __builtin_bit_cast(bf16x8w, xn[kk]);
    load_x(hh + 1, xn);
    f32x4w yc[2];  // clipped rotated values: rows 4 qd + i, column 32 wave + 16 ct + l%16
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4w acc[3];
#pragma unroll
      for (int pc = 0; pc < 3; ++pc) {
        acc[pc] = f32x4w{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc[pc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[kk], rb[ct][kk][pc], acc[pc], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = acc[0][i] + (acc[1][i] + acc[2][i]);
        yc[ct][i] = fminf(fmaxf(y, -clip), clip);
      }
    }
    // min / max of each token over this wave's 32 channels (16 lanes of a row)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo = fminf(yc[0][i], yc[1][i]), hi = fmaxf(yc[0][i], yc[1][i]);
      lo = fminf(lo, row_rot<8>(lo));
      hi = fmaxf(hi, row_rot<8>(hi));
      lo = fminf(lo, row_rot<4>(lo));
      hi = fmaxf(hi, row_rot<4>(hi));
      lo = fminf(lo, row_rot<2>(lo));
      hi = fmaxf(hi, row_rot<2>(hi));
      lo = fminf(lo, row_rot<1>(lo));
      hi = fmaxf(hi, row_rot<1>(hi));
      if (r_a == 0) {
        pmin[hh][4 * qd + i][wave] = lo;
        pmax[hh][4 * qd + i][wave] = hi;
      }
    }
    __syncthreads();  // partials of every wave of the group are in
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * qd + i;
      float lo = pmin[hh][t][WPG * g], hi = pmax[hh][t][WPG * g];
      for (int w = 1; w < WPG; ++w) {
        lo = fminf(lo, pmin[hh][t][WPG * g + w]);
        hi = fmaxf(hi, pmax[hh][t][WPG * g + w]);
      }
      const float s = __half2float(__float2half_rn((hi - lo) / 3.0f));
      const float z = __half2float(__float2half_rn(lo));
      if (r_a == 0 && wave == WPG * g) {
        sz[hh][t][g][0] = s;
        sz[hh][t][g][1] = z;
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        int cd = 0;
        if (s > 0.f) cd = min(3, max(0, int(rintf((yc[ct][i] - z) / s))));
        codes[hh][t][32 * wave + 16 * ct + r_a] = uint8_t(cd);
      }
    }
  }
  __syncthreads();
  // packed store: 128 code dwords per head, then the meta entries
  for (int e = tid; e < nh * 128; e += 256) {
    const int hh = e >> 7, w = e & 127;
    const int ln = w >> 1, d = w & 1, lq = ln >> 4, la = ln & 15;
    uint32_t word = 0, mask = 0;
    for (int u = 0; u < 8; ++u) {
      int t0, t1, c0, c1;
      if (tensor == 0) {
        t0 = t1 = la;
        c0 = 32 * (2 * d + u / 4) + 8 * lq + 2 * (u % 4);
        c1 = c0 + 1;
      } else {
        c0 = c1 = 16 * (4 * d + u / 2) + la;
        t0 = 4 * lq + 2 * (u % 2);
        t1 = t0 + 1;
      }
      if (active_s[t0]) {
        word |= uint32_t(codes[hh][t0][c0]) << slot_lo(u);
        mask |= 3u << slot_lo(u);
      }
      if (active_s[t1]) {
        word |= uint32_t(codes[hh][t1][c1]) << slot_hi(u);
        mask |= 3u << slot_hi(u);
      }
    }
    uint8_t *blk = c.hist + (int64_t(pid) * hkv + h0 + hh) * hist_block_bytes(G);
    uint32_t *area = reinterpret_cast<uint32_t *>(blk + (tensor ? v_codes_off(G) : k_codes_off(G)));
    if (mask == 0xFFFFFFFFu)
      area[w] = word;
    else if (mask)
      area[w] = (area[w] & ~mask) | word;
  }
  for (int e = tid; e < nh * PAGE * NG; e += 256) {
    const int hh = e / (PAGE * NG), t = (e / NG) % PAGE, g = e % NG;
    if (active_s[t]) {
      uint8_t *blk = c.hist + (int64_t(pid) * hkv + h0 + hh) * hist_block_bytes(G);
      __half2 *meta = reinterpret_cast<__half2 *>(blk + (tensor ? v_meta_off(G) : k_meta_off(G)));
      meta[PAGE * g + t] = __halves2half2(__float2half_rn(sz[hh][t][g][0]), __float2half_rn(sz[hh][t][g][1]));
    }
  }
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
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.cu_new = cu_new;
  a.len_before = len_before;
  a.total_tokens = total_tokens;
  a.max_new = max_new;
  // history positions entering in one call span at most max_new + 16 rows
  const int tiles = (max_new + PAGE - 1) / PAGE + 2;
  const dim3 grid((tiles + WPP - 1) / WPP, 2 * ((c.n_kv_heads + WHC - 1) / WHC), batch);
  const KernelEvents ev = take_profile_events();
  switch (c.group) {
    case 32: hipExtLaunchKernelGGL(write_hist_kernel<32>, grid, dim3(256), 0, s, ev.before, ev.after, 0, a); break;
    case 64: hipExtLaunchKernelGGL(write_hist_kernel<64>, grid, dim3(256), 0, s, ev.before, ev.after, 0, a); break;
    default: hipExtLaunchKernelGGL(write_hist_kernel<128>, grid, dim3(256), 0, s, ev.before, ev.after, 0, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(write_raw_kernel, dim3(N_SINK + N_RECENT, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
