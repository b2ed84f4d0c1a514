// Fused KV write: rotate, clip, INT2-pack and page-store history tokens; store
// sink / recent tokens raw.  OSCAR online phase (gist.science nl/fr technical
// summaries, section 2.2.B: history kept as INT2 after the fixed rotation and
// clipping, sink and recent tokens in BF16; arXiv:2605.17757 v2 abstract:
// fused write kernel over a paged cache).
//
// Two launches per call, in stream order:
//   1. write_hist_kernel: one block per (request, touched history page,
//      KV head, K|V).  It gathers the 16 rows of the page that enter history
//      in this call — new tokens, or ring tokens pushed out of the recent
//      window — rotates them (x R, fp32), clips, computes per-group fp16
//      scale / zero and codes, and stores codes and meta in the documented
//      layout (read-modify-write for rows already present).
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

__global__ void __launch_bounds__(128) write_hist_kernel(WriteArgs a) {
  const int b = blockIdx.z;
  const int h = blockIdx.y >> 1;
  const int tensor = blockIdx.y & 1;
  const int tid = threadIdx.x;  // output channel
  const oscar_layer_cache &c = a.c;
  const int hkv = c.n_kv_heads;
  const int G = c.group;
  const int ng = D / G;

  int L0, n;
  if (!request_ok(a, b, L0, n)) {
    if (tid == 0 && blockIdx.x == 0 && blockIdx.y == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  const int L = L0 + n;
  const int hlo = max(N_SINK, L0 - N_RECENT);  // first position entering history
  const int hhi = L - N_RECENT;                 // one past the last
  if (hhi <= hlo) return;
  const int j = (hlo - N_SINK) / PAGE + blockIdx.x;
  const int pos0 = N_SINK + PAGE * j;
  if (pos0 >= hhi) return;
  if (j >= c.hist_pt_stride) {
    if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    return;
  }
  const int pid = c.hist_pt[int64_t(b) * c.hist_pt_stride + j];
  if (pid < 0 || pid >= c.n_hist_pages) {
    if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    return;
  }

  __shared__ float xs[PAGE][D];
  __shared__ float xc[PAGE][D];
  __shared__ uint8_t codes[PAGE][D];
  __shared__ float sc[PAGE][4];
  __shared__ float zc[PAGE][4];
  __shared__ int active[PAGE];
  __shared__ int bad;
  if (tid == 0) bad = 0;
  __syncthreads();

  for (int r = 0; r < PAGE; ++r) {
    const int p = pos0 + r;
    const bool act = p >= hlo && p < hhi;
    float x = 0.f;
    if (act) {
      const uint16_t *row = nullptr;
      if (p < L0) {  // leaves the ring now
        const int slot = p % N_RECENT;
        const int bp = c.bf16_pt[b * BF16_PT + 1 + slot / PAGE];
        if (bp >= 0 && bp < c.n_bf16_pages)
          row = c.bf16 + ((int64_t(bp) * hkv + h) * 2 + tensor) * (PAGE * D) + (slot % PAGE) * D;
        else if (tid == 0)
          bad = 1;
      } else {
        const int64_t src_row = a.cu_new[b] + (p - L0);
        row = a.src[tensor] + (src_row * hkv + h) * D;
      }
      if (row) x = bf16_to_f32(row[tid]);
    }
    xs[r][tid] = x;
    if (tid == 0) active[r] = act;
  }
  __syncthreads();
  if (bad) {
    if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    return;
  }

  // rotation x R (fp32), then clip
  const float *R = reinterpret_cast<const float *>(a.forms[tensor] + FORM_R);
  float acc[PAGE];
#pragma unroll
  for (int r = 0; r < PAGE; ++r) acc[r] = 0.f;
  for (int i = 0; i < D; ++i) {
    const float rij = R[i * D + tid];
#pragma unroll
    for (int r = 0; r < PAGE; ++r) acc[r] = fmaf(xs[r][i], rij, acc[r]);
  }
  const float clip = a.clip[tensor];
#pragma unroll
  for (int r = 0; r < PAGE; ++r) xc[r][tid] = fminf(fmaxf(acc[r], -clip), clip);
  __syncthreads();

  // per (row, group) fp16 zero = min, scale = (max - min)/3
  if (tid < PAGE * ng) {
    const int r = tid / ng, g = tid % ng;
    float lo = xc[r][g * G], hi = lo;
    for (int i = 1; i < G; ++i) {
      lo = fminf(lo, xc[r][g * G + i]);
      hi = fmaxf(hi, xc[r][g * G + i]);
    }
    zc[r][g] = __half2float(__float2half_rn(lo));
    sc[r][g] = __half2float(__float2half_rn((hi - lo) / 3.0f));
  }
  __syncthreads();
  {
    const int g = tid / G;
#pragma unroll
    for (int r = 0; r < PAGE; ++r) {
      const float s = sc[r][g];
      int cd = 0;
      if (s > 0.f) cd = min(3, max(0, int(rintf((xc[r][tid] - zc[r][g]) / s))));
      codes[r][tid] = uint8_t(cd);
    }
  }
  __syncthreads();

  uint8_t *blk = c.hist + (int64_t(pid) * hkv + h) * hist_block_bytes(G);
  uint32_t *area = reinterpret_cast<uint32_t *>(blk + (tensor ? v_codes_off(G) : k_codes_off(G)));
  {
    const int w = tid;  // 128 dwords per code area
    const int lane = w >> 1, d = w & 1, lq = lane >> 4, la = lane & 15;
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
      if (active[t0]) {
        word |= uint32_t(codes[t0][c0]) << slot_lo(u);
        mask |= 3u << slot_lo(u);
      }
      if (active[t1]) {
        word |= uint32_t(codes[t1][c1]) << slot_hi(u);
        mask |= 3u << slot_hi(u);
      }
    }
    if (mask == 0xFFFFFFFFu)
      area[w] = word;
    else if (mask)
      area[w] = (area[w] & ~mask) | word;
  }
  if (tid < PAGE * ng) {
    const int r = tid / ng, g = tid % ng;
    if (active[r]) {
      __half2 *meta = reinterpret_cast<__half2 *>(blk + (tensor ? v_meta_off(G) : k_meta_off(G)));
      meta[PAGE * g + r] = __halves2half2(__float2half_rn(sc[r][g]), __float2half_rn(zc[r][g]));
    }
  }
}

// new tokens that land in the sink or the recent ring: raw bf16 copies
__global__ void __launch_bounds__(256) write_raw_kernel(WriteArgs a) {
  const int b = blockIdx.y;
  const int i = blockIdx.x;
  const oscar_layer_cache &c = a.c;
  int L0, n;
  if (!request_ok(a, b, L0, n)) {
    if (threadIdx.x == 0 && i == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  if (i >= n) return;
  const int L = L0 + n;
  const int p = L0 + i;
  int page, row;
  if (p < N_SINK) {
    page = c.bf16_pt[b * BF16_PT];
    row = p;
  } else if (p >= L - N_RECENT) {
    const int slot = p % N_RECENT;
    page = c.bf16_pt[b * BF16_PT + 1 + slot / PAGE];
    row = slot % PAGE;
  } else {
    return;
  }
  if (page < 0 || page >= c.n_bf16_pages) {
    if (threadIdx.x == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
    return;
  }
  const int hkv = c.n_kv_heads;
  const int64_t src_row = a.cu_new[b] + i;
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
  hipLaunchKernelGGL(write_hist_kernel, dim3(tiles, 2 * c.n_kv_heads, batch), dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(write_raw_kernel, dim3(max_new, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
