// Mixed-precision paged decode attention over the OSCAR cache.
//
// OSCAR online phase (gist.science nl/fr technical summaries, section 2.2.B:
// one fused kernel unpacks, dequantises, undoes the rotation and attends over
// the INT2 history, on paged storage with prefix caching; arXiv:2605.17757 v2
// abstract).  The rotation is never undone per token: history keys stay in
// the rotated basis and are scored against q R_K (an orthogonal R keeps dot
// products), and the history part of the output is rotated back by R_V^T
// once per (request, query head) in the merge.
//
// Kernels, in stream order:
//   qrot:  q_rot = sm_scale * q R_K                           [B][Hq][128]
//   split: one block per (request, KV head, split).  Split 0 covers the raw
//          BF16 sink + recent tokens, split s >= 1 covers history pages
//          [(s-1)P, sP).  Online softmax per query head of the GQA group;
//          writes (acc[128], m, l) per query head.
//   merge: LSE-combines the splits, applies R_V^T to the history part, adds
//          the raw part and normalises.                      [B][Hq][128] fp32
#include "kernels.h"

namespace oscar {

constexpr int MAX_GQA = 16;
constexpr int PART = D + 2;  // acc[128], m, l

SplitPlan plan_int2_splits(int batch, int n_kv_heads, int max_seq_len) {
  const int pages = n_hist_pages(max_seq_len);
  SplitPlan p;
  if (pages == 0) {
    p.pages_per_split = 1;
    p.n_splits = 0;
    return p;
  }
  const int64_t units = int64_t(batch) * n_kv_heads;
  int64_t per = (int64_t(pages) * units + 2047) / 2048;  // about 2048 blocks in all
  if (per < 4) per = 4;
  p.pages_per_split = int(per);
  p.n_splits = int((pages + per - 1) / per);
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t decode_int2_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  const SplitPlan p = plan_int2_splits(batch, n_kv_heads, max_seq_len);
  const size_t qrot = align256(size_t(batch) * n_q_heads * D * sizeof(float));
  const size_t parts = align256(size_t(batch) * n_q_heads * (1 + p.n_splits) * PART * sizeof(float));
  return qrot + parts;
}

struct DecodeArgs {
  oscar_layer_cache c;
  const uint8_t *fk, *fv;
  const uint16_t *q;
  const int32_t *seq_lens;
  int n_q_heads, max_seq_len, pages_per_split, n_splits;
  float sm_scale;
  float *qrot;   // [B][Hq][128]
  float *parts;  // [B][Hq][1 + n_splits][PART]
  float *out;
};

__device__ inline bool valid_len(int L, int max_len) { return L >= 1 && L <= max_len; }

__global__ void __launch_bounds__(128) qrot_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  __shared__ float qs[D];
  qs[j] = bf16_to_f32(a.q[(int64_t(b) * a.n_q_heads + h) * D + j]);
  __syncthreads();
  const float *R = reinterpret_cast<const float *>(a.fk + FORM_R);
  float s = 0.f;
  for (int i = 0; i < D; ++i) s = fmaf(qs[i], R[i * D + j], s);
  a.qrot[(int64_t(b) * a.n_q_heads + h) * D + j] = s * a.sm_scale;
}

// Loads one row of K or V for the split: raw bf16 or dequantised history.
// Raw part: virtual row k of the request's raw token list (sink, then ring).
__device__ inline const uint16_t *raw_row(const oscar_layer_cache &c, int b, int h, int tensor,
                                          int L, int k, bool &bad) {
  const int ns = min(L, N_SINK);
  int page, row;
  if (k < ns) {
    page = c.bf16_pt[b * BF16_PT];
    row = k;
  } else {
    const int p = max(N_SINK, L - N_RECENT) + (k - ns);
    const int slot = p % N_RECENT;
    page = c.bf16_pt[b * BF16_PT + 1 + slot / PAGE];
    row = slot % PAGE;
  }
  if (page < 0 || page >= c.n_bf16_pages) {
    bad = true;
    return nullptr;
  }
  return c.bf16 + ((int64_t(page) * c.n_kv_heads + h) * 2 + tensor) * (PAGE * D) + row * D;
}

__global__ void __launch_bounds__(128) split_kernel(DecodeArgs a) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const oscar_layer_cache &c = a.c;
  const int gqa = a.n_q_heads / c.n_kv_heads;
  const int G = c.group;
  const int L = a.seq_lens[b];

  __shared__ float qs[MAX_GQA][D];
  __shared__ float xs[PAGE][D];
  __shared__ float ps[MAX_GQA][PAGE];
  __shared__ float alpha_s[MAX_GQA];
  __shared__ float m_s[MAX_GQA], l_s[MAX_GQA];
  __shared__ int bad_s;

  float *part0 = a.parts + ((int64_t(b) * a.n_q_heads + hk * gqa) * (1 + a.n_splits) + split) * PART;
  const int64_t head_stride = int64_t(1 + a.n_splits) * PART;

  if (!valid_len(L, a.max_seq_len)) {
    if (tid == 0 && split == 0 && hk == 0) flag_status(c.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  const bool raw = split == 0;
  int rows_total, row0;
  if (raw) {
    rows_total = min(L, N_RAW);
    row0 = 0;
  } else {
    const int nh = n_hist_tokens(L);
    row0 = (split - 1) * a.pages_per_split * PAGE;
    rows_total = min(nh, row0 + a.pages_per_split * PAGE);
  }
  for (int hh = 0; hh < gqa; ++hh) {
    const int hq = hk * gqa + hh;
    qs[hh][tid] = raw ? bf16_to_f32(a.q[(int64_t(b) * a.n_q_heads + hq) * D + tid]) * a.sm_scale
                      : a.qrot[(int64_t(b) * a.n_q_heads + hq) * D + tid];
  }
  if (tid < MAX_GQA) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  if (tid == 0) bad_s = 0;
  float acc[MAX_GQA];
#pragma unroll
  for (int hh = 0; hh < MAX_GQA; ++hh) acc[hh] = 0.f;
  __syncthreads();

  for (int r0 = row0; r0 < rows_total; r0 += PAGE) {
    const int nrow = min(PAGE, rows_total - r0);
    // ---- keys
    const uint8_t *blk = nullptr;
    if (!raw) {
      const int j = r0 / PAGE;
      const int pid = (j < c.hist_pt_stride) ? c.hist_pt[int64_t(b) * c.hist_pt_stride + j] : -1;
      if (pid < 0 || pid >= c.n_hist_pages) {
        if (tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
        continue;  // uniform across the block
      }
      blk = c.hist + (int64_t(pid) * c.n_kv_heads + hk) * hist_block_bytes(G);
    }
    for (int tensor = 0; tensor < 2; ++tensor) {
      for (int r = 0; r < PAGE; ++r) {
        float x = 0.f;
        if (r < nrow) {
          if (raw) {
            bool bad = false;
            const uint16_t *row = raw_row(c, b, hk, tensor, L, r0 + r, bad);
            if (bad) {
              if (tid == 0) bad_s = 1;
            } else {
              x = bf16_to_f32(row[tid]);
            }
          } else {
            int word, bit;
            if (tensor == 0)
              k_code_pos(r, tid, word, bit);
            else
              v_code_pos(r, tid, word, bit);
            const uint32_t *area =
                reinterpret_cast<const uint32_t *>(blk + (tensor ? v_codes_off(G) : k_codes_off(G)));
            const int code = (area[word] >> bit) & 3;
            const __half2 sz = reinterpret_cast<const __half2 *>(
                blk + (tensor ? v_meta_off(G) : k_meta_off(G)))[PAGE * (tid / G) + r];
            x = float(code) * __low2float(sz) + __high2float(sz);
          }
        }
        xs[r][tid] = x;
      }
      __syncthreads();
      if (tensor == 0) {
        // scores for (head, row)
        for (int idx = tid; idx < gqa * PAGE; idx += 128) {
          const int hh = idx / PAGE, r = idx % PAGE;
          float s = 0.f;
          for (int i = 0; i < D; ++i) s = fmaf(qs[hh][i], xs[r][i], s);
          ps[hh][r] = (r < nrow) ? s : -INFINITY;
        }
        __syncthreads();
        if (tid < gqa) {
          float mx = m_s[tid];
          for (int r = 0; r < nrow; ++r) mx = fmaxf(mx, ps[tid][r]);
          const float al = (m_s[tid] == -INFINITY) ? 0.f : expf(m_s[tid] - mx);
          float sum = 0.f;
          for (int r = 0; r < PAGE; ++r) {
            const float p = (r < nrow) ? expf(ps[tid][r] - mx) : 0.f;
            ps[tid][r] = p;
            sum += p;
          }
          l_s[tid] = l_s[tid] * al + sum;
          m_s[tid] = mx;
          alpha_s[tid] = al;
        }
        __syncthreads();
      } else {
        for (int hh = 0; hh < gqa; ++hh) {
          float s = acc[hh] * alpha_s[hh];
          for (int r = 0; r < PAGE; ++r) s = fmaf(ps[hh][r], xs[r][tid], s);
          acc[hh] = s;
        }
        __syncthreads();
      }
    }
  }
  if (bad_s && tid == 0) flag_status(c.status, OSCAR_STATUS_BAD_PAGE);
  for (int hh = 0; hh < gqa; ++hh) {
    float *part = part0 + hh * head_stride;
    part[tid] = acc[hh];
    if (tid == 0) {
      part[D] = m_s[hh];
      part[D + 1] = l_s[hh];
    }
  }
}

__global__ void __launch_bounds__(128) merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_lens[b];
  float *o = a.out + (int64_t(b) * a.n_q_heads + hq) * D;
  if (!valid_len(L, a.max_seq_len)) {
    o[tid] = 0.f;
    return;
  }
  const int used = 1 + (n_hist_pages(L) + a.pages_per_split - 1) / a.pages_per_split;
  const float *parts = a.parts + (int64_t(b) * a.n_q_heads + hq) * (1 + a.n_splits) * PART;
  float m = -INFINITY;
  for (int s = 0; s < used; ++s) m = fmaxf(m, parts[s * PART + D]);
  float l = 0.f, rot = 0.f, plain = 0.f;
  for (int s = 0; s < used; ++s) {
    const float ms = parts[s * PART + D];
    const float w = (ms == -INFINITY) ? 0.f : expf(ms - m);
    l = fmaf(w, parts[s * PART + D + 1], l);
    if (s == 0)
      plain = w * parts[tid];
    else
      rot = fmaf(w, parts[s * PART + tid], rot);
  }
  __shared__ float rs[D];
  rs[tid] = rot;
  __syncthreads();
  const float *RT = reinterpret_cast<const float *>(a.fv + FORM_RT);
  float back = 0.f;  // (rot R_V^T)[tid] = sum_i rot[i] R_V[tid][i]
  for (int i = 0; i < D; ++i) back = fmaf(rs[i], RT[i * D + tid], back);
  o[tid] = (back + plain) / l;
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
  a.qrot = static_cast<float *>(ws);
  a.parts = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                      align256(size_t(batch) * n_q_heads * D * sizeof(float)));
  a.out = out;
  hipLaunchKernelGGL(qrot_kernel, dim3(n_q_heads, batch), dim3(D), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_kernel, dim3(1 + p.n_splits, c.n_kv_heads, batch), dim3(128), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(n_q_heads, batch), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
