// Plain BF16 paged decode attention: the all-BF16 baseline that OSCAR's
// batch-1 decode speed-up is measured against (arXiv:2605.17757 v2 abstract).
// Split-K over pages with an LSE merge, online softmax per query head of the
// GQA group, fp32 accumulation.
#include "kernels.h"

namespace oscar {

constexpr int B_MAX_GQA = 16;
constexpr int B_PART = D + 2;

SplitPlan plan_bf16_splits(int batch, int n_kv_heads, int max_seq_len) {
  const int pages = (max_seq_len + PAGE - 1) / PAGE;
  const int64_t units = int64_t(batch) * n_kv_heads;
  int64_t per = (int64_t(pages) * units + 2047) / 2048;
  if (per < 4) per = 4;
  SplitPlan p;
  p.pages_per_split = int(per);
  p.n_splits = int((pages + per - 1) / per);
  return p;
}

size_t decode_bf16_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  const SplitPlan p = plan_bf16_splits(batch, n_kv_heads, max_seq_len);
  return (size_t(batch) * n_q_heads * p.n_splits * B_PART * sizeof(float) + 255) & ~size_t(255);
}

struct Bf16Args {
  const uint16_t *q, *kv;
  int64_t n_pages;
  const int32_t *pt;
  int pt_stride;
  const int32_t *seq_lens;
  int max_seq_len, n_q_heads, n_kv_heads, pages_per_split, n_splits;
  float sm_scale;
  float *out;
  uint32_t *status;
  float *parts;
};

__global__ void __launch_bounds__(128) bf16_split_kernel(Bf16Args a) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int gqa = a.n_q_heads / a.n_kv_heads;
  const int L = a.seq_lens[b];
  __shared__ float qs[B_MAX_GQA][D];
  __shared__ float xs[PAGE][D];
  __shared__ float ps[B_MAX_GQA][PAGE];
  __shared__ float alpha_s[B_MAX_GQA], m_s[B_MAX_GQA], l_s[B_MAX_GQA];
  if (L < 1 || L > a.max_seq_len) {
    if (tid == 0 && split == 0 && hk == 0) flag_status(a.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  for (int hh = 0; hh < gqa; ++hh)
    qs[hh][tid] = bf16_to_f32(a.q[(int64_t(b) * a.n_q_heads + hk * gqa + hh) * D + tid]) * a.sm_scale;
  if (tid < B_MAX_GQA) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float acc[B_MAX_GQA];
#pragma unroll
  for (int hh = 0; hh < B_MAX_GQA; ++hh) acc[hh] = 0.f;
  __syncthreads();
  const int t_begin = split * a.pages_per_split * PAGE;
  const int t_end = min(L, t_begin + a.pages_per_split * PAGE);
  for (int t0 = t_begin; t0 < t_end; t0 += PAGE) {
    const int nrow = min(PAGE, t_end - t0);
    const int j = t0 / PAGE;
    const int pid = (j < a.pt_stride) ? a.pt[int64_t(b) * a.pt_stride + j] : -1;
    if (pid < 0 || pid >= a.n_pages) {
      if (tid == 0) flag_status(a.status, OSCAR_STATUS_BAD_PAGE);
      continue;
    }
    const uint16_t *base = a.kv + (int64_t(pid) * a.n_kv_heads + hk) * 2 * PAGE * D;
    for (int tensor = 0; tensor < 2; ++tensor) {
      for (int r = 0; r < PAGE; ++r)
        xs[r][tid] = (r < nrow) ? bf16_to_f32(base[tensor * PAGE * D + r * D + tid]) : 0.f;
      __syncthreads();
      if (tensor == 0) {
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
  for (int hh = 0; hh < gqa; ++hh) {
    float *part = a.parts + ((int64_t(b) * a.n_q_heads + hk * gqa + hh) * a.n_splits + split) * B_PART;
    part[tid] = acc[hh];
    if (tid == 0) {
      part[D] = m_s[hh];
      part[D + 1] = l_s[hh];
    }
  }
}

__global__ void __launch_bounds__(128) bf16_merge_kernel(Bf16Args a) {
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_lens[b];
  float *o = a.out + (int64_t(b) * a.n_q_heads + hq) * D;
  if (L < 1 || L > a.max_seq_len) {
    o[tid] = 0.f;
    return;
  }
  const int pages = (L + PAGE - 1) / PAGE;
  const int used = (pages + a.pages_per_split - 1) / a.pages_per_split;
  const float *parts = a.parts + (int64_t(b) * a.n_q_heads + hq) * a.n_splits * B_PART;
  float m = -INFINITY;
  for (int s = 0; s < used; ++s) m = fmaxf(m, parts[s * B_PART + D]);
  float l = 0.f, acc = 0.f;
  for (int s = 0; s < used; ++s) {
    const float ms = parts[s * B_PART + D];
    const float w = (ms == -INFINITY) ? 0.f : expf(ms - m);
    l = fmaf(w, parts[s * B_PART + D + 1], l);
    acc = fmaf(w, parts[s * B_PART + tid], acc);
  }
  o[tid] = acc / l;
}

hipError_t launch_decode_bf16(const uint16_t *q, const uint16_t *kv, int64_t n_pages,
                              const int32_t *pt, int pt_stride, const int32_t *seq_lens, int batch,
                              int max_seq_len, int n_q_heads, int n_kv_heads, float sm_scale,
                              float *out, uint32_t *status, void *ws, hipStream_t s) {
  const SplitPlan p = plan_bf16_splits(batch, n_kv_heads, max_seq_len);
  Bf16Args a;
  a.q = q;
  a.kv = kv;
  a.n_pages = n_pages;
  a.pt = pt;
  a.pt_stride = pt_stride;
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.pages_per_split = p.pages_per_split;
  a.n_splits = p.n_splits;
  a.sm_scale = sm_scale;
  a.out = out;
  a.status = status;
  a.parts = static_cast<float *>(ws);
  hipLaunchKernelGGL(bf16_split_kernel, dim3(p.n_splits, n_kv_heads, batch), dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bf16_merge_kernel, dim3(n_q_heads, batch), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
