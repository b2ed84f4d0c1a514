// Plain BF16 paged decode attention: the all-BF16 baseline that OSCAR's
// batch-1 decode speed-up is measured against (arXiv:2605.17757 v2 abstract).
// Split-K over pages: one workgroup (4 waves, every 4th page each) per
// (request, KV head, split) writes an unnormalised partial per query head; a
// merge kernel LSE-combines them.  Scores on the bf16 matrix cores, PV on the
// vector ALUs, fp32 accumulation throughout.
#include "attn_common.h"

namespace oscar {

SplitPlan plan_bf16_splits(int batch, int n_kv_heads, int max_seq_len) {
  const int pages = (max_seq_len + PAGE - 1) / PAGE;
  const int64_t total = int64_t(pages) * batch * n_kv_heads;
  int64_t pw = (total + int64_t(WAVES) * 1024 - 1) / (int64_t(WAVES) * 1024);
  if (pw < 2) pw = 2;
  if (pw > 32) pw = 32;
  SplitPlan p;
  p.pages_per_split = int(pw) * WAVES;
  p.n_splits = (pages + p.pages_per_split - 1) / p.pages_per_split;
  return p;
}

size_t decode_bf16_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  const SplitPlan p = plan_bf16_splits(batch, n_kv_heads, max_seq_len);
  return (size_t(batch) * n_q_heads * p.n_splits * PART_STRIDE * sizeof(float) + 255) & ~size_t(255);
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

template <int GQA>
__global__ void __launch_bounds__(WAVES * 64) bf16_split_kernel(Bf16Args a) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = a.seq_lens[b];
  __shared__ float o_lds[WAVES * GQA * D];
  __shared__ float m_lds[WAVES * GQA], l_lds[WAVES * GQA];
  if (L < 1 || L > a.max_seq_len) {
    if (tid == 0 && split == 0 && hk == 0) flag_status(a.status, OSCAR_STATUS_BAD_LEN);
    return;
  }
  Bf16Wave<GQA> st;
  st.init(a.q + (int64_t(b) * a.n_q_heads + hk * GQA) * D, a.sm_scale, lane);
  const int pages = (L + PAGE - 1) / PAGE;
  const int j0 = split * a.pages_per_split;
  const int j1 = min(pages, j0 + a.pages_per_split);
  for (int j = j0 + wave; j < j1; j += WAVES) {
    const int pid = __builtin_amdgcn_readfirstlane(a.pt[int64_t(b) * a.pt_stride + j]);
    if (pid < 0 || pid >= a.n_pages) {
      if (lane == 0) flag_status(a.status, OSCAR_STATUS_BAD_PAGE);
      continue;
    }
    const int rows = min(PAGE, L - PAGE * j);
    const uint32_t valid = rows >= PAGE ? 0xFFFFu : ((1u << rows) - 1u);
    const uint16_t *base = a.kv + (int64_t(pid) * a.n_kv_heads + hk) * 2 * PAGE * D;
    st.page(base, base + PAGE * D, valid, lane);
  }
  st.finish(o_lds + wave * GQA * D, m_lds + wave * GQA, l_lds + wave * GQA, lane);
  __syncthreads();
  float *part0 = a.parts + ((int64_t(b) * a.n_q_heads + hk * GQA) * a.n_splits + split) * PART_STRIDE;
  combine_waves<GQA>(o_lds, m_lds, l_lds, part0, int64_t(a.n_splits) * PART_STRIDE, tid);
}

__global__ void __launch_bounds__(256) bf16_merge_kernel(Bf16Args a) {
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_lens[b];
  float *o = a.out + (int64_t(b) * a.n_q_heads + hq) * D;
  if (L < 1 || L > a.max_seq_len) {
    if (tid < D) o[tid] = 0.f;
    return;
  }
  const int pages = (L + PAGE - 1) / PAGE;
  const int used = (pages + a.pages_per_split - 1) / a.pages_per_split;
  const float *parts = a.parts + (int64_t(b) * a.n_q_heads + hq) * a.n_splits * PART_STRIDE;
  __shared__ float red[256];
  __shared__ float acc2[2][D];
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
    l = fmaf((ms == -INFINITY) ? 0.f : fast_exp2(ms - mst), parts[s * PART_STRIDE + D + 1], l);
  }
  red[tid] = l;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const float lsum = red[0];
  const int ch = tid & (D - 1), half = tid >> 7;
  float acc = 0.f;
  for (int s = half; s < used; s += 2) {
    const float ms = parts[s * PART_STRIDE + D];
    const float w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - mst);
    acc = fmaf(w, parts[s * PART_STRIDE + ch], acc);
  }
  acc2[half][ch] = acc;
  __syncthreads();
  if (tid < D) o[tid] = (acc2[0][tid] + acc2[1][tid]) / lsum;
}

template <int GQA>
static hipError_t launch_t(const Bf16Args &a, int batch, hipStream_t s) {
  hipLaunchKernelGGL((bf16_split_kernel<GQA>), dim3(a.n_splits, a.n_kv_heads, batch), dim3(WAVES * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bf16_merge_kernel, dim3(a.n_q_heads, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const uint16_t *q, const uint16_t *kv, int64_t n_pages, const int32_t *pt,
                              int pt_stride, const int32_t *seq_lens, int batch, int max_seq_len,
                              int n_q_heads, int n_kv_heads, float sm_scale, float *out, uint32_t *status,
                              void *ws, hipStream_t s) {
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
  switch (n_q_heads / n_kv_heads) {
    case 1: return launch_t<1>(a, batch, s);
    case 2: return launch_t<2>(a, batch, s);
    case 4: return launch_t<4>(a, batch, s);
    case 8: return launch_t<8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
