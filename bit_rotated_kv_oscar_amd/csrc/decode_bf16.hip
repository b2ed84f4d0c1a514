// Plain BF16 paged decode attention: the all-BF16 baseline that OSCAR's
// batch-1 decode speed-up is measured against (arXiv:2605.17757 v2 abstract).
// One kernel: a workgroup of 8 waves per (request, KV head, split); wave w
// takes every 8th page of the split (page ids preloaded 64 at a time, the
// next page's loads issued into a second register set before the current
// page computes).  Scores on the bf16 matrix
// cores, PV on the vector ALUs, fp32 accumulation.  Each workgroup writes an
// unnormalised partial per query head.  The split plan and the merge are
// those of the INT2 decode: when every (request, KV head) fits one round of
// one workgroup per CU, its pages are spread over as many splits as that
// round holds and the last workgroup of each unit to finish merges the
// partials inside the kernel (agent-scope stores and loads, a counter per
// unit); otherwise splits of 64 pages and a merge kernel (one block per
// (request, KV head)) that LSE-combines them and normalises.
#include "attn_common.h"

namespace oscar {

constexpr int BW = 8;  // waves per workgroup

SplitPlan plan_bf16_splits(int batch, int n_kv_heads, int max_seq_len) {
  // as for the INT2 decode: one round of workgroups, one per CU (the
  // kernel's registers hold one 8-wave workgroup per CU), when every unit
  // gets at least one; else splits of 8 pages per wave
  const int pages = (max_seq_len + PAGE - 1) / PAGE;
  const int64_t units = int64_t(batch) * n_kv_heads;
  const int64_t slots = device_cus();
  SplitPlan p;
  int64_t pps;
  if (units <= slots) {
    const int64_t per_unit = slots / units;
    pps = (pages + per_unit - 1) / per_unit;
    p.fused = true;
  } else {
    pps = 8 * BW;
  }
  if (pps < BW) pps = BW;
  const int64_t min_pps = (pages + MAX_MERGE_SPLITS - 2) / (MAX_MERGE_SPLITS - 1);
  if (pps < min_pps) pps = min_pps;
  p.pages_per_split = int(pps);
  p.n_splits = int((pages + pps - 1) / pps);
  return p;
}

// Partial slots per query head: one per split, and at least the fused
// merge's first register window (loaded without bounds checks).
static int bf16_part_slots(const SplitPlan &p) { return p.n_splits > MERGE_WINDOW ? p.n_splits : MERGE_WINDOW; }

// Workspace: the partials, then one merge counter per (request, KV head)
static size_t count_off(int batch, int n_q_heads, const SplitPlan &p) {
  return (size_t(batch) * n_q_heads * bf16_part_slots(p) * PART_STRIDE * sizeof(float) + 255) & ~size_t(255);
}

size_t decode_bf16_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len) {
  const SplitPlan p = plan_bf16_splits(batch, n_kv_heads, max_seq_len);
  return count_off(batch, n_q_heads, p) + size_t(batch) * n_kv_heads * COUNTER_STRIDE * sizeof(uint32_t);
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
  float *parts;     // [B][Hq][part_slots][PART_STRIDE]
  int part_slots;
  uint32_t *counters;  // [B][Hkv][COUNTER_STRIDE]: word 0 = workgroups done (zero between calls)
};

template <int GQA>
__global__ void __launch_bounds__(1024) bf16_merge_kernel(Bf16Args a) {
  const int hk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;
  const int L = a.seq_lens[b];
  if (L < 1 || L > a.max_seq_len) return;  // output zeroed by the split kernel
  const int pages = (L + PAGE - 1) / PAGE;
  const int used = (pages + a.pages_per_split - 1) / a.pages_per_split;
  const int64_t head_stride = int64_t(a.part_slots) * PART_STRIDE;
  const float *parts0 = a.parts + (int64_t(b) * a.n_q_heads + hk * GQA) * head_stride;
  __shared__ float w_lds[GQA][256];
  __shared__ float lsum[GQA];
  __shared__ float half_o[2][GQA][D];
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
  for (int idx = tid; idx < 2 * GQA * D; idx += 1024) {
    const int hf = idx / (GQA * D), h = (idx / D) % GQA, ch = idx % D;
    const float *ph = parts0 + h * head_stride + ch;
    const int s0 = hf ? used / 2 : 0, s1 = hf ? used : used / 2;
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    int s = s0;
    for (; s + 3 < s1; s += 4) {
      o0 = fmaf(w_lds[h][s], ph[s * PART_STRIDE], o0);
      o1 = fmaf(w_lds[h][s + 1], ph[(s + 1) * PART_STRIDE], o1);
      o2 = fmaf(w_lds[h][s + 2], ph[(s + 2) * PART_STRIDE], o2);
      o3 = fmaf(w_lds[h][s + 3], ph[(s + 3) * PART_STRIDE], o3);
    }
    for (; s < s1; ++s) o0 = fmaf(w_lds[h][s], ph[s * PART_STRIDE], o0);
    half_o[hf][h][ch] = (o0 + o1) + (o2 + o3);
  }
  __syncthreads();
  for (int idx = tid; idx < GQA * D; idx += 1024) {
    const int h = idx / D, ch = idx % D;
    a.out[(int64_t(b) * a.n_q_heads + hk * GQA + h) * D + ch] = (half_o[0][h][ch] + half_o[1][h][ch]) / lsum[h];
  }
}

template <int GQA, bool FUSED>
__global__ void __launch_bounds__(BW * 64) bf16_decode_kernel(Bf16Args a) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int L = a.seq_lens[b];
  __shared__ float lds[BW * GQA * D + 2 * BW * GQA];
  if (L < 1 || L > a.max_seq_len) {
    if (split == 0) {
      if (tid == 0 && hk == 0) flag_status(a.status, OSCAR_STATUS_BAD_LEN);
      for (int e = tid; e < GQA * D; e += BW * 64) a.out[(int64_t(b) * a.n_q_heads + hk * GQA) * D + e] = 0.f;
    }
    return;
  }
  const int pages = (L + PAGE - 1) / PAGE;
  const int used = (pages + a.pages_per_split - 1) / a.pages_per_split;
  if (split >= used) return;
  float *o_lds = lds, *m_lds = lds + BW * GQA * D, *l_lds = m_lds + BW * GQA;
  Bf16Wave<GQA> st;
  st.init(a.q + (int64_t(b) * a.n_q_heads + hk * GQA) * D, a.sm_scale, lane);
  const int j0 = split * a.pages_per_split + wave;
  const int j1 = min(pages, split * a.pages_per_split + a.pages_per_split);
  const int npw = j1 > j0 ? (j1 - j0 + BW - 1) / BW : 0;
  // page ids of pages 64k + lane, loaded per chunk of 64
  const int32_t *pt = a.pt + int64_t(b) * a.pt_stride + j0;
  int my_pid = -1;
  using Loads = typename Bf16Wave<GQA>::Loads;
  auto issue = [&](int i, Loads &ld) -> bool {
    if ((i & 63) == 0) {
      my_pid = (i + lane < npw) ? pt[int64_t(BW) * (i + lane)] : -1;
      // take the wait for this load here, once per 64 pages (see the INT2
      // page loop): later readlanes then wait for nothing
      asm volatile("" : "+v"(my_pid));
    }
    const int pid = __builtin_amdgcn_readlane(my_pid, i & 63);
    if (pid < 0 || pid >= a.n_pages) return false;
    const uint16_t *base = a.kv + (int64_t(pid) * a.n_kv_heads + hk) * 2 * PAGE * D;
    Bf16Wave<GQA>::issue(base, base + PAGE * D, ld, lane);
    return true;
  };
  auto run = [&](const Loads &ld, bool ok, int i) {
    if (!ok) {
      if (lane == 0) flag_status(a.status, OSCAR_STATUS_BAD_PAGE);
      return;
    }
    const int rows = min(PAGE, L - PAGE * (j0 + BW * i));
    st.compute(ld, rows >= PAGE ? 0xFFFFu : ((1u << rows) - 1u), lane);
  };
  // two load buffers used in turn (no copy of in-flight registers)
  Loads ba, bb;
  bool ok_a = npw > 0 ? issue(0, ba) : false, ok_b = false;
  for (int i = 0; i < npw; i += 2) {
    if (i + 1 < npw) ok_b = issue(i + 1, bb);
    run(ba, ok_a, i);
    if (i + 1 >= npw) break;
    if (i + 2 < npw) ok_a = issue(i + 2, ba);
    run(bb, ok_b, i + 1);
  }
  st.finish(o_lds + wave * GQA * D, m_lds + wave * GQA, l_lds + wave * GQA, lane);
  __syncthreads();
  const int64_t head_stride = int64_t(a.part_slots) * PART_STRIDE;
  float *parts0 = a.parts + (int64_t(b) * a.n_q_heads + hk * GQA) * head_stride;
  float *part0 = parts0 + split * PART_STRIDE;
  if constexpr (!FUSED) {
    combine_waves<GQA, BW>(o_lds, m_lds, l_lds, part0, head_stride, tid);
  } else {
    combine_waves<GQA, BW, true>(o_lds, m_lds, l_lds, part0, head_stride, tid);
    // the last workgroup of (b, hk) to finish merges: its partial stores
    // have completed (agent scope) before the counter counts it in; the
    // counter is left at zero for the next call
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (used > 1) {
      __shared__ int last;
      if (tid == 0) {
        uint32_t *cnt = a.counters + COUNTER_STRIDE * (b * a.n_kv_heads + hk);
        const uint32_t done = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = done == uint32_t(used - 1);
        if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (!last) return;
    }
    static_assert(sizeof(MergeWork<GQA>) <= sizeof(lds), "merge work area fits the wave states");
    merge_partials<GQA, BW * 64>(parts0, head_stride, used, a.out + (int64_t(b) * a.n_q_heads + hk * GQA) * D,
                                 tid, *reinterpret_cast<MergeWork<GQA> *>(lds));
  }
}

template <int GQA>
static hipError_t launch_t(const Bf16Args &a, bool fused, int batch, hipStream_t s) {
  const KernelEvents ev = take_profile_events();
  const dim3 grid(a.n_splits, a.n_kv_heads, batch);
  if (fused) {
    hipExtLaunchKernelGGL((bf16_decode_kernel<GQA, true>), grid, dim3(BW * 64), 0, s, ev.before, ev.after, 0, a);
    return hipGetLastError();
  }
  hipExtLaunchKernelGGL((bf16_decode_kernel<GQA, false>), grid, dim3(BW * 64), 0, s, ev.before, ev.after, 0, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bf16_merge_kernel<GQA>), dim3(a.n_kv_heads, batch), dim3(1024), 0, s, a);
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
  a.part_slots = bf16_part_slots(p);
  a.counters = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + count_off(batch, n_q_heads, p));
  switch (n_q_heads / n_kv_heads) {
    case 1: return launch_t<1>(a, p.fused, batch, s);
    case 2: return launch_t<2>(a, p.fused, batch, s);
    case 4: return launch_t<4>(a, p.fused, batch, s);
    case 8: return launch_t<8>(a, p.fused, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
