// extern "C" entry points of liboscar: argument validation, workspace sizing,
// error reporting, and the host side of calibration.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "calib_host.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;
thread_local oscar::KernelEvents g_events;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char *where) {
  return fail(OSCAR_EHIP, "%s: HIP error %d (%s)", where, int(e), hipGetErrorString(e));
}

// The current device must be gfx950; the answer (an immutable property of
// the device) is cached per device id.
int check_device() {
  static std::atomic<int> cached[64];  // 0 unknown, 1 ok, -1 not gfx950
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(OSCAR_ENODEV, "no HIP device (%s)", hipGetErrorString(e));
  if (dev < 64 && cached[dev].load(std::memory_order_relaxed) == 1) return OSCAR_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cached[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  if (!ok) return fail(OSCAR_ENODEV, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  return OSCAR_OK;
}

bool group_ok(int G) { return G == 32 || G == 64 || G == 128; }

int check_cache(const oscar_layer_cache *c) {
  if (!c) return fail(OSCAR_EINVAL, "cache is NULL");
  if (c->n_kv_heads < 1 || c->n_kv_heads > 256)
    return fail(OSCAR_EINVAL, "n_kv_heads %d outside [1, 256]", c->n_kv_heads);
  if (!group_ok(c->group)) return fail(OSCAR_EUNSUPPORTED, "group %d not in {32, 64, 128}", c->group);
  if (c->code_bits != 0 && c->code_bits != 2 && c->code_bits != 4)
    return fail(OSCAR_EUNSUPPORTED, "code_bits %d not in {0 (= 2), 2, 4}", c->code_bits);
  if (c->n_hist_pages < 0 || c->n_bf16_pages < 1)
    return fail(OSCAR_EINVAL, "page counts must be n_hist_pages >= 0 and n_bf16_pages >= 1");
  if (c->n_hist_pages > (int64_t(1) << 31) - 1 || c->n_bf16_pages > (int64_t(1) << 31) - 1)
    return fail(OSCAR_EINVAL, "page counts must fit int32 page ids");
  if (c->n_hist_pages > 0 && !c->hist) return fail(OSCAR_EINVAL, "hist pool is NULL");
  if (!c->bf16) return fail(OSCAR_EINVAL, "bf16 pool is NULL");
  if (!c->hist_pt || c->hist_pt_stride < 1) return fail(OSCAR_EINVAL, "hist_pt NULL or hist_pt_stride < 1");
  if (!c->bf16_pt) return fail(OSCAR_EINVAL, "bf16_pt is NULL");
  return OSCAR_OK;
}

bool clip_ok(float c) { return std::isfinite(c) && c > 0.f && c <= 65504.f; }

// One rotation for the layer (n_heads 0 or 1), or one per KV head (n_heads =
// hkv, at most OSCAR_MAX_HEAD_ROTATIONS, with a host clip per head).
int check_rot(const oscar_rotation *r, const char *name, int32_t hkv) {
  if (!r || !r->forms) return fail(OSCAR_EINVAL, "%s: rotation or its forms is NULL", name);
  if (r->n_heads > 1) {
    if (r->n_heads != hkv || r->n_heads > OSCAR_MAX_HEAD_ROTATIONS)
      return fail(OSCAR_EINVAL, "%s: n_heads %d must be 0, 1 or n_kv_heads %d (at most %d)", name, r->n_heads, hkv,
                  OSCAR_MAX_HEAD_ROTATIONS);
    if (!r->head_clips) return fail(OSCAR_EINVAL, "%s: head_clips is NULL", name);
    for (int h = 0; h < r->n_heads; ++h)
      if (!clip_ok(r->head_clips[h]))
        return fail(OSCAR_EINVAL, "%s: head_clips[%d] = %g must be finite, > 0 and <= 65504", name, h,
                    double(r->head_clips[h]));
    return OSCAR_OK;
  }
  if (r->n_heads < 0) return fail(OSCAR_EINVAL, "%s: n_heads %d < 0", name, r->n_heads);
  if (!clip_ok(r->clip))
    return fail(OSCAR_EINVAL, "%s: clip %g must be finite, > 0 and <= 65504", name, double(r->clip));
  return OSCAR_OK;
}

oscar::RotArg rot_arg(const oscar_rotation *r) {
  oscar::RotArg a{};
  a.forms = static_cast<const uint8_t *>(r->forms);
  a.clip = r->clip;
  if (r->n_heads > 1) {
    a.n_heads = r->n_heads;
    a.stride = int64_t(oscar::FORM_BYTES);
    a.clip = 0.f;
    for (int h = 0; h < r->n_heads; ++h) {
      a.head_clip[h] = r->head_clips[h];
      a.clip = std::max(a.clip, r->head_clips[h]);  // the largest: bounds for every head
    }
  }
  return a;
}

}  // namespace

namespace oscar {
KernelEvents &profile_events() { return g_events; }
}  // namespace oscar

namespace {

// Sweep limit of the eigen-iteration: JACOBI_MAX_SWEEPS (far more than the
// 6-10 sweeps a 128 x 128 moment matrix takes), or the value of the
// environment variable OSCAR_JACOBI_SWEEPS (1..1000), a diagnostic hook that
// lets a test make the iteration stop early and see the error it reports.
int jacobi_sweep_limit() {
  const char *env = std::getenv("OSCAR_JACOBI_SWEEPS");
  if (env) {
    const int v = std::atoi(env);
    if (v >= 1 && v <= 1000) return v;
  }
  return oscar::JACOBI_MAX_SWEEPS;
}

// Eigenbasis (sorted, signed) of the symmetric 128 x 128 matrix at mat (device,
// destroyed) by the device Jacobi iteration; work: device scratch of
// 128 * 128 doubles + one int.  *converged: whether the iteration met its
// tolerance within the sweep limit.
hipError_t device_eigenbasis(double *mat, double *work, hipStream_t s, std::vector<double> &U, bool *converged) {
  const int D = oscar::D;
  int *sweeps = reinterpret_cast<int *>(work + D * D);
  const int limit = jacobi_sweep_limit();
  hipError_t e = oscar::launch_jacobi(mat, work, sweeps, limit, s);
  std::vector<double> VT(D * D), V(D * D), A(D * D), w(D);
  int n_sweeps = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(VT.data(), work, VT.size() * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(A.data(), mat, A.size() * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&n_sweeps, sweeps, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  *converged = n_sweeps < limit;
  for (int i = 0; i < D; ++i) {
    w[i] = A[size_t(i) * D + i];
    for (int j = 0; j < D; ++j) V[size_t(i) * D + j] = VT[size_t(j) * D + i];
  }
  oscar::sorted_basis(V, w, D, U);
  return hipSuccess;
}

// The p quantile (linear interpolation between order statistics, type 7) of
// n non-negative doubles y on the device: the two order statistics by radix
// selection (host memory independent of n), the interpolation as numpy's.
hipError_t device_quantile(const double *y, int64_t n, double p, void *scratch, hipStream_t s, double *q) {
  const double h = double(n - 1) * p;
  int64_t lo = int64_t(std::floor(h));
  if (lo > n - 1) lo = n - 1;
  double a = 0.0, b = 0.0;
  hipError_t e = oscar::select_order_stats(y, n, lo, scratch, s, &a, &b);
  if (e != hipSuccess) return e;
  if (lo >= n - 1) {
    *q = a;
    return hipSuccess;
  }
  const double t = h - double(lo);
  *q = t >= 0.5 ? b - (b - a) * (1.0 - t) : a + (b - a) * t;
  return hipSuccess;
}

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct CalibLayout {
  size_t cov, o, rd, y, part, sel, total;
};
CalibLayout calib_layout(int64_t n_tokens, int32_t hq, int32_t hkv) {
  const size_t D = oscar::D;
  CalibLayout l;
  l.cov = 0;
  l.o = l.cov + al256(2 * D * D * sizeof(double));
  l.rd = l.o + al256(size_t(n_tokens) * hq * D * sizeof(double));
  l.y = l.rd + al256(D * D * sizeof(double));
  l.part = l.y + al256(size_t(n_tokens) * hkv * D * sizeof(double));
  const size_t part = oscar::calib_outer_part_bytes() > D * D * sizeof(double) + 256
                          ? oscar::calib_outer_part_bytes() : D * D * sizeof(double) + 256;
  l.sel = l.part + al256(part);
  l.total = l.sel + al256(oscar::select_scratch_bytes());
  return l;
}

struct AccumLayout {
  size_t o, part, total;
};
AccumLayout accum_layout(int64_t n_tokens, int32_t hq) {
  AccumLayout l;
  l.o = 0;
  l.part = al256(size_t(n_tokens) * hq * oscar::D * sizeof(double));
  l.total = l.part + al256(oscar::calib_outer_part_bytes());
  return l;
}

struct RotationsLayout {
  size_t mat, work, total;
};
RotationsLayout rotations_layout() {
  const size_t D = oscar::D;
  RotationsLayout l;
  l.mat = 0;
  l.work = al256(2 * D * D * sizeof(double));
  l.total = l.work + al256(D * D * sizeof(double) + 256);
  return l;
}

struct ClipLayout {
  size_t rd, y, sel, total;
};
ClipLayout clip_layout(int64_t n_vec) {
  const size_t D = oscar::D;
  ClipLayout l;
  l.rd = 0;
  l.y = al256(D * D * sizeof(double));
  l.sel = l.y + al256(size_t(n_vec) * D * sizeof(double));
  l.total = l.sel + al256(oscar::select_scratch_bytes());
  return l;
}

}  // namespace

extern "C" {

int oscar_profile_events(void *before, void *after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(OSCAR_EINVAL, "profile events: give both events or neither");
  g_events.before = static_cast<hipEvent_t>(before);
  g_events.after = static_cast<hipEvent_t>(after);
  return OSCAR_OK;
}

int oscar_read_probe(const void *buf, int64_t buf_bytes, int64_t n_blocks, int32_t block_bytes, const int32_t *ids,
                     uint32_t *sink, oscar_stream_t stream) {
  if (!buf || !sink) return fail(OSCAR_EINVAL, "read_probe: buf or sink is NULL");
  if (block_bytes < 16 || block_bytes > 4096 || block_bytes % 16)
    return fail(OSCAR_EINVAL, "read_probe: block_bytes %d not a multiple of 16 in [16, 4096]", block_bytes);
  if (n_blocks < 1 || buf_bytes < block_bytes) return fail(OSCAR_EINVAL, "read_probe: no blocks to read");
  if (!ids && n_blocks > buf_bytes / block_bytes)
    return fail(OSCAR_EINVAL, "read_probe: %lld blocks of %d bytes exceed the %lld-byte buffer", (long long)n_blocks,
                block_bytes, (long long)buf_bytes);
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_read_probe(buf, buf_bytes, n_blocks, block_bytes, ids, sink,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read_probe");
  return OSCAR_OK;
}

const char *oscar_last_error(void) { return g_err.c_str(); }

const char *oscar_version(void) { return "oscar-gfx950 0.1"; }

size_t oscar_hist_block_bytes(int32_t group) {
  return group_ok(group) ? size_t(oscar::hist_block_bytes(group)) : 0;
}

size_t oscar_hist_block_bytes_bits(int32_t group, int32_t code_bits) {
  if (!group_ok(group) || (code_bits != 2 && code_bits != 4)) return 0;
  return size_t(oscar::hist_block_bytes(group, code_bits));
}

size_t oscar_rotation_bytes(void) { return oscar::FORM_BYTES; }

int oscar_prepare_rotation(const double *R, void *forms, oscar_stream_t stream) {
  if (!R || !forms) return fail(OSCAR_EINVAL, "R or forms is NULL");
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_prepare_rotation(R, forms, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prepare_rotation");
  return OSCAR_OK;
}

int oscar_write_kv(const oscar_layer_cache *cache, const oscar_rotation *rot_k,
                   const oscar_rotation *rot_v, const uint16_t *k_new, const uint16_t *v_new,
                   const int32_t *cu_new, const int32_t *len_before, int32_t batch,
                   int64_t total_tokens, int32_t max_new, oscar_stream_t stream) {
  if (int rc = check_cache(cache)) return rc;
  if (int rc = check_rot(rot_k, "rot_k", cache->n_kv_heads)) return rc;
  if (int rc = check_rot(rot_v, "rot_v", cache->n_kv_heads)) return rc;
  if (batch < 1 || batch > 65535) return fail(OSCAR_EINVAL, "batch %d outside [1, 65535]", batch);
  if (total_tokens < 0 || max_new < 0) return fail(OSCAR_EINVAL, "negative token counts");
  if (int64_t(max_new) > total_tokens) return fail(OSCAR_EINVAL, "max_new %d > total_tokens %lld", max_new, (long long)total_tokens);
  if (max_new > (1 << 24)) return fail(OSCAR_EINVAL, "max_new %d too large", max_new);
  if (!cu_new || !len_before) return fail(OSCAR_EINVAL, "cu_new or len_before is NULL");
  if (total_tokens > 0 && (!k_new || !v_new)) return fail(OSCAR_EINVAL, "k_new or v_new is NULL");
  if (max_new == 0) return OSCAR_OK;
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_write_kv(*cache, rot_arg(rot_k), rot_arg(rot_v), k_new, v_new, cu_new,
                                        len_before, batch, total_tokens, max_new,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "write_kv");
  return OSCAR_OK;
}

size_t oscar_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t max_seq_len) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || max_seq_len < 1) return 0;
  return oscar::decode_int2_ws_bytes(batch, n_q_heads, n_kv_heads, max_seq_len);
}

static int check_heads(int32_t hq, int32_t hkv) {
  if (hq < 1 || hkv < 1) return fail(OSCAR_EINVAL, "head counts must be >= 1");
  if (hq % hkv) return fail(OSCAR_EUNSUPPORTED, "n_q_heads %d not a multiple of n_kv_heads %d", hq, hkv);
  const int g = hq / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(OSCAR_EUNSUPPORTED, "GQA group %d not in {1, 2, 4, 8}", g);
  return OSCAR_OK;
}

int oscar_decode_attn(const oscar_layer_cache *cache, const oscar_rotation *rot_k,
                      const oscar_rotation *rot_v, const uint16_t *q, int32_t n_q_heads,
                      const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                      float *out, void *workspace, size_t workspace_bytes, oscar_stream_t stream) {
  if (int rc = check_cache(cache)) return rc;
  if (int rc = check_rot(rot_k, "rot_k", cache->n_kv_heads)) return rc;
  if (int rc = check_rot(rot_v, "rot_v", cache->n_kv_heads)) return rc;
  if (int rc = check_heads(n_q_heads, cache->n_kv_heads)) return rc;
  if (batch < 1 || batch > 65535) return fail(OSCAR_EINVAL, "batch %d outside [1, 65535]", batch);
  if (max_seq_len < 1) return fail(OSCAR_EINVAL, "max_seq_len %d < 1", max_seq_len);
  if (oscar::n_hist_pages(max_seq_len) > cache->hist_pt_stride)
    return fail(OSCAR_EINVAL, "max_seq_len %d needs %d history pages, hist_pt_stride is %d", max_seq_len,
                oscar::n_hist_pages(max_seq_len), cache->hist_pt_stride);
  if (!q || !seq_lens || !out) return fail(OSCAR_EINVAL, "q, seq_lens or out is NULL");
  if (!std::isfinite(sm_scale) || sm_scale <= 0.f) return fail(OSCAR_EINVAL, "sm_scale must be finite and > 0");
  const size_t need = oscar::decode_int2_ws_bytes(batch, n_q_heads, cache->n_kv_heads, max_seq_len);
  if (!workspace || workspace_bytes < need)
    return fail(OSCAR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_decode_int2(*cache, rot_arg(rot_k), rot_arg(rot_v), q, n_q_heads, seq_lens,
                                           batch, max_seq_len, sm_scale, out, workspace,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode_attn");
  return OSCAR_OK;
}

size_t oscar_decode_noalloc_max_bytes(void) { return oscar::NOALLOC_SCRATCH_BYTES; }

int oscar_decode_attn_noalloc(const oscar_layer_cache *cache, const oscar_rotation *rot_k,
                              const oscar_rotation *rot_v, const uint16_t *q, int32_t n_q_heads,
                              const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                              float *out, oscar_stream_t stream) {
  if (int rc = check_cache(cache)) return rc;
  if (int rc = check_rot(rot_k, "rot_k", cache->n_kv_heads)) return rc;
  if (int rc = check_rot(rot_v, "rot_v", cache->n_kv_heads)) return rc;
  if (int rc = check_heads(n_q_heads, cache->n_kv_heads)) return rc;
  if (batch < 1 || batch > 65535) return fail(OSCAR_EINVAL, "batch %d outside [1, 65535]", batch);
  if (max_seq_len < 1) return fail(OSCAR_EINVAL, "max_seq_len %d < 1", max_seq_len);
  if (oscar::n_hist_pages(max_seq_len) > cache->hist_pt_stride)
    return fail(OSCAR_EINVAL, "max_seq_len %d needs %d history pages, hist_pt_stride is %d", max_seq_len,
                oscar::n_hist_pages(max_seq_len), cache->hist_pt_stride);
  if (!q || !seq_lens || !out) return fail(OSCAR_EINVAL, "q, seq_lens or out is NULL");
  if (!std::isfinite(sm_scale) || sm_scale <= 0.f) return fail(OSCAR_EINVAL, "sm_scale must be finite and > 0");
  const int64_t units = int64_t(batch) * cache->n_kv_heads;
  const size_t parts = oscar::decode_int2_parts_bytes(batch, n_q_heads, cache->n_kv_heads, max_seq_len);
  const size_t room = oscar::NOALLOC_SCRATCH_BYTES -
                      size_t(oscar::NOALLOC_MAX_UNITS) * 64 * sizeof(uint32_t);
  if (units > oscar::NOALLOC_MAX_UNITS || parts > room)
    return fail(OSCAR_EWORKSPACE,
                "decode_attn_noalloc: %lld (request, KV head) units and %zu bytes of partials exceed the library's "
                "scratch (%d units, %zu bytes); use oscar_decode_attn with a workspace",
                (long long)units, parts, oscar::NOALLOC_MAX_UNITS, room);
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_decode_int2_noalloc(*cache, rot_arg(rot_k), rot_arg(rot_v), q, n_q_heads, seq_lens,
                                                   batch, max_seq_len, sm_scale, out,
                                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode_attn_noalloc");
  return OSCAR_OK;
}

int oscar_decode_step(const oscar_layer_cache *cache, const oscar_rotation *rot_k, const oscar_rotation *rot_v,
                      const uint16_t *k_new, const uint16_t *v_new, const int32_t *len_before,
                      const uint16_t *q, int32_t n_q_heads, int32_t batch, int32_t max_seq_len,
                      float sm_scale, float *out, void *workspace, size_t workspace_bytes,
                      oscar_stream_t stream) {
  if (int rc = check_cache(cache)) return rc;
  if (int rc = check_rot(rot_k, "rot_k", cache->n_kv_heads)) return rc;
  if (int rc = check_rot(rot_v, "rot_v", cache->n_kv_heads)) return rc;
  if (int rc = check_heads(n_q_heads, cache->n_kv_heads)) return rc;
  if (batch < 1 || batch > 65535) return fail(OSCAR_EINVAL, "batch %d outside [1, 65535]", batch);
  if (max_seq_len < 1) return fail(OSCAR_EINVAL, "max_seq_len %d < 1", max_seq_len);
  if (oscar::n_hist_pages(max_seq_len) > cache->hist_pt_stride)
    return fail(OSCAR_EINVAL, "max_seq_len %d needs %d history pages, hist_pt_stride is %d", max_seq_len,
                oscar::n_hist_pages(max_seq_len), cache->hist_pt_stride);
  if (!k_new || !v_new || !len_before || !q || !out)
    return fail(OSCAR_EINVAL, "k_new, v_new, len_before, q or out is NULL");
  if (!std::isfinite(sm_scale) || sm_scale <= 0.f) return fail(OSCAR_EINVAL, "sm_scale must be finite and > 0");
  const size_t need = oscar::decode_int2_ws_bytes(batch, n_q_heads, cache->n_kv_heads, max_seq_len);
  if (!workspace || workspace_bytes < need)
    return fail(OSCAR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_decode_step(*cache, rot_arg(rot_k), rot_arg(rot_v), k_new, v_new, len_before, q,
                                           n_q_heads, nullptr, batch, max_seq_len, sm_scale, out, workspace,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode_step");
  return OSCAR_OK;
}

int oscar_extend_attn(const oscar_layer_cache *cache, const oscar_rotation *rot_k, const oscar_rotation *rot_v,
                      const uint16_t *q, int32_t n_q_heads, const uint16_t *k_new, const uint16_t *v_new,
                      const int32_t *cu_new, const int32_t *len_before, int32_t batch, int64_t total_tokens,
                      int32_t max_new, int32_t max_prefix, float sm_scale, float *out, oscar_stream_t stream) {
  if (int rc = check_cache(cache)) return rc;
  if (int rc = check_rot(rot_k, "rot_k", cache->n_kv_heads)) return rc;
  if (int rc = check_rot(rot_v, "rot_v", cache->n_kv_heads)) return rc;
  if (int rc = check_heads(n_q_heads, cache->n_kv_heads)) return rc;
  if (batch < 1 || batch > 65535) return fail(OSCAR_EINVAL, "batch %d outside [1, 65535]", batch);
  if (total_tokens < 0 || max_new < 0 || max_prefix < 0) return fail(OSCAR_EINVAL, "negative token counts");
  if (int64_t(max_new) > total_tokens) return fail(OSCAR_EINVAL, "max_new %d > total_tokens %lld", max_new, (long long)total_tokens);
  if (max_new > (1 << 24)) return fail(OSCAR_EINVAL, "max_new %d too large", max_new);
  if (oscar::n_hist_pages(max_prefix) > cache->hist_pt_stride)
    return fail(OSCAR_EINVAL, "max_prefix %d needs %d history pages, hist_pt_stride is %d", max_prefix,
                oscar::n_hist_pages(max_prefix), cache->hist_pt_stride);
  if (!cu_new || !len_before) return fail(OSCAR_EINVAL, "cu_new or len_before is NULL");
  if (total_tokens > 0 && (!q || !k_new || !v_new || !out)) return fail(OSCAR_EINVAL, "q, k_new, v_new or out is NULL");
  if (!std::isfinite(sm_scale) || sm_scale <= 0.f) return fail(OSCAR_EINVAL, "sm_scale must be finite and > 0");
  if (max_new == 0) return OSCAR_OK;
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_extend(*cache, rot_arg(rot_k), rot_arg(rot_v), q, n_q_heads, k_new, v_new, cu_new,
                                      len_before, batch, total_tokens, max_new, max_prefix, sm_scale, out,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "extend_attn");
  return OSCAR_OK;
}

size_t oscar_bf16_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t max_seq_len) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || max_seq_len < 1) return 0;
  return oscar::decode_bf16_ws_bytes(batch, n_q_heads, n_kv_heads, max_seq_len);
}

int oscar_bf16_paged_decode(const uint16_t *q, const uint16_t *kv_pages, int64_t n_pages,
                            const int32_t *pt, int32_t pt_stride, const int32_t *seq_lens,
                            int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                            int32_t n_kv_heads, float sm_scale, float *out, uint32_t *status,
                            void *workspace, size_t workspace_bytes, oscar_stream_t stream) {
  if (int rc = check_heads(n_q_heads, n_kv_heads)) return rc;
  if (!q || !kv_pages || !pt || !seq_lens || !out) return fail(OSCAR_EINVAL, "NULL pointer argument");
  if (n_pages < 1 || n_pages > (int64_t(1) << 31) - 1) return fail(OSCAR_EINVAL, "n_pages %lld invalid", (long long)n_pages);
  if (batch < 1 || batch > 65535) return fail(OSCAR_EINVAL, "batch %d outside [1, 65535]", batch);
  if (max_seq_len < 1) return fail(OSCAR_EINVAL, "max_seq_len %d < 1", max_seq_len);
  if (pt_stride < (max_seq_len + OSCAR_PAGE - 1) / OSCAR_PAGE)
    return fail(OSCAR_EINVAL, "pt_stride %d too small for max_seq_len %d", pt_stride, max_seq_len);
  if (!std::isfinite(sm_scale) || sm_scale <= 0.f) return fail(OSCAR_EINVAL, "sm_scale must be finite and > 0");
  const size_t need = oscar::decode_bf16_ws_bytes(batch, n_q_heads, n_kv_heads, max_seq_len);
  if (!workspace || workspace_bytes < need)
    return fail(OSCAR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipError_t e = oscar::launch_decode_bf16(q, kv_pages, n_pages, pt, pt_stride, seq_lens, batch, max_seq_len,
                                           n_q_heads, n_kv_heads, sm_scale, out, status, workspace,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bf16_paged_decode");
  return OSCAR_OK;
}

// ---------------------------------------------------------------- calibration
// Every calibration call works in a caller workspace (no allocation in the
// library): the layouts below, each region 256-byte aligned.

size_t oscar_calibrate_workspace_bytes(int64_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads) {
  if (n_tokens < 1 || n_q_heads < 1 || n_kv_heads < 1) return 0;
  return calib_layout(n_tokens, n_q_heads, n_kv_heads).total;
}

size_t oscar_calib_accumulate_workspace_bytes(int64_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads) {
  if (n_tokens < 1 || n_q_heads < 1 || n_kv_heads < 1) return 0;
  return accum_layout(n_tokens, n_q_heads).total;
}

size_t oscar_calib_rotations_workspace_bytes(void) { return rotations_layout().total; }

size_t oscar_clip_threshold_workspace_bytes(int64_t n_vec) {
  if (n_vec < 1) return 0;
  return clip_layout(n_vec).total;
}

int oscar_calibrate_rotation(const uint16_t *q_cal, const uint16_t *k_cal, const uint16_t *v_cal,
                             int64_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                             double clip_quantile, double *R_K, double *R_V, float *clip_K,
                             float *clip_V, void *workspace, size_t workspace_bytes, oscar_stream_t stream) {
  if (!q_cal || !k_cal || !v_cal) return fail(OSCAR_EINVAL, "calibration inputs NULL");
  if (!R_K || !R_V || !clip_K || !clip_V) return fail(OSCAR_EINVAL, "outputs NULL");
  if (n_tokens < 1 || n_tokens > 65536) return fail(OSCAR_EINVAL, "n_tokens %lld outside [1, 65536]", (long long)n_tokens);
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || n_q_heads > 256)
    return fail(OSCAR_EUNSUPPORTED, "head counts %d/%d unsupported", n_q_heads, n_kv_heads);
  if (!(clip_quantile > 0.0 && clip_quantile <= 1.0)) return fail(OSCAR_EINVAL, "clip_quantile must be in (0, 1]");
  const CalibLayout lay = calib_layout(n_tokens, n_q_heads, n_kv_heads);
  if (!workspace || workspace_bytes < lay.total)
    return fail(OSCAR_EWORKSPACE, "calibrate: workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = oscar::D;
  char *w = static_cast<char *>(workspace);
  double *cov = reinterpret_cast<double *>(w + lay.cov), *o = reinterpret_cast<double *>(w + lay.o);
  double *Rd = reinterpret_cast<double *>(w + lay.rd), *y = reinterpret_cast<double *>(w + lay.y);
  double *part = reinterpret_cast<double *>(w + lay.part);
  void *sel = w + lay.sel;
  const int64_t nq = n_tokens * n_q_heads, nkv = n_tokens * n_kv_heads;
  hipError_t e;
#define CHECK_HIP(expr, where)             \
  do {                                     \
    e = (expr);                            \
    if (e != hipSuccess) return hip_fail(e, where); \
  } while (0)
  CHECK_HIP(oscar::launch_calib_outer(q_cal, nullptr, nq, cov, part, s), "calib C_Q");
  CHECK_HIP(oscar::launch_calib_attention(q_cal, k_cal, v_cal, n_tokens, n_q_heads, n_kv_heads, o, s), "calib attention");
  CHECK_HIP(oscar::launch_calib_outer(nullptr, o, nq, cov + D * D, part, s), "calib C_S");
  // eigenbases of the sums (the 1/(N Hq) scale changes no eigenvector);
  // the Jacobi work area reuses the first partials of the moment step
  std::vector<double> U, Rk, Rv;
  bool conv = true;
  CHECK_HIP(device_eigenbasis(cov, part, s, U, &conv), "eigenbasis C_Q");
  if (!conv) return fail(OSCAR_EINVAL, "calibrate: the eigen-iteration of C_Q did not converge in %d sweeps", jacobi_sweep_limit());
  oscar::compose_rotation(U, Rk);
  CHECK_HIP(device_eigenbasis(cov + D * D, part, s, U, &conv), "eigenbasis C_S");
  if (!conv) return fail(OSCAR_EINVAL, "calibrate: the eigen-iteration of C_S did not converge in %d sweeps", jacobi_sweep_limit());
  oscar::compose_rotation(U, Rv);
  double clips[2];
  const uint16_t *xs[2] = {k_cal, v_cal};
  const std::vector<double> *Rs[2] = {&Rk, &Rv};
  for (int t = 0; t < 2; ++t) {
    CHECK_HIP(hipMemcpyAsync(Rd, Rs[t]->data(), D * D * sizeof(double), hipMemcpyHostToDevice, s), "copy R");
    CHECK_HIP(oscar::launch_calib_rotate_abs(xs[t], nkv, Rd, y, s), "calib |x R|");
    CHECK_HIP(device_quantile(y, nkv * D, clip_quantile, sel, s, &clips[t]), "clip quantile");
  }
#undef CHECK_HIP
  std::memcpy(R_K, Rk.data(), D * D * sizeof(double));
  std::memcpy(R_V, Rv.data(), D * D * sizeof(double));
  *clip_K = float(clips[0]);
  *clip_V = float(clips[1]);
  return OSCAR_OK;
}

int oscar_calib_accumulate(const uint16_t *q_cal, const uint16_t *k_cal, const uint16_t *v_cal,
                           int64_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads, double *sums,
                           void *workspace, size_t workspace_bytes, oscar_stream_t stream) {
  if (!q_cal || !k_cal || !v_cal || !sums) return fail(OSCAR_EINVAL, "calib_accumulate: NULL argument");
  if (n_tokens < 1 || n_tokens > 65536) return fail(OSCAR_EINVAL, "n_tokens %lld outside [1, 65536]", (long long)n_tokens);
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || n_q_heads > 256)
    return fail(OSCAR_EUNSUPPORTED, "head counts %d/%d unsupported", n_q_heads, n_kv_heads);
  const AccumLayout lay = accum_layout(n_tokens, n_q_heads);
  if (!workspace || workspace_bytes < lay.total)
    return fail(OSCAR_EWORKSPACE, "calib_accumulate: workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = oscar::D;
  const int64_t nq = n_tokens * n_q_heads;
  char *w = static_cast<char *>(workspace);
  double *o = reinterpret_cast<double *>(w + lay.o), *part = reinterpret_cast<double *>(w + lay.part);
  hipError_t e = oscar::launch_calib_outer(q_cal, nullptr, nq, sums, part, s, true);
  if (e == hipSuccess) e = oscar::launch_calib_attention(q_cal, k_cal, v_cal, n_tokens, n_q_heads, n_kv_heads, o, s);
  if (e == hipSuccess) e = oscar::launch_calib_outer(nullptr, o, nq, sums + D * D, part, s, true);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "calib_accumulate");
  return OSCAR_OK;
}

int oscar_calib_accumulate_heads(const uint16_t *q_cal, const uint16_t *k_cal, const uint16_t *v_cal,
                                 int64_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads, double *sums,
                                 void *workspace, size_t workspace_bytes, oscar_stream_t stream) {
  if (!q_cal || !k_cal || !v_cal || !sums) return fail(OSCAR_EINVAL, "calib_accumulate_heads: NULL argument");
  if (n_tokens < 1 || n_tokens > 65536) return fail(OSCAR_EINVAL, "n_tokens %lld outside [1, 65536]", (long long)n_tokens);
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || n_q_heads > 256)
    return fail(OSCAR_EUNSUPPORTED, "head counts %d/%d unsupported", n_q_heads, n_kv_heads);
  const AccumLayout lay = accum_layout(n_tokens, n_q_heads);
  if (!workspace || workspace_bytes < lay.total)
    return fail(OSCAR_EWORKSPACE, "calib_accumulate_heads: workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = oscar::D;
  const int gqa = n_q_heads / n_kv_heads;
  const int64_t nv = n_tokens * gqa;  // vectors per KV head
  char *w = static_cast<char *>(workspace);
  double *o = reinterpret_cast<double *>(w + lay.o), *part = reinterpret_cast<double *>(w + lay.part);
  // the attention outputs of every query head once, then per KV head the
  // rows of its query heads (gqa consecutive rows in each token's Hq rows)
  hipError_t e = oscar::launch_calib_attention(q_cal, k_cal, v_cal, n_tokens, n_q_heads, n_kv_heads, o, s);
  for (int h = 0; h < n_kv_heads && e == hipSuccess; ++h) {
    double *sh = sums + int64_t(h) * 2 * D * D;
    e = oscar::launch_calib_outer(q_cal, nullptr, nv, sh, part, s, true, gqa, n_q_heads, int64_t(h) * gqa);
    if (e == hipSuccess)
      e = oscar::launch_calib_outer(nullptr, o, nv, sh + D * D, part, s, true, gqa, n_q_heads, int64_t(h) * gqa);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "calib_accumulate_heads");
  return OSCAR_OK;
}

int oscar_calib_rotations(const double *sums, double count, double *R_K, double *R_V, void *workspace,
                          size_t workspace_bytes, oscar_stream_t stream) {
  if (!sums || !R_K || !R_V) return fail(OSCAR_EINVAL, "calib_rotations: NULL argument");
  if (!(count > 0.0) || !std::isfinite(count)) return fail(OSCAR_EINVAL, "count must be positive and finite");
  const RotationsLayout lay = rotations_layout();
  if (!workspace || workspace_bytes < lay.total)
    return fail(OSCAR_EWORKSPACE, "calib_rotations: workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = oscar::D;
  std::vector<double> c(2 * D * D);
  hipError_t e = hipMemcpyAsync(c.data(), sums, c.size() * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "calib_rotations");
  for (double x : c)
    if (!std::isfinite(x / count)) return fail(OSCAR_EINVAL, "calib_rotations: non-finite moments");
  // the caller's sums stay intact: the iteration runs on a copy (the 1/count
  // scale changes no eigenvector)
  char *w = static_cast<char *>(workspace);
  double *mat = reinterpret_cast<double *>(w + lay.mat), *work = reinterpret_cast<double *>(w + lay.work);
  std::vector<double> U, Rk, Rv;
  bool conv_k = true, conv_v = true;
  e = hipMemcpyAsync(mat, sums, 2 * D * D * sizeof(double), hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = device_eigenbasis(mat, work, s, U, &conv_k);
  if (e == hipSuccess) oscar::compose_rotation(U, Rk);
  if (e == hipSuccess) e = device_eigenbasis(mat + D * D, work, s, U, &conv_v);
  if (e == hipSuccess) oscar::compose_rotation(U, Rv);
  if (e != hipSuccess) return hip_fail(e, "calib_rotations");
  if (!conv_k || !conv_v)
    return fail(OSCAR_EINVAL, "calib_rotations: the eigen-iteration of %s did not converge in %d sweeps",
                conv_k ? "C_S" : "C_Q", jacobi_sweep_limit());
  std::memcpy(R_K, Rk.data(), D * D * sizeof(double));
  std::memcpy(R_V, Rv.data(), D * D * sizeof(double));
  return OSCAR_OK;
}

int oscar_clip_threshold(const uint16_t *x_cal, int64_t n_vec, const double *R, double clip_quantile,
                         float *clip, void *workspace, size_t workspace_bytes, oscar_stream_t stream) {
  if (!x_cal || !R || !clip) return fail(OSCAR_EINVAL, "clip_threshold: NULL argument");
  if (n_vec < 1 || n_vec > (int64_t(1) << 31) - 1)
    return fail(OSCAR_EINVAL, "n_vec %lld outside [1, 2^31 - 1]", (long long)n_vec);
  if (!(clip_quantile > 0.0 && clip_quantile <= 1.0)) return fail(OSCAR_EINVAL, "clip_quantile must be in (0, 1]");
  const ClipLayout lay = clip_layout(n_vec);
  if (!workspace || workspace_bytes < lay.total)
    return fail(OSCAR_EWORKSPACE, "clip_threshold: workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : 0);
  if (int rc = check_device()) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = oscar::D;
  char *w = static_cast<char *>(workspace);
  double *Rd = reinterpret_cast<double *>(w + lay.rd), *y = reinterpret_cast<double *>(w + lay.y);
  double q = 0.0;
  hipError_t e = hipMemcpyAsync(Rd, R, D * D * sizeof(double), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = oscar::launch_calib_rotate_abs(x_cal, n_vec, Rd, y, s);
  if (e == hipSuccess) e = device_quantile(y, n_vec * D, clip_quantile, w + lay.sel, s, &q);
  if (e != hipSuccess) return hip_fail(e, "clip_threshold");
  *clip = float(q);
  return OSCAR_OK;
}

}  // extern "C"
