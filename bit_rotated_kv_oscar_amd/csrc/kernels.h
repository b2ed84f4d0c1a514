// Host-side launchers of the liboscar kernels (implemented in the .hip files).
// They assume validated arguments; api.cpp validates.
#pragma once

#include <hip/hip_ext.h>

#include "common.h"

namespace oscar {

// A rotation as the kernels take it: one form for the layer (stride 0), or
// one per KV head (head h's forms at forms + h * stride, its clip
// head_clip[h]); clip is then the largest head clip.
constexpr int MAX_HEAD_ROT = OSCAR_MAX_HEAD_ROTATIONS;
struct RotArg {
  const uint8_t *forms;  // device forms (FORM_* offsets)
  float clip;
  int n_heads;           // 0: one rotation for every head
  int64_t stride;        // bytes between heads' forms (0: shared)
  float head_clip[MAX_HEAD_ROT];
};

// Events that the next decode launch records around its split-K attention
// kernel (set by oscar_profile_events; per host thread, cleared once used).
struct KernelEvents {
  hipEvent_t before = nullptr, after = nullptr;
};
KernelEvents &profile_events();

// Takes (and clears) the pending profile events.  Launchers pass them to
// hipExtLaunchKernelGGL, which records them when the kernel itself starts
// and ends.
inline KernelEvents take_profile_events() {
  KernelEvents &ev = profile_events();
  const KernelEvents use = ev;
  ev = KernelEvents{};
  return use;
}

hipError_t launch_prepare_rotation(const double *R, void *forms, hipStream_t s);

hipError_t launch_write_kv(const oscar_layer_cache &c, RotArg rk, RotArg rv,
                           const uint16_t *k_new, const uint16_t *v_new,
                           const int32_t *cu_new, const int32_t *len_before,
                           int batch, int64_t total_tokens, int max_new, hipStream_t s);

hipError_t launch_decode_int2(const oscar_layer_cache &c, RotArg rk, RotArg rv,
                              const uint16_t *q, int n_q_heads,
                              const int32_t *seq_lens, int batch, int max_seq_len,
                              float sm_scale, float *out, void *ws, hipStream_t s);

size_t decode_int2_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len);

// Append one token per request (k_new / v_new [B][Hkv][128] at positions
// len_before[b]) and, when q is non-null, decode with lengths len_before + 1.
// counters: the merge counters (null: inside ws, after the partials)
hipError_t launch_decode_step(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *k_new,
                              const uint16_t *v_new, const int32_t *len_before, const uint16_t *q,
                              int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                              float sm_scale, float *out, void *ws, hipStream_t s,
                              uint32_t *counters = nullptr);

// Decode with the library's own per-GPU scratch array instead of a caller
// workspace (no allocation): at most NOALLOC_MAX_UNITS (request, KV head)
// units and NOALLOC_SCRATCH_BYTES of scratch (counters first, then the
// partials, decode_int2_parts_bytes of them).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
constexpr int NOALLOC_MAX_UNITS = 4096;
size_t decode_int2_parts_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len);
hipError_t launch_decode_int2_noalloc(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q,
                                      int n_q_heads, const int32_t *seq_lens, int batch, int max_seq_len,
                                      float sm_scale, float *out, hipStream_t s);

hipError_t launch_decode_bf16(const uint16_t *q, const uint16_t *kv, int64_t n_pages,
                              const int32_t *pt, int pt_stride, const int32_t *seq_lens,
                              int batch, int max_seq_len, int n_q_heads, int n_kv_heads,
                              float sm_scale, float *out, uint32_t *status, void *ws,
                              hipStream_t s);

size_t decode_bf16_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int max_seq_len);

// Extend attention of the new tokens (rows cu_new[b] .. cu_new[b+1]-1 of q,
// k_new, v_new) over the cached prefix of len_before[b] tokens plus the
// chunk itself (causal); out fp32 [total][Hq][128].
hipError_t launch_extend(const oscar_layer_cache &c, RotArg rk, RotArg rv, const uint16_t *q, int n_q_heads,
                         const uint16_t *k_new, const uint16_t *v_new, const int32_t *cu_new,
                         const int32_t *len_before, int batch, int64_t total_tokens, int max_new,
                         int max_prefix, float sm_scale, float *out, hipStream_t s);

// Calibration moments (device fp64).
// cov[128][128] = (accumulate ? cov : 0) + sum over the n_vec vectors of
// x x^T (not divided); part: calib_outer_part_bytes() of device scratch
size_t calib_outer_part_bytes();
// (vector n: row (n / grp) * rstride + roff + n % grp of x; the defaults
// take the rows in order).
hipError_t launch_calib_outer(const uint16_t *x_bf16, const double *x_f64, int64_t n_vec,
                              double *cov, double *part, hipStream_t s, bool accumulate = false, int grp = 1,
                              int64_t rstride = 1, int64_t roff = 0);
// o[N][Hq][128] (fp64) = causal softmax(q k^T / sqrt(128)) v per query head
hipError_t launch_calib_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  int64_t n_tokens, int n_q_heads, int n_kv_heads,
                                  double *o, hipStream_t s);
// Jacobi eigen-decomposition of the symmetric 128 x 128 matrix a (device,
// overwritten: eigenvalues on its diagonal); vt: device [128][128] out, the
// eigenvectors as rows, unsorted; sweeps: device int out, the sweeps done
// (max_sweeps: stopped before reaching the tolerance)
constexpr int JACOBI_MAX_SWEEPS = 60;
hipError_t launch_jacobi(double *a, double *vt, int *sweeps, int max_sweeps, hipStream_t s);
// y[n][128] = |x[n] R| (fp64), x bf16 [n][128]
hipError_t launch_calib_rotate_abs(const uint16_t *x, int64_t n_vec, const double *R,
                                   double *y, hipStream_t s);
// The k-th and (k+1)-th smallest (0-based; the (k+1)-th is the k-th when k
// is the last) of n non-negative doubles y (device), by radix selection;
// scratch: select_scratch_bytes() of device memory.  Synchronises s.
size_t select_scratch_bytes();
hipError_t select_order_stats(const double *y, int64_t n, int64_t k, void *scratch, hipStream_t s, double *vk,
                              double *vk1);

// Read probe: sums (mod 2^32) the words of n_blocks blocks of block_bytes
// bytes into *sink; block i is slot ids[i] of buf (ids null: slot i), slots
// outside the buf_bytes / block_bytes of buf are skipped.
hipError_t launch_read_probe(const void *buf, int64_t buf_bytes, int64_t n_blocks, int block_bytes,
                             const int32_t *ids, uint32_t *sink, hipStream_t s);

}  // namespace oscar
