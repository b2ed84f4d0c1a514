// Rotation forms and the fp64 calibration moments.
//
// Calibration follows the offline phase of OSCAR (gist.science nl/fr
// technical summaries, section 2.2.A; arXiv:2605.17757 v2 abstract): the
// query second moment C_Q and the attention-output second moment C_S, and the
// magnitudes |x R| from which the per-layer clip is taken.  Everything here is
// fp64 so the eigenbases match a double-precision reference to ~1e-14.
#include "kernels.h"

namespace oscar {

// ---------------------------------------------------------------- forms

__global__ void __launch_bounds__(256) prepare_rotation_kernel(const double *__restrict__ R,
                                                               uint8_t *__restrict__ forms) {
  const int e = blockIdx.x * 256 + threadIdx.x;  // e = i*128 + j
  if (e >= D * D) return;
  const int i = e / D, j = e % D;
  const double r = R[e];
  float *R32 = reinterpret_cast<float *>(forms + FORM_R);
  float *RT32 = reinterpret_cast<float *>(forms + FORM_RT);
  __half *hi = reinterpret_cast<__half *>(forms + FORM_RT_HI);
  __half *lo = reinterpret_cast<__half *>(forms + FORM_RT_LO);
  R32[e] = float(r);
  RT32[j * D + i] = float(r);
  const __half h = __float2half_rn(float(r));
  hi[j * D + i] = h;
  lo[j * D + i] = __float2half_rn(float((r - double(__half2float(h))) * 2048.0));
  // three bf16 pieces, each the rounding of what the previous ones leave
  uint16_t *bp = reinterpret_cast<uint16_t *>(forms + FORM_RT_B);
  double rest = r;
  for (int k = 0; k < 3; ++k) {
    uint32_t u = __float_as_uint(float(rest));
    u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
    const uint16_t piece = uint16_t(u >> 16);
    bp[k * D * D + j * D + i] = piece;
    rest -= double(__uint_as_float(uint32_t(piece) << 16));
  }
}

hipError_t launch_prepare_rotation(const double *R, void *forms, hipStream_t s) {
  hipLaunchKernelGGL(prepare_rotation_kernel, dim3(D * D / 256), dim3(256), 0, s, R,
                     static_cast<uint8_t *>(forms));
  return hipGetLastError();
}

// ---------------------------------------------------------------- moments

// cov[i][j] = sum_n x[n][i] x[n][j]; one thread per (i, j), fixed summation
// order (deterministic).  Exactly one of xb (bf16) / xd (fp64) is non-null.
__global__ void __launch_bounds__(256) outer_sum_kernel(const uint16_t *__restrict__ xb,
                                                        const double *__restrict__ xd,
                                                        int64_t n_vec, double *__restrict__ cov) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int i = e / D, j = e % D;
  double acc = 0.0;
  if (xb) {
    for (int64_t n = 0; n < n_vec; ++n) {
      const double a = bf16_to_f32(xb[n * D + i]);
      const double b = bf16_to_f32(xb[n * D + j]);
      acc = fma(a, b, acc);
    }
  } else {
    for (int64_t n = 0; n < n_vec; ++n) acc = fma(xd[n * D + i], xd[n * D + j], acc);
  }
  cov[e] = acc;
}

hipError_t launch_calib_outer(const uint16_t *x_bf16, const double *x_f64, int64_t n_vec,
                              double *cov, hipStream_t s) {
  hipLaunchKernelGGL(outer_sum_kernel, dim3(D * D / 256), dim3(256), 0, s, x_bf16, x_f64, n_vec,
                     cov);
  return hipGetLastError();
}

__device__ inline double block_reduce_max128(double v, double *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int off = 64; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ inline double block_reduce_sum128(double v, double *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int off = 64; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// One block (128 threads) per (query position n, query head h): causal
// softmax attention over keys 0..n in fp64, keys taken 128 at a time with a
// running max / sum.  o[n][h][:] = sum_j p_j v_j.
__global__ void __launch_bounds__(128) calib_attention_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, int n_q_heads, int n_kv_heads, double *__restrict__ o) {
  const int64_t n = blockIdx.x;
  const int h = blockIdx.y;
  const int g = h / (n_q_heads / n_kv_heads);
  const int tid = threadIdx.x;
  __shared__ double qs[D];
  __shared__ double ps[D];
  __shared__ double red[D];
  const double scale = 1.0 / sqrt(double(D));
  qs[tid] = bf16_to_f32(q[(n * n_q_heads + h) * D + tid]) * scale;
  __syncthreads();
  double m = -INFINITY, l = 0.0, acc = 0.0;
  for (int64_t j0 = 0; j0 <= n; j0 += D) {
    const int64_t j = j0 + tid;
    double sc = -INFINITY;
    if (j <= n) {
      const uint16_t *kr = k + (j * n_kv_heads + g) * D;
      double s = 0.0;
      for (int i = 0; i < D; ++i) s = fma(qs[i], double(bf16_to_f32(kr[i])), s);
      sc = s;
    }
    const double mc = block_reduce_max128(sc, red);
    const double mn = fmax(m, mc);
    const double p = (j <= n) ? exp(sc - mn) : 0.0;
    const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mn);
    const double ls = block_reduce_sum128(p, red);
    ps[tid] = p;
    __syncthreads();
    l = l * alpha + ls;
    acc *= alpha;
    const int64_t cnt = (n - j0 + 1 < D) ? (n - j0 + 1) : D;
    for (int t = 0; t < cnt; ++t)
      acc = fma(ps[t], double(bf16_to_f32(v[((j0 + t) * n_kv_heads + g) * D + tid])), acc);
    m = mn;
    __syncthreads();
  }
  o[(n * n_q_heads + h) * D + tid] = acc / l;
}

hipError_t launch_calib_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  int64_t n_tokens, int n_q_heads, int n_kv_heads, double *o,
                                  hipStream_t s) {
  hipLaunchKernelGGL(calib_attention_kernel, dim3(unsigned(n_tokens), n_q_heads), dim3(D), 0, s,
                     q, k, v, n_q_heads, n_kv_heads, o);
  return hipGetLastError();
}

// y[n][j] = |sum_i x[n][i] R[i][j]|, one block per vector.
__global__ void __launch_bounds__(128) rotate_abs_kernel(const uint16_t *__restrict__ x,
                                                         const double *__restrict__ R,
                                                         double *__restrict__ y) {
  const int64_t n = blockIdx.x;
  const int j = threadIdx.x;
  __shared__ double xs[D];
  xs[j] = bf16_to_f32(x[n * D + j]);
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < D; ++i) s = fma(xs[i], R[i * D + j], s);
  y[n * D + j] = fabs(s);
}

hipError_t launch_calib_rotate_abs(const uint16_t *x, int64_t n_vec, const double *R, double *y,
                                   hipStream_t s) {
  hipLaunchKernelGGL(rotate_abs_kernel, dim3(unsigned(n_vec)), dim3(D), 0, s, x, R, y);
  return hipGetLastError();
}

}  // namespace oscar
