// Rotation forms and the fp64 calibration moments.
//
// Calibration follows the offline phase of OSCAR (gist.science nl/fr
// technical summaries, section 2.2.A; arXiv:2605.17757 v2 abstract): the
// query second moment C_Q and the attention-output second moment C_S, and the
// magnitudes |x R| from which the per-layer clip is taken.  Everything here is
// fp64 so the eigenbases match a double-precision reference to ~1e-14.
#include <cstring>

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
}

hipError_t launch_prepare_rotation(const double *R, void *forms, hipStream_t s) {
  hipLaunchKernelGGL(prepare_rotation_kernel, dim3(D * D / 256), dim3(256), 0, s, R,
                     static_cast<uint8_t *>(forms));
  return hipGetLastError();
}

// ---------------------------------------------------------------- moments

// Second moments cov[i][j] = sum_n x[n][i] x[n][j] on the matrix cores, in
// two deterministic steps.  outer_partial_kernel: workgroup w sums rows
// [w rows, (w+1) rows) of x into part[w] with v_mfma_f64_16x16x4_f64 (fp64
// products and sums, four rows per step in a fixed order); wave I owns the
// 16-row block I of cov and all eight column blocks.  outer_reduce_kernel
// adds the partials in workgroup order.  Exactly one of xb (bf16) / xd
// (fp64) is non-null.  Vector n is row (n / grp) * rstride + roff + n % grp
// of x (grp = 1, rstride = 1, roff = 0: the rows in order; per KV head: the
// grp = Hq/Hkv query-head rows of that head in each token's Hq rows).
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int OUTER_WAVES = D / 16;  // one wave per 16-row block
constexpr int OUTER_MAX_PARTS = 256;

struct RowMap {
  int grp;
  int64_t rstride, roff;
  __device__ int64_t row(int64_t n) const { return grp == 1 ? n * rstride + roff : (n / grp) * rstride + roff + n % grp; }
};

__device__ inline double outer_load(const uint16_t *xb, const double *xd, const RowMap &m, int64_t n, int64_t n_end,
                                    int col) {
  if (n >= n_end) return 0.0;
  const int64_t r = m.row(n);
  return xb ? double(bf16_to_f32(xb[r * D + col])) : xd[r * D + col];
}

__global__ void __launch_bounds__(OUTER_WAVES * 64) outer_partial_kernel(const uint16_t *__restrict__ xb,
                                                                       const double *__restrict__ xd,
                                                                       int64_t n_vec, int64_t rows, RowMap map,
                                                                       double *__restrict__ part) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int c = lane & 15, kq = lane >> 4;  // column in a block; row in a step of four
  const int64_t r0 = int64_t(blockIdx.x) * rows;
  const int64_t r1 = min(n_vec, r0 + rows);
  f64x4 acc[D / 16];
#pragma unroll
  for (int jb = 0; jb < D / 16; ++jb) acc[jb] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int64_t n0 = r0; n0 < r1; n0 += 4) {
    const int64_t n = n0 + kq;
    // A: x[n0 + k][16 wave + i] at (i = c, k = kq); B: x[n0 + k][16 jb + j]
    const double a = outer_load(xb, xd, map, n, r1, 16 * wave + c);
    double b[D / 16];
#pragma unroll
    for (int jb = 0; jb < D / 16; ++jb) b[jb] = outer_load(xb, xd, map, n, r1, 16 * jb + c);
#pragma unroll
    for (int jb = 0; jb < D / 16; ++jb) acc[jb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b[jb], acc[jb], 0, 0, 0);
  }
  // the fp64 16x16 result: lane (c, kq), register r holds row kq + 4 r of
  // column c of each tile
  double *P = part + int64_t(blockIdx.x) * D * D;
#pragma unroll
  for (int jb = 0; jb < D / 16; ++jb)
#pragma unroll
    for (int r = 0; r < 4; ++r) P[(16 * wave + kq + 4 * r) * D + 16 * jb + c] = acc[jb][r];
}

__global__ void __launch_bounds__(256) outer_reduce_kernel(const double *__restrict__ part, int n_parts,
                                                           double *__restrict__ cov, bool accumulate) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  double s = 0.0;
  for (int w = 0; w < n_parts; ++w) s += part[int64_t(w) * D * D + e];
  cov[e] = accumulate ? cov[e] + s : s;
}

size_t calib_outer_part_bytes() { return size_t(OUTER_MAX_PARTS) * D * D * sizeof(double); }

hipError_t launch_calib_outer(const uint16_t *x_bf16, const double *x_f64, int64_t n_vec,
                              double *cov, double *part, hipStream_t s, bool accumulate, int grp,
                              int64_t rstride, int64_t roff) {
  // rows per workgroup: a multiple of four, at least 64, at most 256 workgroups
  int64_t rows = (n_vec + OUTER_MAX_PARTS - 1) / OUTER_MAX_PARTS;
  rows = rows < 64 ? 64 : (rows + 3) / 4 * 4;
  const int n_parts = int((n_vec + rows - 1) / rows);
  hipLaunchKernelGGL(outer_partial_kernel, dim3(n_parts), dim3(OUTER_WAVES * 64), 0, s, x_bf16, x_f64, n_vec,
                     rows, RowMap{grp, rstride, roff}, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(outer_reduce_kernel, dim3(D * D / 256), dim3(256), 0, s, part, n_parts, cov, accumulate);
  return hipGetLastError();
}

// Causal attention of the calibration sequence in fp64 on the matrix cores
// (v_mfma_f64_16x16x4_f64).  One wave per (block of 16 query positions,
// query head); key blocks of 16 in order with a running max and sum.  The
// products are taken transposed so that no lane exchange is needed between
// them: S^T = K Q^T (rows keys, columns queries) and O^T += V^T P^T, whose B
// operand for keys 4s .. 4s+3 is register s of P^T in the result layout
// (lane 16 (r mod 4) + c, register r / 4 holds row r, column c).  Lane
// (c, kq) thus holds query c throughout; a query's 16 keys of a block sit in
// its four lanes c, c+16, c+32, c+48 and their four registers.
// o[n][h][:] = sum_j p_j v_j, p = softmax over j <= n of q_n . k_j / sqrt(128).
__device__ inline double lanes4_max_f64(double v) {
  v = fmax(v, __shfl_xor(v, 16));
  return fmax(v, __shfl_xor(v, 32));
}
__device__ inline double lanes4_sum_f64(double v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

__global__ void __launch_bounds__(64) calib_attention_kernel(const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ k,
                                                             const uint16_t *__restrict__ v, int64_t n_tokens,
                                                             int n_q_heads, int n_kv_heads, double *__restrict__ o) {
  const int64_t n0 = int64_t(blockIdx.x) * 16;
  const int h = blockIdx.y;
  const int g = h / (n_q_heads / n_kv_heads);
  const int lane = threadIdx.x;
  const int c = lane & 15, kq = lane >> 4;  // column (query) of the tiles; k row within a step of four
  const double scale = 1.0 / sqrt(double(D));
  // B operand of S^T = K Q^T for channel step t: q[n0 + c][h][4t + kq] / sqrt(128)
  double qb[D / 4];
  {
    const int64_t n = n0 + c;
#pragma unroll
    for (int t = 0; t < D / 4; ++t)
      qb[t] = n < n_tokens ? double(bf16_to_f32(q[(n * n_q_heads + h) * D + 4 * t + kq])) * scale : 0.0;
  }
  f64x4 acc[D / 16];  // O^T tiles: channels 16 ct .. 16 ct + 15 x the 16 queries
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
  double m = -INFINITY, l = 0.0;  // running max / sum of query c
  const int64_t q_last = min(n_tokens, n0 + 16) - 1;
  for (int64_t j0 = 0; j0 <= q_last; j0 += 16) {
    // S^T: A = k[j0 + c] (key c of the block), channels 4t + kq
    f64x4 st = {0.0, 0.0, 0.0, 0.0};
    {
      const int64_t j = j0 + c;
      const uint16_t *kr = k + (j * n_kv_heads + g) * D;
#pragma unroll
      for (int t = 0; t < D / 4; ++t) {
        const double ka = j < n_tokens ? double(bf16_to_f32(kr[4 * t + kq])) : 0.0;
        st = __builtin_amdgcn_mfma_f64_16x16x4f64(ka, qb[t], st, 0, 0, 0);
      }
    }
    // register r: key j0 + kq + 4r of query n0 + c; causal mask
    double mb = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t key = j0 + kq + 4 * r;
      if (key > n0 + c || key >= n_tokens) st[r] = -INFINITY;
      mb = fmax(mb, st[r]);
    }
    mb = lanes4_max_f64(mb);
    const double mn = fmax(m, mb);
    const double alpha = m == -INFINITY ? 0.0 : exp(m - mn);
    double ps = 0.0;
    f64x4 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = st[r] == -INFINITY ? 0.0 : exp(st[r] - mn);
      ps += p[r];
    }
    ps = lanes4_sum_f64(ps);
    l = l * alpha + ps;
    m = mn;
    // every register of the lane belongs to query c: rescale, then
    // O^T += V^T P^T with A = v[j0 + 4s + kq] at channel 16 ct + c, B = p[s]
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[ct][r] *= alpha;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int64_t j = j0 + 4 * s2 + kq;
      const uint16_t *vr = v + (j * n_kv_heads + g) * D;
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) {
        const double va = j < n_tokens ? double(bf16_to_f32(vr[16 * ct + c])) : 0.0;
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(va, p[s2], acc[ct], 0, 0, 0);
      }
    }
  }
  // O^T tile ct, register r: channel 16 ct + kq + 4 r of query n0 + c
  const int64_t n = n0 + c;
  if (n < n_tokens) {
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[(n * n_q_heads + h) * D + 16 * ct + kq + 4 * r] = acc[ct][r] / l;
  }
}

hipError_t launch_calib_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  int64_t n_tokens, int n_q_heads, int n_kv_heads, double *o,
                                  hipStream_t s) {
  hipLaunchKernelGGL(calib_attention_kernel, dim3(unsigned((n_tokens + 15) / 16), n_q_heads), dim3(64), 0, s,
                     q, k, v, n_tokens, n_q_heads, n_kv_heads, o);
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

// ---------------------------------------------------------------- order statistics
// Exact order statistics of non-negative fp64 values (the |x R| of a clip
// quantile) by radix selection on the device, in memory independent of the
// number of values: non-negative IEEE doubles order like their 64-bit
// patterns, so the k-th smallest is found 8 bits at a time, each pass
// counting, among the values whose leading bits equal the prefix found so
// far, how many carry each value of the next 8 bits (a 256-bucket histogram:
// per workgroup in LDS, then added to the global one).

__global__ void __launch_bounds__(256) fill_u64_kernel(unsigned long long *p, int n, unsigned long long v) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = v;
}

__global__ void __launch_bounds__(256) radix_hist_kernel(const unsigned long long *__restrict__ y, int64_t n,
                                                         unsigned long long prefix, int shift,
                                                         unsigned long long *__restrict__ hist) {
  __shared__ unsigned int h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int hi_shift = shift + 8;  // bits above the digit must equal the prefix
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const unsigned long long v = y[i];
    const bool match = hi_shift >= 64 || (v >> hi_shift) == prefix;
    if (match) atomicAdd(&h[(v >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&hist[threadIdx.x], (unsigned long long)h[threadIdx.x]);
}

// *out = min over the values above v (bit patterns), or all ones if none
__global__ void __launch_bounds__(256) next_above_kernel(const unsigned long long *__restrict__ y, int64_t n,
                                                         unsigned long long v, unsigned long long *out) {
  unsigned long long m = ~0ull;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const unsigned long long x = y[i];
    if (x > v && x < m) m = x;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(m, off);
    m = o < m ? o : m;
  }
  if ((threadIdx.x & 63) == 0) atomicMin(out, m);
}

size_t select_scratch_bytes() { return 257 * sizeof(unsigned long long); }

static unsigned select_grid(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return unsigned(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

hipError_t select_order_stats(const double *y, int64_t n, int64_t k, void *scratch, hipStream_t s, double *vk,
                              double *vk1) {
  const unsigned long long *yy = reinterpret_cast<const unsigned long long *>(y);
  unsigned long long *hist = static_cast<unsigned long long *>(scratch);
  unsigned long long prefix = 0, hh[256];
  int64_t rank = k, in_bucket = 0;
  hipError_t e = hipSuccess;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(256), 0, s, hist, 256, 0ull);
    hipLaunchKernelGGL(radix_hist_kernel, dim3(select_grid(n)), dim3(256), 0, s, yy, n, prefix, shift, hist);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(hh, hist, sizeof hh, hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    int d = 0;
    while (d < 255 && rank >= int64_t(hh[d])) rank -= int64_t(hh[d++]);
    in_bucket = int64_t(hh[d]);
    prefix = (prefix << 8) | unsigned(d);
  }
  // prefix: the bit pattern of the k-th smallest; `in_bucket` values equal it
  double v;
  std::memcpy(&v, &prefix, sizeof v);
  *vk = v;
  if (rank + 1 < in_bucket) {
    *vk1 = v;
    return hipSuccess;
  }
  unsigned long long *mn = hist + 256;
  hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(256), 0, s, mn, 1, ~0ull);
  hipLaunchKernelGGL(next_above_kernel, dim3(select_grid(n)), dim3(256), 0, s, yy, n, prefix, mn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  unsigned long long nx = 0;
  if ((e = hipMemcpyAsync(&nx, mn, sizeof nx, hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  if (nx == ~0ull) nx = prefix;  // k is the largest
  std::memcpy(&v, &nx, sizeof v);
  *vk1 = v;
  return hipSuccess;
}

}  // namespace oscar

namespace oscar {

// ---------------------------------------------------------------- eigenbasis

// Cyclic Jacobi eigenvalue iteration for the symmetric 128 x 128 moment
// matrix (Golub & Van Loan, "Matrix Computations", section 8.5, the
// parallel ordering of section 8.5.4): each round applies 64 plane
// rotations on disjoint index pairs at once (a round-robin tournament: slot
// 0 stays, the other 127 slots rotate), 127 rounds per sweep, sweeps until
// the off-diagonal norm is below 1e-16 of the Frobenius norm.  One
// workgroup; the matrix lives in LDS (128 KiB), the accumulated rotation in
// global memory as vt = V^T (a rotation of columns p, q of V is then a
// contiguous update of rows p, q).  On exit a holds the eigenvalues on its
// diagonal and vt the eigenvectors as rows, unsorted.
constexpr int JACOBI_THREADS = 1024;
constexpr int JS = D + 1;  // LDS row stride of the matrix (doubles)

__global__ void __launch_bounds__(JACOBI_THREADS) jacobi_kernel(double *__restrict__ a, double *__restrict__ vt,
                                                               int *__restrict__ sweeps_out, int max_sweeps) {
  __shared__ double A[D * JS];  // rows padded to JS doubles (no bank conflicts down a column)
  __shared__ double cs[D / 2], sn[D / 2];
  __shared__ int pp[D / 2], qq[D / 2];
  __shared__ double red[JACOBI_THREADS / 64];
  const int tid = threadIdx.x;
  double fro = 0.0;
  for (int e = tid; e < D * D; e += JACOBI_THREADS) {
    A[(e / D) * JS + e % D] = a[e];
    vt[e] = (e / D == e % D) ? 1.0 : 0.0;
    fro += a[e] * a[e];
  }
  auto block_sum = [&](double x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    double s = 0.0;
    for (int i = 0; i < JACOBI_THREADS / 64; ++i) s += red[i];
    __syncthreads();
    return s;
  };
  fro = sqrt(block_sum(fro));
  int sweep = 0;
  for (; sweep < max_sweeps; ++sweep) {
    double off = 0.0;
    for (int e = tid; e < D * D; e += JACOBI_THREADS)
      if (e % D > e / D) off += A[(e / D) * JS + e % D] * A[(e / D) * JS + e % D];
    off = block_sum(off);
    if (sqrt(off) <= 1e-16 * fro) break;
    for (int r = 0; r < D - 1; ++r) {
      if (tid < D / 2) {
        auto slot = [&](int s) { return s == 0 ? 0 : (s - 1 + r) % (D - 1) + 1; };
        int p = slot(tid), q = slot(D - 1 - tid);
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        const double apq = A[p * JS + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double theta = (A[q * JS + q] - A[p * JS + p]) / (2.0 * apq);
          const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(t * t + 1.0);
          s = t * c;
        }
        cs[tid] = c;
        sn[tid] = s;
        pp[tid] = p;
        qq[tid] = q;
      }
      __syncthreads();
      // columns p, q of A; rows p, q of V^T
#pragma unroll
      for (int it = 0; it < (D / 2) * D / JACOBI_THREADS; ++it) {
        const int e = tid + JACOBI_THREADS * it;
        const int k = e / D, i = e % D;
        const int p = pp[k], q = qq[k];
        const double c = cs[k], s = sn[k];
        const double x = A[i * JS + p], y = A[i * JS + q];
        A[i * JS + p] = c * x - s * y;
        A[i * JS + q] = s * x + c * y;
        const double vx = vt[p * D + i], vy = vt[q * D + i];
        vt[p * D + i] = c * vx - s * vy;
        vt[q * D + i] = s * vx + c * vy;
      }
      __syncthreads();
      // rows p, q of A
      for (int e = tid; e < (D / 2) * D; e += JACOBI_THREADS) {
        const int k = e / D, j = e % D;
        const int p = pp[k], q = qq[k];
        const double c = cs[k], s = sn[k];
        const double x = A[p * JS + j], y = A[q * JS + j];
        A[p * JS + j] = c * x - s * y;
        A[q * JS + j] = s * x + c * y;
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < D * D; e += JACOBI_THREADS) a[e] = A[(e / D) * JS + e % D];
  if (tid == 0) *sweeps_out = sweep;
}

hipError_t launch_jacobi(double *a, double *vt, int *sweeps, int max_sweeps, hipStream_t s) {
  hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(JACOBI_THREADS), 0, s, a, vt, sweeps, max_sweeps);
  return hipGetLastError();
}

}  // namespace oscar
