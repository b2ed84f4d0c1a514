// Internal definitions shared by the liboscar kernels and host code.
// Storage formats are the ones declared in include/oscar.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

constexpr int D = OSCAR_HEAD_DIM;     // 128
constexpr int PAGE = OSCAR_PAGE;      // 16
constexpr int N_SINK = OSCAR_N_SINK;  // 16
constexpr int N_RECENT = OSCAR_N_RECENT;
constexpr int N_RAW = N_SINK + N_RECENT;  // 144 raw bf16 tokens at most
constexpr int BF16_PT = OSCAR_BF16_PAGES_PER_REQ;
constexpr int CODE_BYTES = 512;       // one INT2 code area: 16 rows x 128 codes x 2 bits

// Byte offsets inside the forms buffer of one rotation.
constexpr size_t FORM_R = 0;                        // fp32 R[i][j]
constexpr size_t FORM_RT = FORM_R + D * D * 4;      // fp32 RT[j][i] = R[i][j]
constexpr size_t FORM_RT_HI = FORM_RT + D * D * 4;  // fp16 hi(R[i][j]) at [j][i]
constexpr size_t FORM_RT_LO = FORM_RT_HI + D * D * 2;  // fp16 2^11 * (R - hi)
constexpr size_t FORM_BYTES = FORM_RT_LO + D * D * 2;

// History blocks of both code widths: [K codes | K meta | V codes | V meta],
// a code area being 16 rows x 128 codes x bits (512 B for INT2, 1 KB for
// INT4).
__host__ __device__ constexpr int n_groups(int G) { return D / G; }
__host__ __device__ constexpr int meta_bytes(int G) { return 64 * (D / G); }
__host__ __device__ constexpr int code_area_bytes(int bits) { return PAGE * D * bits / 8; }
__host__ __device__ constexpr int hist_block_bytes(int G, int bits = 2) {
  return 2 * code_area_bytes(bits) + 128 * (D / G);
}
__host__ __device__ constexpr int k_codes_off(int, int = 2) { return 0; }
__host__ __device__ constexpr int k_meta_off(int, int bits = 2) { return code_area_bytes(bits); }
__host__ __device__ constexpr int v_codes_off(int G, int bits = 2) { return code_area_bytes(bits) + meta_bytes(G); }
__host__ __device__ constexpr int v_meta_off(int G, int bits = 2) { return 2 * code_area_bytes(bits) + meta_bytes(G); }
// the code width of a cache (0 in a zero-initialised struct means INT2)
__host__ __device__ inline int cache_bits(const oscar_layer_cache &c) { return c.code_bits == 4 ? 4 : 2; }

// Slot bit tables of a code dword (first code at LO[u], second at HI[u]).
__host__ __device__ inline int slot_lo(int u) {
  const int t[8] = {8, 6, 12, 10, 4, 2, 16, 14};
  return t[u];
}
__host__ __device__ inline int slot_hi(int u) {
  const int t[8] = {24, 22, 28, 26, 20, 18, 0, 30};
  return t[u];
}

// (word, bit) of the K code of (row t, channel c).
__host__ __device__ inline void k_code_pos(int t, int c, int &word, int &bit) {
  const int k = c >> 5, cb = c & 31;
  const int q = cb >> 3, v = (cb & 7) >> 1;
  const int d = k >> 1, u = 4 * (k & 1) + v;
  word = 2 * (16 * q + t) + d;
  bit = (c & 1) ? slot_hi(u) : slot_lo(u);
}

// (word, bit) of the V code of (row t, channel c).
__host__ __device__ inline void v_code_pos(int t, int c, int &word, int &bit) {
  const int r = c >> 4, m = c & 15;
  const int d = r >> 2, u = 2 * (r & 3) + ((t & 3) >> 1);
  const int q = t >> 2;
  word = 2 * (16 * q + m) + d;
  bit = (t & 1) ? slot_hi(u) : slot_lo(u);
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ inline void flag_status(uint32_t *status, uint32_t bit) {
  if (status) atomicOr(status, bit);
}

// history tokens / pages of a request of length L
__host__ __device__ inline int n_hist_tokens(int L) { return L > N_RAW ? L - N_RAW : 0; }
__host__ __device__ inline int n_hist_pages(int L) { return (n_hist_tokens(L) + PAGE - 1) / PAGE; }

// Decode split plan shared by the workspace sizing and the launch.
struct SplitPlan {
  int pages_per_split;  // history pages per split
  int n_splits;         // history splits (the BF16 part is one more)
  bool fused = false;   // INT2: the attend kernel merges (last workgroup of each unit)
};

// Compute units of the current device (256 when it cannot be queried).
int64_t device_cus();

SplitPlan plan_int2_splits(int batch, int n_kv_heads, int max_seq_len);
SplitPlan plan_bf16_splits(int batch, int n_kv_heads, int max_seq_len);

// Wave index within the workgroup as a scalar: the compiler cannot tell that
// threadIdx.x / 64 is the same in every lane, and a per-lane value would turn
// loop counters and page bookkeeping into vector registers and exec masks.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace oscar
