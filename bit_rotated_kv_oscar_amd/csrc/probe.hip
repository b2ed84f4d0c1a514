// Read-bandwidth probe: the rate at which this GPU streams contiguous memory
// or gathers fixed-size blocks in a given order.  The decode kernels read the
// INT2 history as 1 KB-1.5 KB blocks in page-table order, the write kernel
// streams its input; their achieved bandwidth is reported against these
// measured ceilings as well as against the nominal HBM peak.
#include "kernels.h"

namespace oscar {

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int PROBE_WAVES = 4;   // waves per workgroup
constexpr int PROBE_U = 8;       // blocks in flight per wave
constexpr int PROBE_PIECES = 4;  // 16-byte pieces per lane and block (block_bytes <= 4096)

// Wave v takes the blocks 64 v .. 64 v + 63, then strides by 64 times the
// number of waves: the 64 slot ids arrive with one load (one per lane) and
// are read out lane by lane, so no block waits on a load of its id.  PROBE_U
// blocks are in flight per wave; each lane loads 16-byte pieces lane, lane +
// 64, ... of a block.  The words read are summed (mod 2^32) into *sink, so no
// load can be dropped.
__global__ void __launch_bounds__(64 * PROBE_WAVES)
read_probe_kernel(const uint8_t *buf, int64_t n_slots, int64_t n_blocks, int block_bytes, const int32_t *ids,
                  uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = int64_t(blockIdx.x) * PROBE_WAVES + (threadIdx.x >> 6);
  const int64_t n_waves = int64_t(gridDim.x) * PROBE_WAVES;
  const int pieces = block_bytes / 16;
  uint32_t acc = 0;
  for (int64_t base = wave * 64; base < n_blocks; base += n_waves * 64) {
    const int64_t mine = base + lane;
    int64_t my_slot = -1;
    if (mine < n_blocks) my_slot = ids ? int64_t(ids[mine]) : mine;
    const int lo32 = int(uint64_t(my_slot) & 0xffffffffu), hi32 = int(uint64_t(my_slot) >> 32);
    const int nb = n_blocks - base < 64 ? int(n_blocks - base) : 64;
    for (int k = 0; k < nb; k += PROBE_U) {
      v4u r[PROBE_U][PROBE_PIECES];
#pragma unroll
      for (int u = 0; u < PROBE_U; ++u) {
        int64_t slot = -1;
        if (k + u < nb)
          slot = int64_t((uint64_t(uint32_t(__builtin_amdgcn_readlane(hi32, k + u))) << 32) |
                         uint32_t(__builtin_amdgcn_readlane(lo32, k + u)));
        const bool ok = slot >= 0 && slot < n_slots;
        const uint8_t *blk = buf + (ok ? slot : 0) * int64_t(block_bytes);
#pragma unroll
        for (int p = 0; p < PROBE_PIECES; ++p) {
          const int c = lane + 64 * p;
          r[u][p] = (ok && c < pieces) ? *reinterpret_cast<const v4u *>(blk + 16 * c) : v4u{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < PROBE_U; ++u)
#pragma unroll
        for (int p = 0; p < PROBE_PIECES; ++p) acc += r[u][p][0] + r[u][p][1] + r[u][p][2] + r[u][p][3];
    }
  }
  for (int off = 32; off > 0; off >>= 1) acc += uint32_t(__shfl_xor(int(acc), off));
  if (lane == 0) atomicAdd(sink, acc);
}

}  // namespace

hipError_t launch_read_probe(const void *buf, int64_t buf_bytes, int64_t n_blocks, int block_bytes,
                             const int32_t *ids, uint32_t *sink, hipStream_t s) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // enough waves to keep every CU's memory pipeline full, no more than the
  // blocks need
  const int64_t want = (n_blocks + 64 * PROBE_WAVES - 1) / (64 * PROBE_WAVES);
  const int64_t grid = want < int64_t(cus) * 8 ? want : int64_t(cus) * 8;
  const KernelEvents ev = take_profile_events();
  hipExtLaunchKernelGGL(read_probe_kernel, dim3(unsigned(grid)), dim3(64 * PROBE_WAVES), 0, s, ev.before, ev.after,
                        0, static_cast<const uint8_t *>(buf), buf_bytes / block_bytes, n_blocks, block_bytes, ids,
                        sink);
  return hipGetLastError();
}

}  // namespace oscar
