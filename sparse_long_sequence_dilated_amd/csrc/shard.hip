// Sequence shards: this device's part of the key/value exchange for a
// pattern whose segments span several devices (the gptget.net LongNet
// summary, section 方法论, distributed item: the sequence is cut along its
// length, and devices exchange the sparsified keys and values of a segment
// that crosses them).
//
// out[b][h][i][:] = x[b][(h mod r) + i*r][h][:] for i < N/r: the shard's
// sparse rows of its segment, contiguous, so that gathering the parts of the
// devices of a segment in device order yields [devices, B, H, N/r, D].
#include <algorithm>

#include "dla_kernels.h"

namespace dla {

__global__ __launch_bounds__(256) void shard_gather_kernel(const ShardGatherArgs a) {
  const int64_t total = a.B * a.H * a.cr * 8;          // 16-byte pieces (8 bf16)
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
    const int c = (int)(t & 7);
    const int64_t row = t >> 3;                          // (b*H + h)*cr + i
    const int64_t bh = row / a.cr;
    const int64_t i = row - bh * a.cr;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    const int64_t src = b * a.sb + (h % a.r + i * a.r) * a.sn + h * a.sh + 8 * c;
    ((uint4*)a.out)[t] = *(const uint4*)((const __bf16*)a.x + src);
  }
}

hipError_t launch_shard_gather(const ShardGatherArgs& a, hipStream_t stream) {
  const int64_t total = a.B * a.H * a.cr * 8;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  TimedLaunch tl("shard_gather", stream);
  hipLaunchKernelGGL(shard_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
