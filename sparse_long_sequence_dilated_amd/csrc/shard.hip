// Sequence shards: one device's share of the key/value exchange for patterns
// whose segments span several devices (the gptget.net LongNet summary,
// section 方法论, distributed item: the sequence is cut along its length, and
// devices exchange the sparsified keys and values of a segment that crosses
// them; in the backward the gradients of those keys and values go back).
//
// Layouts: a shard's part of a spanning segment is [B, H, cr, D] with
// cr = N / r (its sparse rows (h mod r) + i*r, i < cr); the exchanged
// segment is [C, B, H, cr, D], C = w / N devices in order; the same segment
// contiguous per (batch, head) is [B, H, C*cr, D].
#include <algorithm>

#include "dla_device.h"

namespace dla {

// out[b][h][out_row0 + i][:] = x[b][(h mod r) + i*r][h][:], rows of out_rows.
__global__ __launch_bounds__(256) void shard_gather_kernel(const ShardGatherArgs a) {
  const int64_t total = a.B * a.H * a.cr * 8;          // 16-byte pieces (8 bf16)
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
    const int c = (int)(t & 7);
    const int64_t row = t >> 3;                          // (b*H + h)*cr + i
    const int64_t bh = row / a.cr;
    const int64_t i = row - bh * a.cr;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    const int64_t src = b * a.sb + (h % a.r + i * a.r) * a.sn + h * a.sh + 8 * c;
    const int64_t dst = (bh * a.out_rows + a.out_row0 + i) * 8 + c;
    ((uint4*)a.out)[dst] = *(const uint4*)((const __bf16*)a.x + src);
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

// The (-LSE * log2 e, -D) pairs of the same rows: out[(b*H + h)*out_rows +
// out_row0 + i] = ld[(b*H + h)*N + (h mod r) + i*r].
__global__ __launch_bounds__(256) void shard_ld_kernel(const ShardLdArgs a) {
  const int64_t total = a.B * a.H * a.cr;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
    const int64_t bh = t / a.cr, i = t - bh * a.cr;
    const int64_t h = bh % a.H;
    a.out[bh * a.out_rows + a.out_row0 + i] = a.ld[bh * a.N + h % a.r + i * a.r];
  }
}

hipError_t launch_shard_ld(const ShardLdArgs& a, hipStream_t stream) {
  const int64_t total = a.B * a.H * a.cr;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  TimedLaunch tl("shard_gather", stream);
  hipLaunchKernelGGL(shard_ld_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// [C, B, H, cr, D] <-> [B, H, C*cr, D] (to_ext: the second into the first),
// rows of `pieces` 16-byte pieces (8 for bf16, 16 for fp32).
__global__ __launch_bounds__(256) void shard_relayout_kernel(const ShardRelayoutArgs a) {
  const int64_t rows = a.C * a.B * a.H * a.cr;
  const int64_t total = rows * a.pieces;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
    const int64_t row = t / a.pieces;
    const int64_t pc = t - row * a.pieces;
    // row indexes the exchange layout: ((c*B + b)*H + h)*cr + i
    const int64_t i = row % a.cr, cbh = row / a.cr;
    const int64_t bh = cbh % (a.B * a.H), c = cbh / (a.B * a.H);
    const int64_t seg_row = bh * (a.C * a.cr) + c * a.cr + i;
    const uint4* src = (const uint4*)a.src;
    uint4* dst = (uint4*)a.dst;
    if (a.to_ext)
      dst[row * a.pieces + pc] = src[seg_row * a.pieces + pc];
    else
      dst[seg_row * a.pieces + pc] = src[row * a.pieces + pc];
  }
}

hipError_t launch_shard_relayout(const ShardRelayoutArgs& a, hipStream_t stream) {
  const int64_t total = a.C * a.B * a.H * a.cr * a.pieces;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  TimedLaunch tl("shard_gather", stream);
  hipLaunchKernelGGL(shard_relayout_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// After the exchange of the gradients: a row n of head h that some spanning
// pattern keeps gets dK (g = 1) and dV (g = 2) as the sum, in descriptor
// order, of the fp32 partials of the local patterns that keep it and the
// exchanged parts of the spanning ones (entry n / r in either), rounded
// once.  32 rows of one (batch, head) per workgroup, 8 lanes per row.
__global__ __launch_bounds__(256) void shard_finish_kernel(const ShardFinishArgs a) {
  const uint32_t b = blockIdx.x / a.nblk;
  const uint32_t n = (blockIdx.x - b * a.nblk) * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  const uint32_t h = blockIdx.y;
  if (n >= (uint32_t)a.N) return;
  uint32_t kept = 0;
  for (int p = 0; p < a.P; ++p) kept |= (uint32_t)((n % (uint32_t)a.r[p]) == (h % (uint32_t)a.r[p])) << p;
  if ((kept & a.span_mask) == 0) return;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t out_off = (int64_t)b * a.sb + (int64_t)n * a.sn + (int64_t)h * a.sh + 8 * c;
  for (int g = 1; g < 3; ++g) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < a.P; ++p) {
      if (!((kept >> p) & 1u)) continue;
      const int64_t row = bh * a.nsp[p] + n / (uint32_t)a.r[p];
      const float* src = ((a.span_mask >> p) & 1u) ? (g == 1 ? a.red_k[p] : a.red_v[p]) : a.part[p][g];
      const float4 x = *(const float4*)(src + row * kD + 8 * c), y = *(const float4*)(src + row * kD + 8 * c + 4);
      acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
      acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
    }
    *(uint4*)((__bf16*)(g == 1 ? a.dk : a.dv) + out_off) =
        uint4{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
              pack_bf16(acc[6], acc[7])};
  }
}

hipError_t launch_shard_finish(const ShardFinishArgs& a, hipStream_t stream) {
  if (a.B * a.N * a.H == 0) return hipSuccess;
  TimedLaunch tl("shard_finish", stream);
  hipLaunchKernelGGL(shard_finish_kernel, dim3((unsigned)(a.B * a.nblk), (unsigned)a.H), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace dla
