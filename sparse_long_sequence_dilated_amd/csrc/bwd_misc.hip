// Backward preprocessing: D = rowsum(dO * O) per (batch, head, row), stored
// negated next to the negated combined LSE (pre-multiplied by log2 e) so
// that the attention backward fetches both with one 8-byte load per row and
// can start its dP accumulator at -D; and zero gradients for rows that no
// pattern keeps (their output is the constant 0).
// Eight lanes per (b, n, h) row, eight d values each; rows walked in
// [B, N, H] order so that O and dO are read contiguously.  HBM bound.
#include "dla_device.h"

namespace dla {

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float v[8]);
template <>
__device__ __forceinline__ void load8f<__bf16>(const __bf16* p, float v[8]) {
  const uint4 a = *(const uint4*)p;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float v[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename T>
__device__ __forceinline__ void zero8(T* p) {
  if (sizeof(T) == 2) {
    *(uint4*)p = uint4{0, 0, 0, 0};
  } else {
    *(uint4*)p = uint4{0, 0, 0, 0};
    *(uint4*)((float*)p + 4) = uint4{0, 0, 0, 0};
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdPrepArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 3;
  const int c = gid & 7;
  if (row >= a.B * a.N * a.H) return;  // whole 8-lane groups leave together
  const int h = (int)(row % a.H);
  const int64_t bn = row / a.H;
  const int64_t n = bn % a.N;
  const int64_t b = bn / a.N;
  const int64_t off = b * a.sb + n * a.sn + h * a.sh + 8 * c;
  float o[8], d[8];
  load8f<T>((const T*)a.o + off, o);
  load8f<T>((const T*)a.dout + off, d);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = __builtin_fmaf(o[i], d[i], s);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (c == 0) {
    const int64_t i = (b * a.H + h) * a.N + n;
    a.ld[i] = float2{-(a.lse[i] * kLog2e), -s};
  }
  const bool pad = n >= batch_len(a.lengths, b, a.N);  // past this batch's length
  if (a.zero_uncovered || pad) {
    bool kept = false;
    for (int p = 0; p < a.P; ++p) kept |= (n % a.r_all[p]) == (h % a.r_all[p]);
    if (!kept || pad) {
      zero8((T*)a.dq + off);
      zero8((T*)a.dk + off);
      zero8((T*)a.dv + off);
    }
  }
}

hipError_t launch_bwd_prep(const BwdPrepArgs& a, int dtype, hipStream_t stream) {
  const int64_t threads = a.B * a.N * a.H * 8;
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  TimedLaunch tl("bwd_prep", stream);
  if (dtype == DLA_F32)
    hipLaunchKernelGGL(bwd_prep_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<__bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Finalize: a row kept by several patterns gets the sum of their fp32 partial
// gradients (each in its pattern's sparse order, where row n is entry n / r),
// rounded once.  Rows kept by one pattern were written by the attention pass
// and rows kept by none by the preprocessing pass.  A workgroup takes 32
// consecutive rows of one (batch, head), eight lanes per row and eight d
// values per lane.  Every load is issued unconditionally (a lane whose row a
// pattern does not keep reads that pattern's first entry and discards it), so
// a wave waits for memory once per tensor.  HBM bound.
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const BwdFinalizeArgs a) {
  const uint32_t b = blockIdx.x / a.nblk;
  const uint32_t n = (blockIdx.x - b * a.nblk) * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  const uint32_t h = blockIdx.y;
  if (n >= (uint32_t)batch_len(a.lengths, b, a.N)) return;  // padding rows were zeroed
  uint32_t kept = 0;
  int cnt = 0;
  uint32_t sp[kMaxP];
  for (int p = 0; p < a.P; ++p) {
    const uint32_t rp = (uint32_t)a.r[p];
    const bool k = a.shift[p] >= 0 ? ((n ^ h) & (rp - 1)) == 0 : (n % rp) == (h % rp);
    sp[p] = a.shift[p] >= 0 ? n >> a.shift[p] : n / rp;
    kept |= (uint32_t)k << p;
    cnt += k;
  }
  // Sequence shard: a row that a spanning pattern keeps has that pattern's
  // dQ partial (finalized here even when no other pattern keeps it) but
  // not its dK/dV, which the shard finish pass adds after the exchange.
  const bool span = (kept & a.span_mask) != 0;
  if (cnt < 2 && !span) return;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t out_off = (int64_t)b * a.sb + (int64_t)n * a.sn + (int64_t)h * a.sh + 8 * c;
  for (int g = 0; g < (span ? 1 : 3); ++g) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < a.P; ++p) {
      const bool k = (kept >> p) & 1;
      const float* src = a.part[p][g] + (k ? (bh * a.nsp[p] + sp[p]) * kD + 8 * c : 0);
      const float4 x = *(const float4*)src, y = *(const float4*)(src + 4);
      if (k) {
        acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
        acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
      }
    }
    *(uint4*)((__bf16*)a.grad[g] + out_off) =
        uint4{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
              pack_bf16(acc[6], acc[7])};
  }
}

// Residue-class variant: rows n = rho + R*t (R = lcm of the rates) of one
// (batch, head) are kept by one set of patterns, so a workgroup of 32 such
// rows has a uniform kept set; classes kept by fewer than two patterns are
// skipped by whole workgroups and each lane loads only the kept partials.
// A workgroup sums one of the three gradients; the patterns go in groups of
// four whose loads issue before the group's adds (which keep descriptor
// order).  Grid: (row blocks, R / cls_step, 3*B*H): when cls_step > 1 the
// classes that only the r = 1 pattern keeps are not launched.
__global__ __launch_bounds__(256) void bwd_finalize_class_kernel(const BwdFinalizeArgs a) {
  const uint32_t g = blockIdx.z % 3u, bhu = blockIdx.z / 3u;
  const uint32_t h = bhu % (uint32_t)a.H, b = bhu / (uint32_t)a.H;
  const uint32_t rho = h % a.cls_step + a.cls_step * blockIdx.y;
  uint32_t kept = 0;
  for (int p = 0; p < a.P; ++p) {
    const uint32_t rp = (uint32_t)a.r[p];
    const bool k = a.shift[p] >= 0 ? ((rho ^ h) & (rp - 1)) == 0 : (rho % rp) == (h % rp);
    kept |= (uint32_t)k << p;
  }
  const bool span = (kept & a.span_mask) != 0;      // see bwd_finalize_kernel
  if (__builtin_popcount(kept) < 2 && !span) return;
  if (span && g != 0) return;                        // dK, dV of such rows: the shard finish pass
  const uint32_t t = blockIdx.x * 32 + (threadIdx.x >> 3);
  if (t >= a.rows_per_class) return;
  const int c = threadIdx.x & 7;
  const uint32_t n = rho + a.R * t;
  if (n >= (uint32_t)batch_len(a.lengths, b, a.N)) return;  // padding rows were zeroed
  const int64_t bh = (int64_t)b * a.H + h;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int p0 = 0; p0 < a.P; p0 += 4) {
    float4 x[4], y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = p0 + j;
      if (p < a.P && ((kept >> p) & 1u)) {            // uniform
        const uint32_t rp = (uint32_t)a.r[p];
        const int64_t row = bh * a.nsp[p] + rho / rp + (a.R / rp) * t;
        const float* src = a.part[p][g] + row * kD + 8 * c;
        x[j] = *(const float4*)src;
        y[j] = *(const float4*)(src + 4);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = p0 + j;
      if (p < a.P && ((kept >> p) & 1u)) {
        acc[0] += x[j].x; acc[1] += x[j].y; acc[2] += x[j].z; acc[3] += x[j].w;
        acc[4] += y[j].x; acc[5] += y[j].y; acc[6] += y[j].z; acc[7] += y[j].w;
      }
    }
  }
  const int64_t out_off = (int64_t)b * a.sb + (int64_t)n * a.sn + (int64_t)h * a.sh + 8 * c;
  *(uint4*)((__bf16*)a.grad[g] + out_off) =
      uint4{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
            pack_bf16(acc[6], acc[7])};
}

hipError_t launch_bwd_finalize(const BwdFinalizeArgs& a, hipStream_t stream) {
  if (a.B * a.N * a.H == 0) return hipSuccess;
  TimedLaunch tl("bwd_finalize", stream);
  if (a.R && 3 * a.B * a.H <= 65535) {
    const dim3 g((a.rows_per_class + 31) / 32, a.R / a.cls_step, (unsigned)(3 * a.B * a.H));
    hipLaunchKernelGGL(bwd_finalize_class_kernel, g, dim3(256), 0, stream, a);
  } else {
    const dim3 grid((unsigned)(a.B * a.nblk), (unsigned)a.H);
    hipLaunchKernelGGL(bwd_finalize_kernel, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dla
