// Backward preprocessing: D = rowsum(dO * O) per (batch, head, row), stored
// next to the combined LSE (pre-multiplied by log2 e) so that the attention
// backward fetches both with one 8-byte load per row; and zero gradients for
// rows that no pattern keeps (their output is the constant 0).
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
    a.ld[i] = float2{a.lse[i] * kLog2e, s};
  }
  if (a.zero_uncovered) {
    bool kept = false;
    for (int p = 0; p < a.P; ++p) kept |= (n % a.r_all[p]) == (h % a.r_all[p]);
    if (!kept) {
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

}  // namespace dla
