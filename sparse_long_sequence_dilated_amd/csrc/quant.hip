// Per-(batch, head) FP8 E4M3 quantization of keys or values (the
// quantization that the gptget.net LongNet summary, section 方法详解, pairs
// with the method).  For each head: amax = max |x| over its N rows and 64
// columns, inv = 448 / amax, code = E4M3(x * inv) rounded to nearest even
// after clamping to +-448, scale = amax / 448 (inv = scale = 1 for an
// all-zero head).  Four launches on the caller's stream: clear the amax
// slots, the amax pass (one vector atomic max per wave on the float bits,
// which order like unsigned integers for non-negative values), the
// quantization pass, and amax -> scale.
#include <algorithm>

#include "dla_device.h"
#include "dla_kernels.h"

namespace dla {

namespace {

constexpr int kQRows = 256;   // rows of one head per workgroup (8 lanes x 8 columns per row)

__global__ __launch_bounds__(256) void q_clear_kernel(float* scale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) scale[i] = 0.f;
}

__device__ __forceinline__ float amax8(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
  }
  return m;
}

// grid (min(ceil(N / 256), kAmaxBlocks), B * H).  The heads' slots share a
// cache line, where atomics serialise, so each workgroup strides over row
// blocks and issues one atomic.
constexpr int kAmaxBlocks = 64;

__global__ __launch_bounds__(256) void q_amax_kernel(QuantArgs a) {
  __shared__ float wmax[4];
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int sub = threadIdx.x & 7, rr = threadIdx.x >> 3;
  const __bf16* x = (const __bf16*)a.x + b * a.sb + h * a.sh + 8 * sub;
  float m = 0.f;
  for (int64_t n = (int64_t)blockIdx.x * 32 + rr; n < a.N; n += (int64_t)gridDim.x * 32)
    m = fmaxf(m, amax8(*(const uint4*)(x + n * a.sn)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax((unsigned int*)(a.scale + bh), __float_as_uint(m));
  }
}

__device__ __forceinline__ float inv_of(float amax) { return amax > 0.f ? __fdiv_rn(448.f, amax) : 1.f; }

__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -448.f), 448.f); }

// grid (ceil(N / 256), B * H); a.scale holds the amax of each head
__global__ __launch_bounds__(256) void q_code_kernel(QuantArgs a) {
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int sub = threadIdx.x & 7, rr = threadIdx.x >> 3;
  const float inv = inv_of(a.scale[bh]);
  const int64_t off = b * a.sb + h * a.sh + 8 * sub;
  for (int i = 0; i < kQRows / 32; ++i) {
    const int64_t n = (int64_t)blockIdx.x * kQRows + 32 * i + rr;
    if (n >= a.N) break;
    const uint4 u = *(const uint4*)((const __bf16*)a.x + off + n * a.sn);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float y[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[2 * k] = clamp448(__uint_as_float(w[k] << 16) * inv);
      y[2 * k + 1] = clamp448(__uint_as_float(w[k] & 0xFFFF0000u) * inv);
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    *(uint2*)(a.x8 + off + n * a.sn) = uint2{(uint32_t)lo, (uint32_t)hi};
  }
}

__global__ __launch_bounds__(256) void q_scale_kernel(float* scale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const float amax = scale[i];
    scale[i] = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream) {
  const int64_t nbh = a.B * a.H;
  if (nbh == 0) return hipSuccess;
  const dim3 small((unsigned)((nbh + 255) / 256));
  TimedLaunch tl("quantize_fp8", stream);
  hipLaunchKernelGGL(q_clear_kernel, small, dim3(256), 0, stream, a.scale, nbh);
  if (a.N > 0) {  // (an empty sequence keeps amax 0, so scale 1)
    const int64_t nblk = (a.N + kQRows - 1) / kQRows;
    const dim3 grid((unsigned)nblk, (unsigned)nbh);
    hipLaunchKernelGGL(q_amax_kernel, dim3((unsigned)std::min<int64_t>(nblk, kAmaxBlocks), (unsigned)nbh),
                       dim3(256), 0, stream, a);
    hipLaunchKernelGGL(q_code_kernel, grid, dim3(256), 0, stream, a);
  }
  hipLaunchKernelGGL(q_scale_kernel, small, dim3(256), 0, stream, a.scale, nbh);
  return hipGetLastError();
}

}  // namespace dla
