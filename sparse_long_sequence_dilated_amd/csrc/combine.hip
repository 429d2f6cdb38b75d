// Multi-pattern merge ("combine/scatter") of dilated attention.
//
// Each pattern p leaves, for the rows it keeps, a normalised output O_p and
// its log-sum-exp LSE_p.  The merged result is one softmax over the union of
// the patterns' keys: LSE = log sum_p exp(LSE_p), O = sum_p exp(LSE_p - LSE)
// O_p, i.e. every pattern weighted by its own softmax denominator so that the
// normaliser they share stays exact (darcstar.tech LongNet page, DarcStar
// commentary; gptget.net LongNet summary, 方法详解: multi-scale mixture).
// A row that no pattern keeps gets O = 0 and LSE = -inf.
//
// The pattern that keeps the most rows wrote straight into o/lse; this pass
// touches only rows that another pattern also keeps (or that none keeps) and
// merges in place.  Eight lanes per (b, n, h) row, eight d values each; rows
// are walked in [B, N, H] order so that o is read and written contiguously.
#include "dla_device.h"

namespace dla {

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float v[8]) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[8]) {
    *(float4*)p = float4{v[0], v[1], v[2], v[3]};
    *(float4*)(p + 4) = float4{v[4], v[5], v[6], v[7]};
  }
};
template <>
struct Vec8<__bf16> {
  static __device__ __forceinline__ void load(const __bf16* p, float v[8]) {
    const uint4 a = *(const uint4*)p;
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  static __device__ __forceinline__ void store(__bf16* p, const float v[8]) {
    *(uint4*)p = uint4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                       pack_bf16(v[6], v[7])};
  }
};

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 3;
  const int c = gid & 7;
  if (row >= a.B * a.N * a.H) return;
  const int h = (int)(row % a.H);
  const int64_t bn = row / a.H;
  const int64_t n = bn % a.N;
  const int64_t b = bn / a.N;

  const int rp = a.r[a.prim];
  const bool prim_kept = (n % rp) == (h % rp);
  int others = 0;
  for (int p = 0; p < a.P; ++p)
    if (p != a.prim && (n % a.r[p]) == (h % a.r[p])) ++others;
  if (prim_kept && others == 0) return;

  const int64_t bh = b * a.H + h;
  T* orow = (T*)a.o + b * a.sb + n * a.sn + h * a.sh + 8 * c;
  float* lse_dst = a.lse + bh * a.N + n;
  const float l_prim = prim_kept ? *lse_dst : -INFINITY;
  float mx = l_prim;
  for (int p = 0; p < a.P; ++p) {
    if (p == a.prim || (n % a.r[p]) != (h % a.r[p])) continue;
    mx = fmaxf(mx, a.part_lse[p][bh * (a.N / a.r[p]) + n / a.r[p]]);
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (mx == -INFINITY) {  // no pattern keeps this row
    Vec8<T>::store(orow, acc);
    if (c == 0) *lse_dst = -INFINITY;
    return;
  }
  float tot = prim_kept ? expf(l_prim - mx) : 0.f;
  for (int p = 0; p < a.P; ++p) {
    if (p == a.prim || (n % a.r[p]) != (h % a.r[p])) continue;
    tot += expf(a.part_lse[p][bh * (a.N / a.r[p]) + n / a.r[p]] - mx);
  }
  const float lse = mx + logf(tot);
  float v[8];
  if (prim_kept) {
    const float wt = expf(l_prim - lse);
    Vec8<T>::load(orow, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = wt * v[i];
  }
  for (int p = 0; p < a.P; ++p) {
    if (p == a.prim || (n % a.r[p]) != (h % a.r[p])) continue;
    const int64_t m = bh * (a.N / a.r[p]) + n / a.r[p];
    const float wt = expf(a.part_lse[p][m] - lse);
    Vec8<T>::load((const T*)a.part_o[p] + m * kD + 8 * c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wt, v[i], acc[i]);
  }
  Vec8<T>::store(orow, acc);
  if (c == 0) *lse_dst = lse;
}

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream) {
  const int64_t threads = a.B * a.N * a.H * 8;
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  TimedLaunch tl("combine", stream);
  if (dtype == DLA_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Integer index map of one pattern, exposed so the address generator can be
// compared bit for bit: out[h*(N/r) + m] = original row of sparse row m.
__global__ __launch_bounds__(256) void row_map_kernel(const RowMapArgs a) {
  const int64_t per_head = a.N / a.r;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= per_head * a.H) return;
  const int h = (int)(gid / per_head);
  const int64_t m = gid - (int64_t)h * per_head;
  const int64_t seg = m / a.L;
  const int64_t row = m - seg * a.L;
  a.out[gid] = (int32_t)(seg_base_row(seg, a.w, a.r, h) + row * a.r);
}

hipError_t launch_row_map(const RowMapArgs& a, hipStream_t stream) {
  const int64_t n = (a.N / a.r) * a.H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(row_map_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
