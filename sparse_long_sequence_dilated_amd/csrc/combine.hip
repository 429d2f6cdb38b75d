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
// merges in place.  A workgroup takes 32 consecutive rows of one (batch,
// head), eight lanes per row and eight d values per lane, so the LSE and
// partial-LSE reads are contiguous; all index arithmetic is 32-bit, with
// shifts for power-of-two rates.
#include "dla_device.h"

namespace dla {

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  struct Raw {
    float4 a, b;
  };
  static __device__ __forceinline__ Raw load_raw(const float* p) {
    return Raw{*(const float4*)p, *(const float4*)(p + 4)};
  }
  static __device__ __forceinline__ void unpack(const Raw& r, float v[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[8]) {
    *(float4*)p = float4{v[0], v[1], v[2], v[3]};
    *(float4*)(p + 4) = float4{v[4], v[5], v[6], v[7]};
  }
};
template <>
struct Vec8<__bf16> {
  typedef uint4 Raw;
  static __device__ __forceinline__ Raw load_raw(const __bf16* p) { return *(const uint4*)p; }
  static __device__ __forceinline__ void unpack(const Raw& a, float v[8]) {
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

// n / r and n mod r for the small set of rates of a launch (shift >= 0 for powers of two).
__device__ __forceinline__ void divmod_r(uint32_t n, uint32_t r, int shift, uint32_t& q, uint32_t& m) {
  if (shift >= 0) {
    q = n >> shift;
    m = n & (r - 1);
  } else {
    q = n / r;
    m = n - q * r;
  }
}

// Block = 32 consecutive rows n of one (batch, head); 8 lanes per row.  NP is
// the number of patterns: fixed at compile time so that the per-pattern loops
// unroll into straight-line code, and every load of a lane issues before the
// first wait.
template <typename T, int NP>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  const uint32_t b = blockIdx.x / a.nblk;
  const uint32_t n = (blockIdx.x - b * a.nblk) * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  const uint32_t h = blockIdx.y;
  if (n >= (uint32_t)batch_len(a.lengths, b, a.N)) return;  // padding: see pad_rows_kernel

  uint32_t kept = 0, sidx[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t q, m, qh, mh;
    divmod_r(n, (uint32_t)a.r[p], a.shift[p], q, m);
    divmod_r(h, (uint32_t)a.r[p], a.shift[p], qh, mh);
    kept |= (uint32_t)(m == mh) << p;
    sidx[p] = q;  // sparse index of row n in pattern p (when it keeps the row)
  }
  const uint32_t prim_bit = 1u << a.prim;
  if (kept == prim_bit) return;  // only the pattern that wrote o keeps this row

  const int64_t bh = (int64_t)b * a.H + h;
  T* orow = (T*)a.o + (int64_t)b * a.sb + (int64_t)n * a.sn + (int64_t)h * a.sh + 8 * c;
  float* lse_dst = a.lse + bh * a.N + n;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (kept == 0) {  // no pattern keeps this row
    Vec8<T>::store(orow, acc);
    if (c == 0) *lse_dst = -INFINITY;
    return;
  }
  // Every load first (LSE and the 8-value slice of each pattern's output), so
  // the memory latencies overlap; then merge.  No branch surrounds a load: the
  // pattern that wrote o/lse and the others differ only in the selected
  // addresses, and a lane whose row pattern p does not keep reads entry 0 of
  // that pattern's buffers and discards it.
  float lv[NP];
  typename Vec8<T>::Raw raw[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const bool k = (kept >> p) & 1u;
    const bool is_prim = p == a.prim;
    const int64_t m = k ? bh * a.nsp[p] + sidx[p] : 0;
    const T* src = is_prim ? (const T*)orow : (const T*)a.part_o[p] + m * kD + (k ? 8 * c : 0);
    const float* lsrc = is_prim ? (const float*)lse_dst : a.part_lse[p] + m;
    const float l = *lsrc;
    raw[p] = Vec8<T>::load_raw(src);
    lv[p] = k ? l : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < NP; ++p) mx = fmaxf(mx, lv[p]);
  float tot = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) tot += (kept >> p) & 1u ? expf(lv[p] - mx) : 0.f;
  const float lse = mx + logf(tot);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    // A pattern that does not keep the row is discarded by selection, not by
    // a zero weight: its load read o itself (the primary pattern's slot,
    // which the primary never wrote for this row) or entry 0 of a partial
    // buffer, and 0 * (NaN or inf) would poison the sum.
    const bool k = (kept >> p) & 1u;
    const float wt = k ? expf(lv[p] - lse) : 0.f;
    float v[8];
    Vec8<T>::unpack(raw[p], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = k ? __builtin_fmaf(wt, v[i], acc[i]) : acc[i];
  }
  Vec8<T>::store(orow, acc);
  if (c == 0) *lse_dst = lse;
}

// Residue-class variant: the set of patterns that keep row n depends only on
// n mod R (R = lcm of the rates) and on the head, so a workgroup that takes 32
// rows n = rho + R*t of one class rho and one (batch, head) has one kept set
// for all its lanes: rows only the primary pattern keeps are skipped by whole
// workgroups, and each lane loads exactly the kept patterns' rows, with no
// divergence and no discarded loads.  Grid: (row blocks, R / cls_step, B*H):
// when cls_step > 1 the classes that only the primary pattern keeps are not
// launched at all (half of the workgroups with geometric rates).
template <typename T, int NP>
__global__ __launch_bounds__(256) void combine_class_kernel(const CombineArgs a) {
  const uint32_t bhu = blockIdx.z;
  const uint32_t h = bhu % (uint32_t)a.H, b = bhu / (uint32_t)a.H;
  const uint32_t rho = h % a.cls_step + a.cls_step * blockIdx.y;
  uint32_t kept = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t q, m, qh, mh;
    divmod_r(rho, (uint32_t)a.r[p], a.shift[p], q, m);
    divmod_r(h, (uint32_t)a.r[p], a.shift[p], qh, mh);
    kept |= (uint32_t)(m == mh) << p;
  }
  if (kept == (1u << a.prim)) return;  // only the pattern that wrote o keeps these rows
  const uint32_t t = blockIdx.x * 32 + (threadIdx.x >> 3);
  if (t >= a.rows_per_class) return;
  const int c = threadIdx.x & 7;
  const uint32_t n = rho + a.R * t;
  if (n >= (uint32_t)batch_len(a.lengths, b, a.N)) return;  // padding: see pad_rows_kernel
  const int64_t bh = (int64_t)b * a.H + h;
  T* orow = (T*)a.o + (int64_t)b * a.sb + (int64_t)n * a.sn + (int64_t)h * a.sh + 8 * c;
  float* lse_dst = a.lse + bh * a.N + n;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (kept == 0) {  // no pattern keeps these rows
    Vec8<T>::store(orow, acc);
    if (c == 0) *lse_dst = -INFINITY;
    return;
  }
  float lv[NP];
  typename Vec8<T>::Raw raw[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    lv[p] = -INFINITY;
    if (!((kept >> p) & 1u)) continue;                 // uniform
    if (p == a.prim) {
      lv[p] = *lse_dst;
      raw[p] = Vec8<T>::load_raw(orow);
    } else {
      // sparse index n / r = rho / r + (R / r) * t
      const uint32_t rp = (uint32_t)a.r[p];
      const int64_t m = bh * a.nsp[p] + rho / rp + (a.R / rp) * t;
      lv[p] = a.part_lse[p][m];
      raw[p] = Vec8<T>::load_raw((const T*)a.part_o[p] + m * kD + 8 * c);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < NP; ++p) mx = fmaxf(mx, lv[p]);
  float tot = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p)
    if ((kept >> p) & 1u) tot += expf(lv[p] - mx);
  const float lse = mx + logf(tot);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (!((kept >> p) & 1u)) continue;
    const float wt = expf(lv[p] - lse);
    float v[8];
    Vec8<T>::unpack(raw[p], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wt, v[i], acc[i]);
  }
  Vec8<T>::store(orow, acc);
  if (c == 0) *lse_dst = lse;
}

template <typename T>
static void launch_combine_np(const CombineArgs& a, dim3 grid, hipStream_t stream) {
  if (a.R) {
    const dim3 g((a.rows_per_class + 31) / 32, a.R / a.cls_step, (unsigned)(a.B * a.H));
    switch (a.P) {
#define DLA_COMBINE_CASE(np) \
      case np: hipLaunchKernelGGL((combine_class_kernel<T, np>), g, dim3(256), 0, stream, a); break;
      DLA_COMBINE_CASE(1) DLA_COMBINE_CASE(2) DLA_COMBINE_CASE(3) DLA_COMBINE_CASE(4)
      DLA_COMBINE_CASE(5) DLA_COMBINE_CASE(6) DLA_COMBINE_CASE(7) DLA_COMBINE_CASE(8)
      DLA_COMBINE_CASE(9) DLA_COMBINE_CASE(10) DLA_COMBINE_CASE(11) DLA_COMBINE_CASE(12)
      DLA_COMBINE_CASE(13) DLA_COMBINE_CASE(14) DLA_COMBINE_CASE(15) DLA_COMBINE_CASE(16)
#undef DLA_COMBINE_CASE
      default: break;
    }
    return;
  }
  switch (a.P) {
#define DLA_COMBINE_CASE(np) \
    case np: hipLaunchKernelGGL((combine_kernel<T, np>), grid, dim3(256), 0, stream, a); break;
    DLA_COMBINE_CASE(1) DLA_COMBINE_CASE(2) DLA_COMBINE_CASE(3) DLA_COMBINE_CASE(4)
    DLA_COMBINE_CASE(5) DLA_COMBINE_CASE(6) DLA_COMBINE_CASE(7) DLA_COMBINE_CASE(8)
    DLA_COMBINE_CASE(9) DLA_COMBINE_CASE(10) DLA_COMBINE_CASE(11) DLA_COMBINE_CASE(12)
    DLA_COMBINE_CASE(13) DLA_COMBINE_CASE(14) DLA_COMBINE_CASE(15) DLA_COMBINE_CASE(16)
#undef DLA_COMBINE_CASE
    default: break;
  }
}

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream) {
  if (a.B * a.N * a.H == 0) return hipSuccess;
  static_assert(kMaxP == 16, "one combine instantiation per pattern count");
  const dim3 grid((unsigned)(a.B * a.nblk), (unsigned)a.H);
  TimedLaunch tl("combine", stream);
  if (dtype == DLA_F32)
    launch_combine_np<float>(a, grid, stream);
  else
    launch_combine_np<__bf16>(a, grid, stream);
  return hipGetLastError();
}

// Rows past a batch's length are padding: output 0, log-sum-exp -inf.
// 32 rows of one (batch, head) per workgroup, 8 lanes per row.
template <typename T>
__global__ __launch_bounds__(256) void pad_rows_kernel(const CombineArgs a) {
  const uint32_t b = blockIdx.x / a.nblk;
  const uint32_t n = (blockIdx.x - b * a.nblk) * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  const uint32_t h = blockIdx.y;
  if (n >= (uint32_t)a.N || n < (uint32_t)batch_len(a.lengths, b, a.N)) return;
  float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  Vec8<T>::store((T*)a.o + (int64_t)b * a.sb + (int64_t)n * a.sn + (int64_t)h * a.sh + 8 * c, zero);
  if (c == 0) a.lse[((int64_t)b * a.H + h) * a.N + n] = -INFINITY;
}

hipError_t launch_pad_rows(const CombineArgs& a, int dtype, hipStream_t stream) {
  if (a.B * a.N * a.H == 0 || !a.lengths) return hipSuccess;
  const dim3 grid((unsigned)(a.B * a.nblk), (unsigned)a.H);
  TimedLaunch tl("combine", stream);
  if (dtype == DLA_F32)
    hipLaunchKernelGGL(pad_rows_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(pad_rows_kernel<__bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Integer index map of one pattern, exposed so the address generator can be
// compared bit for bit: out[h*ceil(N/r) + m] = original row of sparse row m,
// or -1 past the end of a cut-short last segment.
__global__ __launch_bounds__(256) void row_map_kernel(const RowMapArgs a) {
  const int64_t per_head = (a.N + a.r - 1) / a.r;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= per_head * a.H) return;
  const int h = (int)(gid / per_head);
  const int64_t m = gid - (int64_t)h * per_head;
  const int64_t seg = m / a.L;
  const int64_t row = m - seg * a.L;
  const int64_t n = seg_base_row(seg, a.w, a.r, h) + row * a.r;
  a.out[gid] = n < a.N ? (int32_t)n : -1;                // past the end of a cut-short segment
}

hipError_t launch_row_map(const RowMapArgs& a, hipStream_t stream) {
  const int64_t n = ((a.N + a.r - 1) / a.r) * a.H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(row_map_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
