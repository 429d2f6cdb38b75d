// Device helpers shared by the libdla kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dla_kernels.h"

namespace dla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Strided-gather address generator.  Sparse row `a` of segment `seg` of
// pattern (w, r) for head h is original row seg*w + (h mod r) + a*r (the
// gptget.net LongNet summary, section 方法论: equal segments, every r-th row,
// a different offset per head).  Callers keep `seg_base` = seg*w + (h mod r)
// and step by r, so a dilated row is always one contiguous D-element run and
// the sparsified tensors are never materialised.
__device__ __forceinline__ int64_t seg_base_row(int64_t seg, int w, int r, int h) {
  return seg * (int64_t)w + (h % r);
}

// Longest-first unit decode (see Schedule in dla_plan.h).  All quantities fit
// in 32 bits (the planner bounds the unit count by the launch grid), so the
// divisions are 32-bit.
__device__ __forceinline__ void decode_unit(const Schedule& s, uint32_t u, int H,
                                            const int64_t* nseg, int& p, int& b, int& h,
                                            int64_t& seg, int& tile) {
  int j = 0;
  while (j + 1 < s.nband && u >= (uint32_t)s.band_start[j + 1]) ++j;
  const uint32_t rel = u - (uint32_t)s.band_start[j];
  const uint32_t per_level = (uint32_t)s.cum[s.band_npat[j]];
  const uint32_t lvl = rel / per_level;
  uint32_t rem = rel - lvl * per_level;
  tile = s.band_hi[j] - 1 - (int)lvl;
  int i = 0;
  while (rem >= (uint32_t)s.cum[i + 1]) ++i;
  p = s.order[i];
  rem -= (uint32_t)s.cum[i];
  const uint32_t ns = (uint32_t)nseg[p];
  const uint32_t sg = rem % ns;
  rem /= ns;
  h = (int)(rem % (uint32_t)H);
  b = (int)(rem / (uint32_t)H);
  seg = sg;
}

// Bit-cast helpers.
__device__ __forceinline__ float as_float(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_uint(float x) { return __builtin_bit_cast(uint32_t, x); }

// max / sum of a value over lanes l and l^32 (gfx950 v_permlane32_swap).
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(as_uint(x), as_uint(x), false, false);
  return fmaxf(as_float(r[0]), as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(as_uint(x), as_uint(x), false, false);
  return as_float(r[0]) + as_float(r[1]);
}

// Two fp32 values to packed bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t f = {lo, hi};
  bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// acc + lo + hi of a packed bf16 pair, in fp32 (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float dot2_bf16_ones(uint32_t packed, float acc) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2v;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, packed),
                                         __builtin_bit_cast(bf16x2v, 0x3F803F80u), acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return as_float(x & 0xFFFF0000u); }

// LDS layouts of a 64-row x 64-column bf16 tile (rows = sequence, cols = d).
//
// Row-major ("R"): 64 rows of 8 16-byte chunks; chunk c of row i is stored at
// chunk position c ^ t_swz(i).  The 32 lanes of an MFMA operand read (one row
// each, same logical chunk) then hit distinct 16-byte bank groups both within
// any 8 consecutive rows (32 banks x 4 bytes) and within any 16 consecutive
// rows taken modulo 256 bytes (64 banks x 4 bytes).
__device__ __forceinline__ int t_swz(int d);
__device__ __forceinline__ int r_index(int row, int chunk) { return row * 8 + (chunk ^ t_swz(row)); }

// Transposed ("T"): 64 d-rows of 32 words; each word packs the values of two
// consecutive sequence rows.  Within each block of 16 sequence rows the order
// matches the k-slots of a 32x32x16 MFMA operand whose other operand comes
// straight from a 32x32 accumulator: lane group g, element e holds sequence
// row (e/4)*8 + g*4 + e%4.  The 16-byte chunks are swizzled with
// (d ^ (d >> 3)) & 7 so that both the packing writes (fixed d % 8, varying
// d / 8) and the operand reads (varying d % 8) avoid bank conflicts.
__device__ __forceinline__ int t_swz(int d) { return (d ^ (d >> 3)) & 7; }
// word index of (d, sequence rows k and k+1), k even
__device__ __forceinline__ int t_word(int d, int k) {
  const int k16 = k & 15, kk = k >> 4;
  const int g = (k16 & 7) >> 2;
  const int e = ((k16 >> 3) << 2) | (k16 & 3);
  const int chunk = 2 * kk + g;
  return d * 32 + ((chunk ^ t_swz(d)) << 2) + (e >> 1);
}
// uint4 index of the operand chunk of (d, k-step kk, lane group g)
__device__ __forceinline__ int t_chunk(int d, int kk, int g) {
  return d * 8 + ((2 * kk + g) ^ t_swz(d));
}

// Pack two rows' 16-byte chunks (8 bf16 each, same d range) into the 8 words
// (row0[j], row1[j]) for j = 0..7.
__device__ __forceinline__ void pack_pairs(const uint4& r0, const uint4& r1, uint32_t out[8]) {
  const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w};
  const uint32_t b[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __builtin_amdgcn_perm(b[i], a[i], 0x05040100u);
    out[2 * i + 1] = __builtin_amdgcn_perm(b[i], a[i], 0x07060302u);
  }
}

}  // namespace dla
