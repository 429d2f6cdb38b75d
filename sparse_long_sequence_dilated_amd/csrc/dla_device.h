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

// Length of batch b's sequence: lengths[b] clamped to [0, N], or N.
__device__ __forceinline__ int64_t batch_len(const int32_t* lengths, int64_t b, int64_t N) {
  if (!lengths) return N;
  const int64_t x = lengths[b];
  return x < 0 ? 0 : (x > N ? N : x);
}

// Sparse rows of segment seg for head h: L_full = w/r, or fewer in a last
// segment that the end of the sequence cuts short (rows (h mod r) + a*r
// below the N - seg*w rows that remain).
__device__ __forceinline__ int seg_rows(int64_t N, int64_t seg, int w, int r, int h, int L_full) {
  const int64_t left = N - seg * (int64_t)w;
  if (left >= w) return L_full;
  const int off = h % r;
  return left > off ? (int)((left - 1 - off) / r) + 1 : 0;
}

// Longest-first unit decode (see Schedule in dla_plan.h); false for an empty
// unit (a group past a pattern's last segment-head).  All quantities fit
// in 32 bits (the planner bounds the unit count by the launch grid), so the
// divisions are 32-bit.
__device__ __forceinline__ bool decode_unit(const Schedule& s, uint32_t u, int H,
                                            const int64_t* nseg, int& p, int& b, int& h,
                                            int64_t& seg, int& tile) {
  const uint32_t upg = (uint32_t)s.upg;
  const uint32_t grp = u / upg;
  u -= grp * upg;
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
  const int64_t gi = (int64_t)grp * s.chunk[p] + rem;  // segment-head index within the pattern
  if (gi >= s.count[p]) return false;                   // past the pattern's last one
  uint32_t g32 = (uint32_t)gi;
  const uint32_t sg = g32 % ns;
  g32 /= ns;
  h = (int)(g32 % (uint32_t)H);
  b = (int)(g32 / (uint32_t)H);
  seg = sg;
  return true;
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

// Swizzle of the 16-byte chunks of a 64-row x 128-byte LDS tile that is read
// both row-wise (32 lanes on 32 consecutive rows, one chunk each, as an MFMA
// operand) and transposed (ds_read_b64_tr_b16 over 4-row groups): chunk c of
// row i lives at c ^ u_swz(i).  Both access kinds are bank-conflict-free with
// 32 banks x 4 bytes and with 64 banks x 4 bytes.
__device__ __forceinline__ int u_swz(int row) {
  return (((row & 3) << 1) | ((row >> 2) & 1)) ^ (((row >> 3) & 1) << 1);
}

typedef __attribute__((address_space(3))) uint4 lds_u4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) char lds_char;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(1))) void glb_void;
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte operand read of a u-swizzled tile (byte offset within the tile).
__device__ __forceinline__ bf16x8 lds_read_b128(const lds_u4* base, int byte_off) {
  return __builtin_bit_cast(bf16x8, *(const lds_u4*)((const lds_char*)base + byte_off));
}
// MFMA operand with 8 sequence rows of one head dimension from a row-major
// u-swizzled tile: two transposed 8-byte reads, rows +0..3 at byte offset
// `lo` and rows +8..11 at `hi`, matching the k-slot order of an operand that
// comes from a 32x32 accumulator.
__device__ __forceinline__ bf16x8 lds_read_tr8(const lds_u4* base, int lo, int hi) {
  const lds_char* p = (const lds_char*)base;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + lo));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Per-lane byte offsets (lo, hi) of lds_read_tr8 for head-dimension block db
// (32 dims) of the 16-row k-step at rows 0..15 of a tile; k-step kk adds
// kk * 16 * 128 to both (u_swz depends on row % 16 only).  Lane l = 16m + t
// supplies row 4*(m/2) + t/4 (lo) or that + 8 (hi) and dims 32db + 16(m%2) +
// 4(t%4) .. +4, and receives rows 4*(l/32) + {0..3, 8..11} of head dim
// 32db + l%32.  Row + 8 flips bit 1 of the swizzle, i.e. bit 5 of the offset.
__device__ __forceinline__ void tr_offsets(int lane, int db, int& lo, int& hi) {
  const int t = lane & 15, m = lane >> 4;
  const int row = 4 * (m >> 1) + (t >> 2);
  const int chunk = 4 * db + 2 * (m & 1) + ((t & 3) >> 1);
  lo = row * 128 + ((chunk ^ u_swz(row)) << 4) + 8 * (t & 1);
  hi = (lo ^ 32) + 8 * 128;
}
// Per-lane byte offset of the row-wise operand read: row 32*blk + (lane%32),
// logical chunk 2*ks + lane/32.
__device__ __forceinline__ int row_offset(int lane, int blk, int ks) {
  const int row = 32 * blk + (lane & 31);
  return row * 128 + (((2 * ks + (lane >> 5)) ^ u_swz(row)) << 4);
}

// Instruction-interleaving hints for one phase: n MFMAs, each followed by v VALU ops.
#define DLA_INTERLEAVE(n, v)                                   \
  do {                                                         \
    _Pragma("unroll") for (int _i = 0; _i < (n); ++_i) {       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       \
      __builtin_amdgcn_sched_group_barrier(0x002, (v), 0);     \
    }                                                          \
  } while (0)

// Raw buffer resource over [base, base + bytes) (gfx9 dword3 for untyped access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
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
