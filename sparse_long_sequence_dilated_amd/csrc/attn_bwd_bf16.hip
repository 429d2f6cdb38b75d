// Dilated attention backward of one pattern, bf16 in, fp32 accumulation.
//
// The merged forward output is one softmax over the union of each row's keys
// across patterns (darcstar.tech LongNet page, DarcStar commentary: the
// patterns share one denominator), so the gradient of every pattern uses the
// combined LSE and D = rowsum(dO * O):
//   P = exp(S - LSE), dV += P^T dO, dP = dO V^T, dS = P * (dP - D),
//   dQ += scale dS K, dK += scale dS^T Q,
// inside each sparsified segment (gptget.net LongNet summary, section 方法论),
// with rows gathered by the same strided address generator as the forward.
//
// Two launches cover all patterns, one per kind of workgroup (4 waves each):
//   * key units own 128 keys (32 per wave), stream the segment's query rows
//     (Q, dO, and the (LSE, D) pairs) and accumulate dK^T = Q^T dS and
//     dV^T = dO^T P in registers; they need 256 VGPRs, so two workgroups
//     share a CU, with a 4-stage LDS ring (66 KB);
//   * query units own 128 queries (32 per wave), stream key rows (K, V) and
//     accumulate dQ^T = K^T dS^T; they fit in 168 VGPRs and a 3-stage ring
//     (49.5 KB), so three workgroups share a CU.
// The owned rows sit in registers as MFMA B operands; the streamed rows go
// from HBM into the LDS ring with buffer_load ... lds (one 64-row tile per
// stage, refilled as soon as its last reader is past a barrier), in one
// u-swizzled row-major copy that serves both the row-wise operand reads
// (ds_read_b128) and the transposed ones (ds_read_b64_tr_b16) without bank
// conflicts.  S and dP come out of v_mfma_f32_32x32x16_bf16 with the lane on
// the owned row, so P and dS feed the next MFMA as B operands straight from
// registers.
//
// Work runs on 32-row halves h of the streamed side: phase h issues the
// gradient products of half h-1, computes P and dS of half h on the VALU,
// and issues S and dP of half h+1.  Key units interleave the first two by
// hand; query units keep one S/dP set (the third workgroup per CU hides
// their latencies instead).
//
// Per output row the epilogue counts the patterns that keep it: a row kept by
// this pattern alone gets its rounded gradient directly, a row kept by several
// gets this pattern's fp32 partial in the pattern's own sparse-order buffer
// (write-once, contiguous rows), and a finalize pass sums the partials.
#include "dla_device.h"

namespace dla {

constexpr int kBwdRows = 128;   // rows a unit owns (4 waves x 32)
static_assert(kBwdRows == kBwdUnitRows, "the schedules and the kernel must agree on the unit size");
constexpr int kBwdTile = 64;    // streamed rows per LDS tile
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left alone
// (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8); OR-ing in n < 16
// allows n outstanding vector-memory operations.  Issued through the
// builtin, not inline asm, so that the compiler's own wait insertion sees
// it and accounts for every vector-memory operation it has placed.
constexpr int kVmcnt0 = 0x0F70;

struct __align__(16) BwdStage {
  uint4 a[kBwdTile * 8];   // Q (key units) or K (query units): 64 rows x 128 B
  uint4 b[kBwdTile * 8];   // dO (key units) or V (query units)
  // key units: -LSE * log2 e and -D of the tile's rows, in chunks of 16 rows:
  // row i at 32 * (i / 16) + i % 16 and D 16 floats later
  float ld[2 * kBwdTile];
};


// Number of patterns that keep row n of head h (n = h mod r for each).
__device__ __forceinline__ int kept_count(const AttnBwdArgs& a, int n, int h) {
  int c = 0;
  for (int i = 0; i < a.P; ++i) {
    const int ri = a.r[i];
    c += (ri & (ri - 1)) == 0 ? (((n ^ h) & (ri - 1)) == 0) : ((n % ri) == (h % ri));
  }
  return c;
}

__device__ __forceinline__ bf16x8 words_bf16(const uint32_t (&w)[8], int half) {
  return __builtin_bit_cast(bf16x8, uint4{w[4 * half], w[4 * half + 1], w[4 * half + 2], w[4 * half + 3]});
}

// kKV: key unit (dK, dV) or query unit (dQ).  kWin: the launch covers a
// window [qlo, qhi) of a segment's query rows (one sequence shard's queries
// against a gathered segment); every result is then an fp32 partial.  NS:
// LDS ring depth (4: tiles j+2 and j+3 in flight while tile j+1 is read; 3:
// tile j+2 only).
template <bool kKV, bool kWin, int NS>
__device__ __forceinline__ void bwd_unit(const AttnBwdArgs& a, BwdStage* ring, int p, int b, int h,
                                         int64_t seg, int tile) {
  constexpr int kIns = kKV ? 5 : 4;  // DMA instructions per tile and wave
  static_assert((NS - 2) * kIns < 16, "the waits encode vmcnt in 4 bits");
  static_assert(NS == 3 || NS == 4, "ring depth 3 or 4");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int li = lane & 31, lg = lane >> 5;
  const int w = a.w[p], r = a.r[p], L_full = a.L[p];
  // fewer in a cut-short last segment (of the sequence or of this batch's)
  const int L = seg_rows(batch_len(a.lengths, b, a.N), seg, w, r, h, L_full);
  if (tile * kBwdRows >= L) return;                    // nothing of this segment left
  const int64_t base_row = seg_base_row(seg, w, r, h);
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int64_t rstride = (int64_t)r * a.sn;
  const int64_t row_off = head_off + base_row * a.sn;
  const __bf16* Qh = (const __bf16*)a.q + row_off;
  const __bf16* Kh = (const __bf16*)a.k + row_off;
  const __bf16* Vh = (const __bf16*)a.v + row_off;
  const __bf16* Dh = (const __bf16*)a.dout + row_off;
  const float2* ldh = a.ld + ((int64_t)b * a.H + h) * a.N + base_row;  // row stride r
  const float c = a.scale_log2;

  // Owned rows: keys (key units) or queries (query units), 32 per wave.
  const int own0 = tile * kBwdRows + 32 * wave;
  const int own = own0 + li;
  const bool wave_valid = own0 < L;
  const int qlo = kWin ? a.qlo : 0, qhi = kWin ? a.qhi : L;  // query rows that exist
  const int send = kKV ? qhi : L;                    // end of the streamed rows
  const __bf16* srcA = kKV ? Qh : Kh;   // streamed tensors
  const __bf16* srcB = kKV ? Dh : Vh;
  const __bf16* ownA = kKV ? Kh : Qh;   // owned tensors (B operands)
  const __bf16* ownB = kKV ? Vh : Dh;
  bf16x8 opa[4], opb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (own < L) {
      opa[ks] = *(const bf16x8*)(ownA + (int64_t)own * rstride + 16 * ks + 8 * lg);
      opb[ks] = *(const bf16x8*)(ownB + (int64_t)own * rstride + 16 * ks + 8 * lg);
    } else {
      opa[ks] = bf16x8{};
      opb[ks] = bf16x8{};
    }
  }
  float nl2_own = 0.f, nd_own = 0.f;  // query units: -LSE * log2 e and -D of this lane's query
  if (!kKV && own < L) {
    const float2 x = ldh[(int64_t)own * r];
    nl2_own = x.x;
    nd_own = x.y;
  }
  f32x16 nd_tile;  // query units: -D of the lane's query in every element (dP's starting value)
#pragma unroll
  for (int e = 0; e < 16; ++e) nd_tile[e] = nd_own;

  // Streamed range: tiles t = 0..nt-1 start at row 64*(t_first + t); half h
  // covers streamed rows s0(h) = 64*t_first + 32h .. +32.
  int t_first, nt, h_lo, h_hi;
  if (kKV) {
    t_first = a.causal ? 2 * tile : 0;                 // queries >= the first owned key
    if (kWin) t_first = max(t_first, qlo / kBwdTile);
    nt = (send + kBwdTile - 1) / kBwdTile - t_first;
    h_lo = a.causal ? max(0, own0 - kBwdTile * t_first) / 32 : 0;  // first half with a query >= own0
    h_hi = (send - kBwdTile * t_first + 31) / 32;
  } else {
    t_first = 0;
    const int kend = a.causal ? min(L, tile * kBwdRows + kBwdRows) : L;
    nt = (kend + kBwdTile - 1) / kBwdTile;
    h_lo = 0;
    h_hi = a.causal ? min((L + 31) / 32, own0 / 32 + 1) : (L + 31) / 32;
  }
  auto active = [&](int hh) __attribute__((always_inline)) {
    return wave_valid && hh >= h_lo && hh < h_hi;
  };
  auto need_mask = [&](int hh) __attribute__((always_inline)) {
    const int s0 = kBwdTile * t_first + 32 * hh;
    const bool diag = a.causal && (kKV ? own0 + 31 > s0 : s0 + 31 > own0);
    return diag || (s0 + 32 > send) || (own0 + 32 > L);
  };

  // ---- HBM -> LDS: wave w fills rows [16w, 16w+16) of a tile, 8 rows per
  // instruction; lane l lands at row 16w + 8i + l/8, chunk slot l%8, and loads
  // the logical chunk that belongs there (u_swz depends on row % 16 only).
  // Rows past the segment end load row L-1 (finite values, masked later).
  const uint32_t rsb = (uint32_t)(rstride * 2);       // bytes between streamed rows
  const uint32_t span = 63u * rsb + 128u;              // bytes a tile's rows cover
  const int drow = 16 * wave + (lane >> 3);
  uint32_t choff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    choff[i] = 16u * (uint32_t)((lane & 7) ^ u_swz(8 * i + (lane >> 3)));
    voff[i] = (uint32_t)(drow + 8 * i) * rsb + choff[i];
  }
  // (-LSE2, -D) pairs of rows 16w .. 16w+15: lane l < 32 loads component
  // l / 16 of row 16w + l % 16, so the tile holds the two as separate runs.
  const uint32_t ld_voff = (uint32_t)(16 * wave + (lane & 15)) * (uint32_t)(8 * r) + 4u * ((lane >> 4) & 1);
  auto issue_tile = [&](int t, BwdStage* __restrict__ dst) __attribute__((always_inline)) {
    const int trow0 = kBwdTile * (t_first + t);
    const int lim = send - 1 - trow0;                   // last valid row of the tile
    const __amdgpu_buffer_rsrc_t ra = buf_rsrc(srcA + (int64_t)trow0 * rstride, span);
    const __amdgpu_buffer_rsrc_t rb = buf_rsrc(srcB + (int64_t)trow0 * rstride, span);
    uint32_t vo[2] = {voff[0], voff[1]};
    if (lim < kBwdTile - 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i) vo[i] = (uint32_t)min(drow + 8 * i, lim) * rsb + choff[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst->a + 8 * (16 * wave + 8 * i)), 16, vo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dst->b + 8 * (16 * wave + 8 * i)), 16, vo[i], 0, 0, 0);
    }
    if (kKV) {
      // (LSE*log2e, D) of rows 16w .. 16w+15: lanes 0..31 load one float each.
      const __amdgpu_buffer_rsrc_t rl = buf_rsrc(ldh + (int64_t)trow0 * r, 63u * (uint32_t)(8 * r) + 8u);
      uint32_t lo = ld_voff;
      if (lim < kBwdTile - 1)
        lo = (uint32_t)min(16 * wave + (lane & 15), lim) * (uint32_t)(8 * r) + 4u * ((lane >> 4) & 1);
      if (lane < 32)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)((float*)dst->ld + 32 * wave), 4, lo, 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets ----------------------------------------------
  int roff[4];                 // row-wise operand: row 32*blk + li, chunk 2ks + lg (+ blk*4096)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) roff[ks] = row_offset(lane, 0, ks);
  int tlo[2], thi[2];          // transposed operand of head-dim block db (+ kk*2048)
#pragma unroll
  for (int db = 0; db < 2; ++db) tr_offsets(lane, db, tlo[db], thi[db]);

  // ---- accumulators -----------------------------------------------------------
  f32x16 acc0[2], acc1[2];     // key units: dK^T[db], dV^T[db]; query units: dQ^T[db] in acc0
#pragma unroll
  for (int db = 0; db < 2; ++db) { acc0[db] = f32x16{}; acc1[db] = f32x16{}; }

  // ---- pipeline stages ------------------------------------------------------
  // S and dP of half hh (blk = hh & 1 within its tile).
  // The dP accumulator starts at -D of each element's query (key units: from
  // the tile's -D run; query units: the lane's own -D), so that
  // dS = P (dP - D) is one multiply.  (In key units element e = 4g + i of a
  // lane is streamed row 32 blk + 8g + 4 lg + i.)
  auto ld_offset = [&](int blk, int g) __attribute__((always_inline)) {
    return 4 * (32 * (2 * blk + (g >> 1)) + 8 * (g & 1) + 4 * lg);  // bytes; D 64 bytes later
  };
  auto stage_sd = [&](const BwdStage* __restrict__ st, int blk, f32x16& S, f32x16& P) __attribute__((always_inline)) {
    if (kKV) {
      typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 nd = *(const lds_f32x4*)((const lds_char*)st->ld + ld_offset(blk, g) + 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) P[4 * g + i] = nd[i];
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 xa = lds_read_b128((const lds_u4*)st->a, blk * 4096 + roff[ks]);
      const bf16x8 xb = lds_read_b128((const lds_u4*)st->b, blk * 4096 + roff[ks]);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, opa[ks], ks ? S : f32x16{}, 0, 0, 0);
      P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb, opb[ks], ks || kKV ? P : nd_tile, 0, 0, 0);
    }
  };
  // P and dS of half hh from its S and dP, packed to bf16 operand words.
  auto stage_valu = [&](int hh, const BwdStage* __restrict__ st, int blk, const f32x16& S,
                        const f32x16& P, bool masked, uint32_t (&pw)[8], uint32_t (&sw)[8]) __attribute__((always_inline)) {
    const int s0 = kBwdTile * t_first + 32 * hh;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float nl[4];
      if (kKV) {
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
        const f32x4 x = *(const lds_f32x4*)((const lds_char*)st->ld + ld_offset(blk, g));
#pragma unroll
        for (int i = 0; i < 4; ++i) nl[i] = x[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) nl[i] = nl2_own;
      }
      float pv[4], dv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * g + i;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c, nl[i]));
        if (masked) {
          const int srow = s0 + 8 * g + 4 * lg + i;
          const bool dead = kKV ? (srow >= send || own >= L || (a.causal && own > srow))
                                : (srow >= L || own >= L || (a.causal && srow > own));
          if (dead) p = 0.f;
        }
        pv[i] = p;
        dv[i] = p * P[e];
      }
      if (kKV) {
        pw[2 * g] = pack_bf16(pv[0], pv[1]);
        pw[2 * g + 1] = pack_bf16(pv[2], pv[3]);
      }
      sw[2 * g] = pack_bf16(dv[0], dv[1]);
      sw[2 * g + 1] = pack_bf16(dv[2], dv[3]);
    }
  };
  // Gradient products of half hh: key units dV^T += dO^T P, dK^T += Q^T dS;
  // query units dQ^T += K^T dS^T.
  auto stage_grad = [&](const BwdStage* __restrict__ st, int blk, const uint32_t (&pw)[8],
                        const uint32_t (&sw)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kko = (2 * blk + half) * 2048;
      const bf16x8 sb = words_bf16(sw, half);
      if (kKV) {
        const bf16x8 pb = words_bf16(pw, half);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 dta = lds_read_tr8((const lds_u4*)st->b, tlo[db] + kko, thi[db] + kko);
          const bf16x8 qta = lds_read_tr8((const lds_u4*)st->a, tlo[db] + kko, thi[db] + kko);
          acc1[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dta, pb, acc1[db], 0, 0, 0);
          acc0[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, sb, acc0[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 kta = lds_read_tr8((const lds_u4*)st->a, tlo[db] + kko, thi[db] + kko);
          acc0[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kta, sb, acc0[db], 0, 0, 0);
        }
      }
    }
  };

  // VALU chunk g (elements 4g .. 4g+3) of stage_valu with no mask.
  auto valu_chunk = [&](const BwdStage* __restrict__ st, int blk, int g, const f32x16& S,
                        const f32x16& P, uint32_t (&pw)[8], uint32_t (&sw)[8]) __attribute__((always_inline)) {
    float nl[4];
    if (kKV) {
      typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
      const f32x4 x = *(const lds_f32x4*)((const lds_char*)st->ld + ld_offset(blk, g));
#pragma unroll
      for (int i = 0; i < 4; ++i) nl[i] = x[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) nl[i] = nl2_own;
    }
    float pv[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * g + i;
      pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c, nl[i]));
      dv[i] = pv[i] * P[e];
    }
    if (kKV) {
      pw[2 * g] = pack_bf16(pv[0], pv[1]);
      pw[2 * g + 1] = pack_bf16(pv[2], pv[3]);
    }
    sw[2 * g] = pack_bf16(dv[0], dv[1]);
    sw[2 * g + 1] = pack_bf16(dv[2], dv[3]);
  };
  // Steady state of a query unit: gradient products of half hh-1, S/dP of
  // half hh+1 and dS of half hh, hand-interleaved in four groups separated by
  // scheduling fences.  A group issues the LDS reads of its three MFMA
  // operands, then four elements of VALU work (which covers the LDS latency),
  // then the MFMAs, which run while the next group's VALU issues.  (Key units
  // keep the compiler's schedule: their register budget has no room for it.)
  auto fused_q = [&](const BwdStage* __restrict__ sg, int blk_g, const uint32_t (&swp)[8],
                     const BwdStage* __restrict__ ss, int blk_s, f32x16& Sn, f32x16& Pn,
                     int blk_v, const f32x16& S, const f32x16& P, uint32_t (&pw)[8], uint32_t (&sw)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int half = q >> 1, db = q & 1;
      const int kko = (2 * blk_g + half) * 2048;
      const bf16x8 ka = lds_read_tr8((const lds_u4*)sg->a, tlo[db] + kko, thi[db] + kko);
      const bf16x8 xa = lds_read_b128((const lds_u4*)ss->a, blk_s * 4096 + roff[q]);
      const bf16x8 xb = lds_read_b128((const lds_u4*)ss->b, blk_s * 4096 + roff[q]);
      valu_chunk(ss, blk_v, q, S, P, pw, sw);
      acc0[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, words_bf16(swp, half), acc0[db], 0, 0, 0);
      Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, opa[q], q ? Sn : f32x16{}, 0, 0, 0);
      Pn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb, opb[q], q ? Pn : nd_tile, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Steady state of a key unit: gradient products of half hh-1 (dV and dK
  // of one head-dim block and 16-query step per group) interleaved with the
  // P/dS work of half hh, four groups separated by scheduling fences.  A
  // group issues the LDS reads of its two transposed operands, then its
  // four elements of VALU work (which cover the read latency), then its two
  // MFMAs, which run while the next group's VALU issues.
  auto fused_kv = [&](const BwdStage* __restrict__ sg, int blk_g, const uint32_t (&pwp)[8],
                      const uint32_t (&swp)[8], const BwdStage* __restrict__ sv, int blk_v,
                      const f32x16& S, const f32x16& P, uint32_t (&pw)[8], uint32_t (&sw)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int half = q >> 1, db = q & 1;
      const int kko = (2 * blk_g + half) * 2048;
      const bf16x8 dta = lds_read_tr8((const lds_u4*)sg->b, tlo[db] + kko, thi[db] + kko);
      const bf16x8 qta = lds_read_tr8((const lds_u4*)sg->a, tlo[db] + kko, thi[db] + kko);
      valu_chunk(sv, blk_v, q, S, P, pw, sw);
      acc1[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dta, words_bf16(pwp, half), acc1[db], 0, 0, 0);
      acc0[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, words_bf16(swp, half), acc0[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 sx, px, sy, py;                       // S, dP of the even (x) / odd (y) half in flight
  uint32_t pwx[8], swx[8], pwy[8], swy[8];     // packed P, dS of the even / odd half

  // One phase: gradient products of hh-1 (stage sg, block 1-blk), S/dP of
  // hh+1 (stage ss, block 1-blk), P/dS of hh (stage sv, block blk).  In the
  // steady state (all three halves active, no mask) they run in one block:
  //   query units: all three interleaved (S/dP double-buffered);
  //   key units:   gradient MFMAs interleaved with the VALU, then S/dP of hh+1
  //                into the registers the VALU just consumed (their register
  //                budget has no room for a second S/dP set).
  // S/dP of hh+1 is computed whether or not that half is active (on whatever
  // the stage holds; the result is only consumed when it is), so that the
  // registers are written on every path and never copied.  P/dS of a half
  // that does not run is marked dead for the same reason.
#define DLA_DEAD(x) x = __builtin_nondeterministic_value(x)
#define DLA_BWD_PHASE(hh, blk, sg, ss, sv, S_cur, P_cur, S_nxt, P_nxt, pw_cur, sw_cur, pw_prv, sw_prv) \
  do {                                                                                           \
    const bool a_prev = active((hh) - 1), a_cur = active(hh), a_next = active((hh) + 1);        \
    const bool msk = need_mask(hh);                                                              \
    if (!kKV && NS == 4 && a_prev && a_cur && a_next && !msk) {                                 \
      fused_q(sg, 1 - (blk), sw_prv, ss, 1 - (blk), S_nxt, P_nxt, blk, S_cur, P_cur, pw_cur, sw_cur); \
    } else {                                                                                     \
      if (kKV && !kWin && a_prev && a_cur && !msk) {                                             \
        fused_kv(sg, 1 - (blk), pw_prv, sw_prv, sv, blk, S_cur, P_cur, pw_cur, sw_cur);          \
      } else if (kKV && a_prev && a_cur && !msk) {                                               \
        stage_grad(sg, 1 - (blk), pw_prv, sw_prv);                                               \
        stage_valu(hh, sv, blk, S_cur, P_cur, false, pw_cur, sw_cur);                            \
        DLA_INTERLEAVE(8, 10);                                                                   \
      } else {                                                                                   \
        if (a_prev) stage_grad(sg, 1 - (blk), pw_prv, sw_prv);                                   \
        if (a_cur) {                                                                             \
          if (msk) stage_valu(hh, sv, blk, S_cur, P_cur, true, pw_cur, sw_cur);                  \
          else stage_valu(hh, sv, blk, S_cur, P_cur, false, pw_cur, sw_cur);                     \
        } else {                                                                                 \
          _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) { DLA_DEAD(pw_cur[i_]); DLA_DEAD(sw_cur[i_]); } \
        }                                                                                        \
      }                                                                                          \
      stage_sd(ss, 1 - (blk), S_nxt, P_nxt);                                                     \
    }                                                                                            \
    (void)a_next;                                                                                \
  } while (0)

  // Ring step j: phase 2j reads tiles j-1 and j; then wait until tile j+1
  // is in LDS, synchronise, refill the stage of tile j-1 with tile
  // j + NS - 1, and run phase 2j+1 on tiles j and j+1.  The
  // distinct restrict pointers tell the compiler that the DMA target is not
  // read after the refill, so it adds no waits of its own.
  auto ring_step = [&](int j, const BwdStage* __restrict__ sp, const BwdStage* __restrict__ sc,
                       const BwdStage* __restrict__ sn, BwdStage* __restrict__ si) __attribute__((always_inline)) {
    if (kKV || NS == 3) DLA_BWD_PHASE(2 * j, 0, sp, sc, sc, sx, px, sx, px, pwx, swx, pwy, swy);
    else DLA_BWD_PHASE(2 * j, 0, sp, sc, sc, sx, px, sy, py, pwx, swx, pwy, swy);
    // With a 4-stage ring tile j+2 (if it exists) may stay in flight; with 3
    // stages tile j+1 is the newest one issued.
    if (NS == 4 && j + 2 < nt)
      __builtin_amdgcn_s_waitcnt(kVmcnt0 | kIns);
    else
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (j + NS - 1 < nt) issue_tile(j + NS - 1, si);
    if (kKV || NS == 3) DLA_BWD_PHASE(2 * j + 1, 1, sc, sn, sc, sx, px, sx, px, pwy, swy, pwx, swx);
    else DLA_BWD_PHASE(2 * j + 1, 1, sc, sn, sc, sy, py, sx, px, pwy, swy, pwx, swx);
  };

  // Prologue: tiles 0 .. NS-2 in flight, wait for tile 0, S/dP of half 0.
  // (In a query window, a key tile past every query streams nothing and
  // writes zeros.)
  if (!kWin || nt > 0) {
  issue_tile(0, &ring[0]);
  if (nt > 1) issue_tile(1, &ring[1]);
  if (NS == 4 && nt > 2) issue_tile(2, &ring[2]);
  if (NS == 4 && nt > 2)
    __builtin_amdgcn_s_waitcnt(kVmcnt0 | (2 * kIns));   // tiles 1 and 2 may stay in flight
  else if (nt > 1)
    __builtin_amdgcn_s_waitcnt(kVmcnt0 | kIns);
  else
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  stage_sd(&ring[0], 0, sx, px);

  for (int j = 0; j < nt; ++j)
    ring_step(j, &ring[(j + NS - 1) % NS], &ring[j % NS], &ring[(j + 1) % NS], &ring[(j + NS - 1) % NS]);
  // Drain: gradient products of the last half.
  if (active(2 * nt - 1)) stage_grad(&ring[(nt - 1) % NS], 1, pwy, swy);
  }
#undef DLA_BWD_PHASE
#undef DLA_DEAD

  // ---- epilogue: each wave's 32 owned rows go through LDS (chunk c of row i
  // at c ^ (i & 15), 256 B per row and tensor), so that every global store
  // covers 4 whole rows with 16 bytes per lane.  A row kept by this pattern
  // alone gets its rounded gradient; a row that other patterns also keep gets
  // this pattern's fp32 partial (sparse order), summed later by the finalize
  // pass.
  __syncthreads();                                     // the ring is free
  constexpr int kTens = kKV ? 2 : 1;
  char* wbase = (char*)ring + wave * (kTens * 8192);
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  auto put = [&](int t, const f32x16 (&acc)[2], float sc) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        const int ch = 8 * db + 2 * eg + lg;
        const f32x4 v = {sc * acc[db][4 * eg], sc * acc[db][4 * eg + 1], sc * acc[db][4 * eg + 2],
                         sc * acc[db][4 * eg + 3]};
        *(lds_f32x4*)((lds_char*)wbase + t * 8192 + li * 256 + 16 * (ch ^ (li & 15))) = v;
      }
  };
  if (wave_valid) {
    put(0, acc0, a.scale);
    if (kKV) put(1, acc1, 1.f);
    const int cc = lane & 15;
    // (a window's dQ partial holds the window's rows only: nsp_q rows per
    // (batch, head), its base shifted back by qlo rows by the caller)
    const int64_t nsp = (kWin && !kKV) ? a.nsp_q : a.nsp[p];
    const int64_t part_row0 = ((int64_t)b * a.H + h) * nsp + seg * L_full + own0;
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
      const int rr = 4 * it + (lane >> 4);
      const int ownr = own0 + rr;
      if (ownr >= L) continue;
      const int n = (int)base_row + ownr * r;
      const bool shared = kWin || kept_count(a, n, h) > 1;
      const int64_t out_off = head_off + (int64_t)n * a.sn + 4 * cc;
      const int64_t part_off = (part_row0 + rr) * kD + 4 * cc;
#pragma unroll
      for (int t = 0; t < kTens; ++t) {
        const f32x4 v = *(const lds_f32x4*)((const lds_char*)wbase + t * 8192 + rr * 256 + 16 * (cc ^ (rr & 15)));
        const int g = kKV ? 1 + t : 0;               // 0: dQ, 1: dK, 2: dV
        if (shared) {
          *(f32x4*)(a.part[p][g] + part_off) = v;
        } else {
          __bf16* outp = (__bf16*)(g == 0 ? a.dq : g == 1 ? a.dk : a.dv) + out_off;
          *(uint2*)outp = uint2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        }
      }
    }
  }
}

// Key units (dK, dV): 4-stage ring, 256 VGPRs (two waves per SIMD: two
// workgroups per CU).  The schedules hand out the highest tile index first,
// which is the most work for a query tile; under a causal mask a key tile
// has the most work at index 0, so key tiles are taken in reverse.  Units
// that touch the same rows are spread over the launch (a burst of them
// would contend for the same L2 and memory channels).
template <bool kWin>
__global__ __launch_bounds__(256, 2) void attn_bwd_kv_kernel(const AttnBwdArgs a) {
  __shared__ BwdStage ring[4];
  int p, b, h, tile;
  int64_t seg;
  if (!decode_unit(a.sched_kv, blockIdx.x, (int)a.H, a.nseg, p, b, h, seg, tile)) return;
  if (a.causal) tile = (a.L[p] + kBwdRows - 1) / kBwdRows - 1 - tile;
  bwd_unit<true, kWin, 4>(a, ring, p, b, h, seg, tile);
}

// Query units (dQ): 3-stage ring (49.5 KB) and at most 168 VGPRs (three
// waves per SIMD), so that three workgroups share a CU.  They run after the
// key units, in a launch of their own.
template <bool kWin>
__global__ __launch_bounds__(256, 3) void attn_bwd_q_kernel(const AttnBwdArgs a) {
  __shared__ BwdStage ring[3];
  int p, b, h, tile;
  int64_t seg;
  if (!decode_unit(a.sched_q, blockIdx.x, (int)a.H, a.nseg, p, b, h, seg, tile)) return;
  if (kWin) tile += a.qlo / kBwdRows;                // the window's query tiles
  bwd_unit<false, kWin, 3>(a, ring, p, b, h, seg, tile);
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.sched_kv.total + a.sched_q.total == 0) return hipSuccess;
  TimedLaunch tl("attn_bwd", stream);
  if (a.sched_kv.total > 0) {
    if (a.qhi > 0)
      hipLaunchKernelGGL(attn_bwd_kv_kernel<true>, dim3((unsigned)a.sched_kv.total), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_bwd_kv_kernel<false>, dim3((unsigned)a.sched_kv.total), dim3(256), 0, stream, a);
  }
  if (a.sched_q.total > 0) {
    if (a.qhi > 0)
      hipLaunchKernelGGL(attn_bwd_q_kernel<true>, dim3((unsigned)a.sched_q.total), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_bwd_q_kernel<false>, dim3((unsigned)a.sched_q.total), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dla
