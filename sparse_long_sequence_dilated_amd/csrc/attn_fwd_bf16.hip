// Dilated attention forward, bf16 in, fp32 accumulation, gfx950 MFMA.
//
// One workgroup = one unit: 256 consecutive sparse query rows of one
// (pattern, batch, head, segment).  The kernel gathers the dilated rows of
// Q, K and V straight from the [B, N, H, D] tensors (every row a contiguous
// 128-byte run, consecutive sparse rows r*stride_n apart) and runs dense
// softmax attention inside the sparsified segment (the gptget.net LongNet
// summary, sections 方法论 and 方法详解).  Patterns are merged afterwards with
// exp(LSE) weights (darcstar.tech LongNet page, DarcStar commentary); this
// kernel writes each pattern's normalised output and its per-row LSE.
//
// Data movement: K and V tiles of 64 sparse rows go from HBM straight into a
// 4-stage LDS ring (64 KB) with buffer_load_dwordx4 ... lds, three tiles ahead
// of use, so no registers stage them.  Each lane picks the source chunk that
// belongs at its LDS slot, which yields one swizzled row-major layout for K
// and V, chunk c of row i at c ^ u_swz(i), conflict-free both for the K
// operand reads (ds_read_b128) and for the transposed V reads.  V^T operands come from ds_read_b64_tr_b16, which hands each lane
// four consecutive keys of one head dimension.
//
// Compute: 4 waves x 64 query rows, two workgroups per CU.  A wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on the rows, so a lane holds
// one query's scores for 16 keys per block) and O^T += V^T P^T, feeding P^T
// to the MFMA straight from the S^T accumulator layout.  The work runs on
// 32-key half tiles h with the two 32-query halves skewed by one phase:
//   phase A(h): S_{h+1} = K_{h+1} Q^T          || P_h, query half 1
//   phase B(h): O^T += V_h^T P_h (both halves)  || P_{h+1}, query half 0
// Softmax in the exp2 domain with a lazily updated offset: P is computed with
// the current running maximum and accepted unless a lane's partial row sum
// exceeds 2^16 (always the case on the first tile, where the offset is -inf);
// then the true row maximum is taken, P recomputed, and the rescale of O and
// l is applied before O's next update.  Row sums add the bf16-rounded P that
// feeds the MFMA (v_dot2c_f32_bf16).
#include "dla_device.h"

namespace dla {

constexpr int kFwdBM = 256;      // sparse query rows per workgroup
constexpr int kFwdBN = 64;       // keys per LDS tile (two 32-key half tiles)
constexpr int kStages = 4;       // LDS ring depth (tiles in flight: 3)
constexpr float kSumLimit = 65536.f;

struct __align__(16) FwdStage {
  uint4 k[kFwdBN * 8];  // 8 KB
  uint4 v[kFwdBN * 8];  // 8 KB
};

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const AttnFwdArgs a) {
  __shared__ FwdStage ring[kStages];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31, lg = lane >> 5;

  int p, b, h, tile;
  int64_t seg;
  decode_unit(a.sched, blockIdx.x, (int)a.H, a.nseg, p, b, h, seg, tile);
  const int w = a.w[p], r = a.r[p], L = a.L[p];
  const int64_t base_row = seg_base_row(seg, w, r, h);
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int64_t rstride = (int64_t)r * a.sn;  // elements between consecutive sparse rows
  const __bf16* Qh = (const __bf16*)a.q + head_off + base_row * a.sn;
  const __bf16* Kh = (const __bf16*)a.k + head_off + base_row * a.sn;
  const __bf16* Vh = (const __bf16*)a.v + head_off + base_row * a.sn;

  const int q0 = tile * kFwdBM;
  const int qw0 = (q0 + wave * 64);  // wave-uniform (SGPR)
  const int kend = a.causal ? min(L, q0 + kFwdBM) : L;
  const int nkt = (kend + kFwdBN - 1) / kFwdBN;            // LDS tiles the workgroup stages
  const bool wave_active = qw0 < L;
  const int wave_kend = a.causal ? min(L, qw0 + 64) : L;
  const int nh = (wave_active ? (wave_kend + 31) / 32 : 0);  // half tiles this wave computes
  const float c = a.scale_log2;

  // Q as the B operand: lane (query li, group lg) holds d = 16*ks + 8*lg .. +8.
  bf16x8 qop[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw0 + 32 * qb + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qop[qb][ks] = row < L ? *(const bf16x8*)(Qh + (int64_t)row * rstride + 16 * ks + 8 * lg)
                            : bf16x8{};
  }

  // ---- HBM -> LDS: wave w fills rows [16w, 16w+16) of a tile, 8 rows per instruction.
  // Lane l of instruction i lands at row 16w + 8i + l/8, slot l%8; it loads the
  // logical chunk that belongs there.  The tile's first row is the buffer base
  // (scalar), so a lane's byte offset is the same for every tile; rows past the
  // segment end load row L-1 (finite values; the softmax masks those keys).
  const int dma_row0 = 16 * wave + (lane >> 3);
  const int dma_slot = lane & 7;
  const uint32_t rsb = (uint32_t)(rstride * 2);       // bytes between sparse rows
  const uint32_t span = 63u * rsb + 128u;              // bytes a tile's rows cover
  // K and V share one swizzle (u_swz, a function of row % 16 = 8i + l/8), so
  // a lane's source offset is the same for both.
  uint32_t doff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    doff[i] = (uint32_t)(dma_row0 + 8 * i) * rsb + 16u * (uint32_t)(dma_slot ^ u_swz(8 * i + (lane >> 3)));
  auto issue_tile = [&](int kt, lds_u4* __restrict__ kdst, lds_u4* __restrict__ vdst) __attribute__((always_inline)) {
    const int trow0 = kt * kFwdBN;
    const int lim = L - 1 - trow0;                      // last valid row of the tile
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(Kh + (int64_t)trow0 * rstride, span);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(Vh + (int64_t)trow0 * rstride, span);
    uint32_t o[2] = {doff[0], doff[1]};
    if (lim < kFwdBN - 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        o[i] = (uint32_t)min(dma_row0 + 8 * i, lim) * rsb +
               16u * (uint32_t)(dma_slot ^ u_swz(8 * i + (lane >> 3)));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kdst + 8 * (16 * wave + 8 * i)), 16, o[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vdst + 8 * (16 * wave + 8 * i)), 16, o[i], 0, 0, 0);
    }
  };

  // ---- per-lane LDS operand addresses -----------------------------------------
  // K operand (row 32kb + li, logical chunk 2ks + lg): byte offset within a
  // stage's K, + kb * 4096.
  int kaddr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kaddr[ks] = row_offset(lane, 0, ks);
  // V^T operand via transposed reads (keys 16kk + 4*lg + {0..3, 8..11} of head
  // dim 32db + li): byte offsets of the two 4-key halves, + kk * 2048.
  int vlo[2], vhi[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) tr_offsets(lane, db, vlo[db], vhi[db]);

  f32x16 oacc[2][2];  // [db][qb]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  float pend[2] = {1.f, 1.f};   // O rescale factor owed before O's next update

  // ---- building blocks ------------------------------------------------------
  auto read_k = [&](const lds_u4* __restrict__ kst, int kb, bf16x8 (&kop)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kop[ks] = lds_read_b128(kst, kb * 4096 + kaddr[ks]);
  };
  auto read_v = [&](const lds_u4* __restrict__ vst, int half, bf16x8 (&vop)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {
        const int kk = 2 * half + kl;
        vop[db][kl] = lds_read_tr8(vst, vlo[db] + kk * 2048, vhi[db] + kk * 2048);
      }
  };
  auto mfma_s = [&](const bf16x8 (&kop)[4], f32x16 (&s)[2]) __attribute__((always_inline)) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[0][ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[1][ks], s[1], 0, 0, 0);
    }
  };
  auto mfma_o = [&](const bf16x8 (&vop)[2][2], const uint32_t (&p0)[8], const uint32_t (&p1)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, uint4{p0[4 * kl], p0[4 * kl + 1], p0[4 * kl + 2], p0[4 * kl + 3]});
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, uint4{p1[4 * kl], p1[4 * kl + 1], p1[4 * kl + 2], p1[4 * kl + 3]});
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][kl], b0, oacc[db][0], 0, 0, 0);
        oacc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][kl], b1, oacc[db][1], 0, 0, 0);
      }
    }
  };
  // P of one 32x32 block with offset m: 8 packed bf16 words, returns the lane's partial sum.
  auto make_p = [&](const f32x16& s, float m, uint32_t (&pw)[8]) __attribute__((always_inline)) -> float {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], c, -m));
      const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], c, -m));
      pw[i] = pack_bf16(x0, x1);
      if (i & 1) acc1 = dot2_bf16_ones(pw[i], acc1); else acc0 = dot2_bf16_ones(pw[i], acc0);
    }
    return acc0 + acc1;
  };
  // Accept P computed with the running offset, or redo it with the true maximum.
  auto finish_p = [&](const f32x16& s, int qb, float rs, uint32_t (&pw)[8]) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(!(rs <= kSumLimit)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = xhalf_max(mx) * c;
      const float m_new = fmaxf(m_run[qb], mx);
      const float alpha = (m_run[qb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      pend[qb] *= alpha;
      l_run[qb] *= alpha;
      m_run[qb] = m_new;
      rs = make_p(s, m_new == -INFINITY ? 0.f : m_new, pw);
    }
    l_run[qb] += rs;
  };
  // Causal diagonal / ragged tail mask of half tile hh.
  auto mask_s = [&](int hh, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const int k0 = hh * 32;
    if (!((k0 + 32 > L) || (a.causal && k0 + 32 > qw0))) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + (e >> 2) * 8 + lg * 4 + (e & 3);
        const int q = qw0 + 32 * qb + li;
        if (key >= L || (a.causal && key > q)) s[qb][e] = -INFINITY;
      }
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      if (__builtin_amdgcn_ballot_w64(pend[qb] != 1.f) != 0) {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][qb][e] *= pend[qb];
        pend[qb] = 1.f;
      }
  };

  // Four elements (e = 4g .. 4g+3) of P for block s with offset m: two packed
  // bf16 words; the row-sum terms go to two accumulators (short dependency
  // chains).
  auto p_chunk = [&](const f32x16& s, float m, int g, uint32_t (&pw)[8], float& r0, float& r1) __attribute__((always_inline)) {
    const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g], c, -m));
    const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 1], c, -m));
    const float x2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 2], c, -m));
    const float x3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 3], c, -m));
    pw[2 * g] = pack_bf16(x0, x1);
    pw[2 * g + 1] = pack_bf16(x2, x3);
    r0 = dot2_bf16_ones(pw[2 * g], r0);
    r1 = dot2_bf16_ones(pw[2 * g + 1], r1);
  };

  f32x16 sa[2], sb[2];     // S of the current and the next half tile, [qb]
  uint32_t pa[8], pb[8];   // packed P of query half 0, current and next (alternating)
  uint32_t p1[8];          // packed P of query half 1

  // One half-tile step, hand-interleaved: each group of two MFMAs is followed
  // by the softmax VALU work of four elements that does not depend on them,
  // and a scheduling fence keeps the compiler from regrouping (and from
  // hoisting work, which would raise register pressure).
  //   phase A: S_{h+1} = K_{h+1} Q^T (8 MFMAs) || P_h of query half 1
  //   phase B: O^T += V_h^T P_h (8 MFMAs)      || P_{h+1} of query half 0
  // `cur` holds S_h, p0c holds P_h of query half 0, p0n receives P_{h+1}.
  // kst_next: K of the stage holding half tile hh+1; vst: V of hh's stage.
  auto step = [&](int hh, f32x16 (&cur)[2], f32x16 (&nxt)[2], uint32_t (&p0c)[8],
                  uint32_t (&p0n)[8], const lds_u4* __restrict__ kst_next,
                  const lds_u4* __restrict__ vst) __attribute__((always_inline)) {
    const bool has_next = hh + 1 < nh;
    bf16x8 vop[2][2], kop[4];
    if (has_next) {
      read_k(kst_next, (hh + 1) & 1, kop);
      read_v(vst, hh & 1, vop);
      __builtin_amdgcn_sched_barrier(0);
      float r0 = 0.f, r1 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {                   // phase A
        nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[0][ks], ks ? nxt[0] : f32x16{}, 0, 0, 0);
        nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[1][ks], ks ? nxt[1] : f32x16{}, 0, 0, 0);
        p_chunk(cur[1], m_run[1], ks, p1, r0, r1);
        __builtin_amdgcn_sched_barrier(0);
      }
      finish_p(cur[1], 1, r0 + r1, p1);
      mask_s(hh + 1, nxt);
      apply_rescale();
      r0 = 0.f;
      r1 = 0.f;
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {                   // phase B
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, uint4{p0c[4 * kl], p0c[4 * kl + 1], p0c[4 * kl + 2], p0c[4 * kl + 3]});
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, uint4{p1[4 * kl], p1[4 * kl + 1], p1[4 * kl + 2], p1[4 * kl + 3]});
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][kl], b0, oacc[db][0], 0, 0, 0);
          oacc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][kl], b1, oacc[db][1], 0, 0, 0);
          p_chunk(nxt[0], m_run[0], 2 * kl + db, p0n, r0, r1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      finish_p(nxt[0], 0, r0 + r1, p0n);
    } else {
      const float rs1 = make_p(cur[1], m_run[1], p1);
      finish_p(cur[1], 1, rs1, p1);
      apply_rescale();
      read_v(vst, hh & 1, vop);
      mfma_o(vop, p0c, p1);
    }
  };

  // One ring step j >= 0: issue tile j+3, compute half tiles 2j and 2j+1,
  // which read K of tiles j and j+1 and V of tile j, then wait until tile j+2
  // is in LDS (tile j+3 may stay in flight) and synchronise.  Every DMA and
  // every LDS read of the loop lives in this one inlined body, and its
  // distinct restrict pointers tell the compiler that the DMA target never
  // aliases the stages being read, so it adds no waits of its own.
  auto ring_step = [&](int j, lds_u4* __restrict__ dk, lds_u4* __restrict__ dv,
                       const lds_u4* __restrict__ k_j, const lds_u4* __restrict__ v_j,
                       const lds_u4* __restrict__ k_j1) __attribute__((always_inline)) {
    const bool issue = j + 3 < nkt;
    if (issue) issue_tile(j + 3, dk, dv);
    if (2 * j < nh) step(2 * j, sa, sb, pa, pb, k_j, v_j);
    if (2 * j + 1 < nh) step(2 * j + 1, sb, sa, pb, pa, k_j1, v_j);
    if (issue) {
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Prologue (kept out of the loop so that nothing in it is loop-invariant):
  // tiles 0..2 in flight, S and P of half tile 0 once tile 0 has landed.
  issue_tile(0, (lds_u4*)ring[0].k, (lds_u4*)ring[0].v);
  if (nkt > 1) {
    issue_tile(1, (lds_u4*)ring[1].k, (lds_u4*)ring[1].v);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (nkt > 2) issue_tile(2, (lds_u4*)ring[2].k, (lds_u4*)ring[2].v);
  if (nh > 0) {
    bf16x8 kop[4];
    read_k((const lds_u4*)ring[0].k, 0, kop);
    mfma_s(kop, sa);
    mask_s(0, sa);
    const float rs = make_p(sa[0], m_run[0], pa);
    finish_p(sa[0], 0, rs, pa);
  }
  if (nkt > 2) {
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  auto stage_k = [&](int j) __attribute__((always_inline)) { return (lds_u4*)ring[j % kStages].k; };
  auto stage_v = [&](int j) __attribute__((always_inline)) { return (lds_u4*)ring[j % kStages].v; };
  for (int j = 0; j < nkt; ++j)
    ring_step(j, stage_k(j + 3), stage_v(j + 3), stage_k(j), stage_v(j), stage_k(j + 1));

  if (!wave_active) return;
  const bool is_prim = (p == a.prim);
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t nsparse = a.nsp[p];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = xhalf_sum(l_run[qb]);
    const int row = qw0 + 32 * qb + li;
    if (row >= L) continue;
    const float inv = 1.f / lt;
    const float lse = (m_run[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
    __bf16* dst;
    float* lse_dst;
    if (is_prim) {
      const int64_t n = base_row + (int64_t)row * r;
      dst = (__bf16*)a.o + head_off + n * a.sn;
      lse_dst = a.lse + bh * a.N + n;
    } else {
      const int64_t m = seg * L + row;
      dst = (__bf16*)a.part_o[p] + (bh * nsparse + m) * kD;
      lse_dst = a.part_lse[p] + bh * nsparse + m;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        const f32x16& ov = oacc[db][qb];
        uint2 st;
        st.x = pack_bf16(ov[4 * eg] * inv, ov[4 * eg + 1] * inv);
        st.y = pack_bf16(ov[4 * eg + 2] * inv, ov[4 * eg + 3] * inv);
        *(uint2*)(dst + 32 * db + 8 * eg + 4 * lg) = st;
      }
    if (lg == 0) *lse_dst = lse;
  }
}

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a, hipStream_t stream) {
  if (a.sched.total == 0) return hipSuccess;
  TimedLaunch tl("attn_fwd", stream);
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3((unsigned)a.sched.total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
