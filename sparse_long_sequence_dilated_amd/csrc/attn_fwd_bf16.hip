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
// 4-stage LDS ring (64 KB) with global_load_lds_dwordx4, three tiles ahead of
// use, so no registers stage them.  Each lane picks the source chunk that
// belongs at its LDS slot, which yields swizzled layouts: K row-major with
// chunk c of row i at c ^ t_swz(i) (conflict-free MFMA operand reads), V
// row-major with chunk c of row i at c ^ 2*(i & 3) (conflict-free transposed
// reads).  V^T operands come from ds_read_b64_tr_b16, which hands each lane
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

__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 1; }

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const AttnFwdArgs a) {
  __shared__ FwdStage ring[kStages];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const int qw0 = q0 + wave * 64;
  const int kend = a.causal ? min(L, q0 + kFwdBM) : L;
  const int nkt = (kend + kFwdBN - 1) / kFwdBN;            // LDS tiles the workgroup stages
  const bool wave_active = qw0 < L;
  const int wave_kend = a.causal ? min(L, qw0 + 64) : L;
  const int nh = wave_active ? (wave_kend + 31) / 32 : 0;   // half tiles this wave computes
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
  // logical chunk that belongs there.  Rows past the segment end load row L-1
  // (finite values; the softmax masks those keys).
  const int dma_row0 = 16 * wave + (lane >> 3);
  const int dma_slot = lane & 7;
  auto issue_tile = [&](int kt, lds_u4* __restrict__ kdst, lds_u4* __restrict__ vdst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = dma_row0 + 8 * i;
      const int grow = min(kt * kFwdBN + row, L - 1);
      const __bf16* ks = Kh + (int64_t)grow * rstride + 8 * (dma_slot ^ t_swz(row));
      const __bf16* vs = Vh + (int64_t)grow * rstride + 8 * (dma_slot ^ v_swz(row));
      __builtin_amdgcn_global_load_lds((glb_void*)ks, (void __attribute__((address_space(3)))*)(kdst + 8 * (16 * wave + 8 * i)), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void*)vs, (void __attribute__((address_space(3)))*)(vdst + 8 * (16 * wave + 8 * i)), 16, 0, 0);
    }
  };

  // ---- per-lane LDS operand addresses -----------------------------------------
  // K operand (row 32kb + li, logical chunk 2ks + lg): byte offset within a stage's K.
  int kaddr[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kaddr[kb][ks] = 16 * r_index(32 * kb + li, 2 * ks + lg);
  // V^T operand via transposed reads: lane l = 16m + t supplies row
  // 16kk + 8*half + 4*(m/2) + t/4 and head dims 32db + 16(m%2) + 4(t%4) .. +4;
  // it receives keys (16kk + 8*half + 4*lg) .. +3 of head dim 32db + li.
  int vaddr[2];
  {
    const int t = lane & 15, m = lane >> 4;
    const int rowoff = 4 * (m >> 1) + (t >> 2);
    const int dchunk = 2 * (m & 1) + ((t & 3) >> 1);
#pragma unroll
    for (int db = 0; db < 2; ++db)
      vaddr[db] = rowoff * 128 + (((4 * db + dchunk) ^ v_swz(rowoff)) << 4) + 8 * (t & 1);
  }

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
    for (int ks = 0; ks < 4; ++ks)
      kop[ks] = __builtin_bit_cast(bf16x8, *(const lds_u4*)((const lds_char*)kst + kaddr[kb][ks]));
  };
  auto read_v = [&](const lds_u4* __restrict__ vst, int half, bf16x8 (&vop)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {
        const int kk = 2 * half + kl;
        const lds_char* base = (const lds_char*)vst + vaddr[db] + kk * 16 * 128;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + 8 * 128));
        vop[db][kl] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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

  f32x16 sa[2], sb[2];     // S of the current and the next half tile, [qb]
  uint32_t p0[8], p1[8];   // packed P of query halves 0 and 1

  // One half-tile step: `cur` holds S_h, p0 holds P_h of query half 0.
  // kst_next: K of the stage holding half tile hh+1; vst: V of hh's stage.
  auto step = [&](int hh, f32x16 (&cur)[2], f32x16 (&nxt)[2], const lds_u4* __restrict__ kst_next,
                  const lds_u4* __restrict__ vst) __attribute__((always_inline)) {
    const bool has_next = hh + 1 < nh;
    bf16x8 vop[2][2], kop[4];
    if (has_next) {
      read_k(kst_next, (hh + 1) & 1, kop);
      mfma_s(kop, nxt);                                   // phase A
      const float rs1 = make_p(cur[1], m_run[1], p1);
      DLA_INTERLEAVE(8, 6);
      finish_p(cur[1], 1, rs1, p1);
      mask_s(hh + 1, nxt);
      apply_rescale();
      read_v(vst, hh & 1, vop);
      mfma_o(vop, p0, p1);                                // phase B
      const float rs0 = make_p(nxt[0], m_run[0], p0);
      DLA_INTERLEAVE(8, 6);
      finish_p(nxt[0], 0, rs0, p0);
    } else {
      const float rs1 = make_p(cur[1], m_run[1], p1);
      finish_p(cur[1], 1, rs1, p1);
      apply_rescale();
      read_v(vst, hh & 1, vop);
      mfma_o(vop, p0, p1);
    }
  };

  // One ring step j (j >= -3): issue tile j+3; at j == -1 start the pipeline
  // (S_0 and P_0 of query half 0); at j >= 0 compute half tiles 2j and 2j+1,
  // which read K of tiles j and j+1 and V of tile j.  Then wait until tile j+2
  // is in LDS (tile j+3 may stay in flight) and synchronise.  Every DMA and
  // every LDS read of the loop lives in this one inlined body, and its
  // distinct restrict pointers tell the compiler that the DMA target never
  // aliases the stages being read, so it adds no waits of its own.
  auto ring_step = [&](int j, lds_u4* __restrict__ dk, lds_u4* __restrict__ dv,
                       const lds_u4* __restrict__ k_j, const lds_u4* __restrict__ v_j,
                       const lds_u4* __restrict__ k_j1) __attribute__((always_inline)) {
    const bool issue = j + 3 < nkt;
    if (issue) issue_tile(j + 3, dk, dv);
    if (j == -1 && nh > 0) {
      bf16x8 kop[4];
      read_k(k_j1, 0, kop);
      mfma_s(kop, sa);
      mask_s(0, sa);
      const float rs = make_p(sa[0], m_run[0], p0);
      finish_p(sa[0], 0, rs, p0);
    }
    if (j >= 0 && 2 * j < nh) step(2 * j, sa, sb, k_j, v_j);
    if (j >= 0 && 2 * j + 1 < nh) step(2 * j + 1, sb, sa, k_j1, v_j);
    if (issue) {
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  auto stage_k = [&](int j) __attribute__((always_inline)) { return (lds_u4*)ring[(j + kStages) % kStages].k; };
  auto stage_v = [&](int j) __attribute__((always_inline)) { return (lds_u4*)ring[(j + kStages) % kStages].v; };
  for (int j = -3; j < nkt; ++j)
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
