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
// 5-stage LDS ring (80 KB, so two workgroups fill the CU's 160 KB) with
// buffer_load_dwordx4 ... lds, so no registers stage them.  The workgroup
// synchronises once per two tiles: each barrier both publishes the two tiles
// loaded one window earlier and frees the two stages the next loads reuse.  Each lane picks the source chunk that
// belongs at its LDS slot, which yields one swizzled row-major layout for K
// and V, chunk c of row i at c ^ u_swz(i), conflict-free both for the K
// operand reads (ds_read_b128) and for the transposed V reads
// (ds_read_b64_tr_b16, which hands each lane four consecutive keys of one
// head dimension).
//
// Compute: 8 waves x 32 query rows, two workgroups per CU (four waves per
// SIMD, which is what hides the LDS, MFMA and exp latencies; a wave owns few
// rows so that its registers fit that occupancy, and the launch bound holds
// the compiler to the 128 VGPRs it allows).  A wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on the rows, so a lane
// holds one query's scores for 16 keys of a 32-key half tile) and
// O^T += V^T P^T, feeding P^T to the MFMA straight from the S^T accumulator
// layout.  Half tile h runs as one phase:
//   O^T += V_{h-1}^T P_{h-1} (4 MFMAs)  ||  P_h = exp2(S_h c - m)  (VALU)
//   then S_{h+1} = K_{h+1} Q^T (4 MFMAs) into the registers S_h leaves free.
// Softmax in the exp2 domain with a lazily updated offset: a wave's first
// half tile sets it to the exact row maximum; later ones compute P with the
// current offset and accept it unless a lane's partial row sum exceeds 2^16,
// in which case the true row maximum is taken, P recomputed, and the rescale
// of O and l is applied before O's next update.  Row sums add the
// bf16-rounded P that feeds the MFMA (v_dot2c_f32_bf16).
//
// 8-bit keys and values (the quantization the gptget.net page, section
// 方法详解, pairs with the method): K and V arrive as FP8 E4M3 codes with one
// scale per (batch, head).  Every E4M3 value is exact in bf16, so the tiles
// are decoded to bf16 on their way into the same LDS ring and the MFMA loop
// is unchanged; the key scale folds into the softmax constant and the value
// scale into the epilogue.  The codes take a register detour (global load,
// v_cvt_scalef32_pk_bf16_fp8, ds_write) instead of the DMA: each lane loads
// 8 codes of a tile one window ahead and writes their bf16 image after the
// next barrier, into the stage the DMA would have filled.
#include "dla_device.h"

namespace dla {

constexpr int kFwdBM = 256;      // sparse query rows per workgroup (8 waves x 32)
constexpr int kFwdBN = 64;       // keys per LDS tile (two 32-key half tiles)
constexpr int kStages = 5;       // LDS ring depth
constexpr int kFwdWaves = 8;
constexpr float kSumLimit = 65536.f;
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8).  Issued through the builtin, not inline asm, so that the compiler's
// own wait insertion sees them and knows which loads have completed.
constexpr int kVmcnt0 = 0x0F70;
constexpr int kLgkmcnt0 = 0xC07F;  // LDS (and scalar) operations only

struct __align__(16) FwdStage {
  uint4 k[kFwdBN * 8];  // 8 KB
  uint4 v[kFwdBN * 8];  // 8 KB
};

// kShard: some pattern reads gathered keys (a sequence shard); the plain
// instantiation has none of that logic.  kFp8: keys and values are E4M3
// codes (never together with kShard).
template <bool kShard, bool kFp8>
__global__ __launch_bounds__(512, 4) void attn_fwd_bf16_kernel(const AttnFwdArgs a) {
  static_assert(!(kShard && kFp8), "sequence shards read bf16 keys");
  __shared__ FwdStage ring[kStages];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, lg = lane >> 5;

  int p, b, h, tile;
  int64_t seg;
  if (!decode_unit(a.sched, blockIdx.x, (int)a.H, a.nseg, p, b, h, seg, tile)) return;
  // L query rows (local), Lk key rows; local query row i is row qoff + i of
  // the segment (qoff = 0 and Lk = L except for a segment that spans
  // several sequence shards, whose keys come from the gathered buffers).
  const int w = a.w[p], r = a.r[p], L_full = a.L[p];
  // A cut-short last segment holds fewer rows (a pattern spanning shards
  // never has one: its segment is whole by construction).
  const bool ext = kShard && a.ext_k[p] != nullptr;
  const int L = ext ? L_full : seg_rows(batch_len(a.lengths, b, a.N), seg, w, r, h, L_full);
  if (tile * kFwdBM >= L) return;                      // nothing of this segment left
  const int Lk = kShard ? a.Lk[p] : L, qoff = kShard ? a.qoff[p] : 0;
  const int64_t base_row = seg_base_row(seg, w, r, h);
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int64_t rstride = (int64_t)r * a.sn;  // elements between consecutive sparse rows
  const __bf16* Qh = (const __bf16*)a.q + head_off + base_row * a.sn;
  const int64_t cr = a.nsp[p];                 // rows per gathered chunk
  // bf16 keys and values (8-bit ones are addressed in bytes below)
  const __bf16* Kh = kFp8 ? nullptr
                   : ext  ? (const __bf16*)a.ext_k[p] + ((int64_t)b * a.H + h) * cr * kD
                          : (const __bf16*)a.k + head_off + base_row * a.sn;
  const __bf16* Vh = kFp8 ? nullptr
                   : ext  ? (const __bf16*)a.ext_v[p] + ((int64_t)b * a.H + h) * cr * kD
                          : (const __bf16*)a.v + head_off + base_row * a.sn;
  const int64_t kstride = ext ? (int64_t)kD : rstride;   // elements between key rows

  const int q0 = tile * kFwdBM;
  const int qw0 = q0 + wave * 32;                          // this wave's first query row
  const int qg0 = qoff + q0, qgw0 = qoff + qw0;            // the same as rows of the segment
  const int kend = a.causal ? min(Lk, qg0 + kFwdBM) : Lk;
  const int nkt = (kend + kFwdBN - 1) / kFwdBN;            // LDS tiles the workgroup stages
  const bool wave_active = qw0 < L;
  const int wave_kend = a.causal ? min(Lk, qgw0 + 32) : Lk;
  const int nh = wave_active ? (wave_kend + 31) / 32 : 0;  // half tiles this wave computes
  const float c = kFp8 ? a.scale_log2 * a.k_scale[(int64_t)b * a.H + h] : a.scale_log2;

  // Q as the B operand: lane (query li, group lg) holds d = 16*ks + 8*lg .. +8.
  bf16x8 qop[4];
  {
    const int row = qw0 + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qop[ks] = row < L ? *(const bf16x8*)(Qh + (int64_t)row * rstride + 16 * ks + 8 * lg) : bf16x8{};
  }

  // ---- HBM -> LDS: wave w fills rows [8w, 8w+8) of a tile with one
  // instruction per tensor; lane l lands at row 8w + l/8, slot l%8, and loads
  // the logical chunk that belongs there (u_swz depends on row % 16).  The
  // tile's first row is the buffer base (scalar), so a lane's byte offset is
  // the same for every tile; rows past the segment end (only in the tile
  // holding row L-1) load row L-1 (finite values; the softmax masks those
  // keys).  Tiles are issued in order, so the tile base advances by a
  // constant instead of being recomputed.
  const int dma_row = 8 * wave + (lane >> 3);
  const uint32_t rsb = (uint32_t)(kstride * 2);       // bytes between key rows
  const uint32_t span = 63u * rsb + 128u;              // bytes a tile's rows cover
  const uint32_t dchunk = 16u * (uint32_t)((lane & 7) ^ u_swz(dma_row));
  const uint32_t doff = (uint32_t)dma_row * rsb + dchunk;
  const int tail_kt = (Lk - 1) / kFwdBN;
  const uint32_t otail = (uint32_t)min(dma_row, Lk - 1 - tail_kt * kFwdBN) * rsb + dchunk;
  const int64_t tile_bytes = (int64_t)kFwdBN * kstride * 2;
  // Gathered keys: after cr / 64 tiles the next chunk (next device) of this
  // (batch, head) starts B*H chunks further on.
  const int tiles_per_chunk = ext ? (int)(cr / kFwdBN) : 0x7FFFFFFF;
  const int64_t chunk_jump = ext ? ((int64_t)a.B * a.H - 1) * cr * kD * 2 : 0;
  int tc = 0;
  const char* kcur = kFp8 ? (const char*)a.k + head_off + base_row * a.sn : (const char*)Kh;
  const char* vcur = kFp8 ? (const char*)a.v + head_off + base_row * a.sn : (const char*)Vh;
  auto issue_tile = [&](int kt, FwdStage* __restrict__ dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kcur, span);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vcur, span);
    kcur += tile_bytes;
    vcur += tile_bytes;
    if (kShard && ++tc == tiles_per_chunk) {
      tc = 0;
      kcur += chunk_jump;
      vcur += chunk_jump;
    }
    const uint32_t o = kt == tail_kt ? otail : doff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst->k + 8 * (8 * wave)), 16, o, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst->v + 8 * (8 * wave)), 16, o, 0, 0, 0);
  };

  // ---- 8-bit keys and values: lane l of wave w loads the 8 codes of the
  // logical chunk that belongs at LDS slot l % 8 of row 8w + l / 8 (the
  // DMA's placement), tiles one window ahead into stk/stv, and writes their
  // bf16 image to that slot: byte 16 * tid of the stage's K or V tile.
  const uint32_t cchunk8 = 8u * (uint32_t)((lane & 7) ^ u_swz(dma_row));
  const uint32_t doff8 = (uint32_t)dma_row * (uint32_t)kstride + cchunk8;
  const uint32_t otail8 = (uint32_t)min(dma_row, Lk - 1 - tail_kt * kFwdBN) * (uint32_t)kstride + cchunk8;
  const int64_t tile_bytes8 = (int64_t)kFwdBN * kstride;
  uint2 stk[2], stv[2];
  auto load_tile8 = [&](int kt, int slot) __attribute__((always_inline)) {
    const uint32_t o = kt == tail_kt ? otail8 : doff8;
    stk[slot] = *(const uint2*)(kcur + o);
    stv[slot] = *(const uint2*)(vcur + o);
    kcur += tile_bytes8;
    vcur += tile_bytes8;
  };
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x4v lds_u32x4;
  auto decode8 = [](uint2 x) __attribute__((always_inline)) {
    return u32x4v{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true))};
  };
  auto store_tile8 = [&](int slot, FwdStage* __restrict__ dst) __attribute__((always_inline)) {
    *(lds_u32x4*)((lds_char*)(lds_u4*)dst->k + 16 * tid) = decode8(stk[slot]);
    *(lds_u32x4*)((lds_char*)(lds_u4*)dst->v + 16 * tid) = decode8(stv[slot]);
  };

  // ---- per-lane LDS operand offsets -------------------------------------------
  int kaddr[4];   // K operand (row 32*blk + li, logical chunk 2ks + lg), + blk * 4096
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kaddr[ks] = row_offset(lane, 0, ks);
  int vlo[2], vhi[2];  // V^T operand of head-dim block db via transposed reads, + kk * 2048
#pragma unroll
  for (int db = 0; db < 2; ++db) tr_offsets(lane, db, vlo[db], vhi[db]);

  f32x16 oacc[2] = {f32x16{}, f32x16{}};  // O^T[db]
  float m_run = -INFINITY;                // running offset (log2 domain) of this lane's query
  float l_run = 0.f;                      // this lane's half of the row sum
  float pend = 1.f;                       // O rescale factor owed before O's next update
  bool owed = false;                      // (wave-uniform) some lane's pend may differ from 1

  // ---- building blocks --------------------------------------------------------
  // K operand of step ks of S_h = K_h Q^T (half tile h in block blk of its stage).
  auto read_k = [&](const FwdStage* __restrict__ st, int blk, int ks) __attribute__((always_inline)) {
    return lds_read_b128((const lds_u4*)st->k, blk * 4096 + kaddr[ks]);
  };
  // S_h from its four K operands, the first two read ahead by the caller.
  auto mfma_s = [&](const FwdStage* __restrict__ st, int blk, const bf16x8& k0, const bf16x8& k1, f32x16& s) __attribute__((always_inline)) {
    const bf16x8 k2 = read_k(st, blk, 2);
    const bf16x8 k3 = read_k(st, blk, 3);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qop[0], f32x16{}, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qop[1], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k2, qop[2], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k3, qop[3], s, 0, 0, 0);
  };
  // Four elements (e = 4g .. 4g+3) of P with offset m: two packed bf16 words;
  // the row-sum terms go to two accumulators.
  auto p_chunk = [&](const f32x16& s, float m, int g, uint32_t (&pw)[8], float& r0, float& r1) __attribute__((always_inline)) {
    const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g], c, -m));
    const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 1], c, -m));
    const float x2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 2], c, -m));
    const float x3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 3], c, -m));
    pw[2 * g] = pack_bf16(x0, x1);
    pw[2 * g + 1] = pack_bf16(x2, x3);
    if (g == 0) {
      // The first terms start from an inline zero (VOP3P form) instead of a
      // zeroed register, which the accumulating VOP2 form the builtin
      // selects would need: two moves fewer per phase, same arithmetic.
      asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r0) : "v"(pw[0]), "s"(0x3F803F80u));
      asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r1) : "v"(pw[1]), "s"(0x3F803F80u));
    } else {
      r0 = dot2_bf16_ones(pw[2 * g], r0);
      r1 = dot2_bf16_ones(pw[2 * g + 1], r1);
    }
  };
  // V^T operand of one O^T MFMA: head-dim block db, 16-key step kl of the
  // half tile in block blk of stage st.
  auto read_v = [&](const FwdStage* __restrict__ st, int blk, int db, int kl) __attribute__((always_inline)) {
    const int kk = 2 * blk + kl;
    return lds_read_tr8((const lds_u4*)st->v, vlo[db] + kk * 2048, vhi[db] + kk * 2048);
  };
  // One O^T MFMA with the packed P words of that half tile.
  auto mfma_o = [&](const bf16x8& vop, int db, int kl, const uint32_t (&pw)[8]) __attribute__((always_inline)) {
    const bf16x8 pb = __builtin_bit_cast(bf16x8, uint4{pw[4 * kl], pw[4 * kl + 1], pw[4 * kl + 2], pw[4 * kl + 3]});
    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb, oacc[db], 0, 0, 0);
  };
  auto mfma_o1 = [&](const FwdStage* __restrict__ st, int blk, int db, int kl, const uint32_t (&pw)[8]) __attribute__((always_inline)) {
    mfma_o(read_v(st, blk, db, kl), db, kl, pw);
  };
  // Accept P computed with the running offset, or redo it with the true maximum.
  auto finish_p = [&](const f32x16& s, float rs, uint32_t (&pw)[8]) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(!(rs <= kSumLimit)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = xhalf_max(mx) * c;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      pend *= alpha;
      owed = true;
      l_run *= alpha;
      m_run = m_new;
      float r0 = 0.f, r1 = 0.f;
      const float m = m_new == -INFINITY ? 0.f : m_new;
#pragma unroll
      for (int g = 0; g < 4; ++g) p_chunk(s, m, g, pw, r0, r1);
      rs = r0 + r1;
    }
    l_run += rs;
  };
  // P of a wave's first half tile: the offset is still -inf and O and l are
  // zero, so the exact row maximum is taken at once (no rescale is owed)
  // instead of computing P with the running offset first.
  auto first_p = [&](const f32x16& s, uint32_t (&pw)[8]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
    m_run = xhalf_max(mx) * c;
    const float m = m_run == -INFINITY ? 0.f : m_run;
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) p_chunk(s, m, g, pw, r0, r1);
    l_run = r0 + r1;
  };
  // Causal diagonal / ragged tail mask of half tile hh.  Element e of a lane
  // is key k0 + 4*lg + (e/4)*8 + e%4; it is masked when that key exceeds the
  // last visible one (min(q, L-1) under the causal mask, L-1 otherwise), i.e.
  // when the constant (e/4)*8 + e%4 exceeds one per-lane threshold.
  auto mask_s = [&](int hh, f32x16& s) __attribute__((always_inline)) {
    const int k0 = hh * 32;
    if (!((k0 + 32 > Lk) || (a.causal && k0 + 32 > qgw0))) return;
    const int last = a.causal ? min(qgw0 + li, Lk - 1) : Lk - 1;
    const int d = last - k0 - 4 * lg;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((e >> 2) * 8 + (e & 3) > d) s[e] = -INFINITY;
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (owed) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= pend;
      pend = 1.f;
      owed = false;
    }
  };

  f32x16 s;                  // S of the half tile whose P is computed next
  uint32_t pa[8], pb[8];     // packed P of even / odd half tiles

  // Phase hh (the wave has hh < nh): O update with P_{hh-1} (stage so, block
  // 1-blk) interleaved with P_hh (block blk), then S_{hh+1} from stage ss.
  // Hand-interleaved: each O MFMA is followed by four elements of VALU work
  // that do not depend on it, with scheduling fences between the groups.
  // Every LDS operand is read one group ahead of its MFMA: the V^T operand
  // of group g+1 and, in the last group, the first two K operands of
  // S_{hh+1} (both tiles are in LDS for the whole phase).
  auto phase = [&](int hh, int blk, const FwdStage* __restrict__ so, const FwdStage* __restrict__ ss,
                   uint32_t (&pprev)[8], uint32_t (&pcur)[8]) __attribute__((always_inline)) {
    mask_s(hh, s);
    float r0 = 0.f, r1 = 0.f;
    bf16x8 k0, k1;
    if (hh > 0) {
      apply_rescale();
      bf16x8 vn = read_v(so, 1 - blk, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x8 vc = vn;
        if (g < 3) {
          vn = read_v(so, 1 - blk, (g + 1) & 1, (g + 1) >> 1);
        } else {
          k0 = read_k(ss, 1 - blk, 0);
          k1 = read_k(ss, 1 - blk, 1);
        }
        mfma_o(vc, g & 1, g >> 1, pprev);
        p_chunk(s, m_run, g, pcur, r0, r1);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      k0 = read_k(ss, 1 - blk, 0);
      k1 = read_k(ss, 1 - blk, 1);
    }
    if (hh > 0)
      finish_p(s, r0 + r1, pcur);
    else
      first_p(s, pcur);
    if (hh + 1 < nh) mfma_s(ss, 1 - blk, k0, k1, s);
  };

  // Window after barrier B_j (j even): phases 2j+1 .. 2j+4 read tiles j,
  // j+1 and j+2 (V of halves 2j .. 2j+3, K of halves 2j+2 .. 2j+5).  At B_j
  // every wave has finished phase 2j, so the stages of tiles j-2 and j-1 are
  // free and take tiles j+3 and j+4, which the next window's barrier waits
  // for.  Tile t lives in stage t % 5; the distinct restrict pointers tell
  // the compiler that the DMA targets are not read in the window, so it adds
  // no waits of its own.
  // With kFp8 the window writes the bf16 images of tiles j+3 and j+4 (loaded
  // into registers one window earlier) to those stages and loads tiles j+5
  // and j+6; the barrier then waits for the LDS writes instead of the DMA.
  auto window = [&](int j, const FwdStage* __restrict__ s0, const FwdStage* __restrict__ s1,
                    const FwdStage* __restrict__ s2, FwdStage* __restrict__ i3,
                    FwdStage* __restrict__ i4) __attribute__((always_inline)) {
    if (j > 0) {
      __builtin_amdgcn_s_waitcnt(kFp8 ? kLgkmcnt0 : kVmcnt0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if constexpr (kFp8) {
      if (j + 3 < nkt) store_tile8(0, i3);
      if (j + 4 < nkt) store_tile8(1, i4);
      if (j + 5 < nkt) load_tile8(j + 5, 0);
      if (j + 6 < nkt) load_tile8(j + 6, 1);
    } else {
      if (j + 3 < nkt) issue_tile(j + 3, i3);
      if (j + 4 < nkt) issue_tile(j + 4, i4);
    }
    if (2 * j + 1 < nh) phase(2 * j + 1, 1, s0, s1, pa, pb);
    if (2 * j + 2 < nh) phase(2 * j + 2, 0, s0, s1, pb, pa);
    if (2 * j + 3 < nh) phase(2 * j + 3, 1, s1, s2, pa, pb);
    if (2 * j + 4 < nh) phase(2 * j + 4, 0, s1, s2, pb, pa);
  };

  // Prologue: tiles 0..2 in LDS (the first window reads all three; stages 3
  // and 4 are still unused, so B_0 needs no barrier), S and P of half tile 0.
  if constexpr (kFp8) {
    load_tile8(0, 0);
    if (nkt > 1) load_tile8(1, 1);
    store_tile8(0, &ring[0]);
    if (nkt > 1) store_tile8(1, &ring[1]);
    if (nkt > 2) {
      load_tile8(2, 0);
      store_tile8(0, &ring[2]);
    }
    if (nkt > 3) load_tile8(3, 0);
    if (nkt > 4) load_tile8(4, 1);
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
  } else {
    issue_tile(0, &ring[0]);
    if (nkt > 1) issue_tile(1, &ring[1]);
    if (nkt > 2) issue_tile(2, &ring[2]);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (nh > 0) {
    mfma_s(&ring[0], 0, read_k(&ring[0], 0, 0), read_k(&ring[0], 0, 1), s);
    phase(0, 0, &ring[0], &ring[0], pb, pa);
  }
  for (int j = 0, t0 = 0; j < nkt; j += 2) {
    // t0 = j % 5
    const int t1 = t0 == 4 ? 0 : t0 + 1, t2 = t1 == 4 ? 0 : t1 + 1;
    const int t3 = t2 == 4 ? 0 : t2 + 1, t4 = t3 == 4 ? 0 : t3 + 1;
    window(j, &ring[t0], &ring[t1], &ring[t2], &ring[t3], &ring[t4]);
    t0 = t2;
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
      asm volatile("" ::: "memory");

  if (!wave_active) return;
  // Drain: O update with the wave's last P (half nh-1, in tile (nh-1)/2).
  apply_rescale();
  {
    const int hl = nh - 1;
    const FwdStage* st = &ring[(hl >> 1) % kStages];
    if (hl & 1) {
#pragma unroll
      for (int g = 0; g < 4; ++g) mfma_o1(st, 1, g & 1, g >> 1, pb);
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) mfma_o1(st, 0, g & 1, g >> 1, pa);
    }
  }

  const bool is_prim = (p == a.prim);
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t nsparse = a.nsp[p];
  const float lt = xhalf_sum(l_run);
  const int row = qw0 + li;
  if (row >= L) return;
  const float inv = (kFp8 ? a.v_scale[bh] : 1.f) / lt;
  const float lse = (m_run + __builtin_amdgcn_logf(lt)) * kLn2;
  __bf16* dst;
  float* lse_dst;
  if (is_prim) {
    const int64_t n = base_row + (int64_t)row * r;
    dst = (__bf16*)a.o + head_off + n * a.sn;
    lse_dst = a.lse + bh * a.N + n;
  } else {
    const int64_t m = seg * L_full + row;
    dst = (__bf16*)a.part_o[p] + (bh * nsparse + m) * kD;
    lse_dst = a.part_lse[p] + bh * nsparse + m;
  }
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int eg = 0; eg < 4; ++eg) {
      const f32x16& ov = oacc[db];
      uint2 st;
      st.x = pack_bf16(ov[4 * eg] * inv, ov[4 * eg + 1] * inv);
      st.y = pack_bf16(ov[4 * eg + 2] * inv, ov[4 * eg + 3] * inv);
      *(uint2*)(dst + 32 * db + 8 * eg + 4 * lg) = st;
    }
  if (lg == 0) *lse_dst = lse;
}

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a, hipStream_t stream) {
  if (a.sched.total == 0) return hipSuccess;
  bool shard = false;
  for (int i = 0; i < a.P; ++i) shard |= a.ext_k[i] != nullptr;
  if (shard && a.k_scale) return hipErrorInvalidValue;  // not built: the planner rejects it first
  if (a.k_scale) {
    TimedLaunch tl("attn_fwd_fp8", stream);
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<false, true>), dim3((unsigned)a.sched.total),
                       dim3(64 * kFwdWaves), 0, stream, a);
    return hipGetLastError();
  }
  TimedLaunch tl("attn_fwd", stream);
  if (shard)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<true, false>), dim3((unsigned)a.sched.total),
                       dim3(64 * kFwdWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<false, false>), dim3((unsigned)a.sched.total),
                       dim3(64 * kFwdWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
