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
// Tiling: 4 waves x 64 query rows.  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (keys as rows, so a lane holds one query's scores
// for 16 keys) and O^T += V^T P^T, feeding P^T to the MFMA straight from the
// S^T accumulator layout; V^T comes from an LDS tile transposed when staged.
// K and V tiles of 64 rows are double-buffered in LDS (32 KB per workgroup),
// Q stays in registers as the B operand.  Online softmax in the exp2 domain.
#include "dla_device.h"

namespace dla {

constexpr int kFwdBM = 256;  // sparse query rows per workgroup
constexpr int kFwdBN = 64;   // keys per tile
constexpr float kLazyLog2 = 8.f;  // rescale only when a row max grows by > 2^8

struct __align__(16) FwdSmem {
  uint4 k[2][kFwdBN * 8];   // R layout
  uint4 vt[2][kD * 8];      // T layout (as uint4 chunks)
};

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const AttnFwdArgs a) {
  __shared__ FwdSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lg = lane >> 5;

  int p, b, h, tile;
  int64_t seg;
  decode_unit(a.sched, blockIdx.x, a.B, a.H, a.nseg, p, b, h, seg, tile);
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
  const int nkt = (kend + kFwdBN - 1) / kFwdBN;
  const bool wave_active = qw0 < L;
  const int wave_kend = a.causal ? min(L, qw0 + 64) : L;
  const int wave_nkt = wave_active ? (wave_kend + kFwdBN - 1) / kFwdBN : 0;
  const float c = a.scale_log2;

  // Q as the B operand: lane (query li, group lg) holds d = 16*ks + 8*lg .. +8.
  bf16x8 qop[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw0 + 32 * qb + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (row < L) {
        qop[qb][ks] = *(const bf16x8*)(Qh + (int64_t)row * rstride + 16 * ks + 8 * lg);
      } else {
        qop[qb][ks] = bf16x8{};
      }
    }
  }

  // Staging assignment: K rows (tid/8, tid/8 + 32), V rows (2*(tid/8), +1), chunk tid%8.
  const int ld_c = tid & 7;
  const int ld_r = tid >> 3;
  uint4 kreg[2], vreg[2];
  auto load_tile = [&](int kt) {
    const int k0 = kt * kFwdBN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = k0 + ld_r + 32 * i;
      kreg[i] = kr < L ? *(const uint4*)(Kh + (int64_t)kr * rstride + 8 * ld_c) : uint4{0, 0, 0, 0};
      const int vr = k0 + 2 * ld_r + i;
      vreg[i] = vr < L ? *(const uint4*)(Vh + (int64_t)vr * rstride + 8 * ld_c) : uint4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = ld_r + 32 * i;
      sm.k[buf][r_index(kr, ld_c)] = kreg[i];
    }
    uint32_t words[8];
    pack_pairs(vreg[0], vreg[1], words);
    uint32_t* vt = (uint32_t*)sm.vt[buf];
#pragma unroll
    for (int j = 0; j < 8; ++j) vt[t_word(8 * ld_c + j, 2 * ld_r)] = words[j];
  };

  f32x16 oacc[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  if (nkt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
    if (kt < wave_nkt) {
      f32x16 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kop = *(const bf16x8*)&sm.k[buf][r_index(32 * kb + li, 2 * ks + lg)];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[qb][ks], s[kb][qb], 0, 0, 0);
        }
      }
      bf16x8 pop[2][4];
      const int k0 = kt * kFwdBN;
      const bool need_mask = (k0 + kFwdBN > L) || (a.causal && k0 + kFwdBN > qw0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = k0 + 32 * kb + (e >> 2) * 8 + lg * 4 + (e & 3);
              const int q = qw0 + 32 * qb + li;
              if (key >= L || (a.causal && key > q)) s[kb][qb][e] = -INFINITY;
            }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // Row max of this tile (both lane halves hold the same query row).
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
        mx = xhalf_max(mx) * c;
        // Lazy rescaling: keep the running maximum unless this tile exceeds it
        // by more than 2^kLazyLog2 (P then stays <= 2^kLazyLog2, harmless for
        // bf16 and fp32).  The result is the same softmax; only the shared
        // exponent offset differs.  Rare after the first tile.
        if (__builtin_amdgcn_ballot_w64(mx > m_run[qb] + kLazyLog2) != 0) {
          const float m_new = fmaxf(m_run[qb], mx);
          const float alpha = (m_run[qb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][qb][e] *= alpha;
        }
        const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
        // P in bf16 as the MFMA B operand; the row sum adds the same rounded
        // values (v_dot2c_f32_bf16 with (1, 1)), in four independent chains.
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const f32x16& sv = s[kk >> 1][qb];
          const int e0 = 8 * (kk & 1);
          uint32_t wds[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e0 + 2 * i], c, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e0 + 2 * i + 1], c, -m_use));
            wds[i] = pack_bf16(p0, p1);
            rs[i] = dot2_bf16_ones(wds[i], rs[i]);
          }
          pop[qb][kk] = __builtin_bit_cast(bf16x8, uint4{wds[0], wds[1], wds[2], wds[3]});
        }
        l_run[qb] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const bf16x8 vop = *(const bf16x8*)&sm.vt[buf][t_chunk(32 * db + li, kk, lg)];
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[qb][kk], oacc[db][qb], 0, 0, 0);
          }
      }
    }
    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const bool is_prim = (p == a.prim);
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t nsparse = a.N / r;
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
