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
// One launch per pattern holds two kinds of workgroups (4 waves each):
//   * key-tile units (128 keys, 32 per wave) loop over query tiles of 64 rows
//     and accumulate dK^T = Q^T dS and dV^T = dO^T P in registers;
//   * query-tile units (128 queries, 32 per wave) loop over key tiles of 64
//     rows and accumulate dQ^T = K^T dS^T.
// S (or S^T) comes out of v_mfma_f32_32x32x16_bf16 with the lane on the key
// (or query) axis, so P and dS feed the next MFMA as B operands without any
// data movement; the other operand is an LDS tile transposed when staged.
//
// Patterns run one launch after another.  Per output row the epilogue looks
// up which other patterns keep that row: the first pattern to touch it writes
// the fp32 accumulator, later ones add to it, and the last one adds and writes
// the rounded gradient; a row kept by one pattern only is written directly.
#include "dla_device.h"

namespace dla {

constexpr int kBwdT = 128;  // rows per unit (4 waves x 32)
constexpr int kBwdS = 64;   // rows per streamed tile

struct __align__(16) BwdKVSmem {   // staged query tile (for key-tile units)
  uint4 q[kBwdS * 8];              // R layout
  uint4 qt[kD * 8];                // T layout
  uint4 d[kBwdS * 8];              // dO, R layout
  uint4 dt[kD * 8];                // dO, T layout
  float lse2[kBwdS];               // LSE * log2(e)
  float delta[kBwdS];
};
struct __align__(16) BwdQSmem {    // staged key tile (for query-tile units)
  uint4 k[kBwdS * 8];              // R layout
  uint4 kt[kD * 8];                // T layout
  uint4 v[kBwdS * 8];              // R layout
};
union __align__(16) BwdSmem {
  BwdKVSmem kv[2];
  BwdQSmem qs[2];
};

// bit 0: a pattern processed earlier keeps row n of head h; bit 1: a later one does.
__device__ __forceinline__ int cover_state(const AttnBwdArgs& a, int64_t n, int h) {
  int st = 0;
  const int my = a.rank[a.p];
  for (int i = 0; i < a.P; ++i) {
    if (i == a.p) continue;
    const int ri = a.r_all[i];
    if ((n % ri) != (h % ri)) continue;
    st |= (a.rank[i] < my) ? 1 : 2;
  }
  return st;
}

// Write 4 consecutive gradient values of row `n` at d0 following the
// first/middle/last rule above.
__device__ __forceinline__ void emit4(int st, float* acc_row, __bf16* out_row, int d0, float x0,
                                      float x1, float x2, float x3) {
  float4 v = float4{x0, x1, x2, x3};
  if (st & 1) {
    const float4 o = *(const float4*)(acc_row + d0);
    v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
  }
  if (st & 2) {
    *(float4*)(acc_row + d0) = v;
  } else {
    *(uint2*)(out_row + d0) = uint2{pack_bf16(v.x, v.y), pack_bf16(v.z, v.w)};
  }
}

// Stage rows [r0, r0+64) of a gathered tensor: thread loads rows 2*(tid/8)
// and +1, chunk tid%8; writes R layout and (optionally) T layout.
__device__ __forceinline__ void load_pair(const __bf16* base, int64_t rstride, int r0, int L,
                                          int tid, uint4& a0, uint4& a1) {
  const int c = tid & 7, rr = 2 * (tid >> 3);
  const int ra = r0 + rr, rb = ra + 1;
  a0 = ra < L ? *(const uint4*)(base + (int64_t)ra * rstride + 8 * c) : uint4{0, 0, 0, 0};
  a1 = rb < L ? *(const uint4*)(base + (int64_t)rb * rstride + 8 * c) : uint4{0, 0, 0, 0};
}
__device__ __forceinline__ void store_r(uint4* r, int tid, const uint4& a0, const uint4& a1) {
  const int c = tid & 7, rr = 2 * (tid >> 3);
  r[r_index(rr, c)] = a0;
  r[r_index(rr + 1, c)] = a1;
}
__device__ __forceinline__ void store_t(uint4* t, int tid, const uint4& a0, const uint4& a1) {
  const int c = tid & 7, rr = 2 * (tid >> 3);
  uint32_t words[8];
  pack_pairs(a0, a1, words);
  uint32_t* tw = (uint32_t*)t;
#pragma unroll
  for (int j = 0; j < 8; ++j) tw[t_word(8 * c + j, rr)] = words[j];
}

__device__ __forceinline__ bf16x8 slots_bf16(const f32x16& x, int half) {
  const int e0 = 8 * half;
  return __builtin_bit_cast(bf16x8, uint4{pack_bf16(x[e0], x[e0 + 1]), pack_bf16(x[e0 + 2], x[e0 + 3]),
                                          pack_bf16(x[e0 + 4], x[e0 + 5]),
                                          pack_bf16(x[e0 + 6], x[e0 + 7])});
}

// ---------------------------------------------------------------- dK, dV --
__device__ void bwd_kv_unit(const AttnBwdArgs& a, BwdKVSmem* sm, int64_t unit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lg = lane >> 5;
  int pp, b, h, tile;
  int64_t seg;
  decode_unit(a.sched_kv, (uint32_t)unit, (int)a.H, &a.nseg, pp, b, h, seg, tile);
  const int w = a.w, r = a.r, L = a.L;
  // Under a causal mask a key tile's work shrinks with its index: run low tiles first.
  if (a.causal) tile = (L + kBwdT - 1) / kBwdT - 1 - tile;
  const int64_t base_row = seg_base_row(seg, w, r, h);
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int64_t rstride = (int64_t)r * a.sn;
  const int64_t row_off = head_off + base_row * a.sn;
  const __bf16* Qh = (const __bf16*)a.q + row_off;
  const __bf16* Kh = (const __bf16*)a.k + row_off;
  const __bf16* Vh = (const __bf16*)a.v + row_off;
  const __bf16* Dh = (const __bf16*)a.dout + row_off;
  const int64_t bh = (int64_t)b * a.H + h;
  const float* lse_h = a.lse + bh * a.N + base_row;      // stride r
  const float* del_h = a.delta + bh * a.N + base_row;
  const float c = a.scale_log2;

  const int k0 = tile * kBwdT;
  const int kw0 = k0 + 32 * wave;
  const int key = kw0 + li;
  // K and V of this lane's key as B operands (d = 16ks + 8lg .. +8)
  bf16x8 kop[4], vop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (key < L) {
      kop[ks] = *(const bf16x8*)(Kh + (int64_t)key * rstride + 16 * ks + 8 * lg);
      vop[ks] = *(const bf16x8*)(Vh + (int64_t)key * rstride + 16 * ks + 8 * lg);
    } else {
      kop[ks] = bf16x8{};
      vop[ks] = bf16x8{};
    }
  }
  f32x16 dk[2], dv[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) { dk[db] = f32x16{}; dv[db] = f32x16{}; }

  const int nqt = (L + kBwdS - 1) / kBwdS;
  const int qt0 = a.causal ? k0 / kBwdS : 0;
  const bool wave_active = kw0 < L;

  uint4 q0r, q1r, d0r, d1r;
  float lse_r = 0.f, del_r = 0.f;
  auto load = [&](int qt) {
    const int r0 = qt * kBwdS;
    load_pair(Qh, rstride, r0, L, tid, q0r, q1r);
    load_pair(Dh, rstride, r0, L, tid, d0r, d1r);
    if (tid < kBwdS) {
      const int row = r0 + tid;
      lse_r = row < L ? lse_h[(int64_t)row * r] * kLog2e : 0.f;
      del_r = row < L ? del_h[(int64_t)row * r] : 0.f;
    }
  };
  auto store = [&](int buf) {
    store_r(sm[buf].q, tid, q0r, q1r);
    store_t(sm[buf].qt, tid, q0r, q1r);
    store_r(sm[buf].d, tid, d0r, d1r);
    store_t(sm[buf].dt, tid, d0r, d1r);
    if (tid < kBwdS) {
      sm[buf].lse2[tid] = lse_r;
      sm[buf].delta[tid] = del_r;
    }
  };

  if (qt0 < nqt) {
    load(qt0);
    store(0);
  }
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int buf = (qt - qt0) & 1;
    if (qt + 1 < nqt) load(qt + 1);
    const int q0 = qt * kBwdS;
    const bool run = wave_active && (!a.causal || q0 + kBwdS > kw0);
    if (run) {
      const BwdKVSmem& s = sm[buf];
      f32x16 S[2], dP[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) { S[qb] = f32x16{}; dP[qb] = f32x16{}; }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 qa = *(const bf16x8*)&s.q[r_index(32 * qb + li, 2 * ks + lg)];
          const bf16x8 da = *(const bf16x8*)&s.d[r_index(32 * qb + li, 2 * ks + lg)];
          S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kop[ks], S[qb], 0, 0, 0);
          dP[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vop[ks], dP[qb], 0, 0, 0);
        }
      }
      const bool need_mask = (q0 + kBwdS > L) || (kw0 + 32 > L) || (a.causal && q0 < kw0 + 32);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ql = 32 * qb + (e >> 2) * 8 + lg * 4 + (e & 3);
          const float4 ld = float4{s.lse2[ql], s.delta[ql], 0.f, 0.f};
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][e], c, -ld.x));
          if (need_mask) {
            const int q = q0 + ql;
            if (q >= L || key >= L || (a.causal && key > q)) pv = 0.f;
          }
          S[qb][e] = pv;
          dP[qb][e] = pv * (dP[qb][e] - ld.y);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 pb = slots_bf16(S[kk >> 1], kk & 1);
        const bf16x8 sb = slots_bf16(dP[kk >> 1], kk & 1);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 dta = *(const bf16x8*)&s.dt[t_chunk(32 * db + li, kk, lg)];
          const bf16x8 qta = *(const bf16x8*)&s.qt[t_chunk(32 * db + li, kk, lg)];
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dta, pb, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, sb, dk[db], 0, 0, 0);
        }
      }
    }
    if (qt + 1 < nqt) store(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active || key >= L) return;
  const int64_t n = base_row + (int64_t)key * r;
  const int st = cover_state(a, n, h);
  const int64_t acc_off = ((int64_t)b * a.N + n) * a.H * kD + (int64_t)h * kD;
  const int64_t out_off = head_off + n * a.sn;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int eg = 0; eg < 4; ++eg) {
      const int d0 = 32 * db + 8 * eg + 4 * lg;
      const f32x16& kv = dk[db];
      const f32x16& vv = dv[db];
      emit4(st, a.dk_acc + acc_off, (__bf16*)a.dk + out_off, d0, a.scale * kv[4 * eg],
            a.scale * kv[4 * eg + 1], a.scale * kv[4 * eg + 2], a.scale * kv[4 * eg + 3]);
      emit4(st, a.dv_acc + acc_off, (__bf16*)a.dv + out_off, d0, vv[4 * eg], vv[4 * eg + 1],
            vv[4 * eg + 2], vv[4 * eg + 3]);
    }
}

// --------------------------------------------------------------------- dQ --
__device__ void bwd_q_unit(const AttnBwdArgs& a, BwdQSmem* sm, int64_t unit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lg = lane >> 5;
  int pp, b, h, tile;
  int64_t seg;
  decode_unit(a.sched_q, (uint32_t)unit, (int)a.H, &a.nseg, pp, b, h, seg, tile);
  const int w = a.w, r = a.r, L = a.L;
  const int64_t base_row = seg_base_row(seg, w, r, h);
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int64_t rstride = (int64_t)r * a.sn;
  const int64_t row_off = head_off + base_row * a.sn;
  const __bf16* Qh = (const __bf16*)a.q + row_off;
  const __bf16* Kh = (const __bf16*)a.k + row_off;
  const __bf16* Vh = (const __bf16*)a.v + row_off;
  const __bf16* Dh = (const __bf16*)a.dout + row_off;
  const int64_t bh = (int64_t)b * a.H + h;
  const float c = a.scale_log2;

  const int q0 = tile * kBwdT;
  const int qw0 = q0 + 32 * wave;
  const int q = qw0 + li;
  const bool qvalid = q < L;
  bf16x8 qop[4], dop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (qvalid) {
      qop[ks] = *(const bf16x8*)(Qh + (int64_t)q * rstride + 16 * ks + 8 * lg);
      dop[ks] = *(const bf16x8*)(Dh + (int64_t)q * rstride + 16 * ks + 8 * lg);
    } else {
      qop[ks] = bf16x8{};
      dop[ks] = bf16x8{};
    }
  }
  const float lse2 = qvalid ? a.lse[bh * a.N + base_row + (int64_t)q * r] * kLog2e : 0.f;
  const float del = qvalid ? a.delta[bh * a.N + base_row + (int64_t)q * r] : 0.f;
  f32x16 dq[2];
  dq[0] = f32x16{};
  dq[1] = f32x16{};

  const int kend = a.causal ? min(L, q0 + kBwdT) : L;
  const int nkt = (kend + kBwdS - 1) / kBwdS;
  const bool wave_active = qw0 < L;

  uint4 k0r, k1r, v0r, v1r;
  auto load = [&](int kt) {
    load_pair(Kh, rstride, kt * kBwdS, L, tid, k0r, k1r);
    load_pair(Vh, rstride, kt * kBwdS, L, tid, v0r, v1r);
  };
  auto store = [&](int buf) {
    store_r(sm[buf].k, tid, k0r, k1r);
    store_t(sm[buf].kt, tid, k0r, k1r);
    store_r(sm[buf].v, tid, v0r, v1r);
  };
  if (nkt > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load(kt + 1);
    const int kb0 = kt * kBwdS;
    const bool run = wave_active && (!a.causal || kb0 < qw0 + 32);
    if (run) {
      const BwdQSmem& s = sm[buf];
      f32x16 S[2], dP[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) { S[kb] = f32x16{}; dP[kb] = f32x16{}; }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *(const bf16x8*)&s.k[r_index(32 * kb + li, 2 * ks + lg)];
          const bf16x8 va = *(const bf16x8*)&s.v[r_index(32 * kb + li, 2 * ks + lg)];
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[ks], S[kb], 0, 0, 0);
          dP[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dop[ks], dP[kb], 0, 0, 0);
        }
      }
      const bool need_mask = (kb0 + kBwdS > L) || !qvalid || (a.causal && kb0 + kBwdS > qw0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][e], c, -lse2));
          if (need_mask) {
            const int kk = kb0 + 32 * kb + (e >> 2) * 8 + lg * 4 + (e & 3);
            if (!qvalid || kk >= L || (a.causal && kk > q)) pv = 0.f;
          }
          dP[kb][e] = pv * (dP[kb][e] - del);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 sb = slots_bf16(dP[kk >> 1], kk & 1);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 kta = *(const bf16x8*)&s.kt[t_chunk(32 * db + li, kk, lg)];
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kta, sb, dq[db], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nkt) store(buf ^ 1);
    __syncthreads();
  }

  if (!qvalid) return;
  const int64_t n = base_row + (int64_t)q * r;
  const int st = cover_state(a, n, h);
  const int64_t acc_off = ((int64_t)b * a.N + n) * a.H * kD + (int64_t)h * kD;
  const int64_t out_off = head_off + n * a.sn;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int eg = 0; eg < 4; ++eg) {
      const int d0 = 32 * db + 8 * eg + 4 * lg;
      const f32x16& x = dq[db];
      emit4(st, a.dq_acc + acc_off, (__bf16*)a.dq + out_off, d0, a.scale * x[4 * eg],
            a.scale * x[4 * eg + 1], a.scale * x[4 * eg + 2], a.scale * x[4 * eg + 3]);
    }
}

__global__ __launch_bounds__(256, 2) void attn_bwd_bf16_kernel(const AttnBwdArgs a) {
  __shared__ BwdSmem sm;
  const int64_t u = blockIdx.x;
  if (u < a.sched_kv.total) {
    bwd_kv_unit(a, sm.kv, u);
  } else {
    bwd_q_unit(a, sm.qs, u - a.sched_kv.total);
  }
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  const int64_t total = a.sched_kv.total + a.sched_q.total;
  if (total == 0) return hipSuccess;
  TimedLaunch tl("attn_bwd", stream);
  hipLaunchKernelGGL(attn_bwd_bf16_kernel, dim3((unsigned)total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
