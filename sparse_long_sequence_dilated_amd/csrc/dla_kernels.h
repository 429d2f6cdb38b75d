// Kernel argument blocks and launchers of libdla (host and device side).
#pragma once

#include <hip/hip_runtime.h>

#include "dla_plan.h"

namespace dla {

// Attention pass over all patterns (forward), one launch.
struct AttnFwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* part_o[kMaxP];     // per-pattern partial O_p [B,H,N/r,D] (unused for prim)
  float* part_lse[kMaxP];  // per-pattern partial LSE_p [B,H,N/r]
  int64_t sb, sn, sh;
  int64_t B, N, H;
  int P, prim, causal;
  float scale;             // softmax scale
  float scale_log2;        // scale * log2(e)
  int w[kMaxP], r[kMaxP], L[kMaxP];
  int64_t nseg[kMaxP];
  int64_t nsp[kMaxP];      // N / r: sparse rows per (batch, head) of each pattern
  // Sequence shards: a pattern whose segments span several devices reads its
  // keys and values from gathered buffers ext_k/ext_v laid out as
  // [devices of the segment, B, H, nsp, D] (one chunk of nsp sparse rows per
  // device, in segment order); its local query row i is row qoff + i of the
  // segment, which has Lk key rows.  Otherwise Lk == L, qoff == 0 and the
  // ext pointers are null.
  int Lk[kMaxP];
  int qoff[kMaxP];
  const void* ext_k[kMaxP];
  const void* ext_v[kMaxP];
  Schedule sched;
  const int32_t* lengths;  // per-batch sequence lengths (device), null: all N
  // 8-bit keys and values: k and v hold FP8 E4M3 codes (same element
  // strides, one byte each) and the head's K is code * k_scale[b * H + h],
  // likewise V.  Null for bf16 keys and values.
  const float* k_scale;
  const float* v_scale;
};

// Merge of the per-pattern results into o/lse.
struct CombineArgs {
  void* o;
  float* lse;
  const void* part_o[kMaxP];
  const float* part_lse[kMaxP];
  int64_t sb, sn, sh;
  int64_t B, N, H;
  int P, prim;
  int r[kMaxP];
  int64_t nsp[kMaxP];      // N / r
  int shift[kMaxP];        // log2(r) when r is a power of two, else -1
  uint32_t nblk;           // row blocks of 32 per (batch, head)
  // Residue-class launch (R > 0): rows n = rho + R*t with R = lcm of the
  // rates share the set of patterns that keep them.
  uint32_t R;              // 0: per-row launch
  uint32_t rows_per_class; // N / R
  // Classes that only the primary pattern keeps are not launched when every
  // class another pattern keeps satisfies rho = h mod cls_step (grid.y is
  // then R / cls_step and rho = h mod cls_step + cls_step * blockIdx.y);
  // cls_step = 1 launches every class.
  uint32_t cls_step;
  const int32_t* lengths;  // per-batch sequence lengths (device), null: all N
};

// One device's part of the key/value exchange of a spanning pattern.
struct ShardGatherArgs {
  const void* x;           // [B, N, H, D] bf16 with strides sb/sn/sh
  void* out;               // [B, H, out_rows, D]; rows out_row0 .. out_row0 + cr - 1 written
  int64_t sb, sn, sh;
  int64_t B, H;
  int64_t r, cr;           // rate, cr = N / r
  int64_t out_rows, out_row0;
};

struct ShardLdArgs {
  const float2* ld;        // [B, H, N] (-LSE * log2 e, -D) pairs
  float2* out;             // [B, H, out_rows]
  int64_t B, H, N, r, cr, out_rows, out_row0;
};

struct ShardRelayoutArgs {
  const void* src;
  void* dst;
  int64_t C, B, H, cr;     // devices of the segment, rows per device part
  int64_t pieces;          // 16-byte pieces per row
  int to_ext;              // [B,H,C*cr,D] -> [C,B,H,cr,D] (else the reverse)
};

struct ShardFinishArgs {
  const float* part[kMaxP][3];   // local patterns' fp32 partial gradients [B,H,N/r,D]
  const float* red_k[kMaxP];     // spanning patterns: exchanged dK parts [B,H,N/r,D] fp32
  const float* red_v[kMaxP];
  void* dk;
  void* dv;
  int64_t sb, sn, sh;
  int64_t B, N, H;
  int P;
  int r[kMaxP];
  int64_t nsp[kMaxP];
  uint32_t span_mask;
  uint32_t nblk;
};

struct RowMapArgs {
  int32_t* out;
  int64_t N;
  int H, w, r, L;
};

// Backward attention over all patterns in one launch: dK/dV units (one per
// key tile) and dQ units (one per query tile), reading the combined LSE and D.
struct AttnBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float2* ld;        // (-combined LSE * log2 e, -D), D = rowsum(dO*O), [B,H,N]
  float* part[kMaxP][3];   // fp32 partial dQ, dK, dV of pattern p, [B,H,N/r,D] sparse order
  void* dq;                // outputs, input dtype, strides sb/sn/sh
  void* dk;
  void* dv;
  int64_t sb, sn, sh;
  int64_t B, N, H;
  int causal;
  float scale, scale_log2;
  int P;
  int w[kMaxP], r[kMaxP], L[kMaxP];
  int64_t nseg[kMaxP];
  int64_t nsp[kMaxP];      // N / r
  Schedule sched_kv;       // dK/dV units (key tiles), all patterns
  Schedule sched_q;        // dQ units (query tiles), all patterns
  // Query window (one sequence shard's queries in a gathered segment; single
  // pattern, every result an fp32 partial): qhi > 0 selects it.  Query rows
  // [qlo, qhi) exist (multiples of 128); the query schedule covers them only,
  // and dQ partials hold nsp_q rows per (batch, head).
  int qlo, qhi;
  int64_t nsp_q;
  const int32_t* lengths;  // per-batch sequence lengths (device), null: all N
};

// Sum of the per-pattern partial gradients of rows kept by several patterns.
struct BwdFinalizeArgs {
  const float* part[kMaxP][3];
  void* grad[3];           // dq, dk, dv (bf16, strides sb/sn/sh)
  int64_t sb, sn, sh;
  int64_t B, N, H;
  int P;
  int r[kMaxP];
  int64_t nsp[kMaxP];
  int shift[kMaxP];        // log2(r) when r is a power of two, else -1
  uint32_t nblk;           // row blocks of 32 per (batch, head)
  uint32_t R;              // residue-class launch: R = lcm of the rates (0: per row)
  uint32_t rows_per_class; // N / R
  uint32_t cls_step;       // classes launched: rho = h mod cls_step + cls_step * blockIdx.y
  uint32_t span_mask;      // sequence shard: patterns whose segments span devices
  const int32_t* lengths;  // per-batch sequence lengths (device), null: all N
};

struct BwdPrepArgs {
  const void* o;
  const void* dout;
  const float* lse;        // combined LSE [B,H,N]
  float2* ld;              // out: (-LSE * log2 e, -D) [B,H,N]
  void* dq;
  void* dk;
  void* dv;
  int64_t sb, sn, sh;
  int64_t B, N, H;
  int P;
  int r_all[kMaxP];
  int zero_uncovered;      // write zero gradients for rows no pattern keeps
  const int32_t* lengths;  // per-batch sequence lengths (device), null: all N
};

// Scope guard of the opt-in launch timing (dla_timing_enable): records HIP
// events on `stream` around the launches made inside its lifetime.
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t stream);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
  bool active_ = false;
};

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a, hipStream_t stream);

// Per-(batch, head) FP8 E4M3 quantization of a bf16 [B, N, H, D] tensor.
struct QuantArgs {
  const void* x;   // bf16
  uint8_t* x8;     // codes, same element strides
  float* scale;    // [B, H]: the head's amax (as bits) while the pass runs, then the scale
  int64_t sb, sn, sh;
  int64_t B, N, H;
};
hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t stream);
hipError_t launch_shard_gather(const ShardGatherArgs& a, hipStream_t stream);
hipError_t launch_pad_rows(const CombineArgs& a, int dtype, hipStream_t stream);
hipError_t launch_shard_ld(const ShardLdArgs& a, hipStream_t stream);
hipError_t launch_shard_relayout(const ShardRelayoutArgs& a, hipStream_t stream);
hipError_t launch_shard_finish(const ShardFinishArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream);
hipError_t launch_row_map(const RowMapArgs& a, hipStream_t stream);
// Rows a backward work unit owns (the tile size of both schedules).
constexpr int kBwdUnitRows = 128;
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_prep(const BwdPrepArgs& a, int dtype, hipStream_t stream);
hipError_t launch_bwd_finalize(const BwdFinalizeArgs& a, hipStream_t stream);

}  // namespace dla
