// Split-K GQA decode attention over the mixed full-precision / INT2 / tail cache, window scores fused.
//
// What it computes follows the QEvict page ("Mecanismos Principais"): attention over the resident windows (the
// full-precision tier and the INT2 tier, dequantised in registers), the cumulative window score updated from
// each window's attention mass, grouped-query attention (G query heads share one KV head).
//
// decode_partial: one workgroup of WPB waves per (unit, slice); every wave owns ONE task and issues all of its
// loads at once, so a CU keeps its whole share of a step in flight (a decode step moves ~130 KB per CU at the
// 32K-context shape, less than the CU's register file):
//   * dense task: one FULL window (read from its full-precision slot res_slot[f]) or one 32-token tail block: K
//     (8 KiB) and V^T (8 KiB) straight into the MFMA operand registers (16 bytes per lane per instruction);
//   * INT2 task: QW INT2 windows (read from their ledger slots): codes into registers, the per-token scale/zero
//     words through LDS.
//   Tasks of a unit, in launch order: the INT2 windows in groups of QW (their loads are the most scattered and
//   their arithmetic the longest, so they go first), the tail blocks, then FULL window res_list[f] per task.
//   Tasks past the device counts are empty. The INT2 window ids are read at the offset the device count usually
//   has (n_full == max_full) together with the counts, and re-read only when it differs.
//   * q.K^T on MFMA (v_mfma_f32_16x16x32 bf16/f16): A = the G query heads (rows, zero-padded to 16), B = 16
//     tokens x 32 head_dim of K. INT2 keys enter B as 128+c (bf16) / 1024+c (fp16) bit patterns, one group of 32
//     head_dim per MFMA; the group's scale/zero are applied to the fp32 product:  s*acc + (z - magic*s)*sum(q).
//     With G <= 4 an INT2 task puts group k's heads in rows 4k..4k+3 of group k's A, so the four group products
//     share one tile (row block k = group k); each lane scales its own group and cross-row swaps add the groups.
//   * softmax over the task's keys (max, exp, sums by DPP reductions over 16-lane rows); each window's exp-sum and the
//     reference max it is relative to are written for the score. With per-position weights (WEIGHTED: CriticalKV
//     page, "Algoritmo", the projected-value norm plugged into the window score) the window's exp-sum weights each
//     key per head; the weights are loaded with the task's other loads.
//   * P.V on MFMA: A = 16 head_dim x 32 tokens of V (V is stored transposed per window), B = P^T (columns
//     0..G-1) split into a high and a low part that two MFMAs accumulate into the same columns, so the product
//     keeps ~16 bits of P with no merge afterwards. INT2 values enter A as exact fp16 codes and the per-token
//     scale is folded into B (P*s); the zero term sum(P*z) is a VALU bias. With G <= 4, B column 4g + h carries
//     head h scaled by head_dim group g, so one B pair serves every head_dim tile of the window.
//   The workgroup's waves merge their (m, l, o) in LDS into one partial per workgroup.
// decode_combine: merges the partials of a unit in a fixed order (bitwise reproducible), writes o, converts the
// window exp-sums into probability mass, adds it to the cumulative score, finalises the optional probabilities
// and appends the step's token to the tail.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Launch shapes (QW INT2 windows per wave task, WPB waves per workgroup, both template parameters): a step that
// fills the GPU in about one round of workgroups takes (1, 8), the shortest chain per task and the fewest partials;
// a step of many rounds takes (2, 4), more bytes per wave slot and a finer workgroup turnover.
constexpr int kMaxParts = 16384;    // workgroups (partials) per unit
constexpr int kMetaWords = kW * kGroups;  // scale/zero words per window and per K or V
constexpr float kInvSqrtD = 0.088388347648318440550f;  // 1/sqrt(128)
constexpr float kLn32 = 3.4657359027997265471f;          // size correction of a 32-token span summary

struct DecodeParams {
  int NW, TM;
  int FS, LS;              // full-precision and ledger slots per unit
  const uint16_t* k_full;  // [U][FS][W][D]
  const uint16_t* v_full;  // [U][FS][D][W]
  const uint8_t* k_codes;
  const uint16_t* v_codes;
  const uint32_t* k_meta;
  const uint32_t* v_meta;
  uint16_t* k_tail;
  uint16_t* v_tail;
  int32_t* tail_len;
  const int32_t* res_list;
  const int32_t* res_slot;
  const int32_t* n_full;
  const int32_t* n_int2;
  const int32_t* n_windows;
  const int8_t* tier;
  float* cum;
  int32_t* status;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  float* out;
  float* probs;
  float* mass;
  long probs_stride;
  int accumulate;
  int max_full, max_int2, max_tail;
  int n_tb;        // tail-block tasks per unit (bound)
  int n_qt;        // INT2 tasks per unit (bound)
  int P;           // slices (workgroups) per unit
  int CB;          // combine workgroups per unit
  float* part_ml;  // [U][P][G][2]
  float* part_o;   // [U][P][G][D]
  float* wsum;     // [U][NW][G]
  float* wref;     // [U][NW][G]
  int32_t* unit_tl;  // [U] the tail length the step's partials were computed with (before the append)
  const float* wnorm;  // [U][G][wstride] per-head weight of each window position in the score, or null
  long wstride;
  const uint16_t* k_sum;  // [U][SM][D] span summaries (keys), token-major
  const uint16_t* v_sum;  // [U][SM/32][D][32]
  const int32_t* n_sum;   // [U]
  int SM, max_sum;        // capacity; host bound on n_sum (0: no summaries attended)
  int score;              // 0: neither the cumulative score nor the window mass is asked for (a plain decode step)
  int n_sb;               // summary-block tasks per unit (bound)
};

// The compiler fetches kernel arguments on first use, each fetch a round trip it then waits for; these pins make
// it fetch a kernel's arguments together at entry.
__device__ __forceinline__ void fetch_args_partial(const DecodeParams& p) {
  asm volatile("" ::"s"(p.NW), "s"(p.TM), "s"(p.k_full), "s"(p.v_full), "s"(p.k_codes), "s"(p.v_codes), "s"(p.k_meta),
               "s"(p.v_meta), "s"(p.k_tail), "s"(p.v_tail), "s"(p.res_list), "s"(p.n_full), "s"(p.n_int2),
               "s"(p.tail_len), "s"(p.res_slot), "s"(p.FS), "s"(p.LS));
  asm volatile("" ::"s"(p.q), "s"(p.k_new), "s"(p.max_full), "s"(p.max_int2), "s"(p.max_tail), "s"(p.n_tb),
               "s"(p.n_qt), "s"(p.P), "s"(p.part_ml), "s"(p.part_o), "s"(p.wsum), "s"(p.wref), "s"(p.unit_tl),
               "s"(p.wnorm), "s"(p.wstride));
}
__device__ __forceinline__ void fetch_args_combine(const DecodeParams& p) {
  asm volatile("" ::"s"(p.NW), "s"(p.TM), "s"(p.P), "s"(p.CB), "s"(p.out), "s"(p.part_ml), "s"(p.part_o), "s"(p.tier),
               "s"(p.wsum), "s"(p.wref), "s"(p.cum), "s"(p.n_windows), "s"(p.mass), "s"(p.accumulate));
  asm volatile("" ::"s"(p.probs), "s"(p.probs_stride), "s"(p.k_new), "s"(p.v_new), "s"(p.k_tail), "s"(p.v_tail),
               "s"(p.tail_len), "s"(p.unit_tl), "s"(p.n_full), "s"(p.n_int2), "s"(p.max_full), "s"(p.max_int2));
}

// ---- MFMA and conversions per storage dtype ----------------------------------------------------------------
struct MBF16 {
  static constexpr uint32_t kMagic = 0x43004300u;  // two bf16 128.0
  static constexpr float kMagicVal = 128.0f;
  static constexpr uint32_t kOnes = 0x3F803F80u;   // two bf16 1.0
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
  static __device__ __forceinline__ float val(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
};
struct MF16 {
  static constexpr uint32_t kMagic = 0x64006400u;  // two fp16 1024.0
  static constexpr float kMagicVal = 1024.0f;
  static constexpr uint32_t kOnes = 0x3C003C00u;   // two fp16 1.0
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
  static __device__ __forceinline__ float val(uint16_t b) { return float(__builtin_bit_cast(_Float16, b)); }
};
template <class T> struct MfmaOf;
template <> struct MfmaOf<BF16> { using M = MBF16; };
template <> struct MfmaOf<F16> { using M = MF16; };

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ u32x4 zero4u() { return u32x4{0u, 0u, 0u, 0u}; }

// The magic pattern in a VGPR the compiler cannot see through, so that every (x & mask) | magic below is one
// v_and_or_b32 (a literal would need a separate v_or: one instruction takes at most one constant)
__device__ __forceinline__ uint32_t magic_in_vgpr(uint32_t magic) {
  uint32_t v;
  asm("v_mov_b32 %0, %1" : "=v"(v) : "s"(magic));
  return v;
}

// 8 two-bit codes (bits 2e, e = 0..7) -> 8 16-bit values  magic | code,  k-slot e = code e
__device__ __forceinline__ u32x4 expand_codes(uint32_t c16, uint32_t magic) {
  const uint32_t z = c16 | (c16 << 14);  // code 2k at bits 4k, code 2k+1 at bits 4k+16
  return u32x4{(z & 0x00030003u) | magic, ((z >> 4) & 0x00030003u) | magic, ((z >> 8) & 0x00030003u) | magic,
               ((z >> 12) & 0x00030003u) | magic};
}

// exact fp16 codes: (1024 + c) - 1024 (on plain scalars: bit casts of vector elements are avoided)
__device__ __forceinline__ uint32_t f16x2_minus_1024(uint32_t w) {
  f16x2 v = __builtin_bit_cast(f16x2, w);
  const f16x2 m = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  v = v + m;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ u32x4 codes_to_f16(uint32_t c16, uint32_t magic) {
  const u32x4 w = expand_codes(c16, magic);
  return u32x4{f16x2_minus_1024(w.x), f16x2_minus_1024(w.y), f16x2_minus_1024(w.z), f16x2_minus_1024(w.w)};
}

// high or low part of 8 floats in a 16-bit MFMA type (x = hi + lo to ~16 significant bits)
template <class M>
__device__ __forceinline__ u32x4 split8(const float (&x)[8], bool low) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint16_t b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float v = x[2 * k + h];
      const uint16_t hi = M::bits(v);
      b[h] = low ? M::bits(v - M::val(hi)) : hi;
    }
    w[k] = uint32_t(b[0]) | (uint32_t(b[1]) << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// Sum over the four 16-lane rows (lanes l, l^16, l^32, l^48) by cross-row swaps; every lane gets the same bits
// (each step adds the same two values in the same order in both rows of a pair).
__device__ __forceinline__ float sum_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct Ctx {
  int u, lane, q, col;
  int nf, nq, tl, has_new, total_tail;
  size_t unit_win;
};

// Per-lane result of a wave: heads 4*(lane/16) + r for m, l (the 16 lanes of a group agree); O^T tiles acc[dt]
// (column lane%16 = head, for lanes with lane%16 < G; head_dim 16dt + 4*(lane/16) + r); bias[g] = sum P*z of the
// INT2 values of head_dim group g (column lane%16 < G, partial over this lane's tokens).
struct WaveOut {
  float m[4], l[4];
  f32x4 acc[8];
  float bias[4];
};

// Softmax over the task's NWIN windows (S: logits, -inf where masked) -> S holds exp(s - m); m, l per head row,
// ws[i] = exp-sum of window i relative to m.
template <int NWIN>
__device__ __forceinline__ void task_softmax(f32x4 (&S)[NWIN][2], WaveOut& wo, float (&ws)[NWIN][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = fmaxf(S[0][0][r], S[0][1][r]);
#pragma unroll
    for (int i = 1; i < NWIN; ++i) v = fmaxf(v, fmaxf(S[i][0][r], S[i][1][r]));
    wo.m[r] = row_max16(v);
  }
#pragma unroll
  for (int i = 0; i < NWIN; ++i) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[i][t][r] = exp_diff(S[i][t][r], wo.m[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < NWIN; ++i) {
      const float v = row_sum16(S[i][0][r] + S[i][1][r]);
      ws[i][r] = v;
      tot += v;
    }
    wo.l[r] = tot;
  }
}

// Raw logits into the optional probability rows (finalised by the combine kernel).
template <int G>
__device__ __forceinline__ void store_logits(const DecodeParams& p, const Ctx& c, const f32x4 (&S)[2], int pos,
                                             int nvalid) {
  if (4 * c.q >= G) return;
  float* pb = p.probs + size_t(c.u) * G * p.probs_stride + pos;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * c.q + r;
    if (h < G) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (16 * t + c.col < nvalid) pb[size_t(h) * p.probs_stride + 16 * t + c.col] = S[t][r];
      }
    }
  }
}

// P of one window (S layout: lane (token col, head row 4q + r)) -> this lane's B-operand row of P^T: head hcol
// (< G), tokens 8q .. 8q+7, through a per-wave LDS tile [8 heads][32 tokens].
template <int G>
__device__ __forceinline__ void p_to_b(const Ctx& c, const f32x4 (&Pw)[2], float* plds, int hcol, float (&x)[8]) {
  if (4 * c.q < G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * c.q + r;
      if (h < G) {
        plds[h * 32 + c.col] = Pw[0][r];
        plds[h * 32 + 16 + c.col] = Pw[1][r];
      }
    }
  }
  const float4 a0 = *reinterpret_cast<const float4*>(plds + hcol * 32 + 8 * c.q);
  const float4 a1 = *reinterpret_cast<const float4*>(plds + hcol * 32 + 8 * c.q + 4);
  x[0] = a0.x;
  x[1] = a0.y;
  x[2] = a0.z;
  x[3] = a0.w;
  x[4] = a1.x;
  x[5] = a1.y;
  x[6] = a1.z;
  x[7] = a1.w;
}

// Window exp-sums and their reference max, for the score (lanes of column 0 hold one head row each).
template <int G>
__device__ __forceinline__ void store_window_sums(const DecodeParams& p, const Ctx& c, int id, const float (&ws)[4],
                                                  const float (&m)[4]) {
  if (p.score == 0 || c.col != 0 || 4 * c.q >= G) return;  // a plain decode step keeps no window sums
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * c.q + r;
    if (h < G) {
      p.wsum[(c.unit_win + id) * G + h] = ws[r];
      p.wref[(c.unit_win + id) * G + h] = m[r];
    }
  }
}

// Per-head weights of one window's tokens for the weighted score: lane (col, q) takes tokens col and 16 + col of
// head rows 4q + r (rows past G read head G-1; their sums are never stored).
template <int G>
__device__ __forceinline__ void load_weights(const DecodeParams& p, const Ctx& c, int id, float (&wn)[4][2]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float* wp = p.wnorm + (size_t(c.u) * G + min(4 * c.q + r, G - 1)) * p.wstride + size_t(id) * kW;
    wn[r][0] = wp[c.col];
    wn[r][1] = wp[16 + c.col];
  }
}
// Weighted window exp-sums (S holds exp(s - m) of the window's two 16-token tiles).
__device__ __forceinline__ void weighted_sums(const f32x4 (&S)[2], const float (&wn)[4][2], float (&ws)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) ws[r] = row_sum16(S[0][r] * wn[r][0] + S[1][r] * wn[r][1]);
}

// One FULL window (TAIL = false, window id, full-precision slot) or one 32-token tail block (TAIL = true, block
// index blk). SUMM (with TAIL): one 32-summary block of the unit's span summaries, in the tail's layouts, logits +
// ln 32.
template <int G, class T, bool PROBS, bool TAIL, bool WEIGHTED, bool SUMM = false>
__device__ __forceinline__ void dense_task(const DecodeParams& p, const Ctx& c, int id, int slot, int blk, int nvalid,
                                           int pos, const u32x4 (&aq)[4], float* plds, WaveOut& wo) {
  using M = typename MfmaOf<T>::M;
  static_assert(!SUMM || (TAIL && !PROBS), "summary blocks use the tail path and no probabilities");
  const size_t base = TAIL ? (size_t(c.u) * (SUMM ? p.SM : p.TM) + 32 * blk) * kD
                           : (size_t(c.u) * p.FS + slot) * size_t(kW * kD);
  const uint16_t* kb = (TAIL ? (SUMM ? p.k_sum : p.k_tail) : p.k_full) + base;
  const uint16_t* vb = (TAIL ? (SUMM ? p.v_sum : p.v_tail) : p.v_full) + base;
  u32x4 kr[8], vr[8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k) kr[t * 4 + k] = ld16(kb + (16 * t + c.col) * kD + 32 * k + 8 * c.q);
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) vr[dt] = ld16(vb + (16 * dt + c.col) * kW + 8 * c.q);
  float wn[4][2];
  if constexpr (WEIGHTED && !TAIL) load_weights<G>(p, c, id, wn);
  __builtin_amdgcn_sched_barrier(0);  // every load of the task is issued before the first use
  const int tnew = TAIL && !SUMM && c.has_new ? c.tl - 32 * blk : -1;  // the step's token: not in the tail yet
  if (TAIL && !SUMM && c.has_new) {
    u32x4 kn[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) kn[k] = ld16(p.k_new + size_t(c.u) * kD + 32 * k + 8 * c.q);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool is_new = 16 * t + c.col == tnew;
#pragma unroll
      for (int k = 0; k < 4; ++k) kr[t * 4 + k] = is_new ? kn[k] : kr[t * 4 + k];
    }
  }
  f32x4 S[1][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    S[0][t] = zero4();
#pragma unroll
    for (int k = 0; k < 4; ++k) S[0][t] = M::mfma(aq[k], kr[t * 4 + k], S[0][t]);
    const bool ok = 16 * t + c.col < nvalid;
#pragma unroll
    for (int r = 0; r < 4; ++r) S[0][t][r] = ok ? S[0][t][r] * kInvSqrtD + (SUMM ? kLn32 : 0.0f) : -INFINITY;
  }
  if (PROBS) store_logits<G>(p, c, S[0], pos, nvalid);
  float ws[1][4];
  task_softmax<1>(S, wo, ws);
  if constexpr (WEIGHTED && !TAIL) weighted_sums(S[0], wn, ws[0]);
  if (!TAIL) store_window_sums<G>(p, c, id, ws[0], wo.m);
  float x[8];
  p_to_b<G>(c, S[0], plds, c.col < G ? c.col : 0, x);
  // P^T as a high and a low part, accumulated into the same columns by two MFMAs (~16 bits of P); columns G..15
  // repeat head 0 and their results are never read
  const u32x4 Bh = split8<M>(x, false), Bl = split8<M>(x, true);
  if (TAIL) {  // the new token's values from v_new; values past the valid length zeroed (no inf * 0)
    const int t0 = 8 * c.q;
    const int e_new = tnew - t0;
    const int n_ok = min(max(nvalid - t0, 0), 8);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint32_t nv = !SUMM && c.has_new ? uint32_t(p.v_new[size_t(c.u) * kD + 16 * dt + c.col]) : 0u;
      uint32_t w[4] = {vr[dt].x, vr[dt].y, vr[dt].z, vr[dt].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sh = 16 * (e & 1);
        uint32_t v = (w[e >> 1] >> sh) & 0xFFFFu;
        v = e == e_new ? nv : v;
        v = e < n_ok ? v : 0u;
        w[e >> 1] = (w[e >> 1] & ~(0xFFFFu << sh)) | (v << sh);
      }
      vr[dt] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) wo.acc[dt] = M::mfma(vr[dt], Bl, M::mfma(vr[dt], Bh, zero4()));
}

// qsum[k][r] = sum over head_dim group k of q[head 4*(lane/16) + r] in fp32 (rows beyond G: 0)
template <int G, class T>
__device__ __forceinline__ void q_group_sums(const Ctx& c, const u32x4 (&aq)[4], float (&qsum)[4][4]) {
  using M = typename MfmaOf<T>::M;
  float qs[4][G];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w4[4] = {aq[k].x, aq[k].y, aq[k].z, aq[k].w};
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      part += M::val(uint16_t(w4[e] & 0xFFFFu));
      part += M::val(uint16_t(w4[e] >> 16));
    }
    part = xor_sum(part, 16);
    part = xor_sum(part, 32);
#pragma unroll
    for (int h = 0; h < G; ++h) qs[k][h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), h));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = r < G ? qs[k][r < G ? r : 0] : 0.0f;
      if (G > 4 && c.q == 1) v = qs[k][(4 + r) < G ? 4 + r : 0];
      qsum[k][r] = v;
    }
  }
}

// QW INT2 windows: window ids and their ledger slots (ok[i]: window i exists; masked windows read slot 0 and
// contribute nothing).
template <int G, class T, bool PROBS, int QW, bool WEIGHTED>
__device__ __forceinline__ void int2_task(const DecodeParams& p, const Ctx& c, const int (&ids)[QW],
                                          const int (&slots)[QW], const bool (&ok)[QW], int pos0,
                                          const u32x4 (&aq)[4], float* plds, uint32_t* ms, WaveOut& wo) {
  using M = typename MfmaOf<T>::M;
  // all loads first: K codes (tokens col and 16 + col, bytes 8q .. 8q+7), V codes (16 bytes of this lane's
  // operand rows), and 8 bytes of each of the K and V scale/zero tables (lane l: words 2l, 2l+1)
  u32x4 kc[QW], vc[QW];
  uint2 km[QW], vm[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const size_t win = size_t(c.u) * p.LS + slots[i];
    const uint8_t* kcb = p.k_codes + win * (kW * kCodeBytes);
    const uint2 a = ld8(kcb + c.col * kCodeBytes + 8 * c.q);
    const uint2 b = ld8(kcb + (16 + c.col) * kCodeBytes + 8 * c.q);
    kc[i] = u32x4{a.x, a.y, b.x, b.y};
    vc[i] = ld16(p.v_codes + win * (kW * kD / 8) + (c.col * 4 + c.q) * 8);
    km[i] = ld8(p.k_meta + win * kMetaWords + 2 * c.lane);
    vm[i] = ld8(p.v_meta + win * kMetaWords + 2 * c.lane);
  }
  float wn[QW][4][2];
  if constexpr (WEIGHTED) {
#pragma unroll
    for (int i = 0; i < QW; ++i) load_weights<G>(p, c, ids[i], wn[i]);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load of the task is issued before the first use
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const uint2 z2 = {0u, 0u};
    *reinterpret_cast<uint2*>(ms + (2 * i) * kMetaWords + 2 * c.lane) = ok[i] ? km[i] : z2;
    *reinterpret_cast<uint2*>(ms + (2 * i + 1) * kMetaWords + 2 * c.lane) = ok[i] ? vm[i] : z2;
  }
  // logits: one MFMA per (16 tokens, group), the group's scale and zero applied to the fp32 product
  f32x4 S[QW][2];
  if constexpr (G <= 4) {
    // aq[k] holds group k's q in rows 4k .. 4k+3 (head = row % 4) and zeros elsewhere, so the four groups' MFMAs
    // accumulate into one tile: lane (row block q, token col) holds group q's product for heads r = 0..3. Each
    // lane applies its own group's scale and zero, and the four row blocks are summed. The same A against a B of
    // ones gives every lane its group's q sums.
    const u32x4 ones = {M::kOnes, M::kOnes, M::kOnes, M::kOnes};
    const uint32_t mg = magic_in_vgpr(M::kMagic);
    f32x4 qs = zero4();
#pragma unroll
    for (int k = 0; k < 4; ++k) qs = M::mfma(aq[k], ones, qs);
#pragma unroll
    for (int i = 0; i < QW; ++i) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t cw0 = t == 0 ? kc[i].x : kc[i].z;
        const uint32_t cw1 = t == 0 ? kc[i].y : kc[i].w;
        f32x4 o = zero4();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t cw = k < 2 ? cw0 : cw1;
          o = M::mfma(aq[k], expand_codes((cw >> (16 * (k & 1))) & 0xFFFFu, mg), o);
        }
        const uint32_t mw = ms[(2 * i) * kMetaWords + (16 * t + c.col) * kGroups + c.q];
        const float s = half_bits_to_float(mw & 0xFFFFu);
        const float zz = half_bits_to_float(mw >> 16) - M::kMagicVal * s;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = sum_rows4(fmaf(s, o[r], zz * qs[r]));
          S[i][t][r] = ok[i] ? v * kInvSqrtD : -INFINITY;
        }
      }
      if (PROBS && ok[i]) store_logits<G>(p, c, S[i], pos0 + kW * i, kW);
    }
  } else {
    float qsum[4][4];
    q_group_sums<G, T>(c, aq, qsum);
#pragma unroll
    for (int i = 0; i < QW; ++i) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        S[i][t] = zero4();
        const u32x4 meta = ld16(ms + (2 * i) * kMetaWords + (16 * t + c.col) * kGroups);
        const uint32_t cw0 = t == 0 ? kc[i].x : kc[i].z;
        const uint32_t cw1 = t == 0 ? kc[i].y : kc[i].w;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t cw = k < 2 ? cw0 : cw1;
          const uint32_t c16 = (cw >> (16 * (k & 1))) & 0xFFFFu;
          const f32x4 o = M::mfma(aq[k], expand_codes(c16, M::kMagic), zero4());
          const uint32_t mw = k == 0 ? meta.x : (k == 1 ? meta.y : (k == 2 ? meta.z : meta.w));
          const float s = half_bits_to_float(mw & 0xFFFFu);
          const float zz = half_bits_to_float(mw >> 16) - M::kMagicVal * s;
#pragma unroll
          for (int r = 0; r < 4; ++r) S[i][t][r] += s * o[r] + zz * qsum[k][r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) S[i][t][r] = ok[i] ? S[i][t][r] * kInvSqrtD : -INFINITY;
      }
      if (PROBS && ok[i]) store_logits<G>(p, c, S[i], pos0 + kW * i, kW);
    }
  }
  float ws[QW][4];
  task_softmax<QW>(S, wo, ws);
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    if constexpr (WEIGHTED) weighted_sums(S[i], wn[i], ws[i]);
    if (ok[i]) store_window_sums<G>(p, c, ids[i], ws[i], wo.m);
  }
  // P.V: A = exact fp16 codes of 16 head_dim x 32 tokens, B = (P * scale)^T hi/lo, bias = sum P * zero.
  // G <= 4: B column 4g + h carries head h scaled by head_dim group g's value scales, so one B pair serves all
  // eight head_dim tiles and every lane's scaling is used; tile dt's result lies in the columns of its group dt/2,
  // and bias[0] holds the lane's own group. G = 8: one B pair per group, columns = heads, bias[g] per group.
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) wo.acc[dt] = zero4();
  const uint32_t mg16 = magic_in_vgpr(MF16::kMagic);
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const uint32_t* vmw = ms + (2 * i + 1) * kMetaWords + c.q * 32;
    if constexpr (G <= 4) {
      float x[8];
      p_to_b<G>(c, S[i], plds, (c.col & 3) < G ? (c.col & 3) : 0, x);
      const int g = c.col >> 2;
      const u32x4 m0 = ld16(vmw + 8 * g);
      const u32x4 m1 = ld16(vmw + 8 * g + 4);
      const uint32_t mws[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      float y[8];
      float zsum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = x[e] * half_bits_to_float(mws[e] & 0xFFFFu);
        zsum = fmaf(x[e], half_bits_to_float(mws[e] >> 16), zsum);
      }
      wo.bias[0] += zsum;
      const u32x4 Bh = split8<MF16>(y, false), Bl = split8<MF16>(y, true);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t wv = dt < 2 ? vc[i].x : (dt < 4 ? vc[i].y : (dt < 6 ? vc[i].z : vc[i].w));
        const u32x4 a = codes_to_f16((wv >> (16 * (dt & 1))) & 0xFFFFu, mg16);
        wo.acc[dt] = MF16::mfma(a, Bl, MF16::mfma(a, Bh, wo.acc[dt]));
      }
    } else {
      float x[8];
      p_to_b<G>(c, S[i], plds, c.col < G ? c.col : 0, x);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 m0 = ld16(vmw + 8 * g);
        const u32x4 m1 = ld16(vmw + 8 * g + 4);
        const uint32_t mws[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        float y[8];
        float zsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[e] = x[e] * half_bits_to_float(mws[e] & 0xFFFFu);
          zsum = fmaf(x[e], half_bits_to_float(mws[e] >> 16), zsum);
        }
        wo.bias[g] += zsum;
        const u32x4 Bh = split8<MF16>(y, false), Bl = split8<MF16>(y, true);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int dt = 2 * g + h2;
          const uint32_t wv = dt < 2 ? vc[i].x : (dt < 4 ? vc[i].y : (dt < 6 ? vc[i].z : vc[i].w));
          const u32x4 a = codes_to_f16((wv >> (16 * (dt & 1))) & 0xFFFFu, mg16);
          wo.acc[dt] = MF16::mfma(a, Bl, MF16::mfma(a, Bh, wo.acc[dt]));
        }
      }
    }
  }
}

template <int G, class T, bool PROBS, int QW, int WPB, bool WEIGHTED, bool SUMMARY>
__global__ __launch_bounds__(WPB * kWave) __attribute__((amdgpu_waves_per_eu(4))) void decode_partial(DecodeParams p) {
  fetch_args_partial(p);
  // one-round launches (WPB 8) go slice-major, so that every unit's slices are spread over the launch order; many
  // rounds (WPB 4) keep a unit's slices together
  const int nu = int(gridDim.x) / p.P;
  const int u = WPB == 8 ? int(blockIdx.x) % nu : int(blockIdx.x) / p.P;
  const int sl = WPB == 8 ? int(blockIdx.x) / nu : int(blockIdx.x) - u * p.P;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int task = sl * WPB + wave;  // wave-uniform (scalar)

  __shared__ __attribute__((aligned(16))) float sm_o[WPB][G][kD];
  __shared__ float sm_m[WPB][G];
  __shared__ float sm_l[WPB][G];
  __shared__ __attribute__((aligned(16))) float plds_all[WPB][8 * 32];
  __shared__ __attribute__((aligned(16))) uint32_t meta_all[WPB][QW * 2 * kMetaWords];

  Ctx c;
  c.u = u;
  c.lane = lane;
  c.q = lane >> 4;
  c.col = lane & 15;
  c.unit_win = size_t(u) * p.NW;
  const int32_t* res = p.res_list + c.unit_win;
  const int32_t* rslot = p.res_slot + c.unit_win;
  const int MF = p.max_full;
  // task ranges: INT2 tasks, tail blocks, span-summary blocks (SUMMARY only), FULL windows
  const int t_tail = p.n_qt, t_sum = p.n_qt + p.n_tb, t_full = t_sum + (SUMMARY ? p.n_sb : 0), t_end = t_full + MF;
  const int q0 = task * QW;    // INT2 task: first INT2 slot
  const int f = task - t_full;  // FULL task: slot in res_list

  // one vector load gathers the unit's device counts (lanes 0..2), this wave's window ids (lanes 3 .. 3+QW-1)
  // and their slots (lanes 3+QW ..): the FULL window res_list[f] and res_slot[f], or the INT2 windows at the usual
  // offset n_full == max_full (re-read otherwise)
  int gv;
  {
    const int k = lane - 3;
    const bool want_slot = k >= QW;
    const int kk = want_slot ? k - QW : k;
    const int ridx = min(max(task >= t_full ? f : MF + q0 + kk, 0), p.NW - 1);
    const int32_t* cnt = lane == 0 ? p.n_full : (lane == 1 ? p.n_int2 : p.tail_len);
    const int32_t* gp = lane < 3 ? cnt + u : (want_slot ? rslot : res) + ridx;
    if constexpr (SUMMARY) {  // a summary-block task takes the unit's summary count in lane 3
      if (task >= t_sum && task < t_full && lane == 3) gp = p.n_sum + u;
    }
    gv = *gp;
  }
  int sid[QW], sslot[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    sid[i] = __builtin_amdgcn_readlane(gv, 3 + i);
    sslot[i] = __builtin_amdgcn_readlane(gv, 3 + QW + i);
  }
  // device counts are clamped to the host bounds the grid was sized for, so every index stays in range
  const int nf_dev = __builtin_amdgcn_readlane(gv, 0);
  const int nq_dev = __builtin_amdgcn_readlane(gv, 1);
  const int tl_dev = __builtin_amdgcn_readlane(gv, 2);
  c.nf = min(max(nf_dev, 0), p.max_full);
  c.nq = min(max(nq_dev, 0), p.max_int2);
  c.tl = min(max(tl_dev, 0), p.max_tail);
  c.has_new = p.k_new != nullptr ? 1 : 0;
  c.total_tail = c.tl + c.has_new;
  // the combine appends the new token and advances tail_len; its workgroups read this copy instead, so that
  // none of them can see the advanced value
  if (sl == 0 && threadIdx.x == 0) p.unit_tl[u] = c.tl;
  if (sl == 0 && threadIdx.x == 0 && (c.nf != nf_dev || c.nq != nq_dev || c.tl != tl_dev)) {
    atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
  }

  // A operand: the G query heads (rows; rows beyond G repeat head G-1 and their results are never used);
  // k-block k = head_dim 32k + 8*(lane/16) .. +7
  u32x4 aq[4];
  if (G <= 4 && task < t_tail) {
    // INT2 task: the A of head_dim group k holds head h's q in row 4k + h (rows past G repeat head G-1), zero in
    // the other rows, so the groups' products land in different rows of one tile
    const int gk = c.col >> 2;
    const u32x4 v = ld16(p.q + (size_t(u) * G + min(c.col & 3, G - 1)) * kD + 32 * gk + 8 * c.q);
#pragma unroll
    for (int k = 0; k < 4; ++k) aq[k] = gk == k ? v : zero4u();
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) aq[k] = ld16(p.q + (size_t(u) * G + min(c.col, G - 1)) * kD + 32 * k + 8 * c.q);
  }

  WaveOut wo;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    wo.m[r] = -INFINITY;
    wo.l[r] = 0.0f;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) wo.acc[dt] = zero4();
#pragma unroll
  for (int g = 0; g < 4; ++g) wo.bias[g] = 0.0f;
  float* plds = plds_all[wave];
  bool grouped = false;  // the wave ran an INT2 task whose P.V leaves tile dt in the columns of group dt/2

  if (task < t_tail) {
    if (q0 < c.nq) {
      grouped = G <= 4;
      if (c.nf != MF) {
#pragma unroll
        for (int i = 0; i < QW; ++i) {
          sid[i] = res[min(c.nf + q0 + i, p.NW - 1)];
          sslot[i] = rslot[min(c.nf + q0 + i, p.NW - 1)];
        }
      }
      int ids[QW], slots[QW];
      bool ok[QW];
      bool bad = false;
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        const bool in_range = unsigned(sid[i]) < unsigned(p.NW) && unsigned(sslot[i]) < unsigned(p.LS);
        ok[i] = q0 + i < c.nq && in_range;
        bad |= q0 + i < c.nq && !in_range;
        ids[i] = ok[i] ? sid[i] : 0;
        slots[i] = ok[i] ? sslot[i] : 0;
      }
      if (bad && lane == 0) atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
      int2_task<G, T, PROBS, QW, WEIGHTED>(p, c, ids, slots, ok, (c.nf + q0) * kW, aq, plds, meta_all[wave], wo);
    }
  } else if (task < t_sum) {
    const int blk = task - t_tail;
    if (kW * blk < c.total_tail) {
      dense_task<G, T, PROBS, true, WEIGHTED>(p, c, 0, 0, blk, min(kW, c.total_tail - kW * blk),
                                              (c.nf + c.nq + blk) * kW, aq, plds, wo);
    }
  } else if (SUMMARY && task < t_full) {
    if constexpr (SUMMARY) {
      const int blk = task - t_sum;
      const int ns_dev = __builtin_amdgcn_readlane(gv, 3);
      const int ns = min(max(ns_dev, 0), p.max_sum);
      if (blk == 0 && lane == 0 && ns != ns_dev) atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
      if (kW * blk < ns) {
        dense_task<G, T, false, true, WEIGHTED, true>(p, c, 0, 0, blk, min(kW, ns - kW * blk), 0, aq, plds, wo);
      }
    }
  } else if (task < t_end && f < c.nf) {
    const int id = sid[0], slot = sslot[0];
    if (unsigned(id) >= unsigned(p.NW) || unsigned(slot) >= unsigned(p.FS)) {
      if (lane == 0) atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
    } else {
      dense_task<G, T, PROBS, false, WEIGHTED>(p, c, id, slot, 0, kW, f * kW, aq, plds, wo);
    }
  }

  // ---- wave result: O[h][d] = acc + bias of d's head_dim group; merged over the workgroup's waves ----------------
  // (grouped: head h of tile dt in column 4 (dt/2) + h, the lane's group bias in bias[0]; else head h in column h)
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g == 0 || !grouped) {
      wo.bias[g] = xor_sum(wo.bias[g], 16);
      wo.bias[g] = xor_sum(wo.bias[g], 32);
    }
  }
  const int hl = grouped ? (c.col & 3) : c.col;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const bool st = hl < G && (!grouped || (c.col >> 2) == (dt >> 1));
    const float b = grouped ? wo.bias[0] : wo.bias[dt >> 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (st) sm_o[wave][hl][16 * dt + 4 * c.q + r] = wo.acc[dt][r] + b;
    }
  }
  if (c.col == 0 && 4 * c.q < G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * c.q + r;
      if (h < G) {
        sm_m[wave][h] = wo.m[r];
        sm_l[wave][h] = wo.l[r];
      }
    }
  }
  __syncthreads();
  // each wave's rescale factor per head, exp(m_w - max_w m_w), computed once
  __shared__ float sm_sc[WPB][G];
  if (threadIdx.x < WPB * G) {
    const int w = threadIdx.x / G, h = threadIdx.x - w * G;
    float Mx = sm_m[0][h];
#pragma unroll
    for (int w2 = 1; w2 < WPB; ++w2) Mx = fmaxf(Mx, sm_m[w2][h]);
    sm_sc[w][h] = exp_diff(sm_m[w][h], Mx);
    if (w == 0) {
      float L = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < WPB; ++w2) L += sm_l[w2][h] * exp_diff(sm_m[w2][h], Mx);
      const size_t part = size_t(u) * p.P + sl;
      p.part_ml[(part * G + h) * 2 + 0] = Mx;
      p.part_ml[(part * G + h) * 2 + 1] = L;
    }
  }
  __syncthreads();
  const size_t part = size_t(u) * p.P + sl;
  for (int i = threadIdx.x; i < G * kD; i += (WPB * kWave)) {
    const int h = i / kD;
    float O = 0.0f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) O += sm_o[w][h][i % kD] * sm_sc[w][h];
    p.part_o[part * G * kD + i] = O;
  }
}

// Combine: p.CB workgroups per unit; workgroup b owns E = G*D/CB output elements (thread (e, pg): element e,
// partials pg, pg + PG, ... with PG = 256/E, at most kPre of them per thread in the usual case) and a contiguous
// range of the unit's windows. Every load that does not depend on the merged (M, L) — the partial outputs and
// maxima of this thread, its windows' exp-sums, tiers and scores — is issued first; then each workgroup merges
// the partials' (m, l) per head (one pass, fixed order), weights and sums its outputs in a fixed order (bitwise
// reproducible), and turns its windows' exp-sums into probability mass.
constexpr int kPre = 9;  // partials preloaded per thread: 8 groups cover up to 72 (a one-round launch a task over)
constexpr int kMlPre = 4;

// the G per-head values of one window (16-byte aligned rows for G = 4, 8; the workspace is 256-byte aligned)
template <int G>
__device__ __forceinline__ void load_heads(const float* src, float (&dst)[G]) {
  if constexpr (G % 4 == 0) {
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(src)[i];
      dst[4 * i] = v.x;
      dst[4 * i + 1] = v.y;
      dst[4 * i + 2] = v.z;
      dst[4 * i + 3] = v.w;
    }
  } else if constexpr (G == 2) {
    const float2 v = *reinterpret_cast<const float2*>(src);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < G; ++i) dst[i] = src[i];
  }
}

template <int G>
__global__ __launch_bounds__(256) void decode_combine(DecodeParams p) {
  fetch_args_combine(p);
  const int u = blockIdx.x / p.CB;
  const int b = blockIdx.x - u * p.CB;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int CH = p.P;
  const int E = G * kD / p.CB;
  const int PG = 256 / E;
  const int e = threadIdx.x % E, pg = threadIdx.x / E;
  const int idx = b * E + e;
  const int h_out = idx / kD;
  const size_t unit_win = size_t(u) * p.NW;
  // the window range is cut from the capacity, so that no load waits for the unit's window count
  const int wpb = (p.NW + p.CB - 1) / p.CB;
  const int wb = b * wpb;
  const float* ml = p.part_ml + size_t(u) * CH * G * 2;
  const float* po = p.part_o + size_t(u) * CH * G * kD + idx;

  // (m, l) of the partials of the heads this wave merges (h = wave + 4i), the first kMlPre per lane
  constexpr int kHP = (G + 3) / 4;
  float pm[kHP][kMlPre], pl[kHP][kMlPre];
#pragma unroll
  for (int i = 0; i < kHP; ++i) {
    const int h = wave + 4 * i;
#pragma unroll
    for (int k = 0; k < kMlPre; ++k) {
      const int cc = lane + kWave * k;
      const bool in = h < G && cc < CH;
      const float2 v = in ? *reinterpret_cast<const float2*>(ml + (cc * G + h) * 2) : make_float2(-INFINITY, 0.0f);
      pm[i][k] = v.x;
      pl[i][k] = v.y;
    }
  }
  float ov[kPre], mv[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int cc = pg + k * PG;
    const bool in = p.out != nullptr && cc < CH;
    ov[k] = in ? po[size_t(cc) * G * kD] : 0.0f;
    mv[k] = in ? ml[(cc * G + h_out) * 2] : -INFINITY;
  }
  // first window of this thread: unconditional loads (index clamped into the unit), used only if w0 < we
  const int w0 = wb + int(threadIdx.x);
  const int w0c = min(w0, p.NW - 1);
  const int tier0 = p.tier[unit_win + w0c];
  float ws0[G], wr0[G];
  load_heads<G>(p.wsum + (unit_win + w0c) * G, ws0);
  load_heads<G>(p.wref + (unit_win + w0c) * G, wr0);
  const float cum0 = p.cum[unit_win + w0c];
  const int nw = min(max(p.n_windows[u], 0), p.NW);
  const int we = p.score ? min(nw, wb + wpb) : wb;  // a plain decode step (no score, no mass) has no window pass
  // the append's loads (tail length, the new K row and V column), issued with the others
  const int has_new = p.k_new != nullptr ? 1 : 0;
  const int tl = p.unit_tl[u];
  const bool appender = b == 0 && has_new;
  u32x4 kn = u32x4{0u, 0u, 0u, 0u};
  uint16_t vn = 0;
  if (appender && threadIdx.x < 16) kn = reinterpret_cast<const u32x4*>(p.k_new + size_t(u) * kD)[threadIdx.x];
  if (appender && threadIdx.x < kD) vn = p.v_new[size_t(u) * kD + threadIdx.x];

  __shared__ float sM[G], sInvL[G];
  __shared__ float red[256];
#pragma unroll
  for (int i = 0; i < kHP; ++i) {
    const int h = wave + 4 * i;
    if (h >= G) break;
    // the preloaded (m, l) pairs first, the rest (more than 256 partials) in a loop
    float mr = -INFINITY, lr = 0.0f;
#pragma unroll
    for (int k = 0; k < kMlPre; ++k) {
      const float mn = fmaxf(mr, pm[i][k]);
      lr = lr * exp_diff(mr, mn) + pl[i][k] * exp_diff(pm[i][k], mn);
      mr = mn;
    }
    for (int cc = lane + kWave * kMlPre; cc < CH; cc += kWave) {
      const float mc = ml[(cc * G + h) * 2], lc = ml[(cc * G + h) * 2 + 1];
      const float mn = fmaxf(mr, mc);
      lr = lr * exp_diff(mr, mn) + lc * exp_diff(mc, mn);
      mr = mn;
    }
    const float mx = wave_max(mr);
    const float sum = wave_sum(lr * exp_diff(mr, mx));
    if (lane == 0) {
      sM[h] = mx;
      sInvL[h] = sum > 0.0f ? 1.0f / sum : 0.0f;
    }
  }
  __syncthreads();

  if (p.out != nullptr) {
    const float Mh = sM[h_out], iL = sInvL[h_out];
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < kPre; ++k) acc += ov[k] * exp_diff(mv[k], Mh);
    // partials beyond the preloaded ones, eight loads in flight at a time (same sequential order)
    for (int cc0 = pg + kPre * PG; cc0 < CH; cc0 += 8 * PG) {
      float o8[8], m8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int cc = cc0 + k * PG;
        o8[k] = cc < CH ? po[size_t(cc) * G * kD] : 0.0f;
        m8[k] = cc < CH ? ml[(cc * G + h_out) * 2] : -INFINITY;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += o8[k] * exp_diff(m8[k], Mh);
    }
    red[threadIdx.x] = acc * iL;
    __syncthreads();
    if (int(threadIdx.x) < E) {
      // sequential order; eight LDS reads in flight at a time
      float o = 0.0f;
      int g2 = 0;
      for (; g2 + 8 <= PG; g2 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = red[(g2 + j) * E + threadIdx.x];
#pragma unroll
        for (int j = 0; j < 8; ++j) o += v[j];
      }
      for (; g2 < PG; ++g2) o += red[g2 * E + threadIdx.x];
      p.out[size_t(u) * G * kD + idx] = o;
    }
  }
  // window mass = (1/G) sum_h wsum * exp(wref - M_h) / L_h; cumulative score += mass
  for (int w = w0; w < we; w += 256) {
    bool resident = tier0 != KVC_TIER_EVICTED;
    float cw = cum0;
    if (w != w0) {
      resident = p.tier[unit_win + w] != KVC_TIER_EVICTED;
      if (p.accumulate) cw = p.cum[unit_win + w];
    }
    float mass = 0.0f;
    if (resident) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float s = w == w0 ? ws0[h] : p.wsum[(unit_win + w) * G + h];
        const float r = w == w0 ? wr0[h] : p.wref[(unit_win + w) * G + h];
        mass += s * exp_diff(r, sM[h]) * sInvL[h];
      }
      mass *= 1.0f / G;
      if (p.accumulate) p.cum[unit_win + w] = cw + mass;
    }
    if (p.mass != nullptr) p.mass[unit_win + w] = mass;
  }
  if (p.probs != nullptr) {
    const int nf = min(max(p.n_full[u], 0), p.max_full);
    const int nq = min(max(p.n_int2[u], 0), p.max_int2);
    const int n_res = (nf + nq) * kW + tl + has_new;
    for (int h = 0; h < G; ++h) {
      float* pr = p.probs + (size_t(u) * G + h) * p.probs_stride;
      for (int i = b * 256 + threadIdx.x; i < n_res; i += 256 * p.CB) pr[i] = exp_diff(pr[i], sM[h]) * sInvL[h];
    }
  }
  if (appender) {
    // append the step's token to the tail (K row-major, V into its head_dim-major 32-token block)
    if (threadIdx.x < 16) reinterpret_cast<u32x4*>(p.k_tail + (size_t(u) * p.TM + tl) * kD)[threadIdx.x] = kn;
    if (threadIdx.x < kD) p.v_tail[(size_t(u) * p.TM + (tl & ~(kW - 1))) * kD + threadIdx.x * kW + (tl & (kW - 1))] = vn;
    if (threadIdx.x == 0) p.tail_len[u] = tl + 1;
  }
}

struct Shape {
  int qw, wpb;
};

template <int G, class T, int QW, int WPB, bool WEIGHTED>
void launch_partial_w(const DecodeParams& p, int U, hipStream_t s) {
  if (p.max_sum > 0) {  // summaries are attended only without probabilities (checked by the caller)
    hipLaunchKernelGGL((decode_partial<G, T, false, QW, WPB, WEIGHTED, true>), dim3(U * p.P), dim3(WPB * kWave), 0, s,
                       p);
  } else if (p.probs != nullptr) {
    hipLaunchKernelGGL((decode_partial<G, T, true, QW, WPB, WEIGHTED, false>), dim3(U * p.P), dim3(WPB * kWave), 0, s,
                       p);
  } else {
    hipLaunchKernelGGL((decode_partial<G, T, false, QW, WPB, WEIGHTED, false>), dim3(U * p.P), dim3(WPB * kWave), 0,
                       s, p);
  }
}

template <int G, class T, int QW, int WPB>
void launch_partial(const DecodeParams& p, int U, hipStream_t s) {
  if (p.wnorm != nullptr) {
    launch_partial_w<G, T, QW, WPB, true>(p, U, s);
  } else {
    launch_partial_w<G, T, QW, WPB, false>(p, U, s);
  }
}

template <int G, class T>
hipError_t launch_g(const DecodeParams& p, int U, Shape sh, hipStream_t s) {
  if (sh.qw == 1) {
    launch_partial<G, T, 1, 8>(p, U, s);
  } else {
    launch_partial<G, T, 2, 4>(p, U, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine<G>), dim3(U * p.CB), dim3(256), 0, s, p);
  return hipGetLastError();
}

struct TaskCounts {
  int n_tb, n_qt, n_sb, tasks;
};

TaskCounts task_counts(const kvc_decode_args& a, int qw) {
  const int has_new = a.k_new != nullptr ? 1 : 0;
  TaskCounts t;
  t.n_tb = (a.max_tail + has_new + kW - 1) / kW;
  t.n_qt = (a.max_int2 + qw - 1) / qw;
  t.n_sb = (a.max_summary + kW - 1) / kW;
  t.tasks = a.max_full + t.n_tb + t.n_qt + t.n_sb;
  return t;
}

// compute units of the current device (cached per device)
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// (1, 8) while the (1, 8) grid fits in two rounds of resident workgroups (two 8-wave workgroups per CU at four
// waves per SIMD), else (2, 4)
Shape decode_shape(const kvc_cache& c, const kvc_decode_args& a) {
  const TaskCounts t = task_counts(a, 1);
  const int64_t wgs = int64_t(c.n_units) * ((t.tasks + 7) / 8);
  return wgs <= 2 * 2 * int64_t(device_cus()) ? Shape{1, 8} : Shape{2, 4};
}

int combine_blocks(const kvc_cache& c, int P) {
  // partial groups so that a thread holds at most kPre partials, output elements E = 256 / PG (at most G*D); at
  // most 16 groups, so that a workgroup reads at least 16 consecutive floats (64 bytes) of every partial row:
  // with many partials (the full-cache phase), 4-element slices pulled whole 128-byte lines for 16 bytes
  int pg = 1;
  while (pg < 16 && pg * kPre < P) pg *= 2;
  int E = min(256 / pg, c.group * kD);
  int cb = c.group * kD / E;
  // many units: fewer, fuller workgroups (about four per CU in all); a thread then takes more partials, the ones
  // past kPre eight loads at a time
  const int target = max(1, 4 * device_cus() / max(1, c.n_units));
  while (cb > target && cb % 2 == 0 && 2 * E <= 256) {
    E *= 2;
    cb /= 2;
  }
  return cb;
}

}  // namespace

int decode_slices(const kvc_cache& c, const kvc_decode_args& a) {
  const Shape sh = decode_shape(c, a);
  const TaskCounts t = task_counts(a, sh.qw);
  return max(1, (t.tasks + sh.wpb - 1) / sh.wpb);
}

bool decode_supported(const kvc_cache& c, const kvc_decode_args& a) { return decode_slices(c, a) <= kMaxParts; }

size_t decode_workspace_bytes(const kvc_cache& c, const kvc_decode_args& a) {
  const size_t U = size_t(c.n_units), G = size_t(c.group), P = size_t(decode_slices(c, a));
  size_t b = 0;
  b += align_up(U * P * G * 2 * sizeof(float), 256);
  b += align_up(U * P * G * kD * sizeof(float), 256);
  b += 2 * align_up(U * size_t(c.n_windows_max) * G * sizeof(float), 256);
  b += align_up(U * sizeof(int32_t), 256);
  return b;
}

hipError_t launch_decode(const kvc_cache& c, const kvc_decode_args& a, void* ws, hipStream_t s) {
  DecodeParams p{};
  p.NW = c.n_windows_max;
  p.TM = c.tail_max;
  p.FS = c.full_slots;
  p.LS = c.ledger_slots;
  p.k_full = static_cast<const uint16_t*>(c.k_full);
  p.v_full = static_cast<const uint16_t*>(c.v_full);
  p.k_codes = c.k_codes;
  p.v_codes = reinterpret_cast<const uint16_t*>(c.v_codes);
  p.k_meta = c.k_meta;
  p.v_meta = c.v_meta;
  p.k_tail = static_cast<uint16_t*>(c.k_tail);
  p.v_tail = static_cast<uint16_t*>(c.v_tail);
  p.tail_len = c.tail_len;
  p.res_list = c.res_list;
  p.res_slot = c.res_slot;
  p.n_full = c.n_full;
  p.n_int2 = c.n_int2;
  p.n_windows = c.n_windows;
  p.tier = c.tier;
  p.cum = c.cum;
  p.status = c.status;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_new = static_cast<const uint16_t*>(a.k_new);
  p.v_new = static_cast<const uint16_t*>(a.v_new);
  p.out = a.out;
  p.probs = a.probs;
  p.mass = a.mass;
  p.probs_stride = a.probs_stride;
  p.accumulate = a.accumulate_cum;
  p.max_full = a.max_full;
  p.max_int2 = a.max_int2;
  p.max_tail = a.max_tail;
  p.score = (a.accumulate_cum != 0 || a.mass != nullptr) ? 1 : 0;
  p.wnorm = a.token_weight;
  p.wstride = long(a.weight_stride);
  const Shape sh = decode_shape(c, a);
  const TaskCounts tc = task_counts(a, sh.qw);
  p.n_tb = tc.n_tb;
  p.n_qt = tc.n_qt;
  p.n_sb = tc.n_sb;
  p.k_sum = static_cast<const uint16_t*>(c.k_sum);
  p.v_sum = static_cast<const uint16_t*>(c.v_sum);
  p.n_sum = c.n_sum;
  p.SM = c.sum_max;
  p.max_sum = a.max_summary;
  p.P = decode_slices(c, a);
  p.CB = combine_blocks(c, p.P);
  if (p.P > kMaxParts) return hipErrorInvalidValue;
  const size_t U = size_t(c.n_units), G = size_t(c.group), P = size_t(p.P);
  char* w = static_cast<char*>(ws);
  p.part_ml = reinterpret_cast<float*>(w);
  w += align_up(U * P * G * 2 * sizeof(float), 256);
  p.part_o = reinterpret_cast<float*>(w);
  w += align_up(U * P * G * kD * sizeof(float), 256);
  p.wsum = reinterpret_cast<float*>(w);
  w += align_up(U * size_t(c.n_windows_max) * G * sizeof(float), 256);
  p.wref = reinterpret_cast<float*>(w);
  w += align_up(U * size_t(c.n_windows_max) * G * sizeof(float), 256);
  p.unit_tl = reinterpret_cast<int32_t*>(w);
  const int Ui = c.n_units;
  const bool bf = c.kv_dtype == KVC_BF16;
  switch (c.group) {
    case 1: return bf ? launch_g<1, BF16>(p, Ui, sh, s) : launch_g<1, F16>(p, Ui, sh, s);
    case 2: return bf ? launch_g<2, BF16>(p, Ui, sh, s) : launch_g<2, F16>(p, Ui, sh, s);
    case 4: return bf ? launch_g<4, BF16>(p, Ui, sh, s) : launch_g<4, F16>(p, Ui, sh, s);
    case 8: return bf ? launch_g<8, BF16>(p, Ui, sh, s) : launch_g<8, F16>(p, Ui, sh, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvc
