// Split-K GQA decode attention over the mixed full-precision / INT2 / tail cache, window scores fused.
//
// What it computes follows the QEvict page ("Mecanismos Principais"): attention over the resident windows (the
// full-precision tier and the INT2 tier, dequantised in registers), the cumulative window score updated from
// each window's attention mass, grouped-query attention (G query heads share one KV head).
//
// decode_partial: one workgroup (4 waves, one per SIMD) per (unit, slice). A slice is a contiguous share of the
// unit's FULL windows, 32-token tail blocks and INT2 windows ("items"); wave w takes items w, w+4, ...
//   * Items stream through two 16 KiB LDS slots per wave, filled by direct global->LDS loads
//     (global_load_lds_dwordx4), so two items are always in flight without holding VGPRs; the wave waits on
//     vmcnt for the item it is about to use. Each lane later reads back exactly the 16 bytes it brought in, in
//     the lane order the MFMA operands want (conflict-free).
//   * q.K^T on MFMA (v_mfma_f32_16x16x32 bf16/f16): A = the G query heads (rows, zero-padded to 16), B = 16
//     tokens x 32 head_dim of K. INT2 keys enter B as 128+c (bf16) / 1024+c (fp16) bit patterns, one group of 32
//     head_dim per MFMA; the group's scale/zero are applied to the fp32 product:  s*acc + (z - magic*s)*sum(q).
//   * Online softmax at window granularity (running max / sum per head, the output rescaled when the max moves);
//     each window's exp-sum and reference max are kept for the score.
//   * P.V on MFMA: A = 16 head_dim x 32 tokens of V (V is stored transposed per window), B = P^T split into a
//     high and a low part (columns 0..G-1 and G..2G-1) so the product keeps ~16 bits of P. INT2 values enter A as
//     exact fp16 codes and the per-token scale is folded into B (P*s); the zero term sum(P*z) is a VALU bias.
//   The four waves merge their (m, l, o) in LDS into one partial per workgroup.
// decode_combine: merges the partials of a unit in a fixed order (bitwise reproducible), writes o, converts the
// window exp-sums into probability mass, adds it to the cumulative score, finalises the optional probabilities
// and appends the step's token to the tail.
#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;
constexpr int kMaxWgItems = 64;     // windows + tail blocks per workgroup
constexpr int kMaxParts = 4096;     // slices per unit
constexpr int kSlotBytes = 16384;   // one dense item: K (8 KiB) + V^T (8 KiB)
constexpr float kInvSqrtD = 0.088388347648318440550f;  // 1/sqrt(128)

enum ItemKind : int { kFull = 0, kInt2 = 1, kTail = 2 };

struct DecodeParams {
  int NW, TM;
  const uint16_t* k_win;
  const uint16_t* v_win;
  const uint8_t* k_codes;
  const uint16_t* v_codes;
  const uint32_t* k_meta;
  const uint32_t* v_meta;
  uint16_t* k_tail;
  uint16_t* v_tail;
  int32_t* tail_len;
  const int32_t* res_list;
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
  int P;           // slices (workgroups) per unit
  float* part_ml;  // [U][P][G][2]
  float* part_o;   // [U][P][G][D]
  float* wsum;     // [U][NW][G]
  float* wref;     // [U][NW][G]
};

// ---- MFMA and conversions per storage dtype ----------------------------------------------------------------
struct MBF16 {
  static constexpr uint32_t kMagic = 0x43004300u;  // two bf16 128.0
  static constexpr float kMagicVal = 128.0f;
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
__device__ __forceinline__ u32x4 codes_to_f16(uint32_t c16) {
  const uint32_t z = c16 | (c16 << 14);
  const uint32_t w0 = (z & 0x00030003u) | MF16::kMagic;
  const uint32_t w1 = ((z >> 4) & 0x00030003u) | MF16::kMagic;
  const uint32_t w2 = ((z >> 8) & 0x00030003u) | MF16::kMagic;
  const uint32_t w3 = ((z >> 12) & 0x00030003u) | MF16::kMagic;
  return u32x4{f16x2_minus_1024(w0), f16x2_minus_1024(w1), f16x2_minus_1024(w2), f16x2_minus_1024(w3)};
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

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 lds16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// direct global -> LDS copy: every active lane's 16 bytes land at slot + 16 * lane
__device__ __forceinline__ void dma16(const void* g, uint8_t* slot) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(slot), 16, 0, 0);
}

// s_waitcnt vmcnt(N) only (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at max)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct Item {
  int kind;
  int id;      // window id (FULL/INT2) or tail block index (TAIL)
  int pos;     // resident position of its first key (for the optional probabilities)
  int nvalid;  // valid keys (32 for a window, fewer in the last tail block, 0 for a rejected window id)
  int slot;    // index of the item in the slice (LDS score arrays)
};

struct Ctx {
  int u, lane, q, col, tl, total_tail, has_new;
  size_t unit_win;
  const uint16_t* knew;  // LDS copy of k_new[u] (zeros without an append)
  const uint16_t* vnew;  // LDS copy of v_new[u]
};

// Global -> LDS loads of one item (number of load instructions: dense 16, INT2 4).
//   dense (FULL window [32][D] or tail block [32][D] + [D][32]): instruction t*4+k: lane (row, q) brings K tokens
//     16t + row, head_dim 32k + 8q .. +7; instruction 8 + dt: V^T head_dim 16dt + row, tokens 8q .. +7.
//   INT2: plain copies: K codes (1 KiB) at 0, K meta (512 B) at 1024, V codes (1 KiB) at 1536, V meta (512 B) at
//     2560.
constexpr int kDenseLoads = 16;
constexpr int kInt2Loads = 4;

__device__ __forceinline__ void issue_item(const DecodeParams& p, const Ctx& c, const Item& it, uint8_t* slot) {
  const int row = c.col;
  if (it.kind != kInt2) {
    const uint16_t* kb = it.kind == kTail ? p.k_tail + (size_t(c.u) * p.TM + 32 * it.id) * kD
                                          : p.k_win + (c.unit_win + it.id) * size_t(kW * kD);
    const uint16_t* vb = it.kind == kTail ? p.v_tail + (size_t(c.u) * p.TM + 32 * it.id) * kD
                                          : p.v_win + (c.unit_win + it.id) * size_t(kW * kD);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int k = 0; k < 4; ++k) dma16(kb + (16 * t + row) * kD + 32 * k + 8 * c.q, slot + (t * 4 + k) * 1024);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dma16(vb + (16 * dt + row) * kW + 8 * c.q, slot + (8 + dt) * 1024);
  } else {
    const size_t win = c.unit_win + it.id;
    dma16(p.k_codes + win * (kW * kCodeBytes) + 16 * c.lane, slot);
    dma16(p.v_codes + win * (kW * kD / 8) + 8 * c.lane, slot + 1536);
    if (c.lane < 32) {
      dma16(p.k_meta + win * (kW * kGroups) + 4 * c.lane, slot + 1024);
      dma16(p.v_meta + win * (kW * kGroups) + 4 * c.lane, slot + 2560);
    }
  }
}

template <int G>
struct WaveState {
  float m[G], l[G];
  f32x4 acc[8];   // O^T tiles: lane column col (hi/lo head), head_dim 16*dt + 4*(lane/16) + r
  float bias[4];  // sum P*z per group (column col < G: head col)
};

// Online softmax step for one item: S (logits, masked) -> running max/sum, window sum to LDS, rescale of the
// output; returns in x[8] this lane's B-operand row of P^T (head col % G, tokens 8*(lane/16) .. +7).
template <int G, bool PROBS>
__device__ __forceinline__ void softmax_step(const DecodeParams& p, const Ctx& c, const Item& it, f32x4 (&S)[2],
                                             WaveState<G>& st, float* plds, float (*wsl)[G], float (*wrl)[G],
                                             float (&x)[8]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool ok = 16 * t + c.col < it.nvalid;
#pragma unroll
    for (int r = 0; r < 4; ++r) S[t][r] = ok ? S[t][r] * kInvSqrtD : -INFINITY;
  }
  float alpha[G], mnew[G];
  bool any_scale = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int r = h & 3;
    float v = fmaxf(S[0][r], S[1][r]);
    v = xor_max(v, 1);
    v = xor_max(v, 2);
    v = xor_max(v, 4);
    v = xor_max(v, 8);
    const float mwin = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * (h >> 2)));
    mnew[h] = fmaxf(st.m[h], mwin);
    alpha[h] = exp_diff(st.m[h], mnew[h]);
    any_scale |= alpha[h] != 1.0f;
  }
  f32x4 Pp[2];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float mrow = mnew[r < G ? r : 0];
    if (G > 4 && c.q == 1) mrow = mnew[(4 + r) < G ? 4 + r : 0];
#pragma unroll
    for (int t = 0; t < 2; ++t) Pp[t][r] = exp_diff(S[t][r], mrow);
  }
  const bool head_lane = 4 * c.q < G;  // lane group holding real heads
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int r = h & 3;
    float v = Pp[0][r] + Pp[1][r];
    v = xor_sum(v, 1);
    v = xor_sum(v, 2);
    v = xor_sum(v, 4);
    v = xor_sum(v, 8);
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * (h >> 2)));
    st.l[h] = st.l[h] * alpha[h] + ws;
    st.m[h] = mnew[h];
    if (c.lane == 0) {
      wsl[it.slot][h] = ws;
      wrl[it.slot][h] = mnew[h];
    }
  }
  if (PROBS && head_lane) {
    float* pb = p.probs + size_t(c.u) * G * p.probs_stride + it.pos;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * c.q + r;
      if (h < G) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (16 * t + c.col < it.nvalid) pb[size_t(h) * p.probs_stride + 16 * t + c.col] = S[t][r];
        }
      }
    }
  }
  const int hcol = c.col < 2 * G ? (c.col % G) : 0;
  if (any_scale) {
    float a = alpha[0];
#pragma unroll
    for (int h = 1; h < G; ++h) a = hcol == h ? alpha[h] : a;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acc[dt] *= a;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.bias[g] *= a;
  }
  // P^T through LDS (plds[h][token]) into the B operand layout
  if (head_lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * c.q + r;
      if (h < G) {
        plds[h * 32 + c.col] = Pp[0][r];
        plds[h * 32 + 16 + c.col] = Pp[1][r];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
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
  __builtin_amdgcn_wave_barrier();
}

// FULL window or tail block, from its LDS slot
template <int G, class T, bool PROBS>
__device__ __forceinline__ void process_dense(const DecodeParams& p, const Ctx& c, const Item& it, const uint8_t* slot,
                                              const u32x4 (&aq)[4], WaveState<G>& st, float* plds, float (*wsl)[G],
                                              float (*wrl)[G]) {
  using M = typename MfmaOf<T>::M;
  u32x4 kr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kr[j] = lds16(slot + j * 1024 + 16 * c.lane);
  if (it.kind == kTail) {  // the step's new token is not in the tail yet: take it from the LDS copy of k_new
    const int tnew = c.has_new ? c.tl - 32 * it.id : -1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool is_new = 16 * t + c.col == tnew;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 y = *reinterpret_cast<const u32x4*>(c.knew + 32 * k + 8 * c.q);
        kr[t * 4 + k] = is_new ? y : kr[t * 4 + k];
      }
    }
  }
  f32x4 S[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    S[t] = zero4();
#pragma unroll
    for (int k = 0; k < 4; ++k) S[t] = M::mfma(aq[k], kr[t * 4 + k], S[t]);
  }
  float x[8];
  softmax_step<G, PROBS>(p, c, it, S, st, plds, wsl, wrl, x);
  u32x4 B = split8<M>(x, c.col >= G);
  if (c.col >= 2 * G) B = zero4u();
  u32x4 vr[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) vr[dt] = lds16(slot + (8 + dt) * 1024 + 16 * c.lane);
  if (it.kind == kTail) {  // new token from v_new; values past the valid length zeroed (no inf * 0)
    const int t0 = 32 * it.id + 8 * c.q;
    const int e_new = c.has_new ? c.tl - t0 : -1;
    const int n_ok = min(max(c.total_tail - t0, 0), 8);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint32_t nv = c.vnew[16 * dt + c.col];
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
  for (int dt = 0; dt < 8; ++dt) st.acc[dt] = M::mfma(vr[dt], B, st.acc[dt]);
}

// INT2 window, from its LDS slot
template <int G, class T, bool PROBS>
__device__ __forceinline__ void process_int2(const DecodeParams& p, const Ctx& c, const Item& it, const uint8_t* slot,
                                             const u32x4 (&aq)[4], const float (&qsum)[4][4], WaveState<G>& st,
                                             float* plds, float (*wsl)[G], float (*wrl)[G]) {
  using M = typename MfmaOf<T>::M;
  const int row = c.col;
  f32x4 S[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    S[t] = zero4();
    const uint2 cw = *reinterpret_cast<const uint2*>(slot + (16 * t + row) * kCodeBytes + 8 * c.q);
    const u32x4 meta = lds16(slot + 1024 + (16 * t + row) * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = k < 2 ? cw.x : cw.y;
      const uint32_t c16 = (w >> (16 * (k & 1))) & 0xFFFFu;
      const f32x4 o = M::mfma(aq[k], expand_codes(c16, M::kMagic), zero4());
      const uint32_t mw = k == 0 ? meta.x : (k == 1 ? meta.y : (k == 2 ? meta.z : meta.w));
      const float s = half_bits_to_float(mw & 0xFFFFu);
      const float zz = half_bits_to_float(mw >> 16) - M::kMagicVal * s;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[t][r] += s * o[r] + zz * qsum[k][r];
    }
  }
  float x[8];
  softmax_step<G, PROBS>(p, c, it, S, st, plds, wsl, wrl, x);
  const bool live = c.col < 2 * G;
  const bool low = c.col >= G;
  const u32x4 vc = lds16(slot + 1536 + (row * 4 + c.q) * 16);
  const uint8_t* vm = slot + 2560 + c.q * 128;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const u32x4 m0 = lds16(vm + 32 * g);
    const u32x4 m1 = lds16(vm + 32 * g + 16);
    const uint32_t mws[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float y[8];
    float zsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = x[e] * half_bits_to_float(mws[e] & 0xFFFFu);
      zsum = fmaf(x[e], half_bits_to_float(mws[e] >> 16), zsum);
    }
    st.bias[g] += zsum;
    u32x4 B = split8<MF16>(y, low);
    if (!live) B = zero4u();
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int dt = 2 * g + h2;
      const uint32_t wv = dt < 2 ? vc.x : (dt < 4 ? vc.y : (dt < 6 ? vc.z : vc.w));
      const uint32_t c16 = (wv >> (16 * (dt & 1))) & 0xFFFFu;
      st.acc[dt] = MF16::mfma(codes_to_f16(c16), B, st.acc[dt]);
    }
  }
}

template <int G, class T, bool PROBS>
__global__ __launch_bounds__(kBlock) void decode_partial(DecodeParams p) {
  const int u = blockIdx.x / p.P;
  const int sl = blockIdx.x - u * p.P;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;

  // device counts are clamped to the host bounds the grid was sized for, so every index stays in range
  const int nf_dev = p.n_full[u], nq_dev = p.n_int2[u], tl_dev = p.tail_len[u];
  const int nf = min(max(nf_dev, 0), p.max_full);
  const int nq = min(max(nq_dev, 0), p.max_int2);
  const int tl = min(max(tl_dev, 0), p.max_tail);
  const int has_new = p.k_new != nullptr ? 1 : 0;
  if (sl == 0 && threadIdx.x == 0 && (nf != nf_dev || nq != nq_dev || tl != tl_dev)) {
    atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
  }
  Ctx c;
  c.u = u;
  c.lane = lane;
  c.q = lane >> 4;
  c.col = lane & 15;
  c.tl = tl;
  c.has_new = has_new;
  c.total_tail = tl + has_new;
  c.unit_win = size_t(u) * p.NW;

  // this slice's share of FULL windows, tail blocks and INT2 windows (at most kMaxWgItems in all)
  const int n_tb = (c.total_tail + kW - 1) / kW;
  const int f0 = int((long(sl) * nf) / p.P), f1 = int((long(sl + 1) * nf) / p.P);
  const int q0 = int((long(sl) * nq) / p.P), q1 = int((long(sl + 1) * nq) / p.P);
  const int t0 = int((long(sl) * n_tb) / p.P), t1 = int((long(sl + 1) * n_tb) / p.P);
  const int nF = min(f1 - f0, kMaxWgItems);
  const int nT = min(t1 - t0, kMaxWgItems - nF);
  const int nQ = min(q1 - q0, kMaxWgItems - nF - nT);
  const int nD = nF + nT;
  const int n_items = nD + nQ;
  const int tail_pos0 = (nf + nq) * kW;

  __shared__ __attribute__((aligned(16))) uint8_t stage[kWavesPerBlock][2][kSlotBytes];
  __shared__ int ids[kMaxWgItems];
  __shared__ __attribute__((aligned(16))) uint16_t knew_s[kD];
  __shared__ __attribute__((aligned(16))) uint16_t vnew_s[kD];
  __shared__ __attribute__((aligned(16))) float plds_all[kWavesPerBlock][8 * 32];
  __shared__ float wsl[kMaxWgItems][G];  // window exp-sums, relative to wrl
  __shared__ float wrl[kMaxWgItems][G];  // reference max of each window exp-sum
  __shared__ float sm_m[kWavesPerBlock][G];
  __shared__ float sm_l[kWavesPerBlock][G];

  if (threadIdx.x < nF + nQ) {
    const int i = threadIdx.x;
    const int32_t* res = p.res_list + c.unit_win;
    int w = i < nF ? res[f0 + i] : res[nf + q0 + (i - nF)];
    if (unsigned(w) >= unsigned(p.NW)) {
      atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
      w = -1;
    }
    ids[i] = w;
  }
  if (threadIdx.x < 32) {
    const uint16_t* src = threadIdx.x < 16 ? p.k_new : p.v_new;
    u32x4 v = zero4u();
    if (has_new) v = ld16(src + size_t(u) * kD + 8 * (threadIdx.x & 15));
    *reinterpret_cast<u32x4*>((threadIdx.x < 16 ? knew_s : vnew_s) + 8 * (threadIdx.x & 15)) = v;
  }
  c.knew = knew_s;
  c.vnew = vnew_s;

  // A operand: the G query heads (rows), zero rows beyond G; k-block k = head_dim 32k + 8*(lane/16) .. +7
  u32x4 aq[4];
  float qsum[4][4];  // qsum[k][r]: sum over head_dim group k of q[head 4*(lane/16) + r], fp32
  {
    using M = typename MfmaOf<T>::M;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 v = ld16(p.q + (size_t(u) * G + min(c.col, G - 1)) * kD + 32 * k + 8 * c.q);
      aq[k] = c.col < G ? v : zero4u();
    }
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
  __syncthreads();

  // item order inside the slice: dense items first (FULL windows, then tail blocks), then INT2 windows
  auto item_at = [&](int idx) {
    Item it;
    it.slot = idx;
    if (idx < nF) {
      it.kind = kFull;
      it.id = ids[idx];
      it.pos = (f0 + idx) * kW;
      it.nvalid = kW;
    } else if (idx < nD) {
      it.kind = kTail;
      it.id = t0 + idx - nF;
      it.pos = tail_pos0 + 32 * it.id;
      it.nvalid = min(kW, c.total_tail - 32 * it.id);
    } else {
      it.kind = kInt2;
      it.id = ids[nF + idx - nD];
      it.pos = (nf + q0 + idx - nD) * kW;
      it.nvalid = kW;
    }
    if (it.kind != kTail && it.id < 0) {  // rejected window id: read window 0, mask every key
      it.id = 0;
      it.nvalid = 0;
    }
    return it;
  };

  WaveState<G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.0f;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.acc[dt] = zero4();
#pragma unroll
  for (int g = 0; g < 4; ++g) st.bias[g] = 0.0f;
  float* plds = plds_all[wave];
  uint8_t* slots[2] = {stage[wave][0], stage[wave][1]};

  // this wave's items: wave, wave + 4, ...; two in flight (slot i & 1)
  const int my_n = n_items > wave ? (n_items - wave + kWavesPerBlock - 1) / kWavesPerBlock : 0;
  if (my_n > 0) issue_item(p, c, item_at(wave), slots[0]);
  if (my_n > 1) issue_item(p, c, item_at(wave + kWavesPerBlock), slots[1]);
  for (int i = 0; i < my_n; ++i) {
    const Item it = item_at(wave + kWavesPerBlock * i);
    uint8_t* slot = slots[i & 1];
    // wait for this item's loads; the next item's may stay in flight
    if (PROBS || i + 1 >= my_n) {
      wait_vm<0>();
    } else if (item_at(wave + kWavesPerBlock * (i + 1)).kind == kInt2) {
      wait_vm<kInt2Loads>();
    } else {
      wait_vm<kDenseLoads>();
    }
    if (it.kind == kInt2) {
      process_int2<G, T, PROBS>(p, c, it, slot, aq, qsum, st, plds, wsl, wrl);
    } else {
      process_dense<G, T, PROBS>(p, c, it, slot, aq, st, plds, wsl, wrl);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every LDS read of the slot has returned
    if (i + 2 < my_n) issue_item(p, c, item_at(wave + kWavesPerBlock * (i + 2)), slot);
  }

  // ---- wave result: O[h][d] = acc(col h) + acc(col h + G) + bias(group of d); merged over the 4 waves ----
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    st.bias[g] = xor_sum(st.bias[g], 16);
    st.bias[g] = xor_sum(st.bias[g], 32);
  }
  __syncthreads();  // every wave is done with its slots: the staging area now holds the wave outputs
  float* sm_o = reinterpret_cast<float*>(&stage[0][0][0]);  // [4][G][D]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lo = __shfl_down(st.acc[dt][r], G, kWave);
      if (c.col < G) sm_o[(wave * G + c.col) * kD + 16 * dt + 4 * c.q + r] = st.acc[dt][r] + lo + st.bias[dt >> 1];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = st.m[h];
      sm_l[wave][h] = st.l[h];
    }
  }
  __syncthreads();
  const size_t part = size_t(u) * p.P + sl;
  for (int i = threadIdx.x; i < G * kD; i += kBlock) {
    const int h = i / kD;
    float Mx = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) Mx = fmaxf(Mx, sm_m[w][h]);
    float O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) O += sm_o[(w * G + h) * kD + i % kD] * exp_diff(sm_m[w][h], Mx);
    p.part_o[part * G * kD + i] = O;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float Mx = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) Mx = fmaxf(Mx, sm_m[w][h]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) L += sm_l[w][h] * exp_diff(sm_m[w][h], Mx);
    p.part_ml[(part * G + h) * 2 + 0] = Mx;
    p.part_ml[(part * G + h) * 2 + 1] = L;
  }
  for (int i = threadIdx.x; i < (nF + nQ) * G; i += kBlock) {
    const int j = i / G, h = i % G;  // j-th window of the slice (FULL then INT2)
    const int w = ids[j];
    const int idx = j < nF ? j : nD + (j - nF);
    if (w >= 0) {
      p.wsum[(c.unit_win + w) * G + h] = wsl[idx][h];
      p.wref[(c.unit_win + w) * G + h] = wrl[idx][h];
    }
  }
}

// Combine: kCombineBlocks workgroups per unit. Each recomputes the per-head merge weights f[c][h] =
// exp(m_c - M_h) / L_h of the unit's partials, then handles its slice of the outputs, windows and probs.
constexpr int kCombineBlocks = 8;

template <int G>
__global__ __launch_bounds__(256) void decode_combine(DecodeParams p) {
  const int u = blockIdx.x / kCombineBlocks;
  const int b = blockIdx.x - u * kCombineBlocks;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int CH = p.P;
  __shared__ float sM[G], sL[G];
  __shared__ float f[kMaxParts / 4][G];
  __shared__ float red[4][64];
  const float* ml = p.part_ml + size_t(u) * CH * G * 2;
  for (int h = wave; h < G; h += 4) {
    float mx = -INFINITY;
    for (int cc = lane; cc < CH; cc += kWave) mx = fmaxf(mx, ml[(cc * G + h) * 2]);
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int cc = lane; cc < CH; cc += kWave) sum += ml[(cc * G + h) * 2 + 1] * exp_diff(ml[(cc * G + h) * 2], mx);
    sum = wave_sum(sum);
    if (lane == 0) {
      sM[h] = mx;
      sL[h] = sum;
    }
  }
  __syncthreads();
  if (p.out != nullptr) {
    const int per_block = G * kD / kCombineBlocks;
    const float* po = p.part_o + size_t(u) * CH * G * kD;
    const int q4 = threadIdx.x >> 6;
    float acc[(G * kD / kCombineBlocks + 63) / 64];
#pragma unroll
    for (int k = 0; k < (per_block + 63) / 64; ++k) acc[k] = 0.0f;
    for (int c0 = 0; c0 < CH; c0 += kMaxParts / 4) {
      const int cn = min(kMaxParts / 4, CH - c0);
      for (int i = threadIdx.x; i < cn * G; i += 256) {
        const int cc = i / G, h = i - cc * G;
        f[cc][h] = exp_diff(ml[((c0 + cc) * G + h) * 2], sM[h]) / sL[h];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < (per_block + 63) / 64; ++k) {
        const int local = k * 64 + lane;
        if (local < per_block) {
          const int idx = b * per_block + local;
          const int h = idx / kD;
          float a = 0.0f;
#pragma unroll 8
          for (int cc = q4; cc < cn; cc += 4) a += po[size_t(c0 + cc) * G * kD + idx] * f[cc][h];
          acc[k] += a;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < (per_block + 63) / 64; ++k) {
      red[q4][lane] = acc[k];
      __syncthreads();
      const int local = k * 64 + threadIdx.x;
      if (threadIdx.x < 64 && local < per_block) {
        p.out[size_t(u) * G * kD + b * per_block + local] = ((red[0][threadIdx.x] + red[1][threadIdx.x]) +
                                                             red[2][threadIdx.x]) + red[3][threadIdx.x];
      }
      __syncthreads();
    }
  }
  const size_t unit_win = size_t(u) * p.NW;
  const int nw = min(max(p.n_windows[u], 0), p.NW);
  for (int w = b * 256 + threadIdx.x; w < nw; w += 256 * kCombineBlocks) {
    float mass = 0.0f;
    if (p.tier[unit_win + w] != KVC_TIER_EVICTED) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mass += p.wsum[(unit_win + w) * G + h] * exp_diff(p.wref[(unit_win + w) * G + h], sM[h]) / sL[h];
      }
      mass *= 1.0f / G;
      if (p.accumulate) p.cum[unit_win + w] += mass;
    }
    if (p.mass != nullptr) p.mass[unit_win + w] = mass;
  }
  const int has_new = p.k_new != nullptr ? 1 : 0;
  const int tl = min(max(p.tail_len[u], 0), p.max_tail);
  if (p.probs != nullptr) {
    const int nf = min(max(p.n_full[u], 0), p.max_full);
    const int nq = min(max(p.n_int2[u], 0), p.max_int2);
    const int n_res = (nf + nq) * kW + tl + has_new;
    for (int h = 0; h < G; ++h) {
      float* pr = p.probs + (size_t(u) * G + h) * p.probs_stride;
      for (int i = b * 256 + threadIdx.x; i < n_res; i += 256 * kCombineBlocks) pr[i] = exp_diff(pr[i], sM[h]) / sL[h];
    }
  }
  if (b == 0 && has_new) {
    // append the step's token to the tail (K row-major, V into its head_dim-major 32-token block)
    if (threadIdx.x < 16) {
      reinterpret_cast<u32x4*>(p.k_tail + (size_t(u) * p.TM + tl) * kD)[threadIdx.x] =
          reinterpret_cast<const u32x4*>(p.k_new + size_t(u) * kD)[threadIdx.x];
    }
    if (threadIdx.x < kD) {
      p.v_tail[(size_t(u) * p.TM + (tl & ~(kW - 1))) * kD + threadIdx.x * kW + (tl & (kW - 1))] =
          p.v_new[size_t(u) * kD + threadIdx.x];
    }
  }
  __syncthreads();
  if (b == 0 && has_new && threadIdx.x == 0) p.tail_len[u] = tl + 1;
}

template <int G, class T>
hipError_t launch_g(const DecodeParams& p, int U, hipStream_t s) {
  if (p.probs != nullptr) {
    hipLaunchKernelGGL((decode_partial<G, T, true>), dim3(U * p.P), dim3(kBlock), 0, s, p);
  } else {
    hipLaunchKernelGGL((decode_partial<G, T, false>), dim3(U * p.P), dim3(kBlock), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine<G>), dim3(U * kCombineBlocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int decode_slices(const kvc_cache& c, const kvc_decode_args& a) {
  // about one workgroup per CU (the LDS staging allows one per CU) and at least 8 items per workgroup, at most
  // kMaxWgItems per workgroup (slice shares are rounded, hence the margin) and kMaxParts slices per unit
  const int has_new = a.k_new != nullptr ? 1 : 0;
  const int items = a.max_full + a.max_int2 + (a.max_tail + has_new + kW - 1) / kW;
  int P = (256 + c.n_units - 1) / c.n_units;
  P = min(P, max(1, (items + 7) / 8));
  P = max(P, (items + kMaxWgItems - 4) / (kMaxWgItems - 3));
  return max(1, min(P, kMaxParts));
}

size_t decode_workspace_bytes(const kvc_cache& c, const kvc_decode_args& a) {
  const size_t U = size_t(c.n_units), G = size_t(c.group), P = size_t(decode_slices(c, a));
  size_t b = 0;
  b += align_up(U * P * G * 2 * sizeof(float), 256);
  b += align_up(U * P * G * kD * sizeof(float), 256);
  b += 2 * align_up(U * size_t(c.n_windows_max) * G * sizeof(float), 256);
  return b;
}

hipError_t launch_decode(const kvc_cache& c, const kvc_decode_args& a, void* ws, hipStream_t s) {
  DecodeParams p{};
  p.NW = c.n_windows_max;
  p.TM = c.tail_max;
  p.k_win = static_cast<const uint16_t*>(c.k_win);
  p.v_win = static_cast<const uint16_t*>(c.v_win);
  p.k_codes = c.k_codes;
  p.v_codes = reinterpret_cast<const uint16_t*>(c.v_codes);
  p.k_meta = c.k_meta;
  p.v_meta = c.v_meta;
  p.k_tail = static_cast<uint16_t*>(c.k_tail);
  p.v_tail = static_cast<uint16_t*>(c.v_tail);
  p.tail_len = c.tail_len;
  p.res_list = c.res_list;
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
  p.P = decode_slices(c, a);
  const size_t U = size_t(c.n_units), G = size_t(c.group), P = size_t(p.P);
  char* w = static_cast<char*>(ws);
  p.part_ml = reinterpret_cast<float*>(w);
  w += align_up(U * P * G * 2 * sizeof(float), 256);
  p.part_o = reinterpret_cast<float*>(w);
  w += align_up(U * P * G * kD * sizeof(float), 256);
  p.wsum = reinterpret_cast<float*>(w);
  w += align_up(U * size_t(c.n_windows_max) * G * sizeof(float), 256);
  p.wref = reinterpret_cast<float*>(w);
  const int Ui = c.n_units;
  const bool bf = c.kv_dtype == KVC_BF16;
  switch (c.group) {
    case 1: return bf ? launch_g<1, BF16>(p, Ui, s) : launch_g<1, F16>(p, Ui, s);
    case 2: return bf ? launch_g<2, BF16>(p, Ui, s) : launch_g<2, F16>(p, Ui, s);
    case 4: return bf ? launch_g<4, BF16>(p, Ui, s) : launch_g<4, F16>(p, Ui, s);
    case 8: return bf ? launch_g<8, BF16>(p, Ui, s) : launch_g<8, F16>(p, Ui, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvc
