// Internal helpers shared by the gfx950 kernels and the C-ABI layer of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kD = 128;           // head_dim
constexpr int kW = 32;            // window length in tokens
constexpr int kGroupElems = 32;   // INT2 group: 32 contiguous head_dim elements of one token
constexpr int kGroups = kD / kGroupElems;
constexpr int kCodeBytes = kD / 4;  // packed INT2 codes per token row
constexpr int kWave = 64;

// ---- storage conversions (16-bit patterns) ----------------------------------------------------------------
struct BF16 {
  static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }
  static __device__ __forceinline__ float one(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
  // round to nearest even (finite inputs)
  static __device__ __forceinline__ uint16_t from_float(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
  }
};

struct F16 {
  static __device__ __forceinline__ float lo(uint32_t x) { return __half2float(__ushort_as_half(uint16_t(x))); }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return __half2float(__ushort_as_half(uint16_t(x >> 16)));
  }
  static __device__ __forceinline__ float one(uint16_t x) { return __half2float(__ushort_as_half(x)); }
  static __device__ __forceinline__ uint16_t from_float(float f) { return __half_as_ushort(__float2half_rn(f)); }
};

// 8 consecutive storage elements (16 bytes) -> 8 floats
template <class T>
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = T::lo(v.x); f[1] = T::hi(v.x);
  f[2] = T::lo(v.y); f[3] = T::hi(v.y);
  f[4] = T::lo(v.z); f[5] = T::hi(v.z);
  f[6] = T::lo(v.w); f[7] = T::hi(v.w);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) { return __half2float(__ushort_as_half(uint16_t(h))); }

// ---- wave reductions --------------------------------------------------------------------------------------
__device__ __forceinline__ float xor_sum(float v, int mask) { return v + __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ float xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, kWave)); }

// DPP moves inside 16-lane rows (VALU, no LDS round trip). Controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140, row_shl:n = 0x100 + n.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Max / sum over the 16 lanes of a row; every lane of the row gets the same bits (each step combines a value
// with its partner's in a commutative operation).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

// Max / sum over the wave: DPP inside each row, then the four row results through scalar registers (fixed order,
// every lane gets the same bits).
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// exp(a - b) with exp(-inf - x) = 0 and no NaN when both are -inf
__device__ __forceinline__ float exp_diff(float a, float b) { return a == -INFINITY ? 0.0f : __expf(a - b); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Largest entry count of the global top-M and the generic top-k: block counts per row are computed in int32 as
// (row_len + 8191) / 8192, so n (and every row) stays at least one block below 2^31.
constexpr int64_t kTopmMaxN = (int64_t(1) << 31) - 8192 - 16;

// ---- launchers (host) -------------------------------------------------------------------------------------
int decode_slices(const kvc_cache& c, const kvc_decode_args& a);
bool decode_supported(const kvc_cache& c, const kvc_decode_args& a);
size_t decode_workspace_bytes(const kvc_cache& c, const kvc_decode_args& a);
hipError_t launch_decode(const kvc_cache& c, const kvc_decode_args& a, void* ws, hipStream_t s);
// kvc_decode_attn_static: the decode scratch in a static device array of this size (16 MiB per device)
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
int decode_static(const kvc_cache& c, const kvc_decode_args& a, hipStream_t s);
constexpr int kRouteMaxWindows = 4096;  // windows per unit that kvc_route(KVC_ROUTE_TIERS) takes
hipError_t launch_route_tiers(const kvc_tier_route_args& a, hipStream_t s);
hipError_t launch_repack(const kvc_cache& c, void* k_dst, void* v_dst, int32_t dst_slots, hipStream_t s);
hipError_t launch_quantize(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                           int64_t max_total, hipStream_t s);
hipError_t launch_promote(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                          int64_t max_total, hipStream_t s);

hipError_t launch_retention_score(const kvc_retention_args& a, hipStream_t s);

// Global top-M engine (topm.hip): scores from memory, or DBTrimKV's log-retention (t - i) * logf(beta) with i the
// position inside a row, computed where it is used (beta rows need row_len % 16 == 0).
constexpr int kTopmChunk = 2048;  // entries per chunk: one wave's unit of work
struct TopmInput {
  const float* scores;  // [n], or nullptr with beta
  const float* beta;    // [n] when scores is nullptr
  int32_t t;
  int32_t row_len;      // entries per row; n % row_len == 0
  int64_t n;
};
int64_t topm_chunks(int64_t n, int32_t row_len);
size_t topm_engine_workspace(int64_t n, int32_t row_len);
// What the engine writes. keep: one byte (0/1) per entry; or keep_bits, one bit per entry (only for a single row,
// row_len == n: word w holds entries 32 w .. 32 w + 31; topm_chunks * 64 words). row_counts: [n / row_len] or
// nullptr. status: KVC_DEV_NAN_SCORE is ORed in (zeroed first when clear_status).
struct TopmOutput {
  uint8_t* keep = nullptr;
  uint32_t* keep_bits = nullptr;
  int32_t* row_counts = nullptr;
  int32_t* status = nullptr;
  bool clear_status = false;
};
// Kept counts in the workspace once the launches have run: per chunk, and per group of kTopmGroup consecutive
// chunks.
constexpr int kTopmGroup = 64;
struct TopmCounts {
  const int32_t* chunk_kept;
  const int32_t* group_kept;
};
hipError_t launch_topm_engine(const TopmInput& in, int64_t m, const TopmOutput& out, void* ws, hipStream_t s,
                              TopmCounts* counts = nullptr);
size_t topm_workspace_bytes(const kvc_topm_args& a);
hipError_t launch_topm(const kvc_topm_args& a, void* ws, hipStream_t s);
size_t compact_workspace_bytes(const kvc_compact_args& a);
hipError_t launch_compact(const kvc_compact_args& a, void* ws, hipStream_t s);
size_t criticalkv_workspace_bytes(const kvc_criticalkv_args& a);
bool criticalkv_supported(const kvc_criticalkv_args& a);
hipError_t launch_criticalkv(const kvc_criticalkv_args& a, void* ws, hipStream_t s);
size_t two_stage_workspace_bytes(const kvc_two_stage_args& a);
hipError_t launch_two_stage(const kvc_two_stage_args& a, int32_t budget1, void* ws, hipStream_t s);
size_t paged_workspace_bytes(const kvc_paged_decode_args& a);
hipError_t launch_paged_decode(const kvc_paged_decode_args& a, void* ws, hipStream_t s);
hipError_t launch_diagnostics(const kvc_diag_args& a, hipStream_t s);
size_t summarize_workspace_bytes(const kvc_cache& c);
size_t topk_workspace_bytes(int64_t n);
hipError_t launch_topk(const float* scores, int64_t n, int64_t k, int32_t* idx, void* ws, hipStream_t s);
hipError_t launch_summarize(const kvc_cache& c, const int8_t* tier_prev, int32_t max_new, void* ws, hipStream_t s);

}  // namespace kvc
