// Write-once INT2 quantisation ledger and promotion (QEvict page, "Mecanismos Principais": a window is quantised
// only at its first demotion; the low-bit copy is kept and reused for every later promotion and demotion, so the
// approximation error never compounds; promotion dequantises the copy back to full precision).
//
// Both kernels walk a flat list given as per-unit lists + per-unit counts: every workgroup computes the exclusive
// prefix of the counts in LDS, then strides over the flat items (one window per workgroup iteration, so no launch
// depends on a device-side count). A window is 256 (K or V, token, 32-element group) tasks = one per thread.
//
// Quantiser (all decisions in fp32 so that they are bit-reproducible; contraction is disabled for this file):
//   lo, hi = group min / max; zero z = largest fp16 <= lo; scale s = smallest fp16 >= fl32(fl32(hi - z) / 3)
//   (0 if hi == z); code = #{k in 0..2 : fl32(x - z) >= (k + 0.5) * s} (0 if s == 0).
#include "kvc_internal.h"

#pragma clang fp contract(off)

namespace kvc {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ uint16_t f16_next_up(uint16_t h) {
  if ((h & 0x7FFFu) == 0u) return 0x0001u;
  return (h & 0x8000u) ? uint16_t(h - 1u) : uint16_t(h + 1u);
}
__device__ __forceinline__ uint16_t f16_next_down(uint16_t h) {
  if ((h & 0x7FFFu) == 0u) return 0x8001u;
  return (h & 0x8000u) ? uint16_t(h + 1u) : uint16_t(h - 1u);
}
// largest fp16 <= x (|x| < 65504)
__device__ __forceinline__ uint16_t f16_round_down(float x) {
  uint16_t h = __half_as_ushort(__float2half_rn(x));
  if (half_bits_to_float(h) > x) h = f16_next_down(h);
  return h;
}
// smallest fp16 >= x (|x| < 65504)
__device__ __forceinline__ uint16_t f16_round_up(float x) {
  uint16_t h = __half_as_ushort(__float2half_rn(x));
  if (half_bits_to_float(h) < x) h = f16_next_up(h);
  return h;
}

// Exclusive prefix of count[0..U) into pre[0..U], pre[U] = total. Block-wide, deterministic.
__device__ void unit_prefix(const int32_t* count, int U, int stride, int* pre) {
  __shared__ int wave_tot[kBlock / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int seg = (U + kBlock - 1) / kBlock;
  const int lo = min(U, int(threadIdx.x) * seg), hi = min(U, lo + seg);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += min(max(0, count[i]), stride);
  int inc = local;
  for (int d = 1; d < kWave; d <<= 1) {
    const int a = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += a;
  }
  if (lane == kWave - 1) wave_tot[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  int run = base + inc - local;
  for (int i = lo; i < hi; ++i) {
    pre[i] = run;
    run += min(max(0, count[i]), stride);
  }
  if (threadIdx.x == kBlock - 1) pre[U] = run;
  __syncthreads();
}

// unit owning flat item `item`: the last u with pre[u] <= item
__device__ __forceinline__ int find_unit(const int* pre, int U, int item) {
  int lo = 0, hi = U;  // invariant pre[lo] <= item < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

template <class T>
__global__ __launch_bounds__(kBlock) void quantize_kernel(kvc_cache c, const int32_t* list, const int32_t* count,
                                                          int stride) {
  extern __shared__ int pre[];
  __shared__ int s_skip;
  const int U = c.n_units, NW = c.n_windows_max;
  unit_prefix(count, U, stride, pre);
  const int total = pre[U];
  const int kv = threadIdx.x >> 7;          // 0 = K, 1 = V
  const int tok = (threadIdx.x & 127) >> 2;
  const int grp = threadIdx.x & 3;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int u = find_unit(pre, U, item);
    const int w = list[size_t(u) * stride + (item - pre[u])];
    const size_t win = size_t(u) * NW + w;
    if (threadIdx.x == 0) s_skip = unsigned(w) >= unsigned(NW) ? 2 : (c.ledgered[win] != 0 ? 1 : 0);
    __syncthreads();
    if (s_skip) {
      if (threadIdx.x == 0) atomicOr(c.status, s_skip == 1 ? KVC_DEV_LEDGER_REWRITE : KVC_DEV_BOUND_EXCEEDED);
      __syncthreads();
      continue;
    }
    const uint16_t* src = static_cast<const uint16_t*>(kv ? c.v_win : c.k_win) +
                          (win * kW + tok) * kD + grp * kGroupElems;
    float x[kGroupElems];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[q4];
      float f[8];
      unpack8<T>(v, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * q4 + e] = f[e];
    }
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int e = 1; e < kGroupElems; ++e) {
      lo = fminf(lo, x[e]);
      hi = fmaxf(hi, x[e]);
    }
    const uint16_t z16 = f16_round_down(lo);
    const float z = half_bits_to_float(z16);
    uint16_t s16 = 0u;
    if (hi != z) s16 = f16_round_up(__fdiv_rn(__fsub_rn(hi, z), 3.0f));
    const float s = half_bits_to_float(s16);
    const float t0 = __fmul_rn(0.5f, s), t1 = __fmul_rn(1.5f, s), t2 = __fmul_rn(2.5f, s);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < kGroupElems; ++e) {
      const float d = __fsub_rn(x[e], z);
      uint32_t code = uint32_t(d >= t0) + uint32_t(d >= t1) + uint32_t(d >= t2);
      if (s16 == 0u) code = 0u;
      packed[e >> 4] |= code << (2 * (e & 15));
    }
    uint8_t* dst = (kv ? c.v_codes : c.k_codes) + (win * kW + tok) * kCodeBytes + grp * (kGroupElems / 4);
    *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
    uint32_t* meta = (kv ? c.v_meta : c.k_meta) + (win * kW + tok) * kGroups + grp;
    *meta = uint32_t(s16) | (uint32_t(z16) << 16);
    __syncthreads();
    if (threadIdx.x == 0) c.ledgered[win] = 1;
  }
}

template <class T>
__global__ __launch_bounds__(kBlock) void promote_kernel(kvc_cache c, const int32_t* list, const int32_t* count,
                                                         int stride) {
  extern __shared__ int pre[];
  const int U = c.n_units, NW = c.n_windows_max;
  unit_prefix(count, U, stride, pre);
  const int total = pre[U];
  const int kv = threadIdx.x >> 7;
  const int tok = (threadIdx.x & 127) >> 2;
  const int grp = threadIdx.x & 3;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int u = find_unit(pre, U, item);
    const int w = list[size_t(u) * stride + (item - pre[u])];
    if (unsigned(w) >= unsigned(NW)) {
      if (threadIdx.x == 0) atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
      continue;
    }
    const size_t win = size_t(u) * NW + w;
    const uint8_t* codes = (kv ? c.v_codes : c.k_codes) + (win * kW + tok) * kCodeBytes + grp * (kGroupElems / 4);
    const uint2 cw = *reinterpret_cast<const uint2*>(codes);
    const uint32_t mw = (kv ? c.v_meta : c.k_meta)[(win * kW + tok) * kGroups + grp];
    const float s = half_bits_to_float(mw & 0xFFFFu);
    const float z = half_bits_to_float(mw >> 16);
    uint16_t* dst = static_cast<uint16_t*>(kv ? c.v_win : c.k_win) + (win * kW + tok) * kD + grp * kGroupElems;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t bits = (q4 < 2 ? cw.x : cw.y) >> (16 * (q4 & 1));
      uint32_t outw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float a = fmaf(float((bits >> (4 * e2)) & 3u), s, z);
        const float b = fmaf(float((bits >> (4 * e2 + 2)) & 3u), s, z);
        outw[e2] = uint32_t(T::from_float(a)) | (uint32_t(T::from_float(b)) << 16);
      }
      reinterpret_cast<uint4*>(dst)[q4] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
  }
}

int list_grid(int64_t max_total) { return int(max_total < 2048 ? max_total : 2048); }

}  // namespace

hipError_t launch_quantize(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                           int64_t max_total, hipStream_t s) {
  if (max_total <= 0) return hipSuccess;
  const size_t lds = (size_t(c.n_units) + 1) * sizeof(int);
  if (c.kv_dtype == KVC_BF16) {
    hipLaunchKernelGGL(quantize_kernel<BF16>, dim3(list_grid(max_total)), dim3(kBlock), lds, s, c, list, count,
                       stride);
  } else {
    hipLaunchKernelGGL(quantize_kernel<F16>, dim3(list_grid(max_total)), dim3(kBlock), lds, s, c, list, count,
                       stride);
  }
  return hipGetLastError();
}

hipError_t launch_promote(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                          int64_t max_total, hipStream_t s) {
  if (max_total <= 0) return hipSuccess;
  const size_t lds = (size_t(c.n_units) + 1) * sizeof(int);
  if (c.kv_dtype == KVC_BF16) {
    hipLaunchKernelGGL(promote_kernel<BF16>, dim3(list_grid(max_total)), dim3(kBlock), lds, s, c, list, count,
                       stride);
  } else {
    hipLaunchKernelGGL(promote_kernel<F16>, dim3(list_grid(max_total)), dim3(kBlock), lds, s, c, list, count,
                       stride);
  }
  return hipGetLastError();
}

}  // namespace kvc
