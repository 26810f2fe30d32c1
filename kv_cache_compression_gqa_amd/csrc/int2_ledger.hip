// Write-once INT2 quantisation ledger and promotion (QEvict page, "Mecanismos Principais": a window is quantised
// only at its first demotion; the low-bit copy is kept and reused for every later promotion and demotion, so the
// approximation error never compounds; promotion dequantises the copy back to full precision).
//
// Both kernels walk per-unit lists + per-unit counts: workgroup (u, s) of a U x S grid takes items s, s + S, ... of
// unit u (one window per workgroup iteration; S is sized from the host bound, so no launch depends on a
// device-side count). Per window, 128 threads handle K and 128 handle V, one (token, 32-element group) each; V,
// whose storage is transposed, is staged through LDS.
//
// Quantiser (all decisions in fp32 so that they are bit-reproducible; contraction is disabled for this file):
//   lo, hi = group min / max; zero z = largest fp16 <= lo; scale s = smallest fp16 >= fl32(fl32(hi - z) / 3)
//   (0 if hi == z); code = #{k in 0..2 : fl32(x - z) >= (k + 0.5) * s} (0 if s == 0).
// Storage layouts (see include/kvc.h): K codes of a token row: byte 8*s + 2*g + h holds head_dim 32g + 8s + 4h + e
// at bits 2e; V codes: 16-bit word (r, q, dt) of a window holds tokens 8q + e of head_dim 16dt + r at bits 2e;
// V meta: word (q, g, e) = token 8q + e, group g.
#include <algorithm>

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

// One 32-element group: meta word (s | z << 16) and 32 codes (code e at bit 2e of the 64-bit result).
__device__ __forceinline__ uint64_t quantize_group(const float (&x)[kGroupElems], uint32_t& meta) {
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
  uint64_t packed = 0u;
#pragma unroll
  for (int e = 0; e < kGroupElems; ++e) {
    const float d = __fsub_rn(x[e], z);
    uint64_t code = uint64_t(d >= t0) + uint64_t(d >= t1) + uint64_t(d >= t2);
    if (s16 == 0u) code = 0u;
    packed |= code << (2 * e);
  }
  meta = uint32_t(s16) | (uint32_t(z16) << 16);
  return packed;
}

template <class T>
__global__ __launch_bounds__(kBlock) void quantize_kernel(kvc_cache c, const int32_t* list, const int32_t* count,
                                                          int stride) {
  __shared__ uint16_t vt[kD * kW];     // V^T window [d][t]
  __shared__ uint8_t vcode[kD * kW];   // V codes [d][t]
  __shared__ int s_skip;
  const int NW = c.n_windows_max;
  const int u = blockIdx.x;
  const int n = min(max(count[u], 0), stride);
  const int half = threadIdx.x >> 7;         // 0 = K, 1 = V
  const int tok = (threadIdx.x & 127) >> 2;
  const int grp = threadIdx.x & 3;
  for (int j = blockIdx.y; j < n; j += gridDim.y) {
    const int w = list[size_t(u) * stride + j];
    const size_t win = size_t(u) * NW + w;
    if (threadIdx.x == 0) s_skip = unsigned(w) >= unsigned(NW) ? 2 : (c.ledgered[win] != 0 ? 1 : 0);
    __syncthreads();
    if (s_skip) {
      if (threadIdx.x == 0) atomicOr(c.status, s_skip == 1 ? KVC_DEV_LEDGER_REWRITE : KVC_DEV_BOUND_EXCEEDED);
      __syncthreads();
      continue;
    }
    // stage V^T (8 KiB) in LDS: 32 bytes per thread
    {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(c.v_win) + win * kW * kD);
      uint4* dst = reinterpret_cast<uint4*>(vt);
      dst[2 * threadIdx.x] = src[2 * threadIdx.x];
      dst[2 * threadIdx.x + 1] = src[2 * threadIdx.x + 1];
    }
    __syncthreads();
    float x[kGroupElems];
    if (half == 0) {
      const uint16_t* src = static_cast<const uint16_t*>(c.k_win) + (win * kW + tok) * kD + grp * kGroupElems;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float f[8];
        unpack8<T>(reinterpret_cast<const uint4*>(src)[q4], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * q4 + e] = f[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < kGroupElems; ++e) x[e] = T::one(vt[(grp * kGroupElems + e) * kW + tok]);
    }
    uint32_t meta;
    const uint64_t codes = quantize_group(x, meta);
    if (half == 0) {
      uint8_t* row = c.k_codes + (win * kW + tok) * kCodeBytes;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<uint16_t*>(row + 8 * s + 2 * grp) = uint16_t((codes >> (16 * s)) & 0xFFFFu);
      }
      c.k_meta[(win * kW + tok) * kGroups + grp] = meta;
    } else {
#pragma unroll
      for (int e = 0; e < kGroupElems; ++e) vcode[(grp * kGroupElems + e) * kW + tok] = uint8_t((codes >> (2 * e)) & 3u);
      c.v_meta[win * (kW * kGroups) + (tok >> 3) * 32 + grp * 8 + (tok & 7)] = meta;
    }
    __syncthreads();
    // V code words: (r, q, dt) holds tokens 8q..8q+7 of head_dim 16dt + r
    uint16_t* vw = reinterpret_cast<uint16_t*>(c.v_codes) + win * (kW * kD / 8);
    for (int wi = threadIdx.x; wi < kW * kD / 8; wi += kBlock) {
      const int r = wi >> 5, q = (wi >> 3) & 3, dt = wi & 7;
      const uint8_t* src = vcode + (16 * dt + r) * kW + 8 * q;
      uint32_t word = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= uint32_t(src[e]) << (2 * e);
      vw[wi] = uint16_t(word);
    }
    if (threadIdx.x == 0) c.ledgered[win] = 1;
    __syncthreads();
  }
}

template <class T>
__global__ __launch_bounds__(kBlock) void promote_kernel(kvc_cache c, const int32_t* list, const int32_t* count,
                                                         int stride) {
  __shared__ uint16_t vcw[kW * kD / 8];  // V code words of the window
  __shared__ uint32_t vmeta[kW * kGroups];
  __shared__ uint16_t vt[kD * kW];      // promoted V^T [d][t]
  const int NW = c.n_windows_max;
  const int u = blockIdx.x;
  const int n = min(max(count[u], 0), stride);
  const int half = threadIdx.x >> 7;
  const int tok = (threadIdx.x & 127) >> 2;
  const int grp = threadIdx.x & 3;
  for (int j = blockIdx.y; j < n; j += gridDim.y) {
    const int w = list[size_t(u) * stride + j];
    if (unsigned(w) >= unsigned(NW)) {
      if (threadIdx.x == 0) atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
      continue;
    }
    const size_t win = size_t(u) * NW + w;
    {
      const uint16_t* src = reinterpret_cast<const uint16_t*>(c.v_codes) + win * (kW * kD / 8);
      for (int i = threadIdx.x; i < kW * kD / 8; i += kBlock) vcw[i] = src[i];
      if (threadIdx.x < kW * kGroups) vmeta[threadIdx.x] = c.v_meta[win * (kW * kGroups) + threadIdx.x];
    }
    __syncthreads();
    if (half == 0) {
      const uint8_t* row = c.k_codes + (win * kW + tok) * kCodeBytes;
      const uint32_t mw = c.k_meta[(win * kW + tok) * kGroups + grp];
      const float s = half_bits_to_float(mw & 0xFFFFu);
      const float z = half_bits_to_float(mw >> 16);
      uint16_t* dst = static_cast<uint16_t*>(c.k_win) + (win * kW + tok) * kD + grp * kGroupElems;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const uint32_t bits = *reinterpret_cast<const uint16_t*>(row + 8 * sl + 2 * grp);
        uint32_t outw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float a = fmaf(float((bits >> (4 * e2)) & 3u), s, z);
          const float b = fmaf(float((bits >> (4 * e2 + 2)) & 3u), s, z);
          outw[e2] = uint32_t(T::from_float(a)) | (uint32_t(T::from_float(b)) << 16);
        }
        reinterpret_cast<uint4*>(dst)[sl] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
      }
    } else {
      const uint32_t mw = vmeta[(tok >> 3) * 32 + grp * 8 + (tok & 7)];
      const float s = half_bits_to_float(mw & 0xFFFFu);
      const float z = half_bits_to_float(mw >> 16);
#pragma unroll
      for (int e = 0; e < kGroupElems; ++e) {
        const int d = grp * kGroupElems + e;
        const uint32_t word = vcw[(d & 15) * 32 + (tok >> 3) * 8 + (d >> 4)];
        const uint32_t code = (word >> (2 * (tok & 7))) & 3u;
        vt[d * kW + tok] = T::from_float(fmaf(float(code), s, z));
      }
    }
    __syncthreads();
    {
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(c.v_win) + win * kW * kD);
      const uint4* src = reinterpret_cast<const uint4*>(vt);
      dst[2 * threadIdx.x] = src[2 * threadIdx.x];
      dst[2 * threadIdx.x + 1] = src[2 * threadIdx.x + 1];
    }
    __syncthreads();
  }
}

// U x S grid: S workgroups per unit, from the host bound on the items per unit, capped at about 16384 workgroups
dim3 list_grid(int U, int64_t max_total) {
  const int64_t per_unit = (max_total + U - 1) / U;
  const int64_t cap = std::max<int64_t>(1, 16384 / U);
  return dim3(unsigned(U), unsigned(std::max<int64_t>(1, std::min(per_unit, std::min<int64_t>(cap, 65535)))));
}

}  // namespace

hipError_t launch_quantize(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                           int64_t max_total, hipStream_t s) {
  if (max_total <= 0 || c.n_units <= 0) return hipSuccess;
  if (c.kv_dtype == KVC_BF16) {
    hipLaunchKernelGGL(quantize_kernel<BF16>, list_grid(c.n_units, max_total), dim3(kBlock), 0, s, c, list, count, stride);
  } else {
    hipLaunchKernelGGL(quantize_kernel<F16>, list_grid(c.n_units, max_total), dim3(kBlock), 0, s, c, list, count, stride);
  }
  return hipGetLastError();
}

hipError_t launch_promote(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                          int64_t max_total, hipStream_t s) {
  if (max_total <= 0 || c.n_units <= 0) return hipSuccess;
  if (c.kv_dtype == KVC_BF16) {
    hipLaunchKernelGGL(promote_kernel<BF16>, list_grid(c.n_units, max_total), dim3(kBlock), 0, s, c, list, count, stride);
  } else {
    hipLaunchKernelGGL(promote_kernel<F16>, list_grid(c.n_units, max_total), dim3(kBlock), 0, s, c, list, count, stride);
  }
  return hipGetLastError();
}

}  // namespace kvc
