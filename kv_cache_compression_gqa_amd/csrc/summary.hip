// Span summaries of evicted windows for the mixed-resolution attention term.
//
// SEKV page ("Metodologia", sections 2 and 3): every span keeps a light summary vector, and spans that are not
// expanded enter the decode attention as their summaries with a size correction. Here a span is one window; when
// routing evicts a window, its summary key and value (the means of its 32 keys and values) are appended to the
// unit's summary list, which the decode attends after the tail with logit q.k/sqrt(D) + ln 32.
//
// summary_list: one 256-thread workgroup per unit. Windows are taken in chunks of 256 (thread t: window c*256+t);
// a block scan of the "evicted by this event" flags gives each such window its rank, so the list comes out in
// ascending window order. The unit's first slot and the count go to the workspace, and n_sum advances (clamped to
// the capacity, with the bound bit raised past it).
// summary_write: one 128-thread workgroup per (unit, list entry); thread d sums the 32 keys and values at head_dim
// d in fp64 in token order, divides by 32, rounds to fp32 and then to the storage dtype. The values are those of
// the copy the cache held for the window when the event evicted it: its full-precision slot if it was FULL (K rows
// read across threads, coalesced; V as the window's 32 contiguous values of head_dim d, 64 bytes per thread), its
// ledger slot brought back to the storage dtype, RNE(fmaf(code, scale, zero)), if it was INT2.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kListThreads = 256;

__global__ __launch_bounds__(kListThreads) void summary_list(kvc_cache c, const int8_t* tier_prev, int32_t max_new,
                                                             int32_t* list, int32_t* first, int32_t* count) {
  const int u = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t >> 6;
  const int NW = c.n_windows_max;
  const int nw = min(max(c.n_windows[u], 0), NW);
  const size_t base = size_t(u) * NW;
  __shared__ int wsum[kListThreads / kWave];
  int total = 0;
  for (int c0 = 0; c0 < nw; c0 += kListThreads) {
    const int w = c0 + t;
    const bool ev = w < nw && tier_prev[base + w] != KVC_TIER_EVICTED && c.tier[base + w] == KVC_TIER_EVICTED;
    const uint64_t m = __ballot(ev);
    const int below = __popcll(m & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int off = total;
    for (int i = 0; i < wave; ++i) off += wsum[i];
    int chunk = 0;
    for (int i = 0; i < kListThreads / kWave; ++i) chunk += wsum[i];
    if (ev && off + below < max_new) list[base + off + below] = w;
    total += chunk;
    __syncthreads();
  }
  if (t == 0) {
    const int n0 = min(max(c.n_sum[u], 0), c.sum_max);
    int n = min(total, max_new);
    n = min(n, c.sum_max - n0);
    if (n != total || n0 != c.n_sum[u]) atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
    first[u] = n0;
    count[u] = n;
    c.n_sum[u] = n0 + n;
  }
}

// The storage value of head_dim d of token j of ledger slot ls (flat over units): RNE_storage(fmaf(code, s, z)),
// what a promotion writes. K codes: byte 8s + 2g + h of the token row holds head_dim 32g + 8s + 4h + e at bits 2e;
// V codes: 16-bit word (r, q, dt) holds tokens 8q + e of head_dim 16dt + r at bits 2e; V meta word (q, g, e).
template <class T>
__device__ __forceinline__ float ledger_k(const kvc_cache& c, size_t ls, int j, int d) {
  const int g = d >> 5, rem = d & 31;
  const int byte = 8 * (rem >> 3) + 2 * g + ((rem >> 2) & 1);
  const uint32_t code = (c.k_codes[(ls * kW + j) * kCodeBytes + byte] >> (2 * (d & 3))) & 3u;
  const uint32_t m = c.k_meta[(ls * kW + j) * kGroups + g];
  return T::one(T::from_float(fmaf(float(code), half_bits_to_float(m & 0xFFFFu), half_bits_to_float(m >> 16))));
}
template <class T>
__device__ __forceinline__ float ledger_v(const kvc_cache& c, size_t ls, int j, int d) {
  const int q = j >> 3, e = j & 7, g = d >> 5;
  const uint16_t* words = reinterpret_cast<const uint16_t*>(c.v_codes) + ls * (kW * kD / 8);
  const uint32_t code = (uint32_t(words[((d & 15) * 4 + q) * 8 + (d >> 4)]) >> (2 * e)) & 3u;
  const uint32_t m = c.v_meta[ls * (kW * kGroups) + q * 32 + g * 8 + e];
  return T::one(T::from_float(fmaf(float(code), half_bits_to_float(m & 0xFFFFu), half_bits_to_float(m >> 16))));
}

template <class T>
__global__ __launch_bounds__(kD) void summary_write(kvc_cache c, const int8_t* tier_prev, int32_t max_new,
                                                   const int32_t* list, const int32_t* first, const int32_t* count) {
  const int u = blockIdx.x / max_new;
  const int i = blockIdx.x - u * max_new;
  if (i >= count[u]) return;
  const int d = threadIdx.x;
  const int NW = c.n_windows_max;
  const int w = list[size_t(u) * NW + i];
  const int slot = first[u] + i;
  const bool from_full = tier_prev[size_t(u) * NW + w] == KVC_TIER_FULL;
  // the slot the event freed: full-precision for a window evicted from FULL, ledger for one evicted from INT2
  const int src = from_full ? c.full_slot[size_t(u) * NW + w] : c.ledger_slot[size_t(u) * NW + w];
  const int cap = from_full ? c.full_slots : c.ledger_slots;
  double sk = 0.0, sv = 0.0;
  if (unsigned(src) >= unsigned(cap)) {
    if (d == 0) atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
  } else if (from_full) {
    const size_t fs = size_t(u) * c.full_slots + src;
    const uint16_t* kw = static_cast<const uint16_t*>(c.k_full) + fs * (kW * kD);
    const uint16_t* vw = static_cast<const uint16_t*>(c.v_full) + fs * (kW * kD) + d * kW;
#pragma unroll
    for (int j = 0; j < kW; ++j) sk += double(T::one(kw[j * kD + d]));
    const uint4* v4 = reinterpret_cast<const uint4*>(vw);
#pragma unroll
    for (int q = 0; q < kW / 8; ++q) {
      float f[8];
      unpack8<T>(v4[q], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) sv += double(f[e]);
    }
  } else {
    const size_t ls = size_t(u) * c.ledger_slots + src;
#pragma unroll 4
    for (int j = 0; j < kW; ++j) {
      sk += double(ledger_k<T>(c, ls, j, d));
      sv += double(ledger_v<T>(c, ls, j, d));
    }
  }
  const uint16_t kb = T::from_float(float(sk * (1.0 / kW)));
  const uint16_t vb = T::from_float(float(sv * (1.0 / kW)));
  const int SM = c.sum_max;
  static_cast<uint16_t*>(c.k_sum)[(size_t(u) * SM + slot) * kD + d] = kb;
  static_cast<uint16_t*>(c.v_sum)[(size_t(u) * SM + (slot & ~(kW - 1))) * kD + d * kW + (slot & (kW - 1))] = vb;
}

}  // namespace

size_t summarize_workspace_bytes(const kvc_cache& c) {
  return align_up(size_t(c.n_units) * c.n_windows_max * sizeof(int32_t), 256) +
         2 * align_up(size_t(c.n_units) * sizeof(int32_t), 256);
}

hipError_t launch_summarize(const kvc_cache& c, const int8_t* tier_prev, int32_t max_new, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  int32_t* list = reinterpret_cast<int32_t*>(w);
  w += align_up(size_t(c.n_units) * c.n_windows_max * sizeof(int32_t), 256);
  int32_t* first = reinterpret_cast<int32_t*>(w);
  w += align_up(size_t(c.n_units) * sizeof(int32_t), 256);
  int32_t* count = reinterpret_cast<int32_t*>(w);
  hipLaunchKernelGGL(summary_list, dim3(c.n_units), dim3(kListThreads), 0, s, c, tier_prev, max_new, list, first,
                     count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_new == 0) return e;
  const dim3 grid(unsigned(int64_t(c.n_units) * max_new));
  if (c.kv_dtype == KVC_BF16) {
    hipLaunchKernelGGL(summary_write<BF16>, grid, dim3(kD), 0, s, c, tier_prev, max_new, list, first, count);
  } else {
    hipLaunchKernelGGL(summary_write<F16>, grid, dim3(kD), 0, s, c, tier_prev, max_new, list, first, count);
  }
  return hipGetLastError();
}

}  // namespace kvc
