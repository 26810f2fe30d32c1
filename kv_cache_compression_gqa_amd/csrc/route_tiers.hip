// Three-tier window routing under a fixed budget (QEvict page, "Metodologia: QEvict" and "Mecanismos
// Principais"): per unit, resident windows are ranked by (score desc, window asc); the first budget_full go to the
// full-precision tier, the next budget_int2 to the INT2 tier, the rest are evicted for good.
//
// One workgroup per unit. The two rank thresholds are found by an exact MSB-first radix select over
// order-preserving 32-bit keys (4 passes of 8 bits, LDS histogram, one wave scans the 256 bins); keys equal to a
// threshold are admitted lowest index first through an exclusive scan in window order. The new resident lists
// and the quantise / promote lists come from one more in-order scan, so every output is deterministic.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// fp32 -> uint32 with the same order (-0 folded onto +0); NaN is screened out before.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block-wide exclusive scan of 4 counters at once (thread order). Returns the exclusive prefix; totals in tot.
__device__ int4 block_scan4(int4 v, int4* sm_waves, int4& tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  int4 inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int ax = __shfl_up(inc.x, d, kWave);
    const int ay = __shfl_up(inc.y, d, kWave);
    const int az = __shfl_up(inc.z, d, kWave);
    const int aw = __shfl_up(inc.w, d, kWave);
    if (lane >= d) {
      inc.x += ax;
      inc.y += ay;
      inc.z += az;
      inc.w += aw;
    }
  }
  if (lane == kWave - 1) sm_waves[wave] = inc;
  __syncthreads();
  int4 base = make_int4(0, 0, 0, 0);
  int4 all = make_int4(0, 0, 0, 0);
  for (int w = 0; w < kWaves; ++w) {
    const int4 t = sm_waves[w];
    if (w < wave) {
      base.x += t.x;
      base.y += t.y;
      base.z += t.z;
      base.w += t.w;
    }
    all.x += t.x;
    all.y += t.y;
    all.z += t.z;
    all.w += t.w;
  }
  __syncthreads();
  tot = all;
  return make_int4(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z, base.w + inc.w - v.w);
}

struct SelectShared {
  uint32_t hist[256];
  int digit;
  int krem;
};

// Value T of the k-th largest valid key (k >= 1) and how many keys equal to T belong to the top k.
__device__ void radix_kth(const uint32_t* keys, const uint8_t* valid, int n, int k, SelectShared& sh,
                          uint32_t& T, int& need) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  uint32_t prefix = 0u, mask = 0u;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kBlock) sh.hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kBlock) {
      if (valid[i] && (keys[i] & mask) == prefix) atomicAdd(&sh.hist[(keys[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins 4*lane .. 4*lane+3; "above" = keys in bins with a larger digit
      int c[4];
      int own = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        c[b] = int(sh.hist[4 * lane + b]);
        own += c[b];
      }
      // suffix sum over lanes: sum of own over lanes > lane
      int inc = own;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int a = __shfl_down(inc, d, kWave);
        if (lane + d < kWave) inc += a;
      }
      int above = inc - own;
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (above < krem && krem <= above + c[b]) {
          sh.digit = 4 * lane + b;
          sh.krem = krem - above;
        }
        above += c[b];
      }
    }
    __syncthreads();
    const uint32_t d = uint32_t(sh.digit);
    krem = sh.krem;
    prefix |= d << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  T = prefix;
  need = krem;
}

__global__ __launch_bounds__(kBlock) void route_tiers_kernel(kvc_tier_route_args a, kvc_cache c) {
  extern __shared__ uint8_t dyn[];
  const int u = blockIdx.x;
  const int NW = c.n_windows_max;
  uint32_t* keys = reinterpret_cast<uint32_t*>(dyn);
  uint8_t* valid = dyn + size_t(NW) * 4;
  __shared__ SelectShared sh;
  __shared__ int4 sm_waves[kWaves];
  __shared__ int s_flag[2];

  const size_t base = size_t(u) * NW;
  const int n = min(max(c.n_windows[u], 0), NW);
  const float* sc = a.scores != nullptr ? a.scores + base : c.cum + base;
  if (threadIdx.x == 0) {
    s_flag[0] = 0;
    s_flag[1] = 0;
  }
  __syncthreads();
  int nres_local = 0;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const bool v = c.tier[base + i] != KVC_TIER_EVICTED;
    const float f = sc[i];
    if (v && isnan(f)) atomicOr(&s_flag[0], 1);
    valid[i] = v ? 1 : 0;
    keys[i] = order_key(f);
    nres_local += v ? 1 : 0;
  }
  atomicAdd(&s_flag[1], nres_local);
  __syncthreads();
  if (s_flag[0] != 0) {
    if (threadIdx.x == 0) atomicOr(c.status, KVC_DEV_NAN_SCORE);
    return;
  }
  const int n_res = s_flag[1];
  const int bf = max(0, a.budget_full[u]);
  const int bq = max(0, a.budget_int2[u]);
  const int k1 = min(bf, n_res);
  const int k2 = min(bf + bq, n_res);
  uint32_t T1 = 0u, T2 = 0u;
  int need1 = 0, need2 = 0;
  if (k1 > 0) radix_kth(keys, valid, n, k1, sh, T1, need1);
  if (k2 > 0) radix_kth(keys, valid, n, k2, sh, T2, need2);

  // contiguous segment of windows per thread, so that scans follow window order
  const int seg = (n + kBlock - 1) / kBlock;
  const int lo = min(n, int(threadIdx.x) * seg);
  const int hi = min(n, lo + seg);

  // pass 1: rank among keys equal to each threshold
  int4 cnt = make_int4(0, 0, 0, 0);
  for (int i = lo; i < hi; ++i) {
    if (valid[i]) {
      cnt.x += (k1 > 0 && keys[i] == T1) ? 1 : 0;
      cnt.y += (k2 > 0 && keys[i] == T2) ? 1 : 0;
    }
  }
  int4 tot;
  int4 eq = block_scan4(cnt, sm_waves, tot);

  // pass 2: new tier per window, and counts of the four lists
  int4 cnt2 = make_int4(0, 0, 0, 0);
  for (int i = lo; i < hi; ++i) {
    int8_t nt = KVC_TIER_EVICTED;
    if (valid[i]) {
      bool top1 = false, top2 = false;
      if (k1 > 0) {
        if (keys[i] > T1) top1 = true;
        else if (keys[i] == T1) top1 = (eq.x++ < need1);
      }
      if (k2 > 0) {
        if (keys[i] > T2) top2 = true;
        else if (keys[i] == T2) top2 = (eq.y++ < need2);
      }
      nt = top1 ? KVC_TIER_FULL : (top2 ? KVC_TIER_INT2 : KVC_TIER_EVICTED);
    }
    const int8_t old = c.tier[base + i];
    valid[i] = uint8_t(nt);  // reuse: new tier (0, 1, 2)
    cnt2.x += nt == KVC_TIER_FULL;
    cnt2.y += nt == KVC_TIER_INT2;
    cnt2.z += (old == KVC_TIER_FULL && nt == KVC_TIER_INT2 && c.ledgered[base + i] == 0);
    cnt2.w += (old == KVC_TIER_INT2 && nt == KVC_TIER_FULL);
  }
  int4 tot2;
  int4 pos = block_scan4(cnt2, sm_waves, tot2);
  for (int i = lo; i < hi; ++i) {
    const int8_t nt = int8_t(valid[i]);
    const int8_t old = c.tier[base + i];
    if (nt == KVC_TIER_FULL) c.res_list[base + pos.x++] = i;
    if (nt == KVC_TIER_INT2) c.res_list[base + tot2.x + pos.y++] = i;
    if (old == KVC_TIER_FULL && nt == KVC_TIER_INT2 && c.ledgered[base + i] == 0) a.quant_list[base + pos.z++] = i;
    if (old == KVC_TIER_INT2 && nt == KVC_TIER_FULL) a.promo_list[base + pos.w++] = i;
    if (nt == KVC_TIER_EVICTED && old != KVC_TIER_EVICTED) c.ledgered[base + i] = 0;
    c.tier[base + i] = nt;
  }
  if (threadIdx.x == 0) {
    c.n_full[u] = tot2.x;
    c.n_int2[u] = tot2.y;
    a.n_quant[u] = tot2.z;
    a.n_promo[u] = tot2.w;
  }
}

}  // namespace

hipError_t launch_route_tiers(const kvc_tier_route_args& a, hipStream_t s) {
  const kvc_cache& c = *a.cache;
  const size_t lds = size_t(c.n_windows_max) * 5;
  hipLaunchKernelGGL(route_tiers_kernel, dim3(c.n_units), dim3(kBlock), lds, s, a, c);
  return hipGetLastError();
}

}  // namespace kvc
