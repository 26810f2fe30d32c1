// Three-tier window routing under a fixed budget (QEvict page, "Metodologia: QEvict" and "Mecanismos
// Principais"): per unit, resident windows are ranked by (score desc, window asc); the first budget_full go to the
// full-precision tier, the next budget_int2 to the INT2 tier, the rest are evicted for good.
//
// One workgroup per unit. The two rank thresholds are found together by an exact MSB-first radix select over
// order-preserving 32-bit keys (4 passes of 8 bits, per-wave LDS histograms, one wave per threshold scans the 256
// bins); keys equal to a threshold are admitted lowest index first through an exclusive scan in window order. The new resident lists
// and the quantise / promote lists come from one more in-order scan, so every output is deterministic.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
// window flag byte in LDS
constexpr uint8_t kOldTier = 3;     // bits 0-1: tier before routing
constexpr uint8_t kLedgered = 4;    // bit 2: INT2 copy present
constexpr uint8_t kValid = 8;       // bit 3: resident (while loading: the score is NaN)
constexpr int kNewShift = 4;
constexpr uint8_t kNewTier = 0x30;  // bits 4-5: tier after routing

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
  uint32_t hist[2][kWaves][256];  // per selection, per wave
  int digit[2];
  int krem[2];
};

// Both rank thresholds in one series of passes: for s = 0, 1, the value T[s] of the k[s]-th largest valid key
// (k[s] >= 1; k[s] <= 0 leaves selection s idle) and how many keys equal to T[s] belong to the top k[s]. Each pass
// takes 8 bits (MSB first) into per-wave LDS histograms; the top digit, which few distinct values share, groups
// the wave's lanes by bin before one atomic per distinct bin. Wave s then scans selection s's 256 bins.
__device__ void radix_kth2(const uint32_t* keys, const uint8_t* wm, int n, const int (&k)[2], SelectShared& sh,
                           uint32_t (&T)[2], int (&need)[2]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  uint32_t prefix[2] = {0u, 0u}, mask = 0u;
  int krem[2] = {k[0], k[1]};
  const bool active[2] = {k[0] > 0, k[1] > 0};
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 2 * kWaves * 256; i += kBlock) (&sh.hist[0][0][0])[i] = 0u;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += kBlock) {  // uniform trip count (the ballots below need the whole wave)
      const int i = i0 + int(threadIdx.x);
      const bool ok = i < n && (wm[i] & kValid);
      const uint32_t key = ok ? keys[i] : 0u;
      const uint32_t bin = (key >> shift) & 255u;
#pragma unroll
      for (int sel = 0; sel < 2; ++sel) {
        const bool m = ok && active[sel] && (key & mask) == prefix[sel];
        if (shift == 24) {
          uint64_t act = __ballot(m);
          while (act) {
            const int leader = __builtin_ctzll(act);
            const uint32_t lb = uint32_t(__builtin_amdgcn_readlane(int(bin), leader));
            const uint64_t same = __ballot(m && bin == lb);
            if (lane == leader) atomicAdd(&sh.hist[sel][wave][lb], uint32_t(__popcll(same)));
            act &= ~same;
          }
        } else if (m) {
          atomicAdd(&sh.hist[sel][wave][bin], 1u);
        }
      }
    }
    __syncthreads();
    if (wave < 2 && active[wave]) {
      const int sel = wave;
      // lane owns bins 4*lane .. 4*lane+3 (summed over the wave copies); "above" = keys in bins with a larger digit
      int c[4];
      int own = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        int x = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) x += int(sh.hist[sel][w][4 * lane + b]);
        c[b] = x;
        own += x;
      }
      // suffix sum over lanes: sum of own over lanes > lane
      int inc = own;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int a = __shfl_down(inc, d, kWave);
        if (lane + d < kWave) inc += a;
      }
      int above = inc - own;
      const int kr = krem[sel];
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (above < kr && kr <= above + c[b]) {
          sh.digit[sel] = 4 * lane + b;
          sh.krem[sel] = kr - above;
        }
        above += c[b];
      }
    }
    __syncthreads();
#pragma unroll
    for (int sel = 0; sel < 2; ++sel) {
      if (active[sel]) {
        prefix[sel] |= uint32_t(sh.digit[sel]) << shift;
        krem[sel] = sh.krem[sel];
      }
    }
    mask |= 255u << shift;
  }
  T[0] = prefix[0];
  T[1] = prefix[1];
  need[0] = krem[0];
  need[1] = krem[1];
}

__global__ __launch_bounds__(kBlock) void route_tiers_kernel(kvc_tier_route_args a, kvc_cache c) {
  extern __shared__ uint8_t dyn[];
  const int u = blockIdx.x;
  const int NW = c.n_windows_max;
  // per window, in LDS: the key and one byte of flags (old tier, ledgered, valid, new tier)
  uint32_t* keys = reinterpret_cast<uint32_t*>(dyn);
  uint8_t* wm = dyn + size_t(NW) * 4;
  __shared__ SelectShared sh;
  __shared__ int4 sm_waves[kWaves];
  __shared__ int s_flag[2];

  const size_t base = size_t(u) * NW;
  const float* sc = a.scores != nullptr ? a.scores + base : c.cum + base;
  if (threadIdx.x == 0) {
    s_flag[0] = 0;
    s_flag[1] = 0;
  }
  // every window slot's tables are loaded at once (none of the addresses waits for the window count), then read
  // from LDS only
  const int n_raw = c.n_windows[u];
  for (int i0 = threadIdx.x; i0 < NW; i0 += 4 * kBlock) {  // four windows' loads in flight per thread
    float f[4];
    int t[4], lg[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = min(i0 + j * kBlock, NW - 1);
      t[j] = c.tier[base + i];
      f[j] = sc[i];
      lg[j] = c.ledgered[base + i];
    }
    // every use of the twelve loads comes after this point (in/out operands), so none is waited on early
    asm volatile("" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]),
                 "+v"(lg[0]), "+v"(lg[1]), "+v"(lg[2]), "+v"(lg[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * kBlock;
      if (i < NW) {
        keys[i] = order_key(f[j]);
        wm[i] = uint8_t((t[j] & kOldTier) | (lg[j] != 0 ? kLedgered : 0) | (isnan(f[j]) ? kValid : 0));  // kValid: NaN
      }
    }
  }
  const int n = min(max(n_raw, 0), NW);
  __syncthreads();
  int nres_local = 0;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const uint8_t f = wm[i];
    const bool v = (f & kOldTier) != KVC_TIER_EVICTED;
    if (v && (f & kValid)) atomicOr(&s_flag[0], 1);
    wm[i] = uint8_t((f & ~kValid) | (v ? kValid : 0));
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
  const int kk[2] = {k1, k2};
  uint32_t TT[2] = {0u, 0u};
  int nn[2] = {0, 0};
  radix_kth2(keys, wm, n, kk, sh, TT, nn);
  const uint32_t T1 = TT[0], T2 = TT[1];
  const int need1 = nn[0], need2 = nn[1];

  // contiguous segment of windows per thread, so that scans follow window order
  const int seg = (n + kBlock - 1) / kBlock;
  const int lo = min(n, int(threadIdx.x) * seg);
  const int hi = min(n, lo + seg);

  // pass 1: rank among keys equal to each threshold
  int4 cnt = make_int4(0, 0, 0, 0);
  for (int i = lo; i < hi; ++i) {
    if (wm[i] & kValid) {
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
    const uint8_t f = wm[i];
    if (f & kValid) {
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
    const int8_t old = int8_t(f & kOldTier);
    wm[i] = uint8_t((f & ~kNewTier) | (nt << kNewShift));
    cnt2.x += nt == KVC_TIER_FULL;
    cnt2.y += nt == KVC_TIER_INT2;
    cnt2.z += (old == KVC_TIER_FULL && nt == KVC_TIER_INT2 && !(f & kLedgered));
    cnt2.w += (old == KVC_TIER_INT2 && nt == KVC_TIER_FULL);
  }
  int4 tot2;
  int4 pos = block_scan4(cnt2, sm_waves, tot2);
  for (int i = lo; i < hi; ++i) {
    const uint8_t f = wm[i];
    const int8_t nt = int8_t((f & kNewTier) >> kNewShift);
    const int8_t old = int8_t(f & kOldTier);
    if (nt == KVC_TIER_FULL) c.res_list[base + pos.x++] = i;
    if (nt == KVC_TIER_INT2) c.res_list[base + tot2.x + pos.y++] = i;
    if (old == KVC_TIER_FULL && nt == KVC_TIER_INT2 && !(f & kLedgered)) a.quant_list[base + pos.z++] = i;
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
