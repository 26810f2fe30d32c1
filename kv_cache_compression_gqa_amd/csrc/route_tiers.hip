// Three-tier window routing under a fixed budget (QEvict page, "Metodologia: QEvict" and "Mecanismos
// Principais"): per unit, resident windows are ranked by (score desc, window asc); the first budget_full go to the
// full-precision tier, the next budget_int2 to the INT2 tier, the rest are evicted for good. The routing also moves
// the slots of the two pools that hold window data (the cache's memory budget): a window leaving FULL frees its
// full-precision slot, an evicted window its ledger slot, and a window promoted to FULL or demoted for the first
// time takes the lowest free slot of its pool, in ascending window order.
//
// One workgroup per unit. The two rank thresholds are found together by an exact MSB-first radix select over
// order-preserving 32-bit keys (4 passes of 8 bits, per-wave LDS histograms, one wave per threshold scans the 256
// bins); keys equal to a threshold are admitted lowest index first through an exclusive scan in window order. The
// slots still held after the event are marked in two LDS bitmaps, the free slots of each pool are listed
// ascending (a block scan over slot segments), and one more in-order scan writes the new resident lists with their
// slots and the quantise / promote lists, so every output is deterministic.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kSeg = kRouteMaxWindows / kBlock;  // windows per thread segment, at most
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
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int u = blockIdx.x;
  const int NW = c.n_windows_max;
  const int FS = c.full_slots, LS = c.ledger_slots;
  const int fw = (FS + 31) / 32, lw = (LS + 31) / 32;  // words of the two slot bitmaps
  // LDS: per window the key and one byte of flags (old tier, ledgered, valid, new tier); the bitmaps of the
  // full-precision and ledger slots still held; the free slots of each pool, ascending (16-bit slot ids)
  uint32_t* keys = reinterpret_cast<uint32_t*>(dyn);
  uint32_t* used_full = keys + NW;
  uint32_t* used_led = used_full + fw;
  uint16_t* free_full = reinterpret_cast<uint16_t*>(used_led + lw);
  uint16_t* free_led = free_full + FS;
  uint8_t* wm = reinterpret_cast<uint8_t*>(free_led + LS);
  __shared__ SelectShared sh;
  __shared__ int4 sm_waves[kWaves];
  __shared__ int s_flag[3];

  const size_t base = size_t(u) * NW;
  const float* sc = a.scores != nullptr ? a.scores + base : c.cum + base;
  if (threadIdx.x == 0) {
    s_flag[0] = 0;
    s_flag[1] = 0;
    s_flag[2] = 0;
  }
  for (int i = threadIdx.x; i < fw + lw; i += kBlock) used_full[i] = 0u;  // used_led follows used_full
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
  // contiguous segment of windows per thread, so that scans follow window order; the segment's two slot-table
  // entries are loaded now, once, into registers (their latency is taken at the barrier below, not per window)
  const int seg = (n + kBlock - 1) / kBlock;
  const int lo = min(n, int(threadIdx.x) * seg);
  const int hi = min(n, lo + seg);
  int fsr[kSeg] = {}, lsr[kSeg] = {};
#pragma unroll
  for (int k = 0; k < kSeg; ++k) {
    if (k < seg) {  // seg is uniform: no divergence
      const int i = min(lo + k, NW - 1);
      fsr[k] = c.full_slot[base + i];
      lsr[k] = c.ledger_slot[base + i];
    }
  }
  const int bf = max(0, a.budget_full[u]);
  const int bq = max(0, a.budget_int2[u]);
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
  const int k1 = min(bf, n_res);
  const int k2 = min(bf + bq, n_res);
  const int kk[2] = {k1, k2};
  uint32_t TT[2] = {0u, 0u};
  int nn[2] = {0, 0};
  radix_kth2(keys, wm, n, kk, sh, TT, nn);
  const uint32_t T1 = TT[0], T2 = TT[1];
  const int need1 = nn[0], need2 = nn[1];

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

  // pass 2: new tier per window, the slots it keeps, and counts of the four lists
  int4 cnt2 = make_int4(0, 0, 0, 0);
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kSeg; ++k) {
    const int i = lo + k;
    if (i >= hi) break;
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
    if (old == KVC_TIER_FULL && nt == KVC_TIER_FULL) {  // keeps its full-precision slot
      const int sl = fsr[k];
      if (unsigned(sl) < unsigned(FS)) atomicOr(&used_full[sl >> 5], 1u << (sl & 31));
      else bad = true;
    }
    if ((f & kLedgered) && nt != KVC_TIER_EVICTED) {  // keeps its ledger slot
      const int sl = lsr[k];
      if (unsigned(sl) < unsigned(LS)) atomicOr(&used_led[sl >> 5], 1u << (sl & 31));
      else bad = true;
    }
    cnt2.x += nt == KVC_TIER_FULL;
    cnt2.y += nt == KVC_TIER_INT2;
    cnt2.z += (old == KVC_TIER_FULL && nt == KVC_TIER_INT2 && !(f & kLedgered));
    cnt2.w += (old == KVC_TIER_INT2 && nt == KVC_TIER_FULL);
  }
  int4 tot2;
  int4 pos = block_scan4(cnt2, sm_waves, tot2);  // its barriers also publish the bitmaps

  // free slots of each pool, ascending: thread t lists slots [t*sf, t*sf + sf) and [t*sl, t*sl + sl)
  const int sf = (FS + kBlock - 1) / kBlock, sl = (LS + kBlock - 1) / kBlock;
  const int f_lo = min(FS, int(threadIdx.x) * sf), f_hi = min(FS, f_lo + sf);
  const int l_lo = min(LS, int(threadIdx.x) * sl), l_hi = min(LS, l_lo + sl);
  int4 fc = make_int4(0, 0, 0, 0);
  for (int s2 = f_lo; s2 < f_hi; ++s2) fc.x += ((used_full[s2 >> 5] >> (s2 & 31)) & 1u) ? 0 : 1;
  for (int s2 = l_lo; s2 < l_hi; ++s2) fc.y += ((used_led[s2 >> 5] >> (s2 & 31)) & 1u) ? 0 : 1;
  int4 ftot;
  int4 frank = block_scan4(fc, sm_waves, ftot);
  for (int s2 = f_lo; s2 < f_hi; ++s2) {
    if (!((used_full[s2 >> 5] >> (s2 & 31)) & 1u)) free_full[frank.x++] = uint16_t(s2);
  }
  for (int s2 = l_lo; s2 < l_hi; ++s2) {
    if (!((used_led[s2 >> 5] >> (s2 & 31)) & 1u)) free_led[frank.y++] = uint16_t(s2);
  }
  __syncthreads();
  const int nfree_full = ftot.x, nfree_led = ftot.y;

  // pass 3: resident lists with their slots, quantise / promote lists, new slots, tiers
  int32_t* res = c.res_list + base;
  int32_t* rsl = c.res_slot + base;
#pragma unroll
  for (int k = 0; k < kSeg; ++k) {
    const int i = lo + k;
    if (i >= hi) break;
    const uint8_t f = wm[i];
    const int8_t nt = int8_t((f & kNewTier) >> kNewShift);
    const int8_t old = int8_t(f & kOldTier);
    const bool first_quant = old == KVC_TIER_FULL && nt == KVC_TIER_INT2 && !(f & kLedgered);
    const bool promoted = old == KVC_TIER_INT2 && nt == KVC_TIER_FULL;
    if (nt == KVC_TIER_FULL) {
      int slot;
      if (promoted) {
        const int r = pos.w;  // rank among this event's promotions
        slot = r < nfree_full ? int(free_full[r]) : -1;
        c.full_slot[base + i] = slot;
      } else {
        slot = fsr[k];
      }
      bad |= unsigned(slot) >= unsigned(FS);
      rsl[pos.x] = slot;
      res[pos.x++] = i;
    }
    if (nt == KVC_TIER_INT2) {
      int slot;
      if (first_quant) {
        const int r = pos.z;  // rank among this event's first demotions
        slot = r < nfree_led ? int(free_led[r]) : -1;
        c.ledger_slot[base + i] = slot;
      } else {
        slot = lsr[k];
      }
      bad |= unsigned(slot) >= unsigned(LS);
      rsl[tot2.x + pos.y] = slot;
      res[tot2.x + pos.y++] = i;
    }
    if (first_quant) a.quant_list[base + pos.z++] = i;
    if (promoted) a.promo_list[base + pos.w++] = i;
    if (nt == KVC_TIER_EVICTED && old != KVC_TIER_EVICTED) c.ledgered[base + i] = 0;
    c.tier[base + i] = nt;
  }
  if (bad) atomicOr(&s_flag[2], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    c.n_full[u] = tot2.x;
    c.n_int2[u] = tot2.y;
    a.n_quant[u] = tot2.z;
    a.n_promo[u] = tot2.w;
    if (s_flag[2] != 0) atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
  }
}

// repack: one workgroup per (unit, destination slot i): FULL window i of the unit moves from its slot to slot i of
// the new pool (16 KiB: 256 threads x 4 x 16 bytes), then full_slot and res_slot point at i
constexpr int kRepackThreads = 256;

__global__ __launch_bounds__(kRepackThreads) void repack_kernel(kvc_cache c, uint16_t* k_dst, uint16_t* v_dst,
                                                                int dst_slots) {
  const int u = blockIdx.x / dst_slots;
  const int i = blockIdx.x - u * dst_slots;
  const int NW = c.n_windows_max;
  const size_t base = size_t(u) * NW;
  const int nf_dev = c.n_full[u];
  const int nf = min(max(nf_dev, 0), NW);
  if (i == 0 && threadIdx.x == 0 && nf_dev > dst_slots) {
    atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
    for (int j = dst_slots; j < nf; ++j) {  // FULL windows past the new pool: no slot
      c.full_slot[base + c.res_list[base + j]] = -1;
      c.res_slot[base + j] = -1;
    }
  }
  if (i >= nf) return;
  const int w = c.res_list[base + i];
  const int src = c.res_slot[base + i];
  if (unsigned(w) >= unsigned(NW) || unsigned(src) >= unsigned(c.full_slots)) {
    if (threadIdx.x == 0) {
      atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
      c.res_slot[base + i] = -1;
    }
    return;
  }
  constexpr int kVec = kW * kD * 2 / 16;  // 16-byte vectors per K (or V) slot: 512
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(c.k_full) +
                                                   (size_t(u) * c.full_slots + src) * (kW * kD));
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(c.v_full) +
                                                   (size_t(u) * c.full_slots + src) * (kW * kD));
  uint4* kd = reinterpret_cast<uint4*>(k_dst + (size_t(u) * dst_slots + i) * (kW * kD));
  uint4* vd = reinterpret_cast<uint4*>(v_dst + (size_t(u) * dst_slots + i) * (kW * kD));
  uint4 kx[kVec / kRepackThreads], vx[kVec / kRepackThreads];
#pragma unroll
  for (int j = 0; j < kVec / kRepackThreads; ++j) {
    kx[j] = ks[j * kRepackThreads + threadIdx.x];
    vx[j] = vs[j * kRepackThreads + threadIdx.x];
  }
#pragma unroll
  for (int j = 0; j < kVec / kRepackThreads; ++j) {
    kd[j * kRepackThreads + threadIdx.x] = kx[j];
    vd[j * kRepackThreads + threadIdx.x] = vx[j];
  }
  if (threadIdx.x == 0) {
    c.full_slot[base + w] = i;
    c.res_slot[base + i] = i;
  }
}

}  // namespace

size_t route_tiers_lds_bytes(const kvc_cache& c) {
  const size_t words = size_t(c.n_windows_max) + (c.full_slots + 31) / 32 + (c.ledger_slots + 31) / 32;
  return words * 4 + size_t(c.full_slots + c.ledger_slots) * 2 + size_t(c.n_windows_max);
}

hipError_t launch_route_tiers(const kvc_tier_route_args& a, hipStream_t s) {
  const kvc_cache& c = *a.cache;
  hipLaunchKernelGGL(route_tiers_kernel, dim3(c.n_units), dim3(kBlock), route_tiers_lds_bytes(c), s, a, c);
  return hipGetLastError();
}

hipError_t launch_repack(const kvc_cache& c, void* k_dst, void* v_dst, int32_t dst_slots, hipStream_t s) {
  hipLaunchKernelGGL(repack_kernel, dim3(unsigned(int64_t(c.n_units) * dst_slots)), dim3(kRepackThreads), 0, s, c,
                     static_cast<uint16_t*>(k_dst), static_cast<uint16_t*>(v_dst), dst_slots);
  return hipGetLastError();
}

}  // namespace kvc
