// Three-tier window routing under a fixed budget (QEvict page, "Metodologia: QEvict" and "Mecanismos
// Principais"): per unit, resident windows are ranked by (score desc, window asc); the first budget_full go to the
// full-precision tier, the next budget_int2 to the INT2 tier, the rest are evicted for good. The routing also moves
// the slots of the two pools that hold window data (the cache's memory budget): a window leaving FULL frees its
// full-precision slot, an evicted window its ledger slot, and a window promoted to FULL or demoted for the first
// time takes the lowest free slot of its pool, in ascending window order.
//
// One workgroup of TB threads per unit (TB = 64, 256 or 1024: one wave per unit when units are many, 16 waves when
// they are few, so that a unit's chain of dependent steps is short). Thread t holds the windows of one contiguous
// segment of at most kSegMax windows in registers (keys, flags, slots), so every scan follows window order. The two
// rank thresholds are found together by an exact MSB-first radix select over order-preserving 32-bit keys (passes
// of 8 bits into one LDS histogram per threshold; a threshold is settled as soon as its rank takes every key of its
// digit, so later passes are skipped); keys equal to a threshold are admitted lowest index first through an
// exclusive scan in window order, run only when such a tie decides. The slots still held after the event are
// marked in two LDS bitmaps, the free slots of each pool are listed ascending, and the new resident lists with
// their slots and the quantise / promote lists are written in window order, so every output is deterministic.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kSegMax = 4;  // windows per thread segment, at most (the launch picks TB >= NW / kSegMax)

// fp32 -> uint32 with the same order (-0 folded onto +0); NaN is screened out before.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within 16-lane rows, then the row totals carried
// forward by row broadcasts (lanes a DPP move does not write keep 0).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <int TB>
struct RouteShared {
  static constexpr int W = TB / kWave;
  uint32_t hist[2][2][256];  // [pass parity][threshold][digit]
  int digit[2], krem[2], eqc[2];  // per threshold: digit holding the k-th key, its rank in the digit, the digit's count
  int k[2];                       // the two ranks: min(b_full, resident), min(b_full + b_int2, resident)
  int nan;
  int tie[W][2];   // per-wave totals of the tie scan
  int scan[W][6];  // per-wave totals of the list / free-slot scan
};

// Block-wide exclusive scan of N counters in thread order: wave scans, then lane w of every wave reads wave w's
// totals from LDS and one more wave scan gives each wave its base. One barrier (none for a one-wave workgroup);
// `tot` receives the totals.
template <int TB, int N>
__device__ __forceinline__ void block_scan(int (&v)[N], int (&tot)[N], int (*wtot)[N]) {
  constexpr int W = TB / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) inc[j] = wave_incl_scan(v[j]);
  if (W == 1) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      tot[j] = __builtin_amdgcn_readlane(inc[j], kWave - 1);
      v[j] = inc[j] - v[j];
    }
    return;
  }
  if (lane == kWave - 1) {
#pragma unroll
    for (int j = 0; j < N; ++j) wtot[wave][j] = inc[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int x = lane < W ? wtot[lane][j] : 0;
    const int xi = wave_incl_scan(x);
    tot[j] = __builtin_amdgcn_readlane(xi, W - 1);
    v[j] = __builtin_amdgcn_readlane(xi - x, wave) + inc[j] - v[j];
  }
}

// One wave finds, in a 256-bin histogram (larger digit = larger score), the digit holding the kr-th largest key
// (kr >= 1) and stores it with the key's rank inside the digit and the digit's count. Lane l owns bins 4l .. 4l+3.
__device__ __forceinline__ void pick_digit(const uint32_t* h, int kr, int* digit, int* krem, int* eqc) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint4 c4 = *reinterpret_cast<const uint4*>(h + 4 * lane);
  const int c[4] = {int(c4.x), int(c4.y), int(c4.z), int(c4.w)};
  const int own = c[0] + c[1] + c[2] + c[3];
  const int incl = wave_incl_scan(own);
  const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
  int above = total - incl;  // keys in bins of the lanes above this one
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    if (above < kr && kr <= above + c[b]) {
      *digit = 4 * lane + b;
      *krem = kr - above;
      *eqc = c[b];
    }
    above += c[b];
  }
}

template <int TB>
__global__ __launch_bounds__(TB) void route_tiers_kernel(kvc_tier_route_args a, kvc_cache c) {
  constexpr int W = TB / kWave;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  __shared__ __attribute__((aligned(16))) RouteShared<TB> sh;
  const int tid = int(threadIdx.x), lane = tid & (kWave - 1), wave = tid >> 6;
  const int u = blockIdx.x;
  const int NW = c.n_windows_max;
  const int FS = c.full_slots, LS = c.ledger_slots;
  const int fw = (FS + 31) / 32, lw = (LS + 31) / 32;  // words of the two slot bitmaps
  // LDS: the bitmaps of the full-precision and ledger slots still held; the free slots of each pool, ascending
  uint32_t* used_full = reinterpret_cast<uint32_t*>(dyn);
  uint32_t* used_led = used_full + fw;
  uint16_t* free_full = reinterpret_cast<uint16_t*>(used_led + lw);
  uint16_t* free_led = free_full + FS;

  const size_t base = size_t(u) * NW;
  const float* sc = a.scores != nullptr ? a.scores + base : c.cum + base;
  // this thread's segment, cut from the capacity so that no load waits for the window count: every table entry of
  // the segment is loaded at once (indices clamped into the unit; used only for windows below the count)
  const int seg = (NW + TB - 1) / TB;  // <= kSegMax
  const int lo = min(NW, tid * seg);
  float f[kSegMax] = {};
  int t[kSegMax] = {}, lg[kSegMax] = {}, fsr[kSegMax] = {}, lsr[kSegMax] = {};
#pragma unroll
  for (int k = 0; k < kSegMax; ++k) {
    if (k < seg) {  // seg is uniform
      const int i = min(lo + k, NW - 1);
      f[k] = sc[i];
      t[k] = c.tier[base + i];
      lg[k] = c.ledgered[base + i];
      fsr[k] = c.full_slot[base + i];
      lsr[k] = c.ledger_slot[base + i];
    }
  }
  const int n_raw = c.n_windows[u];
  const int bf = max(0, a.budget_full[u]);
  const int bq = max(0, a.budget_int2[u]);
  for (int i = tid; i < fw + lw; i += TB) used_full[i] = 0u;  // used_led follows used_full
  for (int i = tid; i < 2 * 256; i += TB) (&sh.hist[0][0][0])[i] = 0u;
  if (tid == 0) sh.nan = 0;
  __syncthreads();

  // windows of this segment below the count; resident = not evicted before the event
  const int n = min(max(n_raw, 0), NW);
  const int hi = min(n, lo + seg);
  uint32_t key[kSegMax];
  uint32_t res_mask = 0u;  // bit k: window lo + k is resident
  bool nan = false;
#pragma unroll
  for (int k = 0; k < kSegMax; ++k) {
    const bool r = lo + k < hi && (t[k] & 3) != KVC_TIER_EVICTED;
    res_mask |= (r ? 1u : 0u) << k;
    nan |= r && isnan(f[k]);
    key[k] = order_key(f[k]);
  }
  // pass 0 (top 8 bits), shared by both thresholds: the wave's lanes grouped by digit, one atomic per distinct
  // digit (few distinct values share the top digit); the next pass's histograms are cleared meanwhile
  for (int i = tid; i < 2 * 256; i += TB) (&sh.hist[1][0][0])[i] = 0u;
#pragma unroll
  for (int k = 0; k < kSegMax; ++k) {
    const bool m = (res_mask >> k) & 1u;
    const uint32_t bin = key[k] >> 24;
    uint64_t act = __ballot(m);
    while (act) {
      const int leader = __builtin_ctzll(act);
      const uint32_t lb = uint32_t(__builtin_amdgcn_readlane(int(bin), leader));
      const uint64_t same = __ballot(m && bin == lb);
      if (lane == leader) atomicAdd(&sh.hist[0][0][lb], uint32_t(__popcll(same)));
      act &= ~same;
    }
  }
  if (nan) sh.nan = 1;
  __syncthreads();
  if (sh.nan != 0) {
    if (tid == 0) atomicOr(c.status, KVC_DEV_NAN_SCORE);
    return;
  }
  if (wave == 0) {
    // resident count (the histogram's total), the two ranks, and both thresholds' first digits
    const uint4 c4 = *reinterpret_cast<const uint4*>(&sh.hist[0][0][4 * lane]);
    const int n_res = __builtin_amdgcn_readlane(wave_incl_scan(int(c4.x + c4.y + c4.z + c4.w)), kWave - 1);
    const int k1 = min(bf, n_res), k2 = int(min(int64_t(bf) + bq, int64_t(n_res)));  // budgets up to INT_MAX each
    if (lane == 0) {
      sh.k[0] = k1;
      sh.k[1] = k2;
    }
    if (k1 > 0) pick_digit(sh.hist[0][0], k1, &sh.digit[0], &sh.krem[0], &sh.eqc[0]);
    if (k2 > 0) pick_digit(sh.hist[0][0], k2, &sh.digit[1], &sh.krem[1], &sh.eqc[1]);
  }
  __syncthreads();
  const int kk[2] = {sh.k[0], sh.k[1]};
  uint32_t T[2] = {0u, 0u}, M[2] = {0u, 0u};  // threshold digits so far and their mask
  int need[2] = {0, 0}, eqc[2] = {0, 0};
  bool done[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    done[s] = kk[s] <= 0;
    if (!done[s]) {
      T[s] = uint32_t(sh.digit[s]) << 24;
      M[s] = 0xFF000000u;
      need[s] = sh.krem[s];
      eqc[s] = sh.eqc[s];
      done[s] = need[s] == eqc[s];  // the rank takes every key of its digit
    }
  }
  // passes 1..3: each unsettled threshold histograms the next 8 bits of the keys that share its digits so far
  for (int p = 1; p < 4 && !(done[0] && done[1]); ++p) {
    const int shift = 24 - 8 * p;
    const int buf = p & 1;
    for (int i = tid; i < 2 * 256; i += TB) (&sh.hist[buf ^ 1][0][0])[i] = 0u;
#pragma unroll
    for (int k = 0; k < kSegMax; ++k) {
      if ((res_mask >> k) & 1u) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (!done[s] && (key[k] & M[s]) == T[s]) atomicAdd(&sh.hist[buf][s][(key[k] >> shift) & 255u], 1u);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (!done[s] && wave == (W > 1 ? s : 0)) {
        pick_digit(sh.hist[buf][s], need[s], &sh.digit[s], &sh.krem[s], &sh.eqc[s]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (!done[s]) {
        T[s] |= uint32_t(sh.digit[s]) << shift;
        M[s] |= 0xFFu << shift;
        need[s] = sh.krem[s];
        eqc[s] = sh.eqc[s];
        done[s] = need[s] == eqc[s];
      }
    }
  }
  // keys whose masked value equals an unsettled threshold (exact ties after the last pass): rank in window order
  const bool ties = (kk[0] > 0 && need[0] < eqc[0]) || (kk[1] > 0 && need[1] < eqc[1]);
  int eq[2] = {0, 0};
  if (ties) {
    int tot[2];
#pragma unroll
    for (int k = 0; k < kSegMax; ++k) {
      if ((res_mask >> k) & 1u) {
        eq[0] += (key[k] & M[0]) == T[0] ? 1 : 0;
        eq[1] += (key[k] & M[1]) == T[1] ? 1 : 0;
      }
    }
    block_scan<TB, 2>(eq, tot, sh.tie);
  }

  // new tier per window, the slots it keeps, and per-thread counts of the four lists
  int8_t nt[kSegMax];
  int cnt[6] = {0, 0, 0, 0, 0, 0};
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kSegMax; ++k) {
    nt[k] = KVC_TIER_EVICTED;
    if ((res_mask >> k) & 1u) {
      bool top[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t km = key[k] & M[s];
        top[s] = kk[s] > 0 && (km > T[s] || (km == T[s] && (!ties || eq[s] < need[s])));
        if (ties && kk[s] > 0 && km == T[s]) ++eq[s];
      }
      nt[k] = top[0] ? KVC_TIER_FULL : (top[1] ? KVC_TIER_INT2 : KVC_TIER_EVICTED);
    }
    if (lo + k < hi) {
      const int old = t[k] & 3;
      if (old == KVC_TIER_FULL && nt[k] == KVC_TIER_FULL) {  // keeps its full-precision slot
        const int s2 = fsr[k];
        if (unsigned(s2) < unsigned(FS)) atomicOr(&used_full[s2 >> 5], 1u << (s2 & 31));
        else bad = true;
      }
      if (lg[k] != 0 && nt[k] != KVC_TIER_EVICTED) {  // keeps its ledger slot
        const int s2 = lsr[k];
        if (unsigned(s2) < unsigned(LS)) atomicOr(&used_led[s2 >> 5], 1u << (s2 & 31));
        else bad = true;
      }
      cnt[0] += nt[k] == KVC_TIER_FULL;
      cnt[1] += nt[k] == KVC_TIER_INT2;
      cnt[2] += old == KVC_TIER_FULL && nt[k] == KVC_TIER_INT2 && lg[k] == 0;
      cnt[3] += old == KVC_TIER_INT2 && nt[k] == KVC_TIER_FULL;
    }
  }
  __syncthreads();  // the bitmaps are complete
  // free slots of each pool: thread t owns bitmap words [t*wf, t*wf + wf) and [t*wl, t*wl + wl)
  const int wf = (fw + TB - 1) / TB, wl = (lw + TB - 1) / TB;
  const int f_lo = min(fw, tid * wf), f_hi = min(fw, f_lo + wf);
  const int l_lo = min(lw, tid * wl), l_hi = min(lw, l_lo + wl);
  auto free_bits = [](uint32_t used, int w, int slots) {
    const int valid = min(32, slots - 32 * w);
    return ~used & (valid >= 32 ? 0xFFFFFFFFu : ((1u << valid) - 1u));
  };
  for (int w = f_lo; w < f_hi; ++w) cnt[4] += __popc(free_bits(used_full[w], w, FS));
  for (int w = l_lo; w < l_hi; ++w) cnt[5] += __popc(free_bits(used_led[w], w, LS));
  int tot[6];
  block_scan<TB, 6>(cnt, tot, sh.scan);
  for (int w = f_lo; w < f_hi; ++w) {
    for (uint32_t b = free_bits(used_full[w], w, FS); b != 0u; b &= b - 1u) {
      free_full[cnt[4]++] = uint16_t(32 * w + __builtin_ctz(b));
    }
  }
  for (int w = l_lo; w < l_hi; ++w) {
    for (uint32_t b = free_bits(used_led[w], w, LS); b != 0u; b &= b - 1u) {
      free_led[cnt[5]++] = uint16_t(32 * w + __builtin_ctz(b));
    }
  }
  __syncthreads();
  const int nfree_full = tot[4], nfree_led = tot[5];

  // resident lists with their slots, quantise / promote lists, new slots, tiers
  int32_t* res = c.res_list + base;
  int32_t* rsl = c.res_slot + base;
#pragma unroll
  for (int k = 0; k < kSegMax; ++k) {
    const int i = lo + k;
    if (i >= hi) break;
    const int old = t[k] & 3;
    const bool first_quant = old == KVC_TIER_FULL && nt[k] == KVC_TIER_INT2 && lg[k] == 0;
    const bool promoted = old == KVC_TIER_INT2 && nt[k] == KVC_TIER_FULL;
    if (nt[k] == KVC_TIER_FULL) {
      int slot = fsr[k];
      if (promoted) {
        const int r = cnt[3];  // rank among this event's promotions
        slot = r < nfree_full ? int(free_full[r]) : -1;
        c.full_slot[base + i] = slot;
      }
      bad |= unsigned(slot) >= unsigned(FS);
      rsl[cnt[0]] = slot;
      res[cnt[0]++] = i;
    }
    if (nt[k] == KVC_TIER_INT2) {
      int slot = lsr[k];
      if (first_quant) {
        const int r = cnt[2];  // rank among this event's first demotions
        slot = r < nfree_led ? int(free_led[r]) : -1;
        c.ledger_slot[base + i] = slot;
      }
      bad |= unsigned(slot) >= unsigned(LS);
      rsl[tot[0] + cnt[1]] = slot;
      res[tot[0] + cnt[1]++] = i;
    }
    if (first_quant) a.quant_list[base + cnt[2]++] = i;
    if (promoted) a.promo_list[base + cnt[3]++] = i;
    if (nt[k] == KVC_TIER_EVICTED && old != KVC_TIER_EVICTED) c.ledgered[base + i] = 0;
    c.tier[base + i] = nt[k];
  }
  if (bad) atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
  if (tid == 0) {
    c.n_full[u] = tot[0];
    c.n_int2[u] = tot[1];
    a.n_quant[u] = tot[2];
    a.n_promo[u] = tot[3];
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
  const size_t words = (c.full_slots + 31) / 32 + (c.ledger_slots + 31) / 32;
  return words * 4 + size_t(c.full_slots + c.ledger_slots) * 2;
}

// Threads per unit: the fewest that hold the unit in segments of at most kSegMax windows while the launch still
// has 64K threads (four waves per CU); with fewer units, 1024.
int route_tiers_threads(const kvc_cache& c) {
  for (int tb : {64, 256}) {
    if (c.n_windows_max <= tb * kSegMax && int64_t(c.n_units) * tb >= 65536) return tb;
  }
  return 1024;
}

hipError_t launch_route_tiers(const kvc_tier_route_args& a, hipStream_t s) {
  static_assert(kRouteMaxWindows <= 1024 * kSegMax, "1024 threads hold the largest unit");
  const kvc_cache& c = *a.cache;
  const size_t lds = route_tiers_lds_bytes(c);
  switch (route_tiers_threads(c)) {
    case 64: hipLaunchKernelGGL(route_tiers_kernel<64>, dim3(c.n_units), dim3(64), lds, s, a, c); break;
    case 256: hipLaunchKernelGGL(route_tiers_kernel<256>, dim3(c.n_units), dim3(256), lds, s, a, c); break;
    default: hipLaunchKernelGGL(route_tiers_kernel<1024>, dim3(c.n_units), dim3(1024), lds, s, a, c); break;
  }
  return hipGetLastError();
}

hipError_t launch_repack(const kvc_cache& c, void* k_dst, void* v_dst, int32_t dst_slots, hipStream_t s) {
  hipLaunchKernelGGL(repack_kernel, dim3(unsigned(int64_t(c.n_units) * dst_slots)), dim3(kRepackThreads), 0, s, c,
                     static_cast<uint16_t*>(k_dst), static_cast<uint16_t*>(v_dst), dst_slots);
  return hipGetLastError();
}

}  // namespace kvc
