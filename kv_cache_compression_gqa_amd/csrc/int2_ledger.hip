// Write-once INT2 quantisation ledger and promotion (QEvict page, "Mecanismos Principais": a window is quantised
// only at its first demotion; the low-bit copy is kept and reused for every later promotion and demotion, so the
// approximation error never compounds; promotion dequantises the copy back to full precision).
//
// Both kernels take per-unit lists + per-unit counts and spread the listed windows evenly over the whole grid:
// every workgroup first builds, in LDS, the exclusive prefix of the counts of the units it serves (at most kSpan
// units per launch), so flat item f belongs to the unit whose prefix range holds it (binary search). Items go
// round-robin over workgroups (quantiser: one window per workgroup at a time) or over waves (promotion: one window
// per wave at a time); a unit with many listed windows is no longer a serial chain. The grid is sized from the
// host bound and the resident capacity of the GPU, never from a device-side count.
//
// Quantiser (all decisions in fp32 so that they are bit-reproducible; contraction is disabled for this file):
//   lo, hi = group min / max; zero z = largest fp16 <= lo; scale s = smallest fp16 >= fl32(fl32(hi - z) / 3)
//   (0 if hi == z); code = #{k in 0..2 : fl32(x - z) >= (k + 0.5) * s} (0 if s == 0).
// Storage layouts (see include/kvc.h): K codes of a token row: byte 8*s + 2*g + h holds head_dim 32g + 8s + 4h + e
// at bits 2e, so the 16-bit word at byte 8s + 2g holds head_dims 32g + 8s + k (k = 0..7) at bits 2k; V codes:
// 16-bit word (r, q, dt) of a window holds tokens 8q + e of head_dim 16dt + r at bits 2e; V meta: word (q, g, e)
// = token 8q + e, group g.
#include <algorithm>

#include "kvc_internal.h"

#pragma clang fp contract(off)

namespace kvc {
namespace {

constexpr int kBlock = 256;
constexpr int kSpan = 4096;  // units per launch: their count prefix sits in LDS (16 KiB)

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

// The prefix of unit i sits at pre[i + i/16]: one padding dword per 16 units, so that thread t's run of 16
// entries (below) starts 17 dwords after thread t-1's and a wave's accesses to it fall in distinct LDS banks.
constexpr int kPer = kSpan / kBlock;
constexpr int kPreWords = kSpan + kSpan / kPer + 1;
__device__ __forceinline__ int pad_idx(int i) { return i + i / kPer; }

// Exclusive prefix of the clamped counts of units [u0, u0 + nu) into pre (pre[pad_idx(nu)] = total); every thread
// gets the total. The counts are loaded coalesced (unit k*256 + t by thread t, all loads issued at once) into
// LDS; thread t then sums units [kPer*t, kPer*t + kPer) and one block scan places them. Contains the barriers
// that publish pre.
__device__ int unit_prefix(const int32_t* count, int u0, int nu, int stride, int* pre, int* wsum) {
  int v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) v[k] = count[u0 + min(k * kBlock + int(threadIdx.x), nu - 1)];  // unconditional
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = k * kBlock + threadIdx.x;
    if (i < nu) pre[pad_idx(i)] = min(max(v[k], 0), stride);
  }
  __syncthreads();
  const int beg = int(threadIdx.x) * kPer;
  int* mine = pre + pad_idx(beg);
  int n[kPer];
  int own = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    n[k] = beg + k < nu ? mine[k] : 0;
    own += n[k];
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int inc = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  int base = inc - own, total = 0;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) {
    base += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {  // this thread's own run only
    if (beg + k < nu) mine[k] = base;
    base += n[k];
  }
  if (threadIdx.x == 0) pre[pad_idx(nu)] = total;
  __syncthreads();
  return total;
}

// The unit k (0 <= k < nu) with P(k) <= f < P(k + 1), P(i) = pre[pad_idx(i)], for 0 <= f < P(nu) (P(0) = 0).
__device__ __forceinline__ int find_unit(const int* pre, int nu, int f) {
  int lo = 0, hi = nu;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[pad_idx(mid)] <= f) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Unit and window id of flat item f (f < total); window -1 past the end.
__device__ __forceinline__ void resolve_item(const int32_t* list, int stride, const int* pre, int u0, int nu, int total,
                                             int f, int& u, int& w) {
  u = u0;
  w = -1;
  if (f < total) {
    const int k = find_unit(pre, nu, f);
    u = u0 + k;
    w = list[size_t(u) * stride + (f - pre[pad_idx(k)])];
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its global stores (a
// __syncthreads() would also wait until every store of the window had completed).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// What a quantiser thread loads for one window: 32 bytes of V^T and the 64 bytes of the K group (token tok, group
// grp) that thread tok*4 + grp of the K half quantises (the V half loads the same K bytes: every thread then
// issues the same memory operations, so the compiler's waits never fall back to the fewest of two paths).
struct QuantIn {
  uint4 v0, v1, k0, k1, k2, k3;
};

// win: the window's full-precision slot, flat over units (u * FS + slot)
__device__ __forceinline__ QuantIn quant_load(const kvc_cache& c, size_t win, int tok, int grp) {
  QuantIn in;
  const uint4* vsrc = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(c.v_full) + win * kW * kD);
  in.v0 = vsrc[2 * threadIdx.x];
  in.v1 = vsrc[2 * threadIdx.x + 1];
  const uint4* ksrc = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(c.k_full) + (win * kW + tok) * kD +
                                                     grp * kGroupElems);
  in.k0 = ksrc[0];
  in.k1 = ksrc[1];
  in.k2 = ksrc[2];
  in.k3 = ksrc[3];
  return in;
}

static_assert(kW * kCodeBytes == 4 * kBlock && kW * kD / 4 == 4 * kBlock && 2 * kW * kGroups == kBlock,
              "one dword per thread of each ledger array of a window");

struct QuantLds {
  uint16_t vt[kD * kW];           // V^T window [d][t]
  uint8_t vcode[kD * kW];         // V codes [d][t]
  uint32_t kcode[kW * kCodeBytes / 4];  // K code rows of the window, as stored
  uint32_t meta[2 * kW * kGroups];      // K meta words, then V meta words, as stored
};

// Quantise one window from its loaded data (the whole workgroup; LDS-only barriers) into ledger slot win (flat over
// units, u * LS + slot) and mark window flag (u * NW + w) ledgered. Thread t < 128 quantises K group (t/4, t%4),
// thread t >= 128 V group (token (t-128)/4, t%4); the results are staged in LDS and every thread then writes one
// dword each of the K codes, the V code words and the meta words (1 KiB apiece, contiguous).
template <class T>
__device__ __forceinline__ void quant_window(const QuantIn& in, const kvc_cache& c, size_t win, size_t flag,
                                             QuantLds& L, int half, int tok, int grp) {
  {
    uint4* dst = reinterpret_cast<uint4*>(L.vt);
    dst[2 * threadIdx.x] = in.v0;
    dst[2 * threadIdx.x + 1] = in.v1;
  }
  lds_barrier();
  float x[kGroupElems];
  if (half == 0) {
    const uint4 kq[4] = {in.k0, in.k1, in.k2, in.k3};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float f[8];
      unpack8<T>(kq[q4], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * q4 + e] = f[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kGroupElems; ++e) x[e] = T::one(L.vt[(grp * kGroupElems + e) * kW + tok]);
  }
  uint32_t meta;
  const uint64_t codes = quantize_group(x, meta);
  if (half == 0) {
    uint16_t* row = reinterpret_cast<uint16_t*>(L.kcode) + tok * (kCodeBytes / 2);
#pragma unroll
    for (int s = 0; s < 4; ++s) row[4 * s + grp] = uint16_t((codes >> (16 * s)) & 0xFFFFu);
    L.meta[tok * kGroups + grp] = meta;
  } else {
#pragma unroll
    for (int e = 0; e < kGroupElems; ++e) L.vcode[(grp * kGroupElems + e) * kW + tok] = uint8_t((codes >> (2 * e)) & 3u);
    L.meta[kW * kGroups + (tok >> 3) * 32 + grp * 8 + (tok & 7)] = meta;
  }
  lds_barrier();
  // V code words 2t and 2t+1; word (r, q, dt) holds tokens 8q..8q+7 of head_dim 16dt + r
  uint32_t vpair = 0u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int wi = 2 * int(threadIdx.x) + h;
    const int r = wi >> 5, q = (wi >> 3) & 3, dt = wi & 7;
    const uint2 b = *reinterpret_cast<const uint2*>(L.vcode + (16 * dt + r) * kW + 8 * q);
    uint32_t word = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      word |= ((b.x >> (8 * e)) & 3u) << (2 * e);
      word |= ((b.y >> (8 * e)) & 3u) << (2 * e + 8);
    }
    vpair |= word << (16 * h);
  }
  // (each window's K codes, V codes, K meta and V meta are 1 KiB apiece: 256 dwords)
  reinterpret_cast<uint32_t*>(c.k_codes)[win * kBlock + threadIdx.x] = L.kcode[threadIdx.x];
  reinterpret_cast<uint32_t*>(c.v_codes)[win * kBlock + threadIdx.x] = vpair;
  uint32_t* mdst = half == 0 ? c.k_meta + win * (kW * kGroups) : c.v_meta + win * (kW * kGroups) - kW * kGroups;
  mdst[threadIdx.x] = L.meta[threadIdx.x];  // thread t < 128: K word t; t >= 128: V word t - 128
  c.ledgered[flag] = 1;  // every thread, the same byte
  lds_barrier();  // the LDS buffers are rewritten by the next window
}

// One window per workgroup at a time; the next window's loads are issued before this window's stores.
template <class T>
__global__ __launch_bounds__(kBlock) void quantize_kernel(kvc_cache c, const int32_t* list, const int32_t* count,
                                                          int stride, int u0, int nu) {
  __shared__ int pre[kPreWords];
  __shared__ int wsum[kBlock / kWave];
  __shared__ int item_src[kWave], item_dst[kWave], item_flag[kWave], n_items;
  __shared__ QuantLds L;
  const int total = unit_prefix(count, u0, nu, stride, pre, wsum);
  const int NW = c.n_windows_max;
  const int FS = c.full_slots, LS = c.ledger_slots;
  const int NG = gridDim.x;
  const int half = threadIdx.x >> 7;         // 0 = K, 1 = V (uniform per wave)
  const int tok = (threadIdx.x & 127) >> 2;
  const int grp = threadIdx.x & 3;
  // items f0 + i * NG (i < 64) of this workgroup, resolved by its first wave at once with their two slots (the
  // full-precision slot the window held until its demotion, the ledger slot routing gave it); ids or slots out of
  // range and windows already ledgered (write-once) are reported and dropped here, so every window of the loop is
  // written
  for (int f0 = blockIdx.x; f0 < total; f0 += kWave * NG) {
    if (threadIdx.x < kWave) {
      const int f = f0 + int(threadIdx.x) * NG;
      int u, w;
      resolve_item(list, stride, pre, u0, nu, total, f, u, w);
      const bool in_range = f < total && unsigned(w) < unsigned(NW);
      const size_t wi = size_t(u) * NW + (in_range ? w : 0);
      const int fsl = in_range ? c.full_slot[wi] : 0;
      const int lsl = in_range ? c.ledger_slot[wi] : 0;
      const bool led = in_range && c.ledgered[wi] != 0;  // write-once: checked before the slots
      const bool ok = in_range && !led && unsigned(fsl) < unsigned(FS) && unsigned(lsl) < unsigned(LS);
      const uint64_t bad = __ballot(f < total && !led && !ok), rew = __ballot(led), keep = __ballot(ok);
      if (threadIdx.x == 0 && (bad | rew) != 0) {
        atomicOr(c.status, (bad != 0 ? KVC_DEV_BOUND_EXCEEDED : 0) | (rew != 0 ? KVC_DEV_LEDGER_REWRITE : 0));
      }
      if (ok) {
        const int pos = __popcll(keep & ((uint64_t(1) << threadIdx.x) - 1));
        item_src[pos] = u * FS + fsl;
        item_dst[pos] = u * LS + lsl;
        item_flag[pos] = int(wi);
      }
      if (threadIdx.x == 0) n_items = __popcll(keep);
    }
    lds_barrier();
    const int n = n_items;
    auto src_of = [&](int i) { return size_t(item_src[i]); };
    auto dst_of = [&](int i) { return size_t(item_dst[i]); };
    auto flag_of = [&](int i) { return size_t(item_flag[i]); };
    // two buffers, as in the promotion (the load after the last window re-reads it)
    if (n > 0) {
      QuantIn A = quant_load(c, src_of(0), tok, grp);
      QuantIn B = quant_load(c, src_of(min(1, n - 1)), tok, grp);
      quant_window<T>(A, c, dst_of(0), flag_of(0), L, half, tok, grp);
      for (int i = 1; i < n; i += 2) {
        A = quant_load(c, src_of(min(i + 1, n - 1)), tok, grp);
        quant_window<T>(B, c, dst_of(i), flag_of(i), L, half, tok, grp);
        if (i + 1 >= n) break;
        B = quant_load(c, src_of(min(i + 2, n - 1)), tok, grp);
        quant_window<T>(A, c, dst_of(i + 1), flag_of(i + 1), L, half, tok, grp);
      }
    }
    lds_barrier();  // the item lists are rewritten by the next batch
  }
}

// 8 codes (bits 2k of c16) -> 8 storage values rne(fmaf(code_k, s_k, z_k)), packed
template <class T>
__device__ __forceinline__ uint4 dequant8(uint32_t c16, const float (&s)[8], const float (&z)[8]) {
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = fmaf(float((c16 >> (4 * k)) & 3u), s[2 * k], z[2 * k]);
    const float b = fmaf(float((c16 >> (4 * k + 2)) & 3u), s[2 * k + 1], z[2 * k + 1]);
    o[k] = uint32_t(T::from_float(a)) | (uint32_t(T::from_float(b)) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// What one lane loads to promote a window (one window per wave):
//   K: lane l takes token t = l/2 and the 16 code bytes 16h .. 16h+15 (h = l%2) of its row: word i of them holds
//      head_dims 32g + 8s .. +7 with g = i%4, s = 2h + i/4; plus the token's four scale/zero words.
//   V: lane l takes the 8 code words 8l .. 8l+7, i.e. (r, q) = (l/4, l%4) and dt = 0..7: tokens 8q .. 8q+7 of
//      head_dims 16dt + r, with the scale/zero words (q, g, 0..7) of the four groups.
struct PromoteIn {
  uint4 kc, km, vc;
  uint4 vm[8];
};

// win: the ledger slot, flat over units
__device__ __forceinline__ void promote_load(PromoteIn& in, const kvc_cache& c, size_t win, int lane) {
  const int t = lane >> 1, h = lane & 1, q = lane & 3;
  in.kc = *reinterpret_cast<const uint4*>(c.k_codes + (win * kW + t) * kCodeBytes + 16 * h);
  in.km = *reinterpret_cast<const uint4*>(c.k_meta + (win * kW + t) * kGroups);
  in.vc = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(c.v_codes) + win * (kW * kD / 8) +
                                          8 * lane);
  const uint4* vmp = reinterpret_cast<const uint4*>(c.v_meta + win * (kW * kGroups) + 32 * q);
#pragma unroll
  for (int k = 0; k < 8; ++k) in.vm[k] = vmp[k];
}

// One 16-byte store per K word and per V word (for a fixed dt the wave writes 1 KiB contiguously). win: the
// full-precision slot, flat over units.
template <class T>
__device__ __forceinline__ void promote_store(const PromoteIn& in, const kvc_cache& c, size_t win, int lane) {
  const int t = lane >> 1, h = lane & 1;
  const int r = lane >> 2, q = lane & 3;
  uint16_t* krow = static_cast<uint16_t*>(c.k_full) + (win * kW + t) * kD;
  const uint32_t kcw[4] = {in.kc.x, in.kc.y, in.kc.z, in.kc.w};
  const uint32_t kmw[4] = {in.km.x, in.km.y, in.km.z, in.km.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int g = i & 3, s = 2 * h + (i >> 2);
    const uint32_t c16 = (kcw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    const float sc = half_bits_to_float(kmw[g] & 0xFFFFu);
    const float zc = half_bits_to_float(kmw[g] >> 16);
    const float sa[8] = {sc, sc, sc, sc, sc, sc, sc, sc};
    const float za[8] = {zc, zc, zc, zc, zc, zc, zc, zc};
    *reinterpret_cast<uint4*>(krow + 32 * g + 8 * s) = dequant8<T>(c16, sa, za);
  }
  uint16_t* vbase = static_cast<uint16_t*>(c.v_full) + win * (kD * kW) + 8 * q;
  const uint32_t vcw[4] = {in.vc.x, in.vc.y, in.vc.z, in.vc.w};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t mw[8] = {in.vm[2 * g].x,     in.vm[2 * g].y,     in.vm[2 * g].z,     in.vm[2 * g].w,
                            in.vm[2 * g + 1].x, in.vm[2 * g + 1].y, in.vm[2 * g + 1].z, in.vm[2 * g + 1].w};
    float sa[8], za[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sa[e] = half_bits_to_float(mw[e] & 0xFFFFu);
      za[e] = half_bits_to_float(mw[e] >> 16);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int d = 16 * (2 * g + h2) + r;
      const uint32_t c16 = (vcw[g] >> (16 * h2)) & 0xFFFFu;
      *reinterpret_cast<uint4*>(vbase + d * kW) = dequant8<T>(c16, sa, za);
    }
  }
}

// One window per wave at a time, the next window's loads issued before this window's stores.
template <class T>
__global__ __launch_bounds__(kBlock) void promote_kernel(kvc_cache c, const int32_t* list, const int32_t* count,
                                                         int stride, int u0, int nu) {
  __shared__ int pre[kPreWords];
  __shared__ int wsum[kBlock / kWave];
  const int total = unit_prefix(count, u0, nu, stride, pre, wsum);
  const int NW = c.n_windows_max;
  const int FS = c.full_slots, LS = c.ledger_slots;
  const int lane = threadIdx.x & (kWave - 1);
  const int nwaves = int(gridDim.x) * (kBlock / kWave);
  const int gw = int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x >> 6);
  // items f0 + i * nwaves (i < 64) of this wave, one per lane, resolved at once with their ledger slot (source) and
  // full-precision slot (destination); ids or slots out of range are reported and dropped, so every window of the
  // loop is written
  for (int f0 = gw; f0 < total; f0 += kWave * nwaves) {
    const int f = f0 + lane * nwaves;
    int u, w;
    resolve_item(list, stride, pre, u0, nu, total, f, u, w);
    const bool in_range = f < total && unsigned(w) < unsigned(NW);
    const size_t wi = size_t(u) * NW + (in_range ? w : 0);
    const int lsl = in_range ? c.ledger_slot[wi] : 0;
    const int fsl = in_range ? c.full_slot[wi] : 0;
    const bool ok = in_range && unsigned(fsl) < unsigned(FS) && unsigned(lsl) < unsigned(LS);
    if (lane == 0 && __ballot(f < total && !ok) != 0) atomicOr(c.status, KVC_DEV_BOUND_EXCEEDED);
    uint64_t rest = __ballot(ok);
    if (rest == 0) continue;
    const int src = u * LS + lsl, dst = u * FS + fsl;
    auto led_of = [&](int i) { return size_t(__builtin_amdgcn_readlane(src, i)); };
    auto win_of = [&](int i) { return size_t(__builtin_amdgcn_readlane(dst, i)); };
    auto take = [&](int cur) {  // next kept lane, or cur again when none is left
      if (rest == 0) return cur;
      const int i = __builtin_ctzll(rest);
      rest &= rest - 1;
      return i;
    };
    // Two buffers: one window's loads are in flight while the other is dequantised and stored. After the last
    // item the load re-reads it (in bounds, unused), so that every path issues the same memory operations and
    // the wait before each dequantisation never covers the previous window's stores.
    PromoteIn A, B;
    const int i0 = take(-1);
    int ib = take(i0);
    promote_load(A, c, led_of(i0), lane);
    promote_load(B, c, led_of(ib), lane);
    promote_store<T>(A, c, win_of(i0), lane);
    if (ib == i0) continue;
    while (true) {
      const int ia = take(ib);
      promote_load(A, c, led_of(ia), lane);
      promote_store<T>(B, c, win_of(ib), lane);
      if (ia == ib) break;
      ib = take(ia);
      promote_load(B, c, led_of(ib), lane);
      promote_store<T>(A, c, win_of(ia), lane);
      if (ib == ia) break;
    }
  }
}

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

// Workgroups of one launch: enough for the host bound (per_wg windows per workgroup at a time), at most what the
// GPU holds resident at once, so that every workgroup starts at the beginning. One launch per kSpan units.
template <class T, bool QUANT>
hipError_t launch_lists(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                        int64_t max_total, hipStream_t s) {
  const auto kernel = QUANT ? quantize_kernel<T> : promote_kernel<T>;
  const int per_wg = QUANT ? 1 : kBlock / kWave;
  static int resident = 0;  // per (dtype, kernel)
  if (resident == 0) {
    int n = 0;
    resident = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kBlock, 0) == hipSuccess && n > 0 ? n : 1;
  }
  const int64_t want = (max_total + per_wg - 1) / per_wg;
  const int ng = int(std::max<int64_t>(1, std::min<int64_t>(want, int64_t(resident) * device_cus())));
  for (int u0 = 0; u0 < c.n_units; u0 += kSpan) {
    const int nu = std::min(kSpan, c.n_units - u0);
    hipLaunchKernelGGL(kernel, dim3(unsigned(ng)), dim3(kBlock), 0, s, c, list, count, stride, u0, nu);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                           int64_t max_total, hipStream_t s) {
  if (max_total <= 0 || c.n_units <= 0) return hipSuccess;
  return c.kv_dtype == KVC_BF16 ? launch_lists<BF16, true>(c, list, count, stride, max_total, s)
                                : launch_lists<F16, true>(c, list, count, stride, max_total, s);
}

hipError_t launch_promote(const kvc_cache& c, const int32_t* list, const int32_t* count, int32_t stride,
                          int64_t max_total, hipStream_t s) {
  if (max_total <= 0 || c.n_units <= 0) return hipSuccess;
  return c.kv_dtype == KVC_BF16 ? launch_lists<BF16, false>(c, list, count, stride, max_total, s)
                                : launch_lists<F16, false>(c, list, count, stride, max_total, s);
}

}  // namespace kvc
