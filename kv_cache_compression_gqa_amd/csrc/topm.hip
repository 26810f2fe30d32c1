// Global top-M engine: the first m entries of n scores in the order (score desc, index asc), as a keep mask (the
// budgeted selection of the DBTrimKV page, "Metodologia", section 3: every entry of every layer and head competes
// for one global budget; also the generic top-k). Rows of row_len entries only matter for the per-row counts.
//
// Keys are the inverted order-preserving images of the scores (a smaller key is a larger score; +0 == -0). The
// scores are read from memory or computed on the fly as DBTrimKV's log-retention (t - i) * logf(beta) (the
// retention score of section 2; computing it where it is used saves writing and re-reading it). The input is read
// once in full; everything after that touches only the candidates, the entries of a few histogram bins.
// The unit of work is a chunk of 2048 entries inside one row: one wave reads it with eight 16-byte loads per lane.
//   sample     histogram (top 11 key bits) of S = min(65536, n / 4) float4s, one per stratum of n / S entries at a
//              pseudo-random offset inside it (a fixed hash of the stratum number), so that no row structure aliases
//              with the sampling.
//   classify   (16 chunks per 256-thread workgroup, one per wave at a time, no barrier inside the loop): locates in
//              the sample the window [lo, hi] of bins that holds the m-th key with a wide margin (six standard
//              deviations of the sampled count, on the host); entries below lo are kept, entries of lo .. hi go
//              to their chunk's candidate segment in index order, and the exact histogram is built on the way.
//   cand_hist2 (256 chunks' candidates per workgroup): picks the exact bin b1 from that histogram; if the window did
//              not hold it (rare), first classifies its own chunks again against b1 alone; then the histogram of the
//              next 11 key bits of the candidates in b1.
//   cand_hist3 (groups of 64 chunks): picks b2; histogram of the last 10 key bits of the candidates in (b1, b2).
//   cand_mark  (same groups): picks b3, i.e. the threshold key T; keeps every candidate below T and counts the ties
//              (key == T) of its group.
//   tie_fix    (same groups): the ties still needed go to the groups in index order: a group's share follows from
//              the tie counts of the groups before it; it takes them lowest index first. It also adds the groups'
//              final kept counts to their rows.
// Workgroup 0 of a kernel records its pick for the kernels after it; no workgroup waits for another inside a kernel.
#include <algorithm>
#include <cmath>
#include <limits>
#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kChunk = kTopmChunk;        // entries per chunk (inside one row): one wave's unit
constexpr int kU = kChunk / (4 * kWave);  // float4 loads per lane and chunk
constexpr int kBins = 2048;
constexpr int64_t kSampleMax = 65536;      // sampled float4s
constexpr int kSampleTB = 256, kSamplePer = 4;  // sample: threads, float4s per thread
constexpr int kClsTB = 256, kClsPer = 4;   // classify: threads, chunks per wave
constexpr int kH2TB = 1024, kH2G = 256;    // cand_hist2: threads, chunks per workgroup
constexpr int kCandTB = 256, kCandG = kTopmGroup;  // cand_hist3 / cand_mark / tie_fix
static_assert(kCandG <= kWave, "a group's chunk prefix is one wave scan");
static_assert(kH2G <= kH2TB, "one chunk count per thread");

struct State {
  int32_t b1, b2, b3, any;  // any: the threshold key is defined (m > 0)
  uint32_t thr;
  int32_t lo, hi, pad;      // the sampled window of bins
  int64_t need1, need2, need3;
};

struct Ws {
  State* st;
  uint32_t* hist;       // [4][kBins]: exact top bits, candidates' middle bits, last bits, sample
  uint2* cand;          // [nb][kChunk] (key, entry index) per chunk segment, index order
  int32_t* ccnt;        // [nb] candidates per chunk
  int32_t* kept;        // [nb] entries kept per chunk
  uint32_t* tie_cnt;    // [groups of kCandG chunks]
  int32_t* group_kept;  // [groups]
};

// A larger score has a smaller key. Adding +0 turns -0 into +0 (round to nearest), so the two zeros tie; then a
// negative score keeps its bits and a positive one has its 31 low bits flipped.
__device__ __forceinline__ uint32_t desc_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ (~uint32_t(int32_t(u) >> 31) & 0x7FFFFFFFu);
}
struct Chunk {
  int64_t beg, end, row;
};

__device__ __forceinline__ Chunk chunk_of(int64_t b, int32_t row_len) {
  const int64_t per_row = (int64_t(row_len) + kChunk - 1) / kChunk;
  Chunk r;
  r.row = b / per_row;
  const int64_t c = b - r.row * per_row;
  r.beg = r.row * row_len + c * kChunk;
  r.end = r.row * row_len + min((c + 1) * kChunk, int64_t(row_len));
  return r;
}

// A chunk's scores, read by one wave: lane l, slice u holds entries r.beg + 4 (l + 64 u) .. + 3. Every float4 load
// is issued unconditionally at an address clamped into the chunk's last whole float4 (the rows of a chunk are
// 16-byte aligned); only a chunk whose end is not a multiple of 4 (the last one of a ragged kvc_topk input) re-reads
// its last entries one by one. Entries at or past the end are never counted. With beta as input, the log-retention
// is computed in place.
template <bool kBeta>
__device__ __forceinline__ void load_chunk(const TopmInput& in, const Chunk& r, int lane, float4 (&v)[kU]) {
  const float* src = kBeta ? in.beta : in.scores;
  const int64_t last4 = (r.end & ~int64_t(3)) - 4;  // start of the chunk's last whole float4
  if (last4 >= r.beg) {  // uniform: a chunk of fewer than 4 entries is read one by one below
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = r.beg + 4 * (lane + kWave * u);
      v[u] = *reinterpret_cast<const float4*>(src + min(e, last4));
    }
  } else {
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  if ((r.end & 3) != 0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = r.beg + 4 * (lane + kWave * u);
      if (e < r.end && e + 4 > r.end) {
        v[u].x = src[e];
        v[u].y = e + 1 < r.end ? src[e + 1] : 0.0f;
        v[u].z = e + 2 < r.end ? src[e + 2] : 0.0f;
        v[u].w = 0.0f;
      }
    }
  }
  if (kBeta) {  // DBTrimKV log-retention, as kvc_score(KVC_SCORE_RETENTION) computes it
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = int(r.beg - r.row * in.row_len) + 4 * (lane + kWave * u);
      v[u].x = float(in.t - i) * logf(v[u].x);
      v[u].y = float(in.t - i - 1) * logf(v[u].y);
      v[u].z = float(in.t - i - 2) * logf(v[u].z);
      v[u].w = float(in.t - i - 3) * logf(v[u].w);
    }
  }
}

// x OR-ed with the x of the lane that DPP control kCtrl names (all source lanes lie inside the wave here)
template <int kCtrl>
__device__ __forceinline__ uint32_t or_dpp(uint32_t x) {
  return x | uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kCtrl, 0xF, 0xF, false));
}

template <class V, int TB>
__device__ V block_excl_scan(V v, V* wsum, V* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  V inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const V o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  V base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TB / kWave; ++w) {
    base += w < wave ? wsum[w] : V(0);
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// block sum (every thread gets it); two barriers
template <class V, int TB>
__device__ V block_sum(V v, V* wsum) {
  V tot;
  (void)block_excl_scan<V, TB>(v, wsum, &tot);
  return tot;
}

// The bin of global histogram h (nbins = 1024 or 2048) holding the need-th key, and how many keys of that bin are
// needed: pk = {bin, need} ({-1, 0} when need <= 0). Wave 0 alone: lane l owns bins [l * nbins / 64,
// (l + 1) * nbins / 64); the caller publishes pk with a barrier.
__device__ void wave_pick(const uint32_t* h, int nbins, int64_t need, long long* pk) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int per = nbins / kWave;  // 16 or 32
  uint32_t c[32];
  const uint4* hp = reinterpret_cast<const uint4*>(h + lane * per);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 x = q < per / 4 ? hp[q] : make_uint4(0u, 0u, 0u, 0u);
    c[4 * q] = x.x;
    c[4 * q + 1] = x.y;
    c[4 * q + 2] = x.z;
    c[4 * q + 3] = x.w;
  }
  long long own = 0;
#pragma unroll
  for (int k = 0; k < 32; ++k) own += c[k];
  long long inc = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const long long o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  const long long excl = inc - own;
  if (lane == 0) {
    pk[0] = -1;
    pk[1] = 0;
  }
  if (need > 0 && excl < need && need <= inc) {
    long long rem = need - excl;
    int b = 0;
    while (b < per - 1 && rem > (long long)c[b]) rem -= c[b++];
    pk[0] = lane * per + b;
    pk[1] = rem;
  }
}

// Bins of global histogram h holding its lo_pos-th and hi_pos-th keys (1-based): pk[0] = 0 when lo_pos < 1, pk[1] =
// kBins - 1 when hi_pos exceeds the histogram's total. Wave 0 alone; the caller publishes pk with a barrier.
__device__ void wave_locate(const uint32_t* h, int64_t lo_pos, int64_t hi_pos, long long* pk) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  constexpr int per = kBins / kWave;
  uint32_t c[per];
  const uint4* hp = reinterpret_cast<const uint4*>(h + lane * per);
#pragma unroll
  for (int q = 0; q < per / 4; ++q) {
    const uint4 x = hp[q];
    c[4 * q] = x.x;
    c[4 * q + 1] = x.y;
    c[4 * q + 2] = x.z;
    c[4 * q + 3] = x.w;
  }
  long long own = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) own += c[k];
  long long inc = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const long long o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  const long long excl = inc - own;
  if (lane == 0) {
    pk[0] = 0;
    pk[1] = kBins - 1;
  }
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const int64_t pos = which == 0 ? lo_pos : hi_pos;
    if (pos >= 1 && excl < pos && pos <= inc) {
      long long rem = pos - excl;
      int b = 0;
      while (b < per - 1 && rem > (long long)c[b]) rem -= c[b++];
      pk[which] = lane * per + b;
    }
  }
}

// Candidates of the chunks b0 .. b0 + g - 1 as one index-ordered sequence: pref[k] = candidates of the group's chunks
// before chunk k (pref[g] = all). Wave 0 alone; the caller publishes pref with a barrier.
__device__ void group_prefix(const Ws& ws, int64_t b0, int g, int* pref) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int c = lane < g ? ws.ccnt[b0 + lane] : 0;
  int inc = c;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == 0) pref[0] = 0;
  if (lane < g) pref[lane + 1] = inc;
}

// The same for up to TB chunks with the whole workgroup (contains barriers; every thread calls it).
template <int TB>
__device__ void group_prefix_block(const Ws& ws, int64_t b0, int g, int* pref, int* wsum) {
  const int c = int(threadIdx.x) < g ? ws.ccnt[b0 + threadIdx.x] : 0;
  int total;
  const int ex = block_excl_scan<int, TB>(c, wsum, &total);
  if (int(threadIdx.x) < g) pref[threadIdx.x] = ex;
  if (threadIdx.x == 0) pref[g] = total;
  __syncthreads();
}

// chunk k of the group holding the j-th candidate of the sequence: the last k with pref[k] <= j (G = 16 or 64)
template <int G>
__device__ __forceinline__ int chunk_in_group(const int* pref, int g, int j) {
  int lo = 0;
#pragma unroll
  for (int step = G / 2; step >= 1; step >>= 1) {
    if (lo + step < g && pref[lo + step] <= j) lo += step;
  }
  return lo;
}

__device__ __forceinline__ const uint2* seg_of(const Ws& ws, int64_t b) { return ws.cand + size_t(b) * kChunk; }

// set bits of the wave ballot m in the lanes below this one
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

// Adds the kept counts of the chunks b0 .. b0 + g - 1 (thread t < g holds chunk b0 + t's, g <= G) to their rows:
// one global atomic per distinct row, summed in LDS first (slot = row - row of b0; g chunks span at most g rows).
// Every thread calls it (two barriers); rc holds G ints.
template <int G>
__device__ void add_row_counts(int32_t* row_counts, int64_t b0, int g, int cnt, int32_t row_len, int* rc) {
  if (threadIdx.x < G) rc[threadIdx.x] = 0;
  __syncthreads();
  const int64_t per_row = (int64_t(row_len) + kChunk - 1) / kChunk;
  const int64_t row0 = b0 / per_row;
  if (int(threadIdx.x) < g && cnt > 0) atomicAdd(&rc[int((b0 + threadIdx.x) / per_row - row0)], cnt);
  __syncthreads();
  if (threadIdx.x < G && rc[threadIdx.x] > 0) atomicAdd(&row_counts[row0 + threadIdx.x], rc[threadIdx.x]);
}

__global__ __launch_bounds__(256) void eng_clear(Ws ws, int32_t* row_counts, int64_t n_rows, int32_t* status) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < 4 * kBins) ws.hist[i] = 0u;
  if (i < int64_t(sizeof(State) / sizeof(uint32_t))) reinterpret_cast<uint32_t*>(ws.st)[i] = 0u;
  if (row_counts != nullptr && i < n_rows) row_counts[i] = 0;
  if (status != nullptr && i == 0) *status = 0;
}

// One float4 per stratum: stratum j of S covers float4s [j n4 / S, (j + 1) n4 / S); the float4 taken is at the
// fraction (hash(j) mod 2^16) / 2^16 of it (hash(j) = 40503 j + 17).
template <bool kBeta>
__global__ __launch_bounds__(kSampleTB) void eng_sample(TopmInput in, Ws ws, int64_t S) {
  __shared__ uint32_t h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kSampleTB) h[i] = 0u;
  const int64_t n4 = in.n / 4;
  const float* src = kBeta ? in.beta : in.scores;
  float4 x[kSamplePer];
  int64_t e[kSamplePer];
#pragma unroll
  for (int q = 0; q < kSamplePer; ++q) {  // every load first
    const int64_t j = (int64_t(blockIdx.x) * kSamplePer + q) * kSampleTB + threadIdx.x;
    e[q] = -1;
    if (j < S) {
      const int64_t jit = (j * 40503 + 17) & 0xFFFF;
      e[q] = 4 * (((j * 65536 + jit) * n4) / (S * 65536));  // e + 3 < n
      x[q] = *reinterpret_cast<const float4*>(src + e[q]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSamplePer; ++q) {
    if (e[q] < 0) continue;
    float4 y = x[q];
    if (kBeta) {
      const int i = int(e[q] % in.row_len);  // the 4 entries lie in one row (row_len % 16 == 0)
      y.x = float(in.t - i) * logf(y.x);
      y.y = float(in.t - i - 1) * logf(y.y);
      y.z = float(in.t - i - 2) * logf(y.z);
      y.w = float(in.t - i - 3) * logf(y.w);
    }
    atomicAdd(&h[desc_key(y.x) >> 21], 1u);
    atomicAdd(&h[desc_key(y.y) >> 21], 1u);
    atomicAdd(&h[desc_key(y.z) >> 21], 1u);
    atomicAdd(&h[desc_key(y.w) >> 21], 1u);
  }
  __syncthreads();
  for (int bin = threadIdx.x; bin < kBins; bin += kSampleTB) {
    if (h[bin] != 0u) atomicAdd(&ws.hist[3 * kBins + bin], h[bin]);
  }
}

// One wave classifies chunks b, b + stride, ... (at most kPer of them, below nb) against the bins [lo, hi]: entries
// below lo are kept, entries of lo .. hi go to their chunk's candidate segment in index order, and with kHist the
// exact histogram of the top 11 key bits is built in h (LDS) on the way. kBits: the keep mask as bits (one row:
// chunk starts are multiples of 2048), else as bytes; kBeta: scores computed from beta. v holds chunk b's scores,
// loaded by the caller (so that they are in flight during its setup); kPrefetch: the next chunk's loads are issued
// before the current one is classified (32 more VGPRs). Returns whether a NaN score was seen.
template <bool kBits, bool kBeta, bool kHist, bool kPrefetch, int kPer>
__device__ bool classify_chunks(const TopmInput& in, const Ws& ws, int64_t nb, int64_t b, int stride, int lo, int hi,
                                uint8_t* __restrict__ keep, uint32_t* __restrict__ keep_bits, uint32_t* h,
                                float4 (&v)[kU]) {
  const int lane = threadIdx.x & (kWave - 1);
  float4 vn[kU];
  bool nan = false;
  for (int i = 0; i < kPer && b < nb; ++i, b += stride) {  // wave-uniform; no barrier below
    if (kPrefetch && i + 1 < kPer && b + stride < nb) load_chunk<kBeta>(in, chunk_of(b + stride, in.row_len), lane, vn);
    if (!kPrefetch && i > 0) load_chunk<kBeta>(in, chunk_of(b, in.row_len), lane, v);
    const Chunk r = chunk_of(b, in.row_len);
    uint2* seg = ws.cand + size_t(b) * kChunk;
    int base = 0, kept = 0;  // wave-uniform: candidates written so far, entries kept
    // one slice of 256 entries; kFull: the chunk has all 2048 (no entry past its end)
    auto slice = [&](auto full, int u) {
      constexpr bool kFull = decltype(full)::value;
      const int64_t e = r.beg + 4 * (lane + kWave * u);
      const float vs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      nan |= __builtin_isunordered(vs[0], vs[1]) || __builtin_isunordered(vs[2], vs[3]);
      bool k1[4], cd[4];
      unsigned long long K[4], C[4];  // ballots: entry c of every lane kept / a candidate
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool valid = kFull || e + c < r.end;
        const int d = int(desc_key(vs[c]) >> 21);
        if (kHist && valid) atomicAdd(&h[d], 1u);
        k1[c] = valid && d < lo;
        cd[c] = valid && uint32_t(d - lo) <= uint32_t(hi - lo);
        K[c] = __ballot(k1[c]);
        C[c] = __ballot(cd[c]);
      }
      kept += __popcll(K[0]) + __popcll(K[1]) + __popcll(K[2]) + __popcll(K[3]);
      if (kBits) {
        // bit 4 i + c of the word of lanes 8 q .. 8 q + 7 is entry c of lane 8 q + i: each lane puts its four bits in
        // place and the eight lanes' values are OR-ed (neighbours, then pairs, then the mirrored half of 8 lanes)
        const uint32_t nib = (k1[0] ? 1u : 0u) | (k1[1] ? 2u : 0u) | (k1[2] ? 4u : 0u) | (k1[3] ? 8u : 0u);
        uint32_t x = nib << (4 * (lane & 7));
        x = or_dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
        x = or_dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
        x = or_dpp<0x141>(x);  // row_half_mirror
        if ((lane & 7) == 0) keep_bits[e >> 5] = x;
      } else {
        const uint32_t out = (k1[0] ? 1u : 0u) | (k1[1] ? 0x100u : 0u) | (k1[2] ? 0x10000u : 0u) |
                             (k1[3] ? 0x1000000u : 0u);
        if (kFull || e + 4 <= r.end) {
          *reinterpret_cast<uint32_t*>(keep + e) = out;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (e + c < r.end) keep[e + c] = uint8_t((out >> (8 * c)) & 1u);
          }
        }
      }
      // this slice's candidates in index order (lanes in order, then c), after those of the slices before it
      if ((C[0] | C[1] | C[2] | C[3]) != 0ull) {  // wave-uniform
        int p = base + lanes_below(C[0]) + lanes_below(C[1]) + lanes_below(C[2]) + lanes_below(C[3]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (cd[c]) seg[p++] = make_uint2(desc_key(vs[c]), uint32_t(e + c));
        }
        base += __popcll(C[0]) + __popcll(C[1]) + __popcll(C[2]) + __popcll(C[3]);
      }
    };
    if (r.end - r.beg == kChunk) {
#pragma unroll
      for (int u = 0; u < kU; ++u) slice(std::true_type(), u);
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) slice(std::false_type(), u);
    }
    if (lane == 0) {
      ws.ccnt[b] = base;
      ws.kept[b] = kept;
    }
    if (kPrefetch) {
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = vn[u];
    }
  }
  return nan;
}

// The first classification, against the window [lo, hi] of bins that the sample locates around the m-th key,
// building the exact histogram on the way. Four waves per SIMD (at most 128 VGPRs), so that the grid is resident
// in one round.
template <bool kBits, bool kBeta>
__global__ __launch_bounds__(kClsTB) __attribute__((amdgpu_waves_per_eu(4))) void eng_classify(
    TopmInput in, Ws ws, int64_t nb, int64_t lo_pos, int64_t hi_pos, uint8_t* __restrict__ keep,
    uint32_t* __restrict__ keep_bits, int32_t* status) {
  constexpr int W = kClsTB / kWave, kSpan = W * kClsPer;
  __shared__ long long pk[2];
  __shared__ uint32_t h[kBins];
  // the chunk index as a scalar (not for the byte-mask, score-input case, which then spills and measured slower)
  const int wave = (kBits || kBeta) ? __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)) : int(threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b = int64_t(blockIdx.x) * kSpan + wave;
  float4 v[kU];
  if (b < nb) load_chunk<kBeta>(in, chunk_of(b, in.row_len), lane, v);  // the first chunk's loads first
  for (int i = threadIdx.x; i < kBins; i += kClsTB) h[i] = 0u;
  wave_locate(ws.hist + 3 * kBins, lo_pos, hi_pos, pk);
  __syncthreads();
  const int lo = int(pk[0]), hi = int(pk[1]);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.st->lo = lo;
    ws.st->hi = hi;
  }
  const bool nan = classify_chunks<kBits, kBeta, true, true, kClsPer>(in, ws, nb, b, W, lo, hi, keep, keep_bits, h, v);
  if (nan) atomicOr(status, KVC_DEV_NAN_SCORE);
  __syncthreads();
  for (int bin = threadIdx.x; bin < kBins; bin += kClsTB) {
    if (h[bin] != 0u) atomicAdd(&ws.hist[bin], h[bin]);
  }
}

// picks b1; if the sampled window missed it (rare), classifies this workgroup's chunks again against [b1, b1]
// (rewriting their mask, candidates and counts); then the histogram of key bits 20..10 of the candidates in b1
template <bool kBits, bool kBeta>
__global__ __launch_bounds__(kH2TB) void eng_cand_hist2(TopmInput in, Ws ws, int64_t nb, int64_t m,
                                                        uint8_t* __restrict__ keep, uint32_t* __restrict__ keep_bits) {
  __shared__ uint32_t h[kBins];
  __shared__ int pref[kH2G + 1];
  __shared__ int wsum[kH2TB / kWave];
  __shared__ long long pk[2];
  for (int i = threadIdx.x; i < kBins; i += kH2TB) h[i] = 0u;
  const int64_t b0 = int64_t(blockIdx.x) * kH2G;
  const int g = int(min(int64_t(kH2G), nb - b0));
  wave_pick(ws.hist, kBins, m, pk);  // the exact b1 (wave 0, published by the barriers below)
  group_prefix_block<kH2TB>(ws, b0, g, pref, wsum);
  const int b1 = int(pk[0]);
  const int slo = ws.st->lo, shi = ws.st->hi;
  if (!((b1 < 0 && slo == 0) || (slo <= b1 && b1 <= shi))) {  // uniform: the window did not hold b1
    constexpr int W = kH2TB / kWave;  // 16 waves of kH2G / W chunks each
    const int lane = threadIdx.x & (kWave - 1);
    const int w = (kBits || kBeta) ? __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)) : int(threadIdx.x >> 6);
    const int64_t b = b0 + w;  // as in eng_classify
    float4 v[kU];
    if (b < nb) load_chunk<kBeta>(in, chunk_of(b, in.row_len), lane, v);
    (void)classify_chunks<kBits, kBeta, false, false, kH2G / W>(in, ws, nb, b, W, b1, b1, keep, keep_bits, nullptr, v);
    __threadfence_block();  // the rewritten counts and candidates, read below by the workgroup's other waves
    __syncthreads();
    group_prefix_block<kH2TB>(ws, b0, g, pref, wsum);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.st->b1 = b1;
    ws.st->need1 = pk[1];
  }
  const int total = pref[g];
  constexpr int kUn = 4;
  for (int j0 = threadIdx.x; j0 < total; j0 += kH2TB * kUn) {
    uint32_t key[kUn];
#pragma unroll
    for (int q = 0; q < kUn; ++q) {
      const int j = j0 + q * kH2TB;
      key[q] = 0u;
      if (j < total) {
        const int k = chunk_in_group<kH2G>(pref, g, j);
        key[q] = seg_of(ws, b0 + k)[j - pref[k]].x;
      }
    }
#pragma unroll
    for (int q = 0; q < kUn; ++q) {
      if (j0 + q * kH2TB < total && int(key[q] >> 21) == b1) atomicAdd(&h[(key[q] >> 10) & 0x7FFu], 1u);
    }
  }
  __syncthreads();
  for (int bin = threadIdx.x; bin < kBins; bin += kH2TB) {
    if (h[bin] != 0u) atomicAdd(&ws.hist[kBins + bin], h[bin]);
  }
}

// picks b2; histogram of the last 10 key bits of the candidates in (b1, b2)
__global__ __launch_bounds__(kCandTB) void eng_cand_hist3(Ws ws, int64_t nb) {
  __shared__ uint32_t h3[1024];
  __shared__ int pref[kCandG + 1];
  __shared__ long long pk[2];
  for (int i = threadIdx.x; i < 1024; i += kCandTB) h3[i] = 0u;
  const int64_t b0 = int64_t(blockIdx.x) * kCandG;
  const int g = int(min(int64_t(kCandG), nb - b0));
  group_prefix(ws, b0, g, pref);
  wave_pick(ws.hist + kBins, kBins, ws.st->need1, pk);
  __syncthreads();
  const int b2 = int(pk[0]);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.st->b2 = b2;
    ws.st->need2 = pk[1];
  }
  const int b1 = ws.st->b1;
  const int total = (b1 >= 0 && b2 >= 0) ? pref[g] : 0;
  const uint32_t top = (uint32_t(b1) << 11) | uint32_t(b2);  // key bits 31..10 of the candidates counted
  constexpr int kUn = 4;  // loads in flight per thread
  for (int j0 = threadIdx.x; j0 < total; j0 += kCandTB * kUn) {
    uint32_t key[kUn];
#pragma unroll
    for (int q = 0; q < kUn; ++q) {
      const int j = j0 + q * kCandTB;
      key[q] = 0xFFFFFFFFu;
      if (j < total) {
        const int k = chunk_in_group<kCandG>(pref, g, j);
        key[q] = seg_of(ws, b0 + k)[j - pref[k]].x;
      }
    }
#pragma unroll
    for (int q = 0; q < kUn; ++q) {
      if (j0 + q * kCandTB < total && (key[q] >> 10) == top) atomicAdd(&h3[key[q] & 0x3FFu], 1u);
    }
  }
  __syncthreads();
  for (int bin = threadIdx.x; bin < 1024; bin += kCandTB) {
    if (h3[bin] != 0u) atomicAdd(&ws.hist[2 * kBins + bin], h3[bin]);
  }
}

template <bool kBits>
__device__ __forceinline__ void mark_kept(uint8_t* keep, uint32_t* keep_bits, uint32_t i) {
  if (kBits) {
    atomicOr(&keep_bits[i >> 5], 1u << (i & 31u));
  } else {
    keep[i] = 1;
  }
}

// picks b3, i.e. the threshold key T; candidates below T are kept, ties (key == T) counted per group
template <bool kBits>
__global__ __launch_bounds__(kCandTB) void eng_cand_mark(Ws ws, int64_t nb, uint8_t* __restrict__ keep,
                                                         uint32_t* __restrict__ keep_bits) {
  __shared__ int pref[kCandG + 1];
  __shared__ int kc[kCandG];
  __shared__ long long pk[2];
  __shared__ int wsum[kCandTB / kWave];
  if (threadIdx.x < kCandG) kc[threadIdx.x] = 0;
  const int64_t b0 = int64_t(blockIdx.x) * kCandG;
  const int g = int(min(int64_t(kCandG), nb - b0));
  group_prefix(ws, b0, g, pref);
  const int b1 = ws.st->b1, b2 = ws.st->b2;
  wave_pick(ws.hist + 2 * kBins, 1024, ws.st->need2, pk);
  __syncthreads();
  const int b3 = int(pk[0]);
  const bool any = b1 >= 0 && b2 >= 0 && b3 >= 0;  // otherwise nothing is taken among the candidates
  const uint32_t thr = (uint32_t(max(b1, 0)) << 21) | (uint32_t(max(b2, 0)) << 10) | uint32_t(max(b3, 0));
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.st->b3 = b3;
    ws.st->any = any ? 1 : 0;
    ws.st->thr = thr;
    ws.st->need3 = pk[1];
  }
  const int total = any ? pref[g] : 0;
  int ties = 0;
  constexpr int kUn = 4;  // loads in flight per thread
  for (int j0 = threadIdx.x; j0 < total; j0 += kCandTB * kUn) {
    uint2 cdt[kUn];
    int kk[kUn];
#pragma unroll
    for (int q = 0; q < kUn; ++q) {
      const int j = j0 + q * kCandTB;
      cdt[q] = make_uint2(0xFFFFFFFFu, 0u);
      kk[q] = 0;
      if (j < total) {
        kk[q] = chunk_in_group<kCandG>(pref, g, j);
        cdt[q] = seg_of(ws, b0 + kk[q])[j - pref[kk[q]]];
      }
    }
#pragma unroll
    for (int q = 0; q < kUn; ++q) {
      if (j0 + q * kCandTB >= total) continue;
      if (cdt[q].x < thr) {
        mark_kept<kBits>(keep, keep_bits, cdt[q].y);
        atomicAdd(&kc[kk[q]], 1);
      }
      ties += cdt[q].x == thr ? 1 : 0;
    }
  }
  ties = block_sum<int, kCandTB>(ties, wsum);  // its barriers also complete kc
  if (int(threadIdx.x) < g && kc[threadIdx.x] > 0) ws.kept[b0 + threadIdx.x] += kc[threadIdx.x];
  if (threadIdx.x == 0) ws.tie_cnt[blockIdx.x] = uint32_t(ties);
}

// The ties still needed (need3) go to the groups in order: a group takes min(its ties, need3 - ties of the groups
// before it), lowest index first. Also writes the group's final kept count.
template <bool kBits>
__global__ __launch_bounds__(kCandTB) void eng_tie_fix(Ws ws, int64_t nb, uint8_t* __restrict__ keep,
                                                       uint32_t* __restrict__ keep_bits, int32_t* row_counts,
                                                       int32_t row_len) {
  __shared__ int pref[kCandG + 1];
  __shared__ int kc[kCandG], rc[kCandG];
  __shared__ long long lsum[kCandTB / kWave];
  __shared__ uint32_t usum[kCandTB / kWave];
  __shared__ int isum[kCandTB / kWave];
  if (threadIdx.x < kCandG) kc[threadIdx.x] = 0;
  const int64_t b0 = int64_t(blockIdx.x) * kCandG;
  const int g = int(min(int64_t(kCandG), nb - b0));
  group_prefix(ws, b0, g, pref);
  long long before = 0;
  for (int64_t q = threadIdx.x; q < int64_t(blockIdx.x); q += kCandTB) before += ws.tie_cnt[q];
  before = block_sum<long long, kCandTB>(before, lsum);
  const long long mine = ws.tie_cnt[blockIdx.x];
  const uint32_t take = uint32_t(max(0LL, min(mine, ws.st->need3 - before)));
  if (take != 0u) {
    const uint32_t thr = ws.st->thr;
    const int total = pref[g];
    uint32_t done = 0;
    for (int base = 0; base < total && done < take; base += kCandTB) {
      const int j = base + int(threadIdx.x);
      int k = 0;
      uint2 cdt = make_uint2(0xFFFFFFFFu, 0u);
      if (j < total) {
        k = chunk_in_group<kCandG>(pref, g, j);
        cdt = seg_of(ws, b0 + k)[j - pref[k]];
      }
      const uint32_t t = (j < total && cdt.x == thr) ? 1u : 0u;
      uint32_t tot;
      const uint32_t rank = done + block_excl_scan<uint32_t, kCandTB>(t, usum, &tot);
      if (t && rank < take) {
        mark_kept<kBits>(keep, keep_bits, cdt.y);
        atomicAdd(&kc[k], 1);
      }
      done = min(take, done + tot);
    }
  }
  __syncthreads();
  int kept_k = 0;  // chunk b0 + t's final kept count (t < g)
  if (int(threadIdx.x) < g) {
    const int64_t b = b0 + threadIdx.x;
    const int taken = kc[threadIdx.x];
    kept_k = ws.kept[b] + taken;
    if (taken > 0) ws.kept[b] = kept_k;
  }
  const int group_total = block_sum<int, kCandTB>(kept_k, isum);
  if (threadIdx.x == 0) ws.group_kept[blockIdx.x] = group_total;
  if (row_counts != nullptr) add_row_counts<kCandG>(row_counts, b0, g, kept_k, row_len, rc);
}

size_t al(size_t x) { return align_up(x, 256); }

struct Layout {
  int64_t nb, groups;
  size_t st, hist, cand, ccnt, kept, tie_cnt, group_kept, total;
};

Layout layout(int64_t n, int32_t row_len) {
  Layout L;
  L.nb = topm_chunks(n, row_len);
  L.groups = (L.nb + kCandG - 1) / kCandG;
  const size_t nb = size_t(std::max<int64_t>(L.nb, 1)), ng = size_t(std::max<int64_t>(L.groups, 1));
  size_t o = 0;
  L.st = o;
  o += al(sizeof(State));
  L.hist = o;
  o += al(size_t(4) * kBins * 4);
  L.cand = o;
  o += al(nb * kChunk * sizeof(uint2));
  L.ccnt = o;
  o += al(nb * 4);
  L.kept = o;
  o += al(nb * 4);
  L.tie_cnt = o;
  o += al(ng * 4);
  L.group_kept = o;
  o += al(ng * 4);
  L.total = o;
  return L;
}

template <bool kBits, bool kBeta>
void launch_passes(const TopmInput& in, int64_t m, const TopmOutput& out, const Ws& ws, const Layout& L,
                   hipStream_t s) {
  const int64_t nb = L.nb;
  // the sample and the window around the m-th key's expected place in it: six standard deviations of a binomial
  // count plus four, so that a miss (handled by the fallback pass) is rare
  const int64_t S = std::min<int64_t>(kSampleMax, in.n / 4);
  int64_t lo_pos = 0, hi_pos = std::numeric_limits<int64_t>::max();
  if (S > 0) {
    const double st = 4.0 * double(S), q = double(m) / double(in.n);
    const double c = q * st, d = 6.0 * std::sqrt(st * q * (1.0 - q)) + 4.0;
    lo_pos = int64_t(std::floor(c - d));
    hi_pos = int64_t(std::ceil(c + d));
    constexpr int64_t per_wg = int64_t(kSampleTB) * kSamplePer;
    hipLaunchKernelGGL(eng_sample<kBeta>, dim3(unsigned((S + per_wg - 1) / per_wg)), dim3(kSampleTB), 0, s, in, ws, S);
  }
  constexpr int64_t spec_span = int64_t(kClsTB / kWave) * kClsPer;
  hipLaunchKernelGGL((eng_classify<kBits, kBeta>), dim3(unsigned((nb + spec_span - 1) / spec_span)), dim3(kClsTB), 0,
                     s, in, ws, nb, lo_pos, hi_pos, out.keep, out.keep_bits, out.status);
  hipLaunchKernelGGL((eng_cand_hist2<kBits, kBeta>), dim3(unsigned((nb + kH2G - 1) / kH2G)), dim3(kH2TB), 0, s, in,
                     ws, nb, m, out.keep, out.keep_bits);
  const unsigned ng = unsigned(L.groups);
  hipLaunchKernelGGL(eng_cand_hist3, dim3(ng), dim3(kCandTB), 0, s, ws, nb);
  hipLaunchKernelGGL(eng_cand_mark<kBits>, dim3(ng), dim3(kCandTB), 0, s, ws, nb, out.keep, out.keep_bits);
  hipLaunchKernelGGL(eng_tie_fix<kBits>, dim3(ng), dim3(kCandTB), 0, s, ws, nb, out.keep, out.keep_bits,
                     out.row_counts, in.row_len);
}

}  // namespace

int64_t topm_chunks(int64_t n, int32_t row_len) {
  if (n <= 0 || row_len <= 0) return 0;
  return (n / row_len) * ((int64_t(row_len) + kChunk - 1) / kChunk);
}

size_t topm_engine_workspace(int64_t n, int32_t row_len) { return layout(n, row_len).total; }

hipError_t launch_topm_engine(const TopmInput& in, int64_t m, const TopmOutput& out, void* ws_ptr, hipStream_t s,
                              TopmCounts* counts) {
  if ((out.keep == nullptr) == (out.keep_bits == nullptr)) return hipErrorInvalidValue;
  if (out.keep_bits != nullptr && int64_t(in.row_len) != in.n) return hipErrorInvalidValue;  // bits: one row only
  const Layout L = layout(in.n, in.row_len);
  char* w = static_cast<char*>(ws_ptr);
  Ws ws;
  ws.st = reinterpret_cast<State*>(w + L.st);
  ws.hist = reinterpret_cast<uint32_t*>(w + L.hist);
  ws.cand = reinterpret_cast<uint2*>(w + L.cand);
  ws.ccnt = reinterpret_cast<int32_t*>(w + L.ccnt);
  ws.kept = reinterpret_cast<int32_t*>(w + L.kept);
  ws.tie_cnt = reinterpret_cast<uint32_t*>(w + L.tie_cnt);
  ws.group_kept = reinterpret_cast<int32_t*>(w + L.group_kept);
  if (counts != nullptr) {
    counts->chunk_kept = ws.kept;
    counts->group_kept = ws.group_kept;
  }
  const int64_t n_rows = in.row_len > 0 ? in.n / in.row_len : 0;
  const int64_t clear_n = std::max<int64_t>(4 * kBins, out.row_counts != nullptr ? n_rows : 0);
  hipLaunchKernelGGL(eng_clear, dim3(unsigned((clear_n + 255) / 256)), dim3(256), 0, s, ws, out.row_counts, n_rows,
                     out.clear_status ? out.status : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L.nb == 0) return e;
  if (out.keep_bits != nullptr) {
    if (in.scores != nullptr) {
      launch_passes<true, false>(in, m, out, ws, L, s);
    } else {
      return hipErrorInvalidValue;  // the bit mask serves kvc_topk, which reads scores
    }
  } else if (in.scores != nullptr) {
    launch_passes<false, false>(in, m, out, ws, L, s);
  } else {
    launch_passes<false, true>(in, m, out, ws, L, s);
  }
  return hipGetLastError();
}

}  // namespace kvc
