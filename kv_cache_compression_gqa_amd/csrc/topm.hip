// Global top-M engine: the first m entries of n scores in the order (score desc, index asc), as a keep mask (the
// budgeted selection of the DBTrimKV page, "Metodologia", section 3: every entry of every layer and head competes
// for one global budget; also the generic top-k). Rows of row_len entries only matter for the per-row counts.
//
// Keys are the inverted order-preserving images of the scores (a smaller key is a larger score; +0 == -0). The
// scores are read from memory or computed on the fly as DBTrimKV's log-retention (t - i) * logf(beta) (the
// retention score of section 2; computing it where it is used saves writing and re-reading it). Passes over the
// whole input: two; everything after them touches only the entries of one histogram bin.
//   hist1     (chunks of 8192 entries, four per workgroup): 2048-bin histogram of the top 11 key bits (LDS per
//             wave, one global atomic per non-empty bin).
//   classify  (one workgroup per chunk): picks the bin b1 holding the m-th key from the histogram (every workgroup
//             takes the same decision from the same counts), writes the keep mask (1 below b1), and compacts the
//             entries of b1 into the chunk's candidate segment in index order, with a histogram of their next 11
//             bits. Kept entries are counted per chunk and per row.
//   cand_hist3 (per chunk, candidates only): picks b2, histogram of the last 10 bits of the candidates in b2.
//   cand_mark (per chunk, candidates only): picks b3 (threshold key T), keeps every candidate below T and counts the
//             ties (key == T) per chunk.
//   tie_scan  (one workgroup): how many ties each chunk takes, in chunk order, so that ties are taken lowest index
//             first; tie_fix then takes them.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kTB = 256;
constexpr int kChunk = kTopmChunk;             // entries per chunk (inside one row)
constexpr int kU = kChunk / (4 * kTB);         // float4 loads per thread and chunk
constexpr int kBins = 2048;
constexpr int kHistGroup = 4;                  // chunks per histogram workgroup

struct State {
  int32_t b1, b2, b3, pad;
  uint32_t thr;
  uint32_t pad2;
  int64_t need1, need2, need3;
};

struct Ws {
  State* st;
  uint32_t* hist;      // [3][kBins]
  uint2* cand;         // [nb][kChunk] (key, entry index) per chunk segment, index order
  int32_t* ccnt;       // [nb] candidates per chunk
  int32_t* kept;       // [nb] entries kept per chunk
  uint32_t* tie_cnt;   // [nb]
  uint32_t* tie_take;  // [nb]
};

__device__ __forceinline__ uint32_t desc_key(float s) {
  const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
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

// A chunk's scores: thread t, slice u holds entries r.beg + 4 (t + 256 u) .. + 3. Every float4 load is issued
// unconditionally at an address clamped into the chunk's last whole float4 (the rows of a chunk are 16-byte
// aligned); only a chunk whose end is not a multiple of 4 (the last one of a ragged kvc_topk input) re-reads its
// last entries one by one. Entries at or past the end are never counted. With beta as input, the log-retention is
// computed in place.
__device__ __forceinline__ void load_chunk(const TopmInput& in, const Chunk& r, float4 (&v)[kU]) {
  const float* src = in.scores != nullptr ? in.scores : in.beta;
  const int64_t last4 = (r.end & ~int64_t(3)) - 4;  // start of the chunk's last whole float4
  if (last4 >= r.beg) {  // uniform: a chunk of fewer than 4 entries is read one by one below
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = r.beg + 4 * (threadIdx.x + kTB * u);
      v[u] = *reinterpret_cast<const float4*>(src + min(e, last4));
    }
  } else {
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  if ((r.end & 3) != 0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = r.beg + 4 * (threadIdx.x + kTB * u);
      if (e < r.end && e + 4 > r.end) {
        v[u].x = src[e];
        v[u].y = e + 1 < r.end ? src[e + 1] : 0.0f;
        v[u].z = e + 2 < r.end ? src[e + 2] : 0.0f;
        v[u].w = 0.0f;
      }
    }
  }
  if (in.scores == nullptr) {  // DBTrimKV log-retention, as kvc_score(KVC_SCORE_RETENTION) computes it
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = int(r.beg - r.row * in.row_len) + 4 * (threadIdx.x + kTB * u);
      v[u].x = float(in.t - i) * logf(v[u].x);
      v[u].y = float(in.t - i - 1) * logf(v[u].y);
      v[u].z = float(in.t - i - 2) * logf(v[u].z);
      v[u].w = float(in.t - i - 3) * logf(v[u].w);
    }
  }
}

template <class V>
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
  for (int w = 0; w < kTB / kWave; ++w) {
    base += w < wave ? wsum[w] : V(0);
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// The bin of histogram h (nbins = 1024 or 2048) holding the need-th key, and how many keys of that bin are needed:
// pk = {bin, need} ({-1, 0} when need <= 0). Wave 0 alone: lane l owns bins [l * nbins / 64, (l + 1) * nbins / 64);
// the caller publishes pk with a barrier.
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

// Exclusive scan (thread order) of four 16-bit fields packed in a u64 (every field's block total < 65536), and the
// block totals. Contains one barrier; sm must hold kTB / kWave entries and is not reused by the caller.
__device__ __forceinline__ unsigned long long scan_fields(unsigned long long v, unsigned long long* sm,
                                                          unsigned long long& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  unsigned long long inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const unsigned long long o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) sm[wave] = inc;
  __syncthreads();
  unsigned long long base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTB / kWave; ++w) {
    base += w < wave ? sm[w] : 0ull;
    tot += sm[w];
  }
  total = tot;
  return base + inc - v;
}

__global__ __launch_bounds__(kTB) void eng_clear(Ws ws, int32_t* row_counts, int64_t n_rows) {
  const int64_t i = int64_t(blockIdx.x) * kTB + threadIdx.x;
  if (i < 3 * kBins) ws.hist[i] = 0u;
  if (row_counts != nullptr && i < n_rows) row_counts[i] = 0;
}

__global__ __launch_bounds__(kTB) void eng_hist1(TopmInput in, Ws ws, int64_t nb) {
  __shared__ uint32_t h[kTB / kWave][kBins];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < (kTB / kWave) * kBins; i += kTB) (&h[0][0])[i] = 0u;
  __syncthreads();
  const int64_t b0 = int64_t(blockIdx.x) * kHistGroup;
  const int nc = int(min(int64_t(kHistGroup), nb - b0));
  auto load = [&](int k, float4 (&v)[kU]) { load_chunk(in, chunk_of(b0 + k, in.row_len), v); };
  float4 v[kU], vn[kU];
  load(0, v);
  for (int k = 0; k < nc; ++k) {
    if (k + 1 < nc) load(k + 1, vn);
    const Chunk r = chunk_of(b0 + k, in.row_len);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = r.beg + 4 * (threadIdx.x + kTB * u);
      const float vs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (e + c < r.end) atomicAdd(&h[wave][desc_key(vs[c]) >> 21], 1u);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = vn[u];
  }
  __syncthreads();
  for (int bin = threadIdx.x; bin < kBins; bin += kTB) {
    const uint32_t s = h[0][bin] + h[1][bin] + h[2][bin] + h[3][bin];
    if (s != 0u) atomicAdd(&ws.hist[bin], s);
  }
}

__global__ __launch_bounds__(kTB) void eng_classify(TopmInput in, Ws ws, int64_t m, uint8_t* __restrict__ keep,
                                                    int32_t* row_counts, int32_t* status) {
  __shared__ long long pk[2];
  __shared__ unsigned long long sm[3][kTB / kWave];
  __shared__ uint32_t h2[kBins];
  const Chunk r = chunk_of(blockIdx.x, in.row_len);
  float4 v[kU];
  load_chunk(in, r, v);  // the chunk's loads first
  for (int i = threadIdx.x; i < kBins; i += kTB) h2[i] = 0u;
  wave_pick(ws.hist, kBins, m, pk);
  __syncthreads();
  const int b1 = int(pk[0]);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.st->b1 = b1;
    ws.st->need1 = pk[1];
  }
  uint32_t cand_bits = 0u;
  unsigned long long f0 = 0ull, f1 = 0ull, f2 = 0ull;  // candidates per slice (16-bit fields), kept (f2)
  bool nan = false;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t e = r.beg + 4 * (threadIdx.x + kTB * u);
    const float vs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    uint32_t out = 0u;
    unsigned long long cu = 0ull;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool valid = e + c < r.end;
      const uint32_t key = desc_key(vs[c]);
      nan |= valid && vs[c] != vs[c];
      const int d = int(key >> 21);
      const bool k1 = valid && d < b1;
      const bool cd = valid && d == b1;
      f2 += k1 ? 1ull : 0ull;
      out |= (k1 ? 1u : 0u) << (8 * c);
      cand_bits |= (cd ? 1u : 0u) << (4 * u + c);
      cu += cd ? 1ull : 0ull;
      if (cd) atomicAdd(&h2[(key >> 10) & 0x7FFu], 1u);
    }
    if (u < 4) f0 += cu << (16 * u);
    else f1 += cu << (16 * (u - 4));
    if (e + 4 <= r.end) {
      *reinterpret_cast<uint32_t*>(keep + e) = out;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (e + c < r.end) keep[e + c] = uint8_t((out >> (8 * c)) & 1u);
      }
    }
  }
  if (nan) atomicOr(status, KVC_DEV_NAN_SCORE);
  // candidates in index order: slice u before slice u + 1, threads in order inside a slice (one scan of packed
  // per-slice counts)
  unsigned long long t0, t1, t2;
  const unsigned long long e0 = scan_fields(f0, sm[0], t0);
  const unsigned long long e1 = scan_fields(f1, sm[1], t1);
  (void)scan_fields(f2, sm[2], t2);
  int base = 0;
  uint2* seg = ws.cand + size_t(blockIdx.x) * kChunk;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const unsigned long long ex = u < 4 ? e0 : e1;
    const unsigned long long tt = u < 4 ? t0 : t1;
    const int sh = 16 * (u & 3);
    int p = base + int((ex >> sh) & 0xFFFFull);
    const int64_t e = r.beg + 4 * (threadIdx.x + kTB * u);
    const float vs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((cand_bits >> (4 * u + c)) & 1u) seg[p++] = make_uint2(desc_key(vs[c]), uint32_t(e + c));
    }
    base += int((tt >> sh) & 0xFFFFull);
  }
  const int ktot = int(t2);
  if (threadIdx.x == 0) {
    ws.ccnt[blockIdx.x] = base;
    ws.kept[blockIdx.x] = ktot;
    if (row_counts != nullptr && ktot > 0) atomicAdd(&row_counts[r.row], ktot);
  }
  if (base > 0) {  // h2 complete: the scans' barriers follow every atomic
    for (int bin = threadIdx.x; bin < kBins; bin += kTB) {
      if (h2[bin] != 0u) atomicAdd(&ws.hist[kBins + bin], h2[bin]);
    }
  }
}

// candidates of bin b2 (picked from the second histogram): histogram of their last 10 bits
__global__ __launch_bounds__(kTB) void eng_cand_hist3(Ws ws) {
  __shared__ long long pk[2];
  __shared__ uint32_t h3[1024];
  const int nc = ws.ccnt[blockIdx.x];
  if (nc == 0 && blockIdx.x != 0) return;  // workgroup 0 always records the pick
  const int64_t need1 = ws.st->need1;
  wave_pick(ws.hist + kBins, kBins, need1, pk);
  __syncthreads();
  const int b2 = int(pk[0]);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.st->b2 = b2;
    ws.st->need2 = pk[1];
  }
  if (nc == 0) return;
  for (int i = threadIdx.x; i < 1024; i += kTB) h3[i] = 0u;
  __syncthreads();
  const uint2* seg = ws.cand + size_t(blockIdx.x) * kChunk;
  for (int i = threadIdx.x; i < nc; i += kTB) {
    const uint32_t key = seg[i].x;
    if (int((key >> 10) & 0x7FFu) == b2) atomicAdd(&h3[key & 0x3FFu], 1u);
  }
  __syncthreads();
  for (int bin = threadIdx.x; bin < 1024; bin += kTB) {
    if (h3[bin] != 0u) atomicAdd(&ws.hist[2 * kBins + bin], h3[bin]);
  }
}

// threshold key T from the third histogram; candidates below T kept, ties counted
__global__ __launch_bounds__(kTB) void eng_cand_mark(Ws ws, uint8_t* __restrict__ keep, int32_t* row_counts,
                                                     int32_t row_len) {
  __shared__ long long pk[2];
  __shared__ int red[2][kTB / kWave];
  const int nc = ws.ccnt[blockIdx.x];
  if (nc == 0 && blockIdx.x != 0) {
    if (threadIdx.x == 0) ws.tie_cnt[blockIdx.x] = 0u;
    return;
  }
  const int b1 = ws.st->b1, b2 = ws.st->b2;
  const int64_t need2 = ws.st->need2;
  wave_pick(ws.hist + 2 * kBins, 1024, need2, pk);
  __syncthreads();
  const int b3 = int(pk[0]);
  const uint32_t thr = (uint32_t(b1) << 21) | (uint32_t(b2) << 10) | uint32_t(b3 < 0 ? 0 : b3);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.st->b3 = b3;
    ws.st->thr = thr;
    ws.st->need3 = pk[1];
  }
  const bool any = b1 >= 0 && b2 >= 0 && b3 >= 0;  // otherwise nothing is taken among the candidates
  const uint2* seg = ws.cand + size_t(blockIdx.x) * kChunk;
  int kept = 0, ties = 0;
  for (int i = threadIdx.x; i < nc; i += kTB) {
    const uint2 cdt = seg[i];
    if (any && cdt.x < thr) {
      keep[cdt.y] = 1;
      ++kept;
    }
    ties += (any && cdt.x == thr) ? 1 : 0;
  }
  kept = wave_sum_int(kept);
  ties = wave_sum_int(ties);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[0][threadIdx.x >> 6] = kept;
    red[1][threadIdx.x >> 6] = ties;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int k = 0, t = 0;
    for (int w = 0; w < kTB / kWave; ++w) {
      k += red[0][w];
      t += red[1][w];
    }
    ws.tie_cnt[blockIdx.x] = uint32_t(t);
    if (k > 0) {
      ws.kept[blockIdx.x] += k;
      if (row_counts != nullptr) atomicAdd(&row_counts[chunk_of(blockIdx.x, row_len).row], k);
    }
  }
}

// one workgroup: exclusive scan of the chunks' tie counts -> how many ties each chunk takes
__global__ __launch_bounds__(kTB) void eng_tie_scan(Ws ws, int64_t nb) {
  __shared__ long long wsum[kTB / kWave];
  const int64_t per = (nb + kTB - 1) / kTB;
  const int64_t b0 = min(nb, int64_t(threadIdx.x) * per), b1 = min(nb, b0 + per);
  long long mine = 0;
  for (int64_t b = b0; b < b1; ++b) mine += ws.tie_cnt[b];
  long long total;
  long long off = block_excl_scan<long long>(mine, wsum, &total);
  const long long need = ws.st->need3;
  for (int64_t b = b0; b < b1; ++b) {
    const long long c = ws.tie_cnt[b];
    ws.tie_take[b] = uint32_t(max(0LL, min(c, need - off)));
    off += c;
  }
}

// chunks holding kept ties: take the first tie_take of their ties, in index order (= candidate order)
__global__ __launch_bounds__(kTB) void eng_tie_fix(Ws ws, uint8_t* __restrict__ keep, int32_t* row_counts,
                                                   int32_t row_len) {
  const uint32_t take = ws.tie_take[blockIdx.x];
  if (take == 0u) return;
  __shared__ uint32_t wsum[kTB / kWave];
  const uint32_t thr = ws.st->thr;
  const int nc = ws.ccnt[blockIdx.x];
  const uint2* seg = ws.cand + size_t(blockIdx.x) * kChunk;
  uint32_t done = 0;
  for (int base = 0; base < nc; base += kTB) {
    const int i = base + int(threadIdx.x);
    const uint2 cdt = i < nc ? seg[i] : make_uint2(0xFFFFFFFFu, 0u);
    const uint32_t t = (i < nc && cdt.x == thr) ? 1u : 0u;
    uint32_t tot;
    const uint32_t rank = done + block_excl_scan<uint32_t>(t, wsum, &tot);
    if (t && rank < take) keep[cdt.y] = 1;
    done += tot;
    if (done >= take) break;
  }
  if (threadIdx.x == 0) {
    ws.kept[blockIdx.x] += int(take);
    if (row_counts != nullptr) atomicAdd(&row_counts[chunk_of(blockIdx.x, row_len).row], int(take));
  }
}

size_t al(size_t x) { return align_up(x, 256); }

struct Layout {
  int64_t nb;
  size_t st, hist, cand, ccnt, kept, tie_cnt, tie_take, total;
};

Layout layout(int64_t n, int32_t row_len) {
  Layout L;
  L.nb = topm_chunks(n, row_len);
  const size_t nb = size_t(std::max<int64_t>(L.nb, 1));
  size_t o = 0;
  L.st = o;
  o += al(sizeof(State));
  L.hist = o;
  o += al(3 * kBins * 4);
  L.cand = o;
  o += al(nb * kChunk * sizeof(uint2));
  L.ccnt = o;
  o += al(nb * 4);
  L.kept = o;
  o += al(nb * 4);
  L.tie_cnt = o;
  o += al(nb * 4);
  L.tie_take = o;
  o += al(nb * 4);
  L.total = o;
  return L;
}

}  // namespace

int64_t topm_chunks(int64_t n, int32_t row_len) {
  if (n <= 0 || row_len <= 0) return 0;
  return (n / row_len) * ((int64_t(row_len) + kChunk - 1) / kChunk);
}

size_t topm_engine_workspace(int64_t n, int32_t row_len) { return layout(n, row_len).total; }

hipError_t launch_topm_engine(const TopmInput& in, int64_t m, uint8_t* keep, int32_t* row_counts, int32_t* status,
                              void* ws_ptr, int32_t** chunk_kept, hipStream_t s) {
  const Layout L = layout(in.n, in.row_len);
  char* w = static_cast<char*>(ws_ptr);
  Ws ws;
  ws.st = reinterpret_cast<State*>(w + L.st);
  ws.hist = reinterpret_cast<uint32_t*>(w + L.hist);
  ws.cand = reinterpret_cast<uint2*>(w + L.cand);
  ws.ccnt = reinterpret_cast<int32_t*>(w + L.ccnt);
  ws.kept = reinterpret_cast<int32_t*>(w + L.kept);
  ws.tie_cnt = reinterpret_cast<uint32_t*>(w + L.tie_cnt);
  ws.tie_take = reinterpret_cast<uint32_t*>(w + L.tie_take);
  if (chunk_kept != nullptr) *chunk_kept = ws.kept;
  const int64_t n_rows = in.row_len > 0 ? in.n / in.row_len : 0;
  const int64_t clear_n = std::max<int64_t>(3 * kBins, row_counts != nullptr ? n_rows : 0);
  hipLaunchKernelGGL(eng_clear, dim3(unsigned((clear_n + kTB - 1) / kTB)), dim3(kTB), 0, s, ws, row_counts, n_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L.nb == 0) return e;
  const unsigned nb = unsigned(L.nb);
  hipLaunchKernelGGL(eng_hist1, dim3(unsigned((L.nb + kHistGroup - 1) / kHistGroup)), dim3(kTB), 0, s, in, ws, L.nb);
  hipLaunchKernelGGL(eng_classify, dim3(nb), dim3(kTB), 0, s, in, ws, m, keep, row_counts, status);
  hipLaunchKernelGGL(eng_cand_hist3, dim3(nb), dim3(kTB), 0, s, ws);
  hipLaunchKernelGGL(eng_cand_mark, dim3(nb), dim3(kTB), 0, s, ws, keep, row_counts, in.row_len);
  hipLaunchKernelGGL(eng_tie_scan, dim3(1), dim3(kTB), 0, s, ws, L.nb);
  hipLaunchKernelGGL(eng_tie_fix, dim3(nb), dim3(kTB), 0, s, ws, keep, row_counts, in.row_len);
  return hipGetLastError();
}

}  // namespace kvc
