// DBTrimKV global retention budget: log-retention scores, one global top-M, per-row paged compaction.
//
// What it computes follows the DBTrimKV page ("Make Each Token Count: Towards Improving Long-Context
// Performance with KV Cache Eviction"), "Metodologia: Evicção Baseada em Retenção Global":
//   * section 2: token i's retention weight at step t is beta_i^(t - i). It is ranked through its logarithm
//     (t - i) * ln(beta_i): the map is monotone, and the power itself underflows for most entries at long
//     contexts, which would leave the order to ties;
//   * section 3: every entry of every layer and head competes for one global budget M; the order is
//     (score desc, flat index asc), which makes the kept set unique;
//   * section 4: paged storage where each (layer, head) row keeps a variable-length sequence. The kept positions
//     of a row, ascending, are copied out of place into fresh pages, row after row.
//
// Kernels (all HBM-bound streaming passes, 256 threads, 16-byte vector accesses):
//   retention_score: score = float(t - i) * logf(beta).
//   top-M: a three-pass radix select on the order-preserving 32-bit image of the score (11 + 11 + 10 bits).
//   Each pass streams the scores and builds a 2048-bin histogram of the next digit of the keys that match the
//   prefix chosen so far, in four per-wave LDS copies, merged into global bins with one atomic per non-empty
//   bin. A single workgroup then picks the bin holding the M-th key. The mark pass keeps every key below the
//   threshold and counts the threshold ties per block. A scan of those counts gives each block its share of
//   the ties, which a fix-up pass takes in index order (only blocks with ties do work).
//   compaction: per (row, chunk) counts, one workgroup that scans rows and chunks (lengths, page offsets), an
//   index pass that writes the source pool row of every output row (-1 for the unused rows of a row's last
//   page), and a gather in output order (16 lanes x 16 bytes per 128-element row, eight rows per lane group in
//   flight) that copies each row or writes zeros.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTB = 256;
constexpr int kChunk = 8192;     // entries per top-M block (inside one row)
constexpr int kCChunk = 4096;    // positions per compaction block (inside one row)
constexpr int kBins = 2048;
constexpr int kVecPerThread = kChunk / (4 * kTB);  // float4 loads per thread and top-M block

// ---- retention score ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(kTB) void retention_score_kernel(const float* __restrict__ beta, float* __restrict__ score,
                                                              int64_t n, int32_t n_tokens, int32_t t) {
  const int64_t stride = int64_t(gridDim.x) * kTB * 4;
  for (int64_t e0 = (int64_t(blockIdx.x) * kTB + threadIdx.x) * 4; e0 < n; e0 += stride) {
    const int i = int(e0 % n_tokens);  // n_tokens % 4 == 0: the 4 entries share a row
    const float4 b = *reinterpret_cast<const float4*>(beta + e0);
    float4 s;
    s.x = float(t - i) * logf(b.x);
    s.y = float(t - i - 1) * logf(b.y);
    s.z = float(t - i - 2) * logf(b.z);
    s.w = float(t - i - 3) * logf(b.w);
    *reinterpret_cast<float4*>(score + e0) = s;
  }
}

// ---- global top-M --------------------------------------------------------------------------------------------
struct TopmState {
  uint32_t prefix;  // key bits chosen so far
  uint32_t pad;
  int64_t need;     // entries still to take among the keys that match the prefix
};

struct TopmWs {
  TopmState* state;
  uint32_t* hist;      // [3][kBins]
  uint32_t* tie_cnt;   // [blocks]
  uint32_t* tie_take;  // [blocks]
};

// order-preserving image of a finite score, inverted so that a smaller key is a larger score (+0 == -0)
__device__ __forceinline__ uint32_t desc_key(float s) {
  const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

struct BlockRange {
  int64_t beg, end;
  int64_t row;
};

__device__ __forceinline__ BlockRange block_range(int64_t b, int32_t row_len, int chunk) {
  const int per_row = (row_len + chunk - 1) / chunk;
  BlockRange r;
  r.row = b / per_row;
  const int c = int(b - r.row * per_row);
  r.beg = r.row * row_len + int64_t(c) * chunk;
  r.end = r.row * row_len + min(int64_t(c + 1) * chunk, int64_t(row_len));
  return r;
}

// exclusive prefix (thread order) of one value per thread over a 256-thread block; *total gets the block sum
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

__global__ __launch_bounds__(kTB) void topm_clear(TopmWs ws, int32_t* row_counts, int64_t n_rows) {
  const int64_t i = int64_t(blockIdx.x) * kTB + threadIdx.x;
  if (i < 3 * kBins) ws.hist[i] = 0u;
  if (i < n_rows) row_counts[i] = 0;
}

// digit of a key in pass P, and whether the key matches the prefix chosen by the earlier passes
template <int P>
__device__ __forceinline__ bool digit_of(uint32_t key, uint32_t prefix, uint32_t& bin) {
  if (P == 0) {
    bin = key >> 21;
    return true;
  } else if (P == 1) {
    bin = (key >> 10) & 0x7FFu;
    return (key >> 21) == prefix;
  } else {
    bin = key & 0x3FFu;
    return (key >> 10) == prefix;
  }
}

// A histogram workgroup of pass P takes hist_group(P) consecutive chunks of one row: one LDS clear and one flush
// of the 2048 bins to the global histogram serve all of them (the flush's global atomics land on the same few
// hot bins from every workgroup). Passes 0 and 1 gain; pass 2, with few matching keys, runs one chunk each. The
// next chunk's loads are issued before the current chunk's atomics.
constexpr int hist_group(int P) { return P == 2 ? 1 : 4; }

template <int P>
__global__ __launch_bounds__(kTB) void topm_hist(const float* __restrict__ scores, TopmWs ws, int32_t row_len) {
  __shared__ uint32_t h[4][kBins];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kBins; i += kTB) (&h[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t prefix = P == 0 ? 0u : ws.state->prefix;
  const int per_row = (row_len + kChunk - 1) / kChunk;
  constexpr int kG = hist_group(P);
  const int groups = (per_row + kG - 1) / kG;
  const int64_t row = blockIdx.x / groups;
  const int c0 = int(blockIdx.x - row * groups) * kG;
  const int nc = min(kG, per_row - c0);
  // every load of a chunk in flight at once (clamped into the chunk's range)
  auto load = [&](int c, float4 (&v)[kVecPerThread]) {
    const BlockRange r = block_range(row * per_row + c, row_len, kChunk);
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const int64_t e = min(r.beg + 4 * (threadIdx.x + kTB * u), r.end - 4);
      v[u] = *reinterpret_cast<const float4*>(scores + e);
    }
  };
  float4 v[kVecPerThread], vn[kVecPerThread];
  load(c0, v);
  for (int k = 0; k < nc; ++k) {
    if (k + 1 < nc) load(c0 + k + 1, vn);
    const BlockRange r = block_range(row * per_row + c0 + k, row_len, kChunk);
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      if (r.beg + 4 * (threadIdx.x + kTB * u) >= r.end) break;
      const float vs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t bin;
        if (digit_of<P>(desc_key(vs[c]), prefix, bin)) atomicAdd(&h[wave][bin], 1u);
      }
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) v[u] = vn[u];
  }
  __syncthreads();
  for (int bin = threadIdx.x; bin < kBins; bin += kTB) {
    const uint32_t s = h[0][bin] + h[1][bin] + h[2][bin] + h[3][bin];
    if (s != 0u) atomicAdd(&ws.hist[P * kBins + bin], s);
  }
}

// one workgroup: the bin of pass P that holds the need-th key (1-based) of the current prefix
template <int P>
__global__ __launch_bounds__(kTB) void topm_pick(TopmWs ws, int64_t m) {
  constexpr int nb = P == 2 ? 1024 : kBins;
  constexpr int per = nb / kTB;
  constexpr int bits = P == 2 ? 10 : 11;
  __shared__ long long wsum[kTB / kWave];
  const long long need = P == 0 ? m : ws.state->need;
  const uint32_t prev = P == 0 ? 0u : ws.state->prefix;
  const uint32_t* hp = ws.hist + P * kBins + threadIdx.x * per;
  uint32_t c[per];
  long long mine = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    c[k] = hp[k];
    mine += c[k];
  }
  long long total;
  const long long excl = block_excl_scan<long long>(mine, wsum, &total);
  // the thread whose bins hold the need-th key (need <= 0: nothing to take, bin 0; need > total cannot happen)
  const bool mine_bin = need <= 0 ? threadIdx.x == 0 : (excl < need && excl + mine >= need);
  if (mine_bin) {
    long long rem = need - excl;
    int b = 0;
    while (b < per - 1 && rem > c[b]) rem -= c[b++];
    ws.state->prefix = (prev << bits) | uint32_t(threadIdx.x * per + b);
    ws.state->need = need <= 0 ? 0 : rem;
  }
}

// keep every key below the threshold; count the threshold ties of the block
__global__ __launch_bounds__(kTB) void topm_mark(const float* __restrict__ scores, uint8_t* __restrict__ keep,
                                                 int32_t* row_counts, TopmWs ws, int32_t row_len, int32_t* status) {
  __shared__ uint32_t red[2][kTB / kWave];
  const uint32_t thr = ws.state->prefix;
  const BlockRange r = block_range(blockIdx.x, row_len, kChunk);
  uint32_t kept = 0, ties = 0;
  bool nan = false;
  float4 vv[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int64_t e = min(r.beg + 4 * (threadIdx.x + kTB * u), r.end - 4);
    vv[u] = *reinterpret_cast<const float4*>(scores + e);
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int64_t e = r.beg + 4 * (threadIdx.x + kTB * u);
    if (e >= r.end) break;
    const float4 v = vv[u];
    const float vs[4] = {v.x, v.y, v.z, v.w};
    uint32_t out = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t key = desc_key(vs[c]);
      nan |= vs[c] != vs[c];
      const uint32_t k1 = key < thr ? 1u : 0u;
      kept += k1;
      ties += key == thr ? 1u : 0u;
      out |= k1 << (8 * c);
    }
    *reinterpret_cast<uint32_t*>(keep + e) = out;
  }
  if (nan) atomicOr(status, KVC_DEV_NAN_SCORE);
  kept = uint32_t(wave_sum_int(int(kept)));
  ties = uint32_t(wave_sum_int(int(ties)));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = kept;
    red[1][wave] = ties;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t k = 0, t = 0;
    for (int w = 0; w < kTB / kWave; ++w) {
      k += red[0][w];
      t += red[1][w];
    }
    if (k != 0u) atomicAdd(&row_counts[r.row], int(k));
    ws.tie_cnt[blockIdx.x] = t;
  }
}

// one workgroup: exclusive scan of the blocks' tie counts -> how many ties each block takes
__global__ __launch_bounds__(kTB) void topm_tie_scan(TopmWs ws, int64_t n_blocks) {
  __shared__ long long wsum[kTB / kWave];
  const int64_t per = (n_blocks + kTB - 1) / kTB;
  const int64_t b0 = threadIdx.x * per, b1 = min(n_blocks, b0 + per);
  long long mine = 0;
  for (int64_t b = b0; b < b1; ++b) mine += ws.tie_cnt[b];
  long long total;
  long long off = block_excl_scan<long long>(mine, wsum, &total);
  const long long need = ws.state->need;
  for (int64_t b = b0; b < b1; ++b) {
    const long long c = ws.tie_cnt[b];
    ws.tie_take[b] = uint32_t(max(0LL, min(c, need - off)));
    off += c;
  }
}

// blocks holding kept ties: take the first tie_take of them in index order
__global__ __launch_bounds__(kTB) void topm_fix(const float* __restrict__ scores, uint8_t* __restrict__ keep,
                                                int32_t* row_counts, TopmWs ws, int32_t row_len) {
  const uint32_t take = ws.tie_take[blockIdx.x];
  if (take == 0u) return;
  __shared__ uint32_t wsum[kTB / kWave];
  const uint32_t thr = ws.state->prefix;
  const BlockRange r = block_range(blockIdx.x, row_len, kChunk);
  uint32_t done = 0;  // ties already seen before this iteration, in index order
  for (int64_t base = r.beg; base < r.end; base += 4 * kTB) {
    const int64_t e = base + 4 * threadIdx.x;
    uint32_t flags = 0, cnt = 0;
    if (e < r.end) {
      const float4 v = *reinterpret_cast<const float4*>(scores + e);
      const float vs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (desc_key(vs[c]) == thr) {
          flags |= 1u << c;
          ++cnt;
        }
      }
    }
    uint32_t tot;
    uint32_t rank = done + block_excl_scan<uint32_t>(cnt, wsum, &tot);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((flags >> c) & 1u) {
        if (rank < take) keep[e + c] = 1;
        ++rank;
      }
    }
    done += tot;
    if (done >= take) break;
  }
  if (threadIdx.x == 0) atomicAdd(&row_counts[r.row], int(take));
}

// ---- compaction ----------------------------------------------------------------------------------------------
struct CompactWs {
  int32_t* chunk_cnt;   // [rows * chunks]
  int32_t* chunk_off;   // [rows * chunks] position of the chunk's first kept entry within its row
  int32_t* src_of_dst;  // [out_pages_max * page] source pool row of each output row, -1 for a zero row
};

__global__ __launch_bounds__(kTB) void compact_count(const uint8_t* __restrict__ keep, CompactWs ws, int32_t row_len) {
  __shared__ int red[kTB / kWave];
  const BlockRange r = block_range(blockIdx.x, row_len, kCChunk);
  int cnt = 0;
  for (int64_t e = r.beg + 16 * threadIdx.x; e < r.end; e += 16 * kTB) {
    const uint4 v = *reinterpret_cast<const uint4*>(keep + e);
    cnt += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);  // bytes are 0 or 1
  }
  cnt = wave_sum_int(cnt);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) ws.chunk_cnt[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// one workgroup: row lengths, pages, page offsets (consecutive in row order) and chunk offsets
__global__ __launch_bounds__(kTB) void compact_plan(CompactWs ws, int64_t n_rows, int32_t chunks, int32_t page,
                                                    int32_t* lengths, int32_t* page_offset, int32_t* n_pages,
                                                    int64_t out_pages_max, int32_t* status) {
  __shared__ long long wsum[kTB / kWave];
  const int64_t per = (n_rows + kTB - 1) / kTB;
  const int64_t r0 = threadIdx.x * per, r1 = min(n_rows, r0 + per);
  long long mine = 0;
  for (int64_t row = r0; row < r1; ++row) {
    int off = 0;
    for (int c = 0; c < chunks; ++c) {
      ws.chunk_off[row * chunks + c] = off;
      off += ws.chunk_cnt[row * chunks + c];
    }
    lengths[row] = off;
    const int np = (off + page - 1) / page;
    n_pages[row] = np;
    mine += np;
  }
  long long total;
  long long off = block_excl_scan<long long>(mine, wsum, &total);
  if (threadIdx.x == 0 && total > out_pages_max) atomicOr(status, KVC_DEV_BOUND_EXCEEDED);
  for (int64_t row = r0; row < r1; ++row) {
    page_offset[row] = int32_t(off);
    off += n_pages[row];
  }
}

// source row of every output row, per (row, chunk): the chunk's page ids go to LDS in one coalesced read, ranks
// come from a block scan over 16-position runs; a rejected page id gives -1, and so do the unused rows of a row's
// last page (marked by the block holding the row's last chunk)
__global__ __launch_bounds__(kTB) void compact_index(const uint8_t* __restrict__ keep, const int32_t* __restrict__ pt,
                                                     CompactWs ws, const int32_t* __restrict__ lengths,
                                                     const int32_t* __restrict__ page_offset,
                                                     const int32_t* __restrict__ n_pages, int32_t row_len,
                                                     int32_t page, int64_t n_src_pages, int64_t out_pages_max,
                                                     int32_t* status) {
  __shared__ int32_t src_s[kCChunk];
  extern __shared__ int32_t pg_s[];  // page id per block of `page` positions of the chunk (sized at launch)
  __shared__ int wsum[kTB / kWave];
  const BlockRange r = block_range(blockIdx.x, row_len, kCChunk);
  const int64_t pos0 = r.beg - r.row * row_len;  // first position of the chunk within its row
  const int npg = int((r.end - r.beg + page - 1) / page);
  const int32_t* ptr = pt + r.row * (row_len / page) + pos0 / page;
  for (int i = threadIdx.x; i < npg; i += kTB) pg_s[i] = ptr[i];
  const int64_t e = r.beg + 16 * threadIdx.x;
  uint32_t bits = 0;
  if (e < r.end) {
    const uint4 v = *reinterpret_cast<const uint4*>(keep + e);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) bits |= ((w[j >> 2] >> (8 * (j & 3))) & 1u) << j;
  }
  int nk;
  int k = block_excl_scan<int>(__popc(bits), wsum, &nk);  // (contains the barrier that publishes pg_s)
  bool bad = false;
  for (int j = 0; j < 16; ++j) {
    if ((bits >> j) & 1u) {
      const int p = 16 * threadIdx.x + j;  // position within the chunk (pos0 is a multiple of page)
      const int64_t src_page = pg_s[p / page];
      const bool ok = src_page >= 0 && src_page < n_src_pages;
      bad |= !ok;
      src_s[k++] = ok ? int32_t(src_page * page + p % page) : -1;
    }
  }
  if (bad) atomicOr(status, KVC_DEV_BOUND_EXCEEDED);
  __syncthreads();
  const int64_t base = int64_t(page_offset[r.row]) * page;
  const int64_t dst0 = base + ws.chunk_off[blockIdx.x];
  const int64_t cap = out_pages_max * page;
  for (int i = threadIdx.x; i < nk; i += kTB) {
    if (dst0 + i < cap) ws.src_of_dst[dst0 + i] = src_s[i];
  }
  if (r.end == (r.row + 1) * int64_t(row_len)) {
    const int64_t last = min(base + int64_t(n_pages[r.row]) * page, cap);
    for (int64_t d = base + lengths[r.row] + threadIdx.x; d < last; d += kTB) ws.src_of_dst[d] = -1;
  }
}

// the copy itself, in output order: 16 lanes move one 128-element row (one 16-byte access each for K and V), kGU
// rows per lane group with every load issued before the stores; source -1 writes zeros
constexpr int kGU = 8;
constexpr int kGRows = (kTB / 16) * kGU;  // output rows per workgroup
__global__ __launch_bounds__(kTB) void compact_gather(const int32_t* __restrict__ src_of_dst,
                                                      const uint4* __restrict__ k_pool,
                                                      const uint4* __restrict__ v_pool, uint4* __restrict__ k_out,
                                                      uint4* __restrict__ v_out,
                                                      const int32_t* __restrict__ page_offset,
                                                      const int32_t* __restrict__ n_pages, int64_t n_rows,
                                                      int32_t page, int64_t out_pages_max) {
  const int64_t total = min((int64_t(page_offset[n_rows - 1]) + n_pages[n_rows - 1]) * page, out_pages_max * page);
  const int64_t d0 = int64_t(blockIdx.x) * kGRows;
  if (d0 >= total) return;
  const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
  int src[kGU];
#pragma unroll
  for (int u = 0; u < kGU; ++u) {
    const int64_t d = d0 + grp + 16 * u;
    src[u] = d < total ? src_of_dst[d] : -2;
  }
  u32x4 kv[kGU], vv[kGU];
#pragma unroll
  for (int u = 0; u < kGU; ++u) {
    const size_t si = size_t(max(src[u], 0)) * 16 + sub;  // row 0 stands in for a zero row
    kv[u] = reinterpret_cast<const u32x4*>(k_pool)[si];
    vv[u] = reinterpret_cast<const u32x4*>(v_pool)[si];
  }
  // keep the loads ahead of the conditional stores (else each pair is sunk into its store's branch)
#pragma unroll
  for (int u = 0; u < kGU; ++u) asm volatile("" ::"v"(kv[u]), "v"(vv[u]));
  const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < kGU; ++u) {
    if (src[u] >= -1) {
      const size_t di = size_t(d0 + grp + 16 * u) * 16 + sub;
      reinterpret_cast<u32x4*>(k_out)[di] = src[u] >= 0 ? kv[u] : z;
      reinterpret_cast<u32x4*>(v_out)[di] = src[u] >= 0 ? vv[u] : z;
    }
  }
}

size_t al(size_t x) { return align_up(x, 256); }

}  // namespace

// ---- launchers ---------------------------------------------------------------------------------------------
hipError_t launch_retention_score(const kvc_retention_args& a, hipStream_t s) {
  const int64_t n = a.n_rows * int64_t(a.n_tokens);
  const int64_t blocks = std::min<int64_t>((n / 4 + kTB - 1) / kTB, 65536);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(retention_score_kernel, dim3(unsigned(blocks)), dim3(kTB), 0, s, a.beta, a.score, n,
                     a.n_tokens, a.t);
  return hipGetLastError();
}

int64_t topm_blocks(const kvc_topm_args& a) {
  const int64_t per_row = (a.row_len + kChunk - 1) / kChunk;
  return (a.n / a.row_len) * per_row;
}

size_t topm_workspace_bytes(const kvc_topm_args& a) {
  const int64_t nb = topm_blocks(a);
  return al(sizeof(TopmState)) + al(3 * kBins * sizeof(uint32_t)) + 2 * al(size_t(nb) * sizeof(uint32_t));
}

hipError_t launch_topm(const kvc_topm_args& a, void* ws_ptr, hipStream_t s) {
  char* w = static_cast<char*>(ws_ptr);
  TopmWs ws;
  ws.state = reinterpret_cast<TopmState*>(w);
  w += al(sizeof(TopmState));
  ws.hist = reinterpret_cast<uint32_t*>(w);
  w += al(3 * kBins * sizeof(uint32_t));
  const int64_t nb = topm_blocks(a);
  ws.tie_cnt = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(nb) * sizeof(uint32_t));
  ws.tie_take = reinterpret_cast<uint32_t*>(w);
  const int64_t n_rows = a.n / a.row_len;
  const int64_t clear_n = std::max<int64_t>(3 * kBins, n_rows);
  hipLaunchKernelGGL(topm_clear, dim3(unsigned((clear_n + kTB - 1) / kTB)), dim3(kTB), 0, s, ws, a.row_counts, n_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n == 0) return e;
  // m == 0 and m == n need no special case: the picks then select the first key's bin with nothing to take, or
  // the last key's bin with every key taken
  const dim3 grid{unsigned(nb), 1, 1};
  const int64_t per_row = (a.row_len + kChunk - 1) / kChunk;
  auto hgrid = [&](int g) { return dim3{unsigned(n_rows * ((per_row + g - 1) / g)), 1, 1}; };
  hipLaunchKernelGGL(topm_hist<0>, hgrid(hist_group(0)), dim3(kTB), 0, s, a.scores, ws, a.row_len);
  hipLaunchKernelGGL(topm_pick<0>, dim3(1), dim3(kTB), 0, s, ws, a.m);
  hipLaunchKernelGGL(topm_hist<1>, hgrid(hist_group(1)), dim3(kTB), 0, s, a.scores, ws, a.row_len);
  hipLaunchKernelGGL(topm_pick<1>, dim3(1), dim3(kTB), 0, s, ws, a.m);
  hipLaunchKernelGGL(topm_hist<2>, hgrid(hist_group(2)), dim3(kTB), 0, s, a.scores, ws, a.row_len);
  hipLaunchKernelGGL(topm_pick<2>, dim3(1), dim3(kTB), 0, s, ws, a.m);
  hipLaunchKernelGGL(topm_mark, grid, dim3(kTB), 0, s, a.scores, a.keep, a.row_counts, ws, a.row_len, a.status);
  hipLaunchKernelGGL(topm_tie_scan, dim3(1), dim3(kTB), 0, s, ws, nb);
  hipLaunchKernelGGL(topm_fix, grid, dim3(kTB), 0, s, a.scores, a.keep, a.row_counts, ws, a.row_len);
  return hipGetLastError();
}

int64_t compact_blocks(const kvc_compact_args& a) {
  return a.n_rows * int64_t((a.n_tokens + kCChunk - 1) / kCChunk);
}

size_t compact_workspace_bytes(const kvc_compact_args& a) {
  return 2 * al(size_t(compact_blocks(a)) * sizeof(int32_t)) + al(size_t(a.out_pages_max) * a.page * sizeof(int32_t));
}

hipError_t launch_compact(const kvc_compact_args& a, void* ws_ptr, hipStream_t s) {
  char* w = static_cast<char*>(ws_ptr);
  const int64_t nb = compact_blocks(a);
  if (nb == 0) return hipSuccess;  // no rows
  CompactWs ws;
  ws.chunk_cnt = reinterpret_cast<int32_t*>(w);
  w += al(size_t(nb) * sizeof(int32_t));
  ws.chunk_off = reinterpret_cast<int32_t*>(w);
  w += al(size_t(nb) * sizeof(int32_t));
  ws.src_of_dst = reinterpret_cast<int32_t*>(w);
  const int chunks = (a.n_tokens + kCChunk - 1) / kCChunk;
  hipLaunchKernelGGL(compact_count, dim3(unsigned(nb)), dim3(kTB), 0, s, a.keep, ws, a.n_tokens);
  hipLaunchKernelGGL(compact_plan, dim3(1), dim3(kTB), 0, s, ws, a.n_rows, chunks, a.page, a.lengths, a.page_offset,
                     a.n_pages, a.out_pages_max, a.status);
  const size_t pg_lds = size_t((kCChunk + a.page - 1) / a.page) * sizeof(int32_t);
  hipLaunchKernelGGL(compact_index, dim3(unsigned(nb)), dim3(kTB), pg_lds, s, a.keep, a.page_table, ws, a.lengths,
                     a.page_offset, a.n_pages, a.n_tokens, a.page, a.n_src_pages, a.out_pages_max, a.status);
  const int64_t cap_rows = a.out_pages_max * a.page;
  const int64_t gb = (cap_rows + kGRows - 1) / kGRows;
  if (gb > 0) {
    hipLaunchKernelGGL(compact_gather, dim3(unsigned(gb)), dim3(kTB), 0, s, ws.src_of_dst,
                       static_cast<const uint4*>(a.k_pool), static_cast<const uint4*>(a.v_pool),
                       static_cast<uint4*>(a.k_out), static_cast<uint4*>(a.v_out), a.page_offset, a.n_pages,
                       a.n_rows, a.page, a.out_pages_max);
  }
  return hipGetLastError();
}

}  // namespace kvc
