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
//   top-M: the engine of topm.hip (two passes over the scores, or over beta with the score computed in place).
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
constexpr int kCChunk = 4096;    // positions per compaction block (inside one row)

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

// ---- shared helpers ------------------------------------------------------------------------------------------
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

size_t topm_workspace_bytes(const kvc_topm_args& a) { return topm_engine_workspace(a.n, a.row_len); }

hipError_t launch_topm(const kvc_topm_args& a, void* ws, hipStream_t s) {
  TopmInput in;
  in.scores = a.scores;
  in.beta = a.scores == nullptr ? a.beta : nullptr;
  in.t = a.t;
  in.row_len = a.row_len;
  in.n = a.n;
  TopmOutput out;
  out.keep = a.keep;
  out.row_counts = a.row_counts;
  out.status = a.status;
  return launch_topm_engine(in, a.m, out, ws, s);
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
