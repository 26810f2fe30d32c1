// Generic budgeted top-k: the k largest of n scores, ties to the lower index, written as their indices in
// ascending order. Every selection on the pages is a budgeted top-k under this order: QEvict's tiers, CriticalKV's
// two stages, DBTrimKV's global top-M; this entry point exposes the selection itself.
//
// The kept set is found by the global top-M engine (topm.hip) over one row of n entries (any n: the last chunk is
// ragged, nothing is padded). It leaves a bit mask (one bit per entry) and the kept counts of its chunks and of their
// groups. topk_write handles four blocks of 8192 entries per workgroup (their mask words loaded up front): the
// first block's place in the output is the sum of the counts before it, each next one follows the previous; per
// block, each thread expands its mask word into LDS at its prefix position (16-bit offsets), and the workgroup then
// stores the run contiguously.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kKThreads = 256;
constexpr int kBlock = 8192;                         // entries per block
constexpr int kWords = kBlock / 32;                  // mask words per block: one per thread
constexpr int kSub = 4;                              // blocks per workgroup
constexpr int kChunksPerBlock = kBlock / kTopmChunk;  // engine chunks per block
static_assert(kWords == kKThreads, "one mask word per thread and block");
static_assert(kTopmGroup % (kSub * kChunksPerBlock) == 0, "a workgroup's chunks lie in one group");

// exclusive prefix over the workgroup (thread order) and the total; two barriers
__device__ int block_scan_int(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < kKThreads / kWave; ++q) {
    base += q < wave ? wsum[q] : 0;
    tot += wsum[q];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__device__ long long block_sum_ll(long long v, long long* wsum) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
  if (lane == 0) wsum[wave] = v;
  __syncthreads();
  long long tot = 0;
#pragma unroll
  for (int q = 0; q < kKThreads / kWave; ++q) tot += wsum[q];
  __syncthreads();
  return tot;
}

__global__ __launch_bounds__(kKThreads) void topk_write(const uint32_t* __restrict__ bits,
                                                        const int32_t* __restrict__ chunk_kept,
                                                        const int32_t* __restrict__ group_kept, int64_t n,
                                                        int64_t k, int32_t* __restrict__ idx) {
  __shared__ uint16_t stage[kBlock];  // offsets (entry - block start) of the block's kept entries, in order
  __shared__ int wsum[kKThreads / kWave];
  __shared__ long long bsum[kKThreads / kWave];
  const int64_t blk0 = int64_t(blockIdx.x) * kSub;
  // only entries below n count: the engine clears the bits past n in its last chunk, and the words past that chunk
  // are never written
  uint32_t w[kSub];
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    const int64_t word = (blk0 + b) * kWords + threadIdx.x;
    const int64_t lo = word * 32;
    w[b] = lo >= n ? 0u : (lo + 32 <= n ? bits[word] : bits[word] & ((1u << (n - lo)) - 1u));
  }
  // kept entries before this workgroup's first chunk: whole groups, then the group's chunks before it
  const int64_t c0 = blk0 * kChunksPerBlock;
  const int64_t grp = c0 / kTopmGroup, gfirst = grp * kTopmGroup;
  long long before = 0;
  for (int64_t q = threadIdx.x; q < grp; q += kKThreads) before += group_kept[q];
  if (int64_t(threadIdx.x) < c0 - gfirst) before += chunk_kept[gfirst + threadIdx.x];
  long long base = block_sum_ll(before, bsum);
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    int total;
    int p = block_scan_int(__popc(w[b]), wsum, &total);  // its barriers also order the previous block's stage reads
    uint32_t x = w[b];
    while (x) {
      const int j = __builtin_ctz(x);
      x &= x - 1;
      stage[p++] = uint16_t(32 * threadIdx.x + j);
    }
    __syncthreads();
    const int32_t first = int32_t((blk0 + b) * kBlock);
    for (int i = threadIdx.x; i < total; i += kKThreads) {
      if (base + i < k) idx[base + i] = first + int32_t(stage[i]);
    }
    base += total;
  }
}

struct TopkLayout {
  int64_t nb;
  size_t bits_off, misc_off, engine_off, total;
};

TopkLayout topk_layout(int64_t n) {
  TopkLayout L;
  L.nb = (n + int64_t(kSub) * kBlock - 1) / (int64_t(kSub) * kBlock);  // workgroups of topk_write
  const size_t nb = size_t(std::max<int64_t>(L.nb, 1)) * kSub;
  size_t o = 0;
  L.bits_off = o;
  o += align_up(nb * kWords * sizeof(uint32_t), 256);
  L.misc_off = o;  // the engine's status word
  o += 256;
  L.engine_off = o;
  o += topm_engine_workspace(n, int32_t(n));
  L.total = o;
  return L;
}

}  // namespace

size_t topk_workspace_bytes(int64_t n) { return topk_layout(n).total; }

hipError_t launch_topk(const float* scores, int64_t n, int64_t k, int32_t* idx, void* ws, hipStream_t s) {
  const TopkLayout L = topk_layout(n);
  char* w = static_cast<char*>(ws);
  TopmInput in;
  in.scores = scores;
  in.beta = nullptr;
  in.t = 0;
  in.row_len = int32_t(n);
  in.n = n;
  TopmOutput out;
  out.keep_bits = reinterpret_cast<uint32_t*>(w + L.bits_off);
  out.status = reinterpret_cast<int32_t*>(w + L.misc_off);
  out.clear_status = true;
  TopmCounts counts;
  hipError_t e = launch_topm_engine(in, k, out, w + L.engine_off, s, &counts);
  if (e != hipSuccess || L.nb == 0) return e;
  hipLaunchKernelGGL(topk_write, dim3(unsigned(L.nb)), dim3(kKThreads), 0, s, out.keep_bits, counts.chunk_kept,
                     counts.group_kept, n, k, idx);
  return hipGetLastError();
}

}  // namespace kvc
