// Generic budgeted top-k: the k largest of n scores, ties to the lower index, written as their indices in
// ascending order. Every selection on the pages is a budgeted top-k under this order: QEvict's tiers, CriticalKV's
// two stages, DBTrimKV's global top-M; this entry point exposes the selection itself.
//
// The kept set is found by the global top-M engine (topm.hip) over one row of n entries (any n: the last chunk is
// ragged, nothing is padded); it leaves a byte mask and the kept count of every 8192-entry chunk. topk_offsets
// turns the counts into exclusive offsets (one workgroup), and topk_write writes each chunk's kept indices at its
// offset in ascending order (a block scan of per-thread counts, the indices staged in LDS and stored as one run).
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kKThreads = 256;
constexpr int kKChunk = kTopmChunk;           // 8192 entries: the engine's chunks
constexpr int kKPer = kKChunk / kKThreads;    // 32 mask bytes per thread

// exclusive offsets of nb chunk counts, one 1024-thread workgroup: thread t sums a contiguous run of chunks, a
// wave-shuffle scan plus one LDS step places the runs
__global__ __launch_bounds__(1024) void topk_offsets(const int32_t* __restrict__ counts, int64_t nb,
                                                     int32_t* __restrict__ offsets) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t >> 6;
  const int64_t per = (nb + 1023) / 1024;
  const int64_t lo = min(nb, t * per), hi = min(nb, lo + per);
  int s = 0;
  for (int64_t i = lo; i < hi; ++i) s += counts[i];
  int inc = s;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  __shared__ int wsum[1024 / kWave];
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  int run = base + inc - s;
  for (int64_t i = lo; i < hi; ++i) {
    offsets[i] = run;
    run += counts[i];
  }
}

__global__ __launch_bounds__(kKThreads) void topk_write(const uint8_t* __restrict__ keep, int64_t n,
                                                        const int32_t* __restrict__ offsets, int64_t k,
                                                        int32_t* __restrict__ idx) {
  const int64_t beg = int64_t(blockIdx.x) * kKChunk + int64_t(threadIdx.x) * kKPer;
  uint32_t bits = 0u;  // bit j: entry beg + j kept
  if (beg + kKPer <= n) {
    const uint4 v0 = *reinterpret_cast<const uint4*>(keep + beg);
    const uint4 v1 = *reinterpret_cast<const uint4*>(keep + beg + 16);
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int j = 0; j < kKPer; ++j) bits |= ((w[j >> 2] >> (8 * (j & 3))) & 1u) << j;
  } else {
    for (int j = 0; j < kKPer; ++j) bits |= (beg + j < n ? uint32_t(keep[beg + j] & 1) : 0u) << j;
  }
  const int c = __popc(bits);
  // exclusive prefix of the per-thread counts over the workgroup (thread order = index order)
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int inc = c;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  __shared__ int wsum[kKThreads / kWave];
  __shared__ int32_t stage[kKChunk];  // the chunk's kept indices in order, written out as one contiguous run
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  int lpos = inc - c, total = 0;
#pragma unroll
  for (int w = 0; w < kKThreads / kWave; ++w) {
    if (w < wave) lpos += wsum[w];
    total += wsum[w];
  }
  while (bits) {
    const int j = __builtin_ctz(bits);
    bits &= bits - 1;
    stage[lpos++] = int32_t(beg + j);
  }
  __syncthreads();
  const int64_t base = offsets[blockIdx.x];
  for (int i = threadIdx.x; i < total; i += kKThreads) {
    if (base + i < k) idx[base + i] = stage[i];
  }
}

struct TopkLayout {
  int64_t nb;
  size_t keep_off, offsets_off, misc_off, engine_off, total;
};

TopkLayout topk_layout(int64_t n) {
  TopkLayout L;
  L.nb = topm_chunks(n, int32_t(n));
  size_t o = 0;
  L.keep_off = o;
  o += align_up(size_t(std::max<int64_t>(n, 1)) + 32, 256);
  L.offsets_off = o;
  o += align_up(size_t(std::max<int64_t>(L.nb, 1)) * sizeof(int32_t), 256);
  L.misc_off = o;  // row count + status of the engine
  o += 256;
  L.engine_off = o;
  o += topm_engine_workspace(n, int32_t(n));
  L.total = o;
  return L;
}

__global__ void topk_zero(int32_t* __restrict__ w) {
  if (threadIdx.x == 0) w[0] = 0;
}

}  // namespace

size_t topk_workspace_bytes(int64_t n) { return topk_layout(n).total; }

hipError_t launch_topk(const float* scores, int64_t n, int64_t k, int32_t* idx, void* ws, hipStream_t s) {
  const TopkLayout L = topk_layout(n);
  char* w = static_cast<char*>(ws);
  uint8_t* keep = reinterpret_cast<uint8_t*>(w + L.keep_off);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.offsets_off);
  int32_t* misc = reinterpret_cast<int32_t*>(w + L.misc_off);
  hipLaunchKernelGGL(topk_zero, dim3(1), dim3(kWave), 0, s, misc + 1);  // the engine's status word (a kernel: graphs)
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TopmInput in;
  in.scores = scores;
  in.beta = nullptr;
  in.t = 0;
  in.row_len = int32_t(n);
  in.n = n;
  int32_t* chunk_kept = nullptr;
  e = launch_topm_engine(in, k, keep, nullptr, misc + 1, w + L.engine_off, &chunk_kept, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_offsets, dim3(1), dim3(1024), 0, s, chunk_kept, L.nb, offsets);
  hipLaunchKernelGGL(topk_write, dim3(unsigned(L.nb)), dim3(kKThreads), 0, s, keep, n, offsets, k, idx);
  return hipGetLastError();
}

}  // namespace kvc
