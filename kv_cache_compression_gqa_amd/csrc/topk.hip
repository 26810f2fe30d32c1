// Generic budgeted top-k: the k largest of n scores, ties to the lower index, written as their indices in
// ascending order. Every selection on the pages is a budgeted top-k under this order: QEvict's tiers, CriticalKV's
// two stages, DBTrimKV's global top-M; this entry point exposes the selection itself.
//
// The kept set is found by the global top-M kernels (radix passes over the scores, a tie scan, a mark pass into a
// byte mask); then topk_count counts the kept entries of every 4096-entry chunk, topk_offsets turns the counts into
// exclusive offsets (one workgroup), and topk_write writes each chunk's kept indices at its offset in ascending
// order (a block scan of per-thread counts). Inputs whose length is not a multiple of 16 are first copied into the
// workspace with -FLT_MAX padding: padded entries come after every real entry in the order (equal or smaller
// score, larger index), so they are never among the first k <= n.
#include <float.h>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kKChunk = 4096;
constexpr int kKThreads = 256;
constexpr int kKPer = kKChunk / kKThreads;  // 16 mask bytes per thread

__global__ __launch_bounds__(kKThreads) void topk_pad(const float* __restrict__ src, float* __restrict__ dst,
                                                      int64_t n, int64_t n_pad) {
  const int64_t i = int64_t(blockIdx.x) * kKThreads + threadIdx.x;
  if (i < n_pad) dst[i] = i < n ? src[i] : -FLT_MAX;
}

__global__ void topk_zero(int32_t* __restrict__ w) {
  if (threadIdx.x == 0) w[0] = 0;
}

__global__ __launch_bounds__(kKThreads) void topk_count(const uint8_t* __restrict__ keep, int64_t n,
                                                        int32_t* __restrict__ counts) {
  const int64_t beg = int64_t(blockIdx.x) * kKChunk + int64_t(threadIdx.x) * kKPer;
  int c = 0;
  if (beg + kKPer <= n) {
    const uint4 v = *reinterpret_cast<const uint4*>(keep + beg);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) c += __popc(w[j] & 0x01010101u);
  } else {
    for (int64_t i = beg; i < n; ++i) c += keep[i] & 1;
  }
  c = wave_sum_int(c);
  __shared__ int ws[kKThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) ws[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) counts[blockIdx.x] = ws[0] + ws[1] + ws[2] + ws[3];
}

// exclusive offsets of nb chunk counts, one 1024-thread workgroup (thread t owns a contiguous run of chunks)
__global__ __launch_bounds__(1024) void topk_offsets(const int32_t* __restrict__ counts, int64_t nb,
                                                     int32_t* __restrict__ offsets) {
  const int t = threadIdx.x;
  const int64_t per = (nb + 1023) / 1024;
  const int64_t lo = min(nb, t * per), hi = min(nb, lo + per);
  int s = 0;
  for (int64_t i = lo; i < hi; ++i) s += counts[i];
  __shared__ int sh[1024];
  sh[t] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan over the 1024 run sums
    const int v = t >= d ? sh[t - d] : 0;
    __syncthreads();
    sh[t] += v;
    __syncthreads();
  }
  int run = sh[t] - s;
  for (int64_t i = lo; i < hi; ++i) {
    offsets[i] = run;
    run += counts[i];
  }
}

__global__ __launch_bounds__(kKThreads) void topk_write(const uint8_t* __restrict__ keep, int64_t n,
                                                        const int32_t* __restrict__ offsets, int64_t k,
                                                        int32_t* __restrict__ idx) {
  const int64_t beg = int64_t(blockIdx.x) * kKChunk + int64_t(threadIdx.x) * kKPer;
  uint8_t b[kKPer];
  if (beg + kKPer <= n) {
    const uint4 v = *reinterpret_cast<const uint4*>(keep + beg);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < kKPer; ++j) b[j] = uint8_t((w[j >> 2] >> (8 * (j & 3))) & 1u);
  } else {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) b[j] = beg + j < n ? (keep[beg + j] & 1) : 0;
  }
  int c = 0;
#pragma unroll
  for (int j = 0; j < kKPer; ++j) c += b[j];
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
#pragma unroll
  for (int j = 0; j < kKPer; ++j) {
    if (b[j]) stage[lpos++] = int32_t(beg + j);
  }
  __syncthreads();
  const int64_t base = offsets[blockIdx.x];
  for (int i = threadIdx.x; i < total; i += kKThreads) {
    if (base + i < k) idx[base + i] = stage[i];
  }
}

struct TopkLayout {
  int64_t n_pad, nb;
  size_t pad_off, keep_off, counts_off, offsets_off, misc_off, topm_off, total;
};

TopkLayout topk_layout(int64_t n) {
  TopkLayout L;
  L.n_pad = (n + 15) / 16 * 16;
  if (L.n_pad == 0) L.n_pad = 16;
  L.nb = (L.n_pad + kKChunk - 1) / kKChunk;
  size_t o = 0;
  L.pad_off = o;
  o += (L.n_pad != n) ? align_up(size_t(L.n_pad) * sizeof(float), 256) : 0;
  L.keep_off = o;
  o += align_up(size_t(L.n_pad), 256);
  L.counts_off = o;
  o += align_up(size_t(L.nb) * sizeof(int32_t), 256);
  L.offsets_off = o;
  o += align_up(size_t(L.nb) * sizeof(int32_t), 256);
  L.misc_off = o;  // row count + status of the top-M kernels
  o += 256;
  L.topm_off = o;
  kvc_topm_args a{};
  a.n = L.n_pad;
  a.row_len = int32_t(L.n_pad);
  o += topm_workspace_bytes(a);
  L.total = o;
  return L;
}

}  // namespace

size_t topk_workspace_bytes(int64_t n) { return topk_layout(n).total; }

hipError_t launch_topk(const float* scores, int64_t n, int64_t k, int32_t* idx, void* ws, hipStream_t s) {
  const TopkLayout L = topk_layout(n);
  char* w = static_cast<char*>(ws);
  const float* sc = scores;
  if (L.n_pad != n) {
    float* pad = reinterpret_cast<float*>(w + L.pad_off);
    hipLaunchKernelGGL(topk_pad, dim3(unsigned((L.n_pad + kKThreads - 1) / kKThreads)), dim3(kKThreads), 0, s,
                       scores, pad, n, L.n_pad);
    sc = pad;
  }
  uint8_t* keep = reinterpret_cast<uint8_t*>(w + L.keep_off);
  int32_t* counts = reinterpret_cast<int32_t*>(w + L.counts_off);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.offsets_off);
  int32_t* misc = reinterpret_cast<int32_t*>(w + L.misc_off);
  hipLaunchKernelGGL(topk_zero, dim3(1), dim3(kWave), 0, s, misc + 1);  // the top-M status word (a kernel: graphs)
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kvc_topm_args a{};
  a.scores = sc;
  a.n = L.n_pad;
  a.m = k;
  a.row_len = int32_t(L.n_pad);
  a.keep = keep;
  a.row_counts = misc;
  a.status = misc + 1;
  e = launch_topm(a, w + L.topm_off, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_count, dim3(unsigned(L.nb)), dim3(kKThreads), 0, s, keep, L.n_pad, counts);
  hipLaunchKernelGGL(topk_offsets, dim3(1), dim3(1024), 0, s, counts, L.nb, offsets);
  hipLaunchKernelGGL(topk_write, dim3(unsigned(L.nb)), dim3(kKThreads), 0, s, keep, L.n_pad, offsets, k, idx);
  return hipGetLastError();
}

}  // namespace kvc
