// HBM read probes (measurement utilities, see include/kvc_probe.h): a grid-stride streaming read and a per-wave
// read of contiguous 16 KiB tasks with every load issued before the first use (the decode kernel's pattern for a
// full-precision window). Each folds what it reads into one word per workgroup so that no load is dead.
#include "kvc_internal.h"
#include "kvc_probe.h"

namespace kvc {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;
constexpr int kWaveTaskBytes = 16384;
constexpr int kWaveLoads = kWaveTaskBytes / (16 * kWave);  // 16 loads of 16 bytes per lane
constexpr int kWavesPerWg = 8;

__global__ __launch_bounds__(kStreamThreads) void stream_read(const uint4* __restrict__ buf, int64_t n16,
                                                              uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * kStreamThreads;
  int64_t i = int64_t(blockIdx.x) * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) v[k] = buf[i + k * stride];
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kStreamThreads / kWave];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), m, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(kWavesPerWg * kWave) void wave_read(const uint4* __restrict__ buf, int64_t tasks,
                                                                 uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t task = int64_t(blockIdx.x) * kWavesPerWg + (threadIdx.x >> 6);
  uint32_t acc = 0;
  if (task < tasks) {
    const uint4* p = buf + task * (kWaveTaskBytes / 16);
    uint4 v[kWaveLoads];
#pragma unroll
    for (int k = 0; k < kWaveLoads; ++k) v[k] = p[k * kWave + lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kWaveLoads; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  __shared__ uint32_t red[kWavesPerWg];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), m, kWave));
  if (lane == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerWg; ++w) x ^= red[w];
    sink[blockIdx.x] = x;
  }
}

int stream_workgroups(int32_t workgroups) {
  if (workgroups > 0) return workgroups;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    cus = 256;
  }
  return 8 * cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace kvc

extern "C" {

int kvc_probe_stream_workgroups(int32_t workgroups) { return workgroups < 0 ? 0 : kvc::stream_workgroups(workgroups); }

int kvc_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || !kvc::aligned16(buf) || bytes % 16 != 0 || workgroups < 0) {
    return KVC_E_INVALID;
  }
  if (bytes > (size_t(1) << 40)) return KVC_E_UNSUPPORTED;
  const int wgs = kvc::stream_workgroups(workgroups);
  hipLaunchKernelGGL(kvc::stream_read, dim3(wgs), dim3(kvc::kStreamThreads), 0, stream,
                     static_cast<const uint4*>(buf), int64_t(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_probe_wave_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || !kvc::aligned16(buf) || bytes % kvc::kWaveTaskBytes != 0) {
    return KVC_E_INVALID;
  }
  if (bytes > (size_t(1) << 36)) return KVC_E_UNSUPPORTED;
  const int64_t tasks = int64_t(bytes / kvc::kWaveTaskBytes);
  if (tasks == 0) return KVC_OK;
  const int64_t wgs = (tasks + kvc::kWavesPerWg - 1) / kvc::kWavesPerWg;
  hipLaunchKernelGGL(kvc::wave_read, dim3(unsigned(wgs)), dim3(kvc::kWavesPerWg * kvc::kWave), 0, stream,
                     static_cast<const uint4*>(buf), tasks, sink);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_HIP;
}

}  // extern "C"
