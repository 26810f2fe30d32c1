// Routing diagnostics of a compressed-cache decode run, one routing event or one step at a time.
//
// QEvict page ("Principais Contribuições", item 1) characterises cache dynamics under a policy by the future
// missed mass (the share of later attention that falls on states the policy has dropped), the global latent
// importance reactivation (windows that had left the active set coming back) and the selection churn (how much the
// assignment changes between consecutive routing steps). CriticalKV page ("Framework Teórico") measures a kept
// subset by the L1 distance between the attention output over the full cache and over the subset.
//
// diag_kernel: one 256-thread workgroup per unit. Thread d < 128 first loads |o_full - o| at head_dim d of every
// query head; thread t then takes windows t, t + 256, ... (ascending) and counts tier changes, entries into FULL,
// FULL and resident windows, and sums the full-cache mass of the EVICTED windows. Every sum is taken per wave
// (DPP row sums, then the four rows in order) and then over the four waves in order, so the results are bitwise
// reproducible. Everything it reads is a few KB per unit: the kernel is latency-bound.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kDiagThreads = 256;
constexpr int kDiagWaves = kDiagThreads / kWave;

template <int G>
__global__ __launch_bounds__(kDiagThreads) void diag_kernel(kvc_diag_args a) {
  const int u = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t >> 6;
  const int NW = a.n_windows_max;
  const int nw = min(max(a.n_windows[u], 0), NW);
  const size_t base = size_t(u) * NW;
  float part[1 + G];
  const bool have_o = a.o_full != nullptr && a.o != nullptr;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    part[1 + h] = 0.0f;
    if (have_o && t < kD) {
      const size_t i = (size_t(u) * G + h) * kD + t;
      part[1 + h] = fabsf(a.o_full[i] - a.o[i]);
    }
  }
  int ch = 0, re = 0, nf = 0, nr = 0;
  float fmm = 0.0f;
  for (int w = t; w < nw; w += kDiagThreads) {
    const int now = a.tier[base + w];
    const int prev = a.tier_prev != nullptr ? int(a.tier_prev[base + w]) : now;
    ch += now != prev ? 1 : 0;
    re += (now == KVC_TIER_FULL && prev != KVC_TIER_FULL) ? 1 : 0;
    nf += now == KVC_TIER_FULL ? 1 : 0;
    nr += now != KVC_TIER_EVICTED ? 1 : 0;
    if (a.mass_full != nullptr && now == KVC_TIER_EVICTED) fmm += a.mass_full[base + w];
  }
  part[0] = fmm;
  __shared__ int cnt[4][kDiagWaves];
  __shared__ float vred[1 + G][kDiagWaves];
  ch = wave_sum_int(ch);
  re = wave_sum_int(re);
  nf = wave_sum_int(nf);
  nr = wave_sum_int(nr);
#pragma unroll
  for (int i = 0; i < 1 + G; ++i) part[i] = wave_sum(part[i]);
  if (lane == 0) {
    cnt[0][wave] = ch;
    cnt[1][wave] = re;
    cnt[2][wave] = nf;
    cnt[3][wave] = nr;
#pragma unroll
    for (int i = 0; i < 1 + G; ++i) vred[i][wave] = part[i];
  }
  __syncthreads();
  if (t < 4) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < kDiagWaves; ++i) s += cnt[t][i];
    a.counts[size_t(u) * 4 + t] = s;
  } else if (t >= kWave && t < kWave + 1 + G) {
    const int i = t - kWave;
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kDiagWaves; ++k) s += vred[i][k];
    a.values[size_t(u) * (1 + G) + i] = s;
  }
}

}  // namespace

hipError_t launch_diagnostics(const kvc_diag_args& a, hipStream_t s) {
  const dim3 grid(unsigned(a.n_units)), block(kDiagThreads);
  switch (a.group) {
    case 1: hipLaunchKernelGGL(diag_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(diag_kernel<2>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(diag_kernel<4>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(diag_kernel<8>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace kvc
