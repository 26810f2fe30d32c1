// Split-K GQA decode attention over per-head variable-length page lists (DBTrimKV page, "Metodologia: Evicção
// Baseada em Retenção Global", section 4: after the global budget every (layer, KV head) row keeps a sequence of
// its own length in PagedAttention pages; decoding attends over the row's kept tokens). Token i of a row is row
// i % page of pool page page_list[i / page]; the G query heads of the row use standard scaled dot-product
// attention.
//
// paged_partial: one wave per (row, slice of kSliceTok tokens); a workgroup holds four consecutive slices of one
// row. A wave walks its slice in 32-token chunks (two 16-token MFMA tiles; page is a multiple of 16, so a tile
// never straddles two pages) with an online softmax:
//   * the slice's page ids are gathered once, one per lane;
//   * q.K^T on MFMA (v_mfma_f32_16x16x32 bf16/f16): A = the G query heads (rows), B = 16 tokens x 32 head_dim of
//     K (token-major pages: one 16-byte load per lane per operand);
//   * P.V on the fp32 VALU: V pages are token-major, so lane l holds 8 consecutive tokens 8*(l/16) .. +7 of the
//     chunk at head_dim 8*(l%16) .. +7 (eight 16-byte loads) and accumulates o[h][8 head_dim] += p[h][t] v[t][d]
//     for all G heads; P reaches the lanes through a per-wave LDS tile. The four lanes that share a head_dim
//     group are summed at the end of the slice.
//   Every load of a chunk (K and V) is issued before its first use.
// paged_combine: one workgroup per row merges the row's slices in a fixed order (bitwise reproducible): the per-head
// (max, sum) first, then the outputs with eight partial loads in flight per thread.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 pf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t pu32x4 __attribute__((ext_vector_type(4)));

constexpr int kSliceTok = 256;              // tokens per wave slice
constexpr int kChunk = 32;                  // tokens per chunk
constexpr int kPWaves = 4;                  // waves (slices) per workgroup
constexpr float kScale = 0.088388347648318440550f;  // 1/sqrt(128)

template <class T> struct PMfma;
template <> struct PMfma<BF16> {
  static __device__ __forceinline__ pf32x4 mfma(pu32x4 a, pu32x4 b, pf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pbf16x8, a), __builtin_bit_cast(pbf16x8, b),
                                                   c, 0, 0, 0);
  }
};
template <> struct PMfma<F16> {
  static __device__ __forceinline__ pf32x4 mfma(pu32x4 a, pu32x4 b, pf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(pf16x8, a), __builtin_bit_cast(pf16x8, b), c,
                                                  0, 0, 0);
  }
};

__device__ __forceinline__ pu32x4 pld16(const uint16_t* p) { return *reinterpret_cast<const pu32x4*>(p); }

}  // namespace

struct PagedParams {
  const uint16_t* q;       // [rows][G][128]
  const uint16_t* k_pool;  // [n_pool][page][128]
  const uint16_t* v_pool;
  const int32_t* page_list;  // [rows][page_stride]
  const int32_t* lengths;    // [rows]
  float* part_ml;            // [rows][slices][G][2]
  float* part_o;             // [rows][slices][G][128]
  float* out;                // [rows][G][128]
  int32_t* status;
  int64_t page_stride;
  int64_t n_pool;
  int32_t n_rows, page, slices, max_tokens;
};

namespace {

template <int G, class T>
__global__ __launch_bounds__(kPWaves * kWave) void paged_partial(PagedParams p) {
  using M = PMfma<T>;
  const int wg_per_row = (p.slices + kPWaves - 1) / kPWaves;
  const int row = int(blockIdx.x) / wg_per_row;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = (int(blockIdx.x) - row * wg_per_row) * kPWaves + wave;
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane & 15, qd = lane >> 4;
  __shared__ __attribute__((aligned(16))) float plds_all[kPWaves][G * kChunk];
  float* plds = plds_all[wave];

  const int len_dev = p.lengths[row];
  const int len = min(max(len_dev, 0), p.max_tokens);
  if (slice == 0 && lane == 0 && len != len_dev) atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
  const int t_beg = slice * kSliceTok;
  if (slice >= p.slices || t_beg >= len) return;  // wave-uniform; the combine reads slices < ceil(len / kSliceTok)
  const int t_end = min(t_beg + kSliceTok, len);

  // page ids of the slice's 16-token tiles: lane i holds tile i (16 tiles per slice)
  const int tiles = (t_end - t_beg + 15) >> 4;
  int pid_l = 0;
  {
    const int tok = t_beg + 16 * min(lane, tiles - 1);
    const int pid = p.page_list[size_t(row) * p.page_stride + tok / p.page];
    const bool bad = lane < tiles && (pid < 0 || int64_t(pid) >= p.n_pool);
    if (__ballot(bad) != 0 && lane == 0) atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
    pid_l = bad ? -1 : pid;  // a bad id: the tile reads page 0 (in bounds) and is masked
  }

  // A operand: the G query heads (rows; rows beyond G repeat head G-1 and are never used), k-block k = head_dim
  // 32k + 8*(lane/16) .. +7
  pu32x4 aq[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) aq[k] = pld16(p.q + (size_t(row) * G + min(col, G - 1)) * kD + 32 * k + 8 * qd);

  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.0f;
  }
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
  }

  for (int t0 = t_beg; t0 < t_end; t0 += kChunk) {
    const int tile0 = (t0 - t_beg) >> 4;
    // pool rows of the chunk's two tiles; a masked tile reads page 0
    int64_t base[2];
    bool tile_ok[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = t0 + 16 * tt;
      const int pid = __builtin_amdgcn_readlane(pid_l, min(tile0 + tt, tiles - 1));
      tile_ok[tt] = tok < t_end && pid >= 0;
      base[tt] = tile_ok[tt] ? int64_t(pid) * p.page + tok % p.page : 0;
    }
    pu32x4 kr[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int k = 0; k < 4; ++k) kr[tt * 4 + k] = pld16(p.k_pool + size_t(base[tt] + col) * kD + 32 * k + 8 * qd);
    }
    // V: lane holds tokens 8*qd + j (j = 0..7) of the chunk, head_dim 8*col .. +7
    pu32x4 vr[8];
    {
      const int tt = qd >> 1;
      const int64_t b = base[tt] + 8 * (qd & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[j] = pld16(p.v_pool + size_t(b + j) * kD + 8 * col);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the chunk is issued before the first use

    pf32x4 S[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      S[tt] = pf32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 4; ++k) S[tt] = M::mfma(aq[k], kr[tt * 4 + k], S[tt]);
      const bool ok = tile_ok[tt] && t0 + 16 * tt + col < t_end;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[tt][r] = ok ? S[tt][r] * kScale : -INFINITY;
    }
    // online softmax per head row (lane (col, qd) holds heads 4*qd + r of tokens col and 16 + col)
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mc = row_max16(fmaxf(S[0][r], S[1][r]));
      const float mn = fmaxf(m_run[r], mc);
      alpha[r] = exp_diff(m_run[r], mn);
      S[0][r] = exp_diff(S[0][r], mn);
      S[1][r] = exp_diff(S[1][r], mn);
      l_run[r] = l_run[r] * alpha[r] + row_sum16(S[0][r] + S[1][r]);
      m_run[r] = mn;
    }
    // P to the lanes that hold the values: plds[h][token]
    if (4 * qd < G) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * qd + r;
        if (h < G) {
          plds[h * kChunk + col] = S[0][r];
          plds[h * kChunk + 16 + col] = S[1][r];
        }
      }
    }
    // lane's tokens 8*qd + j: values past the length or on a bad page count as zero (p is 0 there; no 0 * inf)
    const int tv = t0 + 8 * qd;
    const bool vtile_ok = tile_ok[qd >> 1];
    float pj[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = lane_f(alpha[h & 3], 16 * (h >> 2));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= a;
      const float4 p0 = *reinterpret_cast<const float4*>(plds + h * kChunk + 8 * qd);
      const float4 p1 = *reinterpret_cast<const float4*>(plds + h * kChunk + 8 * qd + 4);
      pj[h][0] = p0.x;
      pj[h][1] = p0.y;
      pj[h][2] = p0.z;
      pj[h][3] = p0.w;
      pj[h][4] = p1.x;
      pj[h][5] = p1.y;
      pj[h][6] = p1.z;
      pj[h][7] = p1.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = vtile_ok && tv + j < t_end;
      const uint32_t w4[4] = {ok ? vr[j].x : 0u, ok ? vr[j].y : 0u, ok ? vr[j].z : 0u, ok ? vr[j].w : 0u};
      float vv[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        vv[2 * e2] = T::lo(w4[e2]);
        vv[2 * e2 + 1] = T::hi(w4[e2]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pj[h][j], vv[e], o[h][e]);
      }
    }
  }

  // the four lanes of a head_dim group hold disjoint tokens: sum them (fixed order)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[h][e] = xor_sum(o[h][e], 16);
      o[h][e] = xor_sum(o[h][e], 32);
    }
  }
  const size_t part = size_t(row) * p.slices + slice;
  if (qd == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(p.part_o + (part * G + h) * kD + 8 * col);
      dst[0] = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
      dst[1] = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
    }
  }
  if (col == 0 && 4 * qd < G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * qd + r;
      if (h < G) {
        p.part_ml[(part * G + h) * 2 + 0] = m_run[r];
        p.part_ml[(part * G + h) * 2 + 1] = l_run[r];
      }
    }
  }
}

// One workgroup per row. Wave w merges the (m, l) of heads w, w + 4 over the row's slices (lanes over slices in
// a fixed order, then a wave reduction); thread t then owns float4 column c = t % C4 of the row's G*128 outputs
// (C4 = 32 G) for slices pg, pg + PG, ... (PG = 256 / C4), eight loads in flight, and the PG sums are added in LDS
// in order (bitwise reproducible).
template <int G>
__global__ __launch_bounds__(256) void paged_combine(PagedParams p) {
  constexpr int C4 = G * kD / 4;
  constexpr int PG = 256 / C4;
  const int row = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int len = min(max(p.lengths[row], 0), p.max_tokens);
  const int ns = min((len + kSliceTok - 1) / kSliceTok, p.slices);
  const float* ml = p.part_ml + size_t(row) * p.slices * G * 2;
  const float4* po = reinterpret_cast<const float4*>(p.part_o + size_t(row) * p.slices * G * kD);
  __shared__ float sM[G], sInvL[G];
  __shared__ float4 red[256];
  for (int h = wave; h < G; h += 4) {
    float mr = -INFINITY, lr = 0.0f;
    for (int s = lane; s < ns; s += kWave) {
      const float2 v = *reinterpret_cast<const float2*>(ml + (s * G + h) * 2);
      const float mn = fmaxf(mr, v.x);
      lr = lr * exp_diff(mr, mn) + v.y * exp_diff(v.x, mn);
      mr = mn;
    }
    const float mx = wave_max(mr);
    const float sum = wave_sum(lr * exp_diff(mr, mx));
    if (lane == 0) {
      sM[h] = mx;
      sInvL[h] = sum > 0.0f ? 1.0f / sum : 0.0f;
    }
  }
  __syncthreads();
  const int c = int(threadIdx.x) % C4, pg = int(threadIdx.x) / C4;
  const int h = 4 * c / kD;
  const float Mh = sM[h];
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = pg; s0 < ns; s0 += 8 * PG) {
    float4 o8[8];
    float m8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = s0 + k * PG;
      o8[k] = s < ns ? po[size_t(s) * C4 + c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      m8[k] = s < ns ? ml[(s * G + h) * 2] : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = exp_diff(m8[k], Mh);
      acc.x += o8[k].x * w;
      acc.y += o8[k].y * w;
      acc.z += o8[k].z * w;
      acc.w += o8[k].w * w;
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  if (int(threadIdx.x) < C4) {
    float4 o = red[threadIdx.x];
#pragma unroll
    for (int g = 1; g < PG; ++g) {
      const float4 v = red[g * C4 + threadIdx.x];
      o.x += v.x;
      o.y += v.y;
      o.z += v.z;
      o.w += v.w;
    }
    const float iL = sInvL[h];
    reinterpret_cast<float4*>(p.out + size_t(row) * G * kD)[c] = make_float4(o.x * iL, o.y * iL, o.z * iL, o.w * iL);
  }
}

template <int G, class T>
hipError_t launch_g(const PagedParams& p, hipStream_t s) {
  const int wg_per_row = (p.slices + kPWaves - 1) / kPWaves;
  hipLaunchKernelGGL((paged_partial<G, T>), dim3(unsigned(int64_t(p.n_rows) * wg_per_row)), dim3(kPWaves * kWave),
                     0, s, p);
  hipLaunchKernelGGL((paged_combine<G>), dim3(unsigned(p.n_rows)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <class T>
hipError_t launch_t(const PagedParams& p, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_g<1, T>(p, s);
    case 2: return launch_g<2, T>(p, s);
    case 4: return launch_g<4, T>(p, s);
    default: return launch_g<8, T>(p, s);
  }
}

int paged_slices(const kvc_paged_decode_args& a) {
  const int64_t max_tokens = int64_t(a.max_pages) * a.page;
  return int((max_tokens + kSliceTok - 1) / kSliceTok);
}

}  // namespace

size_t paged_workspace_bytes(const kvc_paged_decode_args& a) {
  const size_t per = size_t(a.n_rows) * size_t(std::max(paged_slices(a), 1)) * size_t(a.group);
  return align_up(per * 2 * sizeof(float), 256) + align_up(per * kD * sizeof(float), 256);
}

hipError_t launch_paged_decode(const kvc_paged_decode_args& a, void* ws, hipStream_t s) {
  PagedParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_pool = static_cast<const uint16_t*>(a.k_pool);
  p.v_pool = static_cast<const uint16_t*>(a.v_pool);
  p.page_list = a.page_list;
  p.lengths = a.lengths;
  p.out = a.out;
  p.status = a.status;
  p.page_stride = a.page_stride;
  p.n_pool = a.n_pool_pages;
  p.n_rows = int32_t(a.n_rows);
  p.page = a.page;
  p.slices = std::max(paged_slices(a), 1);
  p.max_tokens = a.max_pages * a.page;
  const size_t per = size_t(a.n_rows) * size_t(p.slices) * size_t(a.group);
  char* w = static_cast<char*>(ws);
  p.part_ml = reinterpret_cast<float*>(w);
  p.part_o = reinterpret_cast<float*>(w + align_up(per * 2 * sizeof(float), 256));
  return a.kv_dtype == KVC_BF16 ? launch_t<BF16>(p, a.group, s) : launch_t<F16>(p, a.group, s);
}

}  // namespace kvc
