// Split-K GQA decode attention over the mixed full-precision / INT2 / tail cache, with the window scores fused.
//
// What it computes follows the QEvict page ("Mecanismos Principais"): attention over the resident windows
// (full-precision tier and INT2 tier, the latter dequantised in registers), the cumulative window score
// updated from the attention mass of each window, GQA (G query heads per KV head).
//
// Two kernels per step:
//   decode_partial  one workgroup per (unit, chunk). A chunk is up to 8 full windows, 16 INT2 windows or 256
//                   tail tokens. Each wave streams 32-token windows: lane (r, j) owns token slot r (0..3) of
//                   every 4-token row and head_dim slice [8j, 8j+8); K rows arrive as 16-byte loads (256 B per
//                   token, 1 KiB per wave instruction), logits are reduced over the 16 lanes of a slot, the
//                   softmax is online at window granularity, and the window's exp-sum (with its reference max)
//                   is written for the score. The four waves are merged in LDS into one (m, l, o) partial.
//   decode_combine  one workgroup per unit: merges the chunk partials in fixed order (bitwise reproducible),
//                   writes o, turns the window exp-sums into probability mass, adds it to the cumulative score,
//                   optionally rewrites the stored logits as probabilities, and advances the tail.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;
constexpr int kFullWinPerChunk = 8;
constexpr int kInt2WinPerChunk = 16;
constexpr int kTailTokPerChunk = 256;
constexpr float kInvSqrtD = 0.088388347648318440550f;  // 1/sqrt(128)

struct DecodeParams {
  int NW, TM;
  const uint16_t* k_win;
  const uint16_t* v_win;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint32_t* k_meta;
  const uint32_t* v_meta;
  uint16_t* k_tail;
  uint16_t* v_tail;
  int32_t* tail_len;
  const int32_t* res_list;
  const int32_t* n_full;
  const int32_t* n_int2;
  const int32_t* n_windows;
  const int8_t* tier;
  float* cum;
  int32_t* status;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  float* out;
  float* probs;
  float* mass;
  long probs_stride;
  int accumulate;
  int max_full, max_int2, max_tail;
  int CF, CQ, CT, CH;
  float* part_ml;  // [U][CH][G][2]
  float* part_o;   // [U][CH][G][D]
  float* wsum;     // [U][NW][G]
  float* wref;     // [U][NW][G]
};

// ---- K/V sources: 8 consecutive elements (dims 8j..8j+7) of one token --------------------------------------
template <class T>
struct FullSrc {
  const uint16_t* k;
  const uint16_t* v;
  __device__ void load_k(int tok, int j, float (&f)[8]) const {
    unpack8<T>(*reinterpret_cast<const uint4*>(k + size_t(tok) * kD + 8 * j), f);
  }
  __device__ void load_v(int tok, int j, float (&f)[8]) const {
    unpack8<T>(*reinterpret_cast<const uint4*>(v + size_t(tok) * kD + 8 * j), f);
  }
};

struct Int2Src {
  const uint8_t* kc;
  const uint8_t* vc;
  const uint32_t* km;
  const uint32_t* vm;
  static __device__ void deq(const uint8_t* codes, const uint32_t* meta, int tok, int j, float (&f)[8]) {
    const uint32_t bits = *reinterpret_cast<const uint16_t*>(codes + tok * kCodeBytes + 2 * j);
    const uint32_t mw = meta[tok * kGroups + (j >> 2)];
    const float s = half_bits_to_float(mw & 0xFFFFu);
    const float z = half_bits_to_float(mw >> 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = fmaf(float((bits >> (2 * e)) & 3u), s, z);
  }
  __device__ void load_k(int tok, int j, float (&f)[8]) const { deq(kc, km, tok, j, f); }
  __device__ void load_v(int tok, int j, float (&f)[8]) const { deq(vc, vm, tok, j, f); }
};

// Tail tokens base + tok; position tl is the new token (read from k_new/v_new and written into the tail).
template <class T>
struct TailSrc {
  uint16_t* kt;
  uint16_t* vt;
  const uint16_t* kn;
  const uint16_t* vn;
  int tl, base;
  __device__ void load(uint16_t* tail, const uint16_t* nw, int tok, int j, float (&f)[8]) const {
    const int i = base + tok;
    uint4 x;
    if (i < tl) {
      x = *reinterpret_cast<const uint4*>(tail + size_t(i) * kD + 8 * j);
    } else {
      x = *reinterpret_cast<const uint4*>(nw + 8 * j);
      *reinterpret_cast<uint4*>(tail + size_t(i) * kD + 8 * j) = x;
    }
    unpack8<T>(x, f);
  }
  __device__ void load_k(int tok, int j, float (&f)[8]) const { load(kt, kn, tok, j, f); }
  __device__ void load_v(int tok, int j, float (&f)[8]) const { load(vt, vn, tok, j, f); }
};

// One (pseudo-)window of up to 32 tokens for one wave. Lane (r, j): tokens 4t + r, dims [8j, 8j+8).
template <int G, class Src>
__device__ __forceinline__ void attend_window(const Src& src, int n_valid, int r, int j, int lane,
                                              const float (&qf)[G][8], float (&m)[G], float (&l)[G],
                                              float (&o)[G][8], float* probs_base, long stride, float* wsum,
                                              float* wref) {
  float s[8][G];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int tok = 4 * t + r;
    float kf[8];
    if (tok < n_valid) {
      src.load_k(tok, j, kf);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(qf[h][e], kf[e], acc);
      acc = xor_sum(acc, 1);
      acc = xor_sum(acc, 2);
      acc = xor_sum(acc, 4);
      acc = xor_sum(acc, 8);
      s[t][h] = tok < n_valid ? acc : -INFINITY;
    }
  }
  float pw[8][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mw = s[0][h];
#pragma unroll
    for (int t = 1; t < 8; ++t) mw = fmaxf(mw, s[t][h]);
    mw = xor_max(mw, 16);
    mw = xor_max(mw, 32);
    const float mnew = fmaxf(m[h], mw);
    const float alpha = exp_diff(m[h], mnew);
    l[h] *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
    m[h] = mnew;
    float ssum = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      pw[t][h] = exp_diff(s[t][h], mnew);
      ssum += pw[t][h];
    }
    ssum = xor_sum(ssum, 16);
    ssum = xor_sum(ssum, 32);
    l[h] += ssum;
    if (wsum != nullptr && lane == 0) {
      wsum[h] = ssum;
      wref[h] = mnew;
    }
  }
  if (probs_base != nullptr && j == 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tok = 4 * t + r;
      if (tok < n_valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) probs_base[h * stride + tok] = s[t][h];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int tok = 4 * t + r;
    if (tok < n_valid) {
      float vf[8];
      src.load_v(tok, j, vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pw[t][h], vf[e], o[h][e]);
      }
    }
  }
}

template <int G, class T>
__global__ __launch_bounds__(kBlock) void decode_partial(DecodeParams p) {
  const int u = blockIdx.x / p.CH;
  const int c = blockIdx.x - u * p.CH;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 4;
  const int j = lane & 15;

  // device counts are clamped to the host bounds the grid was sized for, so every index stays in range
  const int nf_dev = p.n_full[u], nq_dev = p.n_int2[u], tl_dev = p.tail_len[u];
  const int nf = min(max(nf_dev, 0), p.max_full);
  const int nq = min(max(nq_dev, 0), p.max_int2);
  const int tl = min(max(tl_dev, 0), p.max_tail);
  const int has_new = p.k_new != nullptr ? 1 : 0;
  if (c == 0 && threadIdx.x == 0 && (nf != nf_dev || nq != nq_dev || tl != tl_dev)) {
    atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
  }

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    unpack8<T>(*reinterpret_cast<const uint4*>(p.q + (size_t(u) * G + h) * kD + 8 * j), qf[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[h][e] *= kInvSqrtD;
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
  }

  const size_t unit_win = size_t(u) * p.NW;
  float* probs_u = p.probs != nullptr ? p.probs + size_t(u) * G * p.probs_stride : nullptr;
  const int* res = p.res_list + unit_win;

  if (c < p.CF) {
    const int per_wave = kFullWinPerChunk / kWavesPerBlock;
    for (int k = 0; k < per_wave; ++k) {
      const int rp = c * kFullWinPerChunk + wave * per_wave + k;  // position among FULL windows
      if (rp >= nf) break;
      const int w = res[rp];
      if (unsigned(w) >= unsigned(p.NW)) {
        if (lane == 0) atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
        break;
      }
      const size_t off = (unit_win + w) * size_t(kW) * kD;
      FullSrc<T> src{p.k_win + off, p.v_win + off};
      attend_window<G>(src, kW, r, j, lane, qf, m, l, o, probs_u ? probs_u + size_t(rp) * kW : nullptr,
                       p.probs_stride, p.wsum + (unit_win + w) * G, p.wref + (unit_win + w) * G);
    }
  } else if (c < p.CF + p.CQ) {
    const int per_wave = kInt2WinPerChunk / kWavesPerBlock;
    for (int k = 0; k < per_wave; ++k) {
      const int rq = (c - p.CF) * kInt2WinPerChunk + wave * per_wave + k;  // position among INT2 windows
      if (rq >= nq) break;
      const int w = res[nf + rq];
      if (unsigned(w) >= unsigned(p.NW)) {
        if (lane == 0) atomicOr(p.status, KVC_DEV_BOUND_EXCEEDED);
        break;
      }
      const size_t tok0 = (unit_win + w) * size_t(kW);
      Int2Src src{p.k_codes + tok0 * kCodeBytes, p.v_codes + tok0 * kCodeBytes, p.k_meta + tok0 * kGroups,
                  p.v_meta + tok0 * kGroups};
      attend_window<G>(src, kW, r, j, lane, qf, m, l, o, probs_u ? probs_u + size_t(nf + rq) * kW : nullptr,
                       p.probs_stride, p.wsum + (unit_win + w) * G, p.wref + (unit_win + w) * G);
    }
  } else {
    const int total = tl + has_new;
    const int per_wave = kTailTokPerChunk / kWavesPerBlock;  // 64 tokens = 2 pseudo-windows
    const int base0 = (c - p.CF - p.CQ) * kTailTokPerChunk + wave * per_wave;
    for (int k = 0; k < per_wave / kW; ++k) {
      const int base = base0 + k * kW;
      if (base >= total) break;
      const int n_valid = min(kW, total - base);
      TailSrc<T> src{p.k_tail + size_t(u) * p.TM * kD, p.v_tail + size_t(u) * p.TM * kD,
                     has_new ? p.k_new + size_t(u) * kD : nullptr, has_new ? p.v_new + size_t(u) * kD : nullptr,
                     tl, base};
      attend_window<G>(src, n_valid, r, j, lane, qf, m, l, o,
                       probs_u ? probs_u + size_t(nf + nq) * kW + base : nullptr, p.probs_stride, nullptr, nullptr);
    }
  }

  // merge the four token slots of the wave (m and l are already wave-uniform)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[h][e] = xor_sum(o[h][e], 16);
      o[h][e] = xor_sum(o[h][e], 32);
    }
  }
  __shared__ float sm_m[kWavesPerBlock][G];
  __shared__ float sm_l[kWavesPerBlock][G];
  __shared__ float sm_o[kWavesPerBlock][G][kD];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][h][8 * j + e] = o[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  const size_t part = size_t(u) * p.CH + c;
  for (int idx = threadIdx.x; idx < G * kD; idx += kBlock) {
    const int h = idx / kD;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) M = fmaxf(M, sm_m[w][h]);
    float O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) O += sm_o[w][h][idx % kD] * exp_diff(sm_m[w][h], M);
    p.part_o[part * G * kD + idx] = O;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) L += sm_l[w][h] * exp_diff(sm_m[w][h], M);
    p.part_ml[(part * G + h) * 2 + 0] = M;
    p.part_ml[(part * G + h) * 2 + 1] = L;
  }
}

// Combine: kCombineBlocks workgroups per unit. Each recomputes the per-head merge weights f[c][h] =
// exp(m_c - M_h) / L_h of the unit's chunks (cheap), then handles its slice of the outputs, windows and probs.
constexpr int kCombineBlocks = 8;
constexpr int kMaxChunks = 1024;

template <int G>
__global__ __launch_bounds__(256) void decode_combine(DecodeParams p) {
  const int u = blockIdx.x / kCombineBlocks;
  const int b = blockIdx.x - u * kCombineBlocks;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  __shared__ float sM[G], sL[G];
  __shared__ float f[kMaxChunks / 4][G];   // reused in 4 slices when CH > kMaxChunks / 4
  __shared__ float red[4][64];
  const float* ml = p.part_ml + size_t(u) * p.CH * G * 2;
  for (int h = wave; h < G; h += 4) {
    float mx = -INFINITY;
    for (int c = lane; c < p.CH; c += kWave) mx = fmaxf(mx, ml[(c * G + h) * 2]);
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int c = lane; c < p.CH; c += kWave) sum += ml[(c * G + h) * 2 + 1] * exp_diff(ml[(c * G + h) * 2], mx);
    sum = wave_sum(sum);
    if (lane == 0) {
      sM[h] = mx;
      sL[h] = sum;
    }
  }
  __syncthreads();
  if (p.out != nullptr) {
    // this block's 64 outputs (of G*D); 4 threads per output, each over a fixed quarter of the chunks
    const int per_block = G * kD / kCombineBlocks;
    const float* po = p.part_o + size_t(u) * p.CH * G * kD;
    const int q4 = threadIdx.x >> 6;
    float acc[(G * kD / kCombineBlocks + 63) / 64];
#pragma unroll
    for (int k = 0; k < (per_block + 63) / 64; ++k) acc[k] = 0.0f;
    for (int c0 = 0; c0 < p.CH; c0 += kMaxChunks / 4) {
      const int cn = min(kMaxChunks / 4, p.CH - c0);
      for (int i = threadIdx.x; i < cn * G; i += 256) {
        const int c = i / G, h = i - c * G;
        f[c][h] = exp_diff(ml[((c0 + c) * G + h) * 2], sM[h]) / sL[h];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < (per_block + 63) / 64; ++k) {
        const int local = k * 64 + lane;
        if (local < per_block) {
          const int idx = b * per_block + local;
          const int h = idx / kD;
          float a = 0.0f;
#pragma unroll 8
          for (int c = q4; c < cn; c += 4) a += po[size_t(c0 + c) * G * kD + idx] * f[c][h];
          acc[k] += a;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < (per_block + 63) / 64; ++k) {
      red[q4][lane] = acc[k];
      __syncthreads();
      const int local = k * 64 + threadIdx.x;
      if (threadIdx.x < 64 && local < per_block) {
        p.out[size_t(u) * G * kD + b * per_block + local] = ((red[0][threadIdx.x] + red[1][threadIdx.x]) +
                                                             red[2][threadIdx.x]) + red[3][threadIdx.x];
      }
      __syncthreads();
    }
  }
  const size_t unit_win = size_t(u) * p.NW;
  const int nw = min(max(p.n_windows[u], 0), p.NW);
  for (int w = b * 256 + threadIdx.x; w < nw; w += 256 * kCombineBlocks) {
    float mass = 0.0f;
    if (p.tier[unit_win + w] != KVC_TIER_EVICTED) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mass += p.wsum[(unit_win + w) * G + h] * exp_diff(p.wref[(unit_win + w) * G + h], sM[h]) / sL[h];
      }
      mass *= 1.0f / G;
      if (p.accumulate) p.cum[unit_win + w] += mass;
    }
    if (p.mass != nullptr) p.mass[unit_win + w] = mass;
  }
  const int has_new = p.k_new != nullptr ? 1 : 0;
  const int tl = min(max(p.tail_len[u], 0), p.max_tail);
  if (p.probs != nullptr) {
    const int nf = min(max(p.n_full[u], 0), p.max_full);
    const int nq = min(max(p.n_int2[u], 0), p.max_int2);
    const int n_res = (nf + nq) * kW + tl + has_new;
    for (int h = 0; h < G; ++h) {
      float* pr = p.probs + (size_t(u) * G + h) * p.probs_stride;
      for (int i = b * 256 + threadIdx.x; i < n_res; i += 256 * kCombineBlocks) pr[i] = exp_diff(pr[i], sM[h]) / sL[h];
    }
  }
  __syncthreads();
  if (b == 0 && has_new && threadIdx.x == 0) p.tail_len[u] = tl + 1;
}

template <int G, class T>
hipError_t launch_g(const DecodeParams& p, int U, hipStream_t s) {
  hipLaunchKernelGGL((decode_partial<G, T>), dim3(U * p.CH), dim3(kBlock), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine<G>), dim3(U * kCombineBlocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

DecodeGrid decode_grid(const kvc_decode_args& a) {
  DecodeGrid g;
  const int has_new = a.k_new != nullptr ? 1 : 0;
  g.chunks_full = (a.max_full + kFullWinPerChunk - 1) / kFullWinPerChunk;
  g.chunks_int2 = (a.max_int2 + kInt2WinPerChunk - 1) / kInt2WinPerChunk;
  g.chunks_tail = (a.max_tail + has_new + kTailTokPerChunk - 1) / kTailTokPerChunk;
  return g;
}

size_t decode_workspace_bytes(const kvc_cache& c, const kvc_decode_args& a) {
  const DecodeGrid g = decode_grid(a);
  const size_t U = size_t(c.n_units), G = size_t(c.group), CH = size_t(g.chunks());
  size_t b = 0;
  b += align_up(U * CH * G * 2 * sizeof(float), 256);
  b += align_up(U * CH * G * kD * sizeof(float), 256);
  b += 2 * align_up(U * size_t(c.n_windows_max) * G * sizeof(float), 256);
  return b;
}

hipError_t launch_decode(const kvc_cache& c, const kvc_decode_args& a, void* ws, hipStream_t s) {
  const DecodeGrid g = decode_grid(a);
  DecodeParams p{};
  p.NW = c.n_windows_max;
  p.TM = c.tail_max;
  p.k_win = static_cast<const uint16_t*>(c.k_win);
  p.v_win = static_cast<const uint16_t*>(c.v_win);
  p.k_codes = c.k_codes;
  p.v_codes = c.v_codes;
  p.k_meta = c.k_meta;
  p.v_meta = c.v_meta;
  p.k_tail = static_cast<uint16_t*>(c.k_tail);
  p.v_tail = static_cast<uint16_t*>(c.v_tail);
  p.tail_len = c.tail_len;
  p.res_list = c.res_list;
  p.n_full = c.n_full;
  p.n_int2 = c.n_int2;
  p.n_windows = c.n_windows;
  p.tier = c.tier;
  p.cum = c.cum;
  p.status = c.status;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_new = static_cast<const uint16_t*>(a.k_new);
  p.v_new = static_cast<const uint16_t*>(a.v_new);
  p.out = a.out;
  p.probs = a.probs;
  p.mass = a.mass;
  p.probs_stride = a.probs_stride;
  p.accumulate = a.accumulate_cum;
  p.max_full = a.max_full;
  p.max_int2 = a.max_int2;
  p.max_tail = a.max_tail;
  p.CF = g.chunks_full;
  p.CQ = g.chunks_int2;
  p.CT = g.chunks_tail;
  p.CH = g.chunks();
  const size_t U = size_t(c.n_units), G = size_t(c.group), CH = size_t(p.CH);
  char* w = static_cast<char*>(ws);
  p.part_ml = reinterpret_cast<float*>(w);
  w += align_up(U * CH * G * 2 * sizeof(float), 256);
  p.part_o = reinterpret_cast<float*>(w);
  w += align_up(U * CH * G * kD * sizeof(float), 256);
  p.wsum = reinterpret_cast<float*>(w);
  w += align_up(U * size_t(c.n_windows_max) * G * sizeof(float), 256);
  p.wref = reinterpret_cast<float*>(w);
  const int Ui = c.n_units;
  const bool bf = c.kv_dtype == KVC_BF16;
  switch (c.group) {
    case 1: return bf ? launch_g<1, BF16>(p, Ui, s) : launch_g<1, F16>(p, Ui, s);
    case 2: return bf ? launch_g<2, BF16>(p, Ui, s) : launch_g<2, F16>(p, Ui, s);
    case 4: return bf ? launch_g<4, BF16>(p, Ui, s) : launch_g<4, F16>(p, Ui, s);
    case 8: return bf ? launch_g<8, BF16>(p, Ui, s) : launch_g<8, F16>(p, Ui, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvc
