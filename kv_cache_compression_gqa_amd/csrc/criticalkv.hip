// CriticalKV scores for one layer at prefill (the two-stage selection that uses them is in two_stage.hip).
//
// What it computes follows the CriticalKV page ("Resumo Técnico: CriticalKV"):
//   * "Framework Teórico": the output perturbation of dropping an entry is bounded through its attention weight A
//     and its value projected by the output matrix, V W_O;
//   * "Algoritmo: Seleção Constrainda por Perturbação" (Algorithm 1): a first budget b' = alpha * b goes to the
//     entries of highest attention weight, the rest to the entries of highest A_i * |V_i W_O|_1 (the printed
//     formula drops W_O; the bound and the prose are about the projected values, so they are used). A comes from
//     the host method's observation window (the trailing prompt queries, causal).
//   Per KV head g with query heads h of its group: A_{h,i} = (1/T) sum_j p_{h,j,i} over the T observation
//   queries; N_{h,i} = sum_c |sum_d V_{g,i,d} W_O[h*D + d, c]|; A_g = mean_h A_{h,i}; S2_g = mean_h A_{h,i} N_{h,i}.
//
// Kernels:
//   wo_transpose: W_O [Hq*D][d_model] -> [Hq][d_model][D], so that every MFMA B fragment is one 16-byte load.
//   proj_norm: N on MFMA (v_mfma_f32_32x32x16): a workgroup keeps 256 tokens of V_g in registers (4 waves x 2
//     tiles of 32 tokens x 128 head_dim) and streams W_O,h through LDS in blocks of 32 output columns (double
//     buffered, rows padded to 272 bytes so the 16-byte reads are conflict-free); after each block's 8 k-steps the
//     |.| of the 32x32 products is added to per-row partial sums, so the tokens x d_model product is never stored.
//   obs_attn<1>: per (KV head, chunk of keys) the logits of the G*T observation rows against the chunk on MFMA in
//     the transposed orientation (A = 16 keys x 32 head_dim, B = 16 query rows), online (max, sum) per row;
//   obs_combine: merges the chunks' (max, sum) per row;
//   obs_attn<2>: recomputes the logits, p = exp(s - m) / l, and sums each head's T rows with DPP row reductions
//     into A_{h,i};
//   group_scores: A_g and S2_g.
#include <algorithm>
#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kObs = 32;           // observation queries
constexpr int kObsChunk = 512;     // keys per obs_attn workgroup
constexpr int kTokBlk = 256;       // tokens per proj_norm workgroup
constexpr int kColBlk = 64;        // output columns per LDS block
static_assert(kColBlk == 64, "proj_norm's pipeline is written for two 32-column sub-blocks per W block");
constexpr float kInvSqrtD = 0.088388347648318440550f;

template <class T> struct Mfma;
template <> struct Mfma<BF16> {
  static __device__ __forceinline__ f32x4 m16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 m32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};
template <> struct Mfma<F16> {
  static __device__ __forceinline__ f32x4 m16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  static __device__ __forceinline__ f32x16 m32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---- W_O transpose: wt[h][c][d] = w_o[h*D + d][c] -----------------------------------------------------------------
__global__ __launch_bounds__(256) void wo_transpose(const uint16_t* __restrict__ w_o, uint16_t* __restrict__ wt,
                                                    int dm) {
  __shared__ uint16_t tile[64][66];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;  // r = h*D + d; 64 rows never straddle a head
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    tile[rr][cc] = w_o[size_t(r0 + rr) * dm + c0 + cc];
  }
  __syncthreads();
  const int h = r0 / kD, d0 = r0 % kD;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    wt[(size_t(h) * dm + c0 + cc) * kD + d0 + rr] = tile[rr][cc];
  }
}

// ---- N = |V_g W_O,h|_1 per token ------------------------------------------------------------------------------
// W blocks reach LDS through the load unit directly (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at
// M0 + 16 i), issued as inline asm so that the compiler, which cannot tell which LDS bytes such a load writes, does
// not wait for it before every LDS read; the kernel waits for it explicitly before the barrier that publishes it.
// Nothing else in proj_norm uses M0.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}

// Column c of an LDS W block holds its 16 chunks of 8 head_dim values with chunk q at slot q ^ (c % 16), so the
// 16 columns of one B-fragment read hit 16 distinct 16-byte bank groups.
template <class T>
__global__ __launch_bounds__(256) void proj_norm(const uint16_t* __restrict__ v, const uint16_t* __restrict__ wt,
                                                 float* __restrict__ norm, int n, int group, int dm) {
  __shared__ __attribute__((aligned(16))) uint16_t wl[2][kColBlk * kD];
  const int h = blockIdx.y, g = h / group;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok0 = blockIdx.x * kTokBlk + 64 * wave;
  // A fragments: tile t = tokens tok0 + 32t + lane%32; k-step j = head_dim 16j + 8*(lane/32) .. +7
  u32x4 a[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = min(tok0 + 32 * t + (lane & 31), n - 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[t][j] = ld16(v + (size_t(g) * n + tok) * kD + 16 * j + 8 * (lane >> 5));
  }
  const uint16_t* wh = wt + size_t(h) * dm * kD;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)(&wl[0][0])));
  // block cb -> buffer buf: the wave's instruction k moves columns 4m .. 4m+3 (m = 4k + wave), 1 KB
  auto dma_block = [&](int cb, int buf) {
#pragma unroll
    for (int k = 0; k < kColBlk / 16; ++k) {
      const int m = 4 * k + wave;
      const int c = 4 * m + (lane >> 4);
      const int q = (lane & 15) ^ (c & 15);
      dma16(wh + size_t(kColBlk * cb + c) * kD + 8 * q, lds0 + uint32_t(buf * kColBlk * kD * 2 + m * 1024));
    }
  };
  // B fragments of columns 32sb .. 32sb+31 of buffer buf: column lane%32, k = 16j + 8*(lane/32) .. +7
  auto read_b = [&](int buf, int sb, u32x4 (&b)[8]) {
    const int c = 32 * sb + (lane & 31);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = 2 * j + (lane >> 5);
      b[j] = *reinterpret_cast<const u32x4*>(&wl[buf][c * kD + 8 * (q ^ (c & 15))]);
    }
  };
  f32x16 part0 = f32x16{}, part1 = f32x16{};
  // One sub-block of 32 columns: two independent MFMA chains (tiles 0 and 1), with the |.| sums of the previous
  // sub-block's products (x, y) and the LDS reads of the next sub-block's B fragments interleaved between them.
  auto sub = [&](u32x4 (&b)[8], f32x16& x, f32x16& y, int nbuf, int nsb) {
    f32x16 nx = Mfma<T>::m32(a[0][0], b[0], f32x16{});
    f32x16 ny = Mfma<T>::m32(a[1][0], b[0], f32x16{});
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      nx = Mfma<T>::m32(a[0][j], b[j], nx);
      ny = Mfma<T>::m32(a[1][j], b[j], ny);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      part0[i] += fabsf(x[i]);
      part1[i] += fabsf(y[i]);
    }
    read_b(nbuf, nsb, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    asm volatile("" : "+v"(nx), "+v"(ny));
    __builtin_amdgcn_sched_barrier(0);
    x = nx;
    y = ny;
  };
  const int ncb = dm / kColBlk;
  dma_block(0, 0);
  dma_block(min(1, ncb - 1), 1);
  // The compiler waits for the A fragments here (it does not count the copies), so no wait for them is left
  // inside the loop, where it would also wait for the copy in flight.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(a[t][j]));
  }
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kColBlk / 16) : "memory");  // block 0 landed
  __syncthreads();
  u32x4 b[8];
  read_b(0, 0, b);
  f32x16 x = f32x16{}, y = f32x16{};
  for (int cb = 0; cb < ncb; ++cb) {
    const int cur = cb & 1;
    sub(b, x, y, cur, 1);  // columns 0..31 of block cb; fetches the B fragments of columns 32..63
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of block cb + 1 has landed
    __syncthreads();       // everyone's has, and block cb's buffer is no longer read
    dma_block(min(cb + 2, ncb - 1), cur);
    sub(b, x, y, cur ^ 1, 0);  // columns 32..63; fetches block cb + 1's first B fragments (unused after the last)
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    part0[i] += fabsf(x[i]);
    part1[i] += fabsf(y[i]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy into LDS outlives the workgroup
  const f32x16 part[2] = {part0, part1};
  // row sums over the 32 columns (lanes of one half-wave); D row of acc[i]: 8*(i/4) + 4*(lane/32) + i%4
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = row_sum16(part[t][i]);
      s += __shfl_xor(s, 16, kWave);
      const int tok = tok0 + 32 * t + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if ((lane & 31) == 0 && tok < n) norm[size_t(h) * n + tok] = s;
    }
  }
}

// ---- observation-window attention -----------------------------------------------------------------------------
// One workgroup = the G heads of KV head g (one wave per head) x one chunk of keys. Per wave: B = the head's 32
// query rows (2 column tiles), A = 16 keys per tile. S^T lane layout: column = query row 16ct + lane%16, rows =
// keys 4*(lane/16) + r of the tile.
template <class T, int PASS>
__global__ __launch_bounds__(512) void obs_attn(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                int n, int group, int chunks, float* __restrict__ part_ml,
                                                const float* __restrict__ row_ml, float* __restrict__ a_head) {
  const int g = blockIdx.y, ch = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = g * group + wave;
  const int col = lane & 15, qq = lane >> 4;
  u32x4 bq[2][4];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bq[ct][kk] = ld16(q + (size_t(h) * kObs + 16 * ct + col) * kD + 32 * kk + 8 * qq);
  }
  float m[2], l[2], rm[2], ril[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    m[ct] = -INFINITY;
    l[ct] = 0.0f;
    if (PASS == 2) {
      const int row = wave * kObs + 16 * ct + col;
      rm[ct] = row_ml[(size_t(g) * group * kObs + row) * 2];
      const float lt = row_ml[(size_t(g) * group * kObs + row) * 2 + 1];
      ril[ct] = lt > 0.0f ? 1.0f / lt : 0.0f;
    }
  }
  const int key0 = ch * kObsChunk;
  const int nkeys = min(kObsChunk, n - key0);
  const uint16_t* kg = k + size_t(g) * n * kD;
  // The workgroup's waves (one per query head) share the chunk's keys: batches of kBatch key tiles (64 keys,
  // 16 KiB) are copied global -> LDS by the load unit (global_load_lds_dwordx4; the next batch while the current
  // one is computed) instead of every wave loading the same keys. Key row r's 16-byte chunk q sits at slot
  // q ^ (r % 16), so each A-fragment read (16 rows, one chunk each) is conflict-free.
  constexpr int kBatch = 4;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kBatch * 16 * kD];
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const uint32_t ks0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)(&ks[0][0])));
  const int ntiles = (nkeys + 15) / 16;
  const int nbatch = (ntiles + kBatch - 1) / kBatch;
  // batch bt -> buffer buf: instruction m (of 16, taken by the waves in turn) moves key rows 4m .. 4m+3
  auto copy_batch = [&](int bt, int buf) {
    for (int m = wave; m < kBatch * 4; m += group) {
      const int row = 4 * m + (lane >> 4);
      const int qc = (lane & 15) ^ (row & 15);
      const int tok = min(key0 + kBatch * 16 * bt + row, n - 1);
      dma16(kg + size_t(tok) * kD + 8 * qc, ks0 + uint32_t(buf * kBatch * 16 * kD * 2 + m * 1024));
    }
  };
  // MASKED: the chunk holds keys past the end or inside the observation window (causal mask), which only the last
  // chunks do; the others skip the per-element checks
  auto sweep = [&](auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    for (int bt = 0; bt < nbatch; ++bt) {
      const int cur = bt & 1;
      if (bt + 1 < nbatch) copy_batch(bt + 1, cur ^ 1);
      const int tb = bt * kBatch;
      u32x4 ka[kBatch][4];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int row = 16 * b + col;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          ka[b][kk] = *reinterpret_cast<const u32x4*>(&ks[cur][row * kD + 8 * ((4 * kk + qq) ^ col)]);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int tile_key0 = key0 + 16 * (tb + b);
        if (tile_key0 >= key0 + nkeys) break;
        f32x4 s[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          s[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) s[ct] = Mfma<T>::m16(ka[b][kk], bq[ct][kk], s[ct]);
        }
        float pv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int obs_pos = n - kObs + 16 * ct + col;  // position of this column's query
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = tile_key0 + 4 * qq + r;
            const bool ok = !MASKED || (key < n && key <= obs_pos);
            const float sv = ok ? s[ct][r] * kInvSqrtD : -INFINITY;
            if (PASS == 1) {
              s[ct][r] = sv;
            } else {
              pv[r] += exp_diff(sv, rm[ct]) * ril[ct];
            }
          }
          if (PASS == 1) {
            const float mt = fmaxf(fmaxf(s[ct][0], s[ct][1]), fmaxf(s[ct][2], s[ct][3]));
            const float mn = fmaxf(m[ct], mt);
            float add = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) add += exp_diff(s[ct][r], mn);
            l[ct] = l[ct] * exp_diff(m[ct], mn) + add;
            m[ct] = mn;
          }
        }
        if (PASS == 2) {
          // sum over the head's 32 query rows: the two column tiles are already added; now the 16 columns
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float tot = row_sum16(pv[r]) * (1.0f / kObs);
            const int key = tile_key0 + 4 * qq + r;
            if (col == 0 && key < n) a_head[size_t(h) * n + key] = tot;
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of the next batch has landed
      __syncthreads();                                   // everyone's has, and the current buffer is free
    }
  };
  copy_batch(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (key0 + kObsChunk <= n - kObs) {
    sweep(std::false_type{});
  } else {
    sweep(std::true_type{});
  }
  if (PASS == 1) {
    // merge the four 16-lane groups (different keys, same query rows)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int x = 16; x <= 32; x <<= 1) {
        const float mo = __shfl_xor(m[ct], x, kWave), lo = __shfl_xor(l[ct], x, kWave);
        const float mn = fmaxf(m[ct], mo);
        l[ct] = l[ct] * exp_diff(m[ct], mn) + lo * exp_diff(mo, mn);
        m[ct] = mn;
      }
      if (qq == 0) {
        const int row = wave * kObs + 16 * ct + col;
        float* o = part_ml + ((size_t(g) * chunks + ch) * group * kObs + row) * 2;
        o[0] = m[ct];
        o[1] = l[ct];
      }
    }
  }
}

// one wave per observation row: lanes merge strided chunks, then a butterfly merges the lanes (fixed order)
__global__ __launch_bounds__(256) void obs_combine(const float* __restrict__ part_ml, float* __restrict__ row_ml,
                                                   int rows_per_g, int chunks) {
  const int g = blockIdx.y;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= rows_per_g) return;
  float m = -INFINITY, l = 0.0f;
  for (int c = lane; c < chunks; c += kWave) {
    const float* p = part_ml + ((size_t(g) * chunks + c) * rows_per_g + row) * 2;
    const float mn = fmaxf(m, p[0]);
    l = l * exp_diff(m, mn) + p[1] * exp_diff(p[0], mn);
    m = mn;
  }
#pragma unroll
  for (int x = 1; x < kWave; x <<= 1) {
    const float mo = __shfl_xor(m, x, kWave), lo = __shfl_xor(l, x, kWave);
    const float mn = fmaxf(m, mo);
    // combine in lane order so that every lane gets the same bits
    const bool first = (lane & x) == 0;
    const float la = first ? l : lo, ma = first ? m : mo, lb = first ? lo : l, mb = first ? mo : m;
    l = la * exp_diff(ma, mn) + lb * exp_diff(mb, mn);
    m = mn;
  }
  if (lane == 0) {
    row_ml[(size_t(g) * rows_per_g + row) * 2] = m;
    row_ml[(size_t(g) * rows_per_g + row) * 2 + 1] = l;
  }
}

__global__ __launch_bounds__(256) void group_scores(const float* __restrict__ a_head, const float* __restrict__ norm,
                                                    float* __restrict__ a_group, float* __restrict__ s2_group, int n,
                                                    int hkv, int group) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(n) * hkv) return;
  const int g = int(i / n), key = int(i - int64_t(g) * n);
  float a = 0.0f, s2 = 0.0f;
  for (int hh = 0; hh < group; ++hh) {
    const size_t idx = size_t(g * group + hh) * n + key;
    a += a_head[idx];
    s2 += a_head[idx] * norm[idx];
  }
  a_group[i] = a / group;
  s2_group[i] = s2 / group;
}

size_t al(size_t x) { return align_up(x, 256); }

int obs_chunks(const kvc_criticalkv_args& a) { return (a.n_keys + kObsChunk - 1) / kObsChunk; }

}  // namespace

size_t criticalkv_workspace_bytes(const kvc_criticalkv_args& a) {
  const size_t G = size_t(a.hq / a.hkv);
  return al(size_t(a.hq) * a.d_model * kD * 2) + al(size_t(a.hkv) * obs_chunks(a) * G * kObs * 2 * 4) +
         al(size_t(a.hkv) * G * kObs * 2 * 4);
}

bool criticalkv_supported(const kvc_criticalkv_args& a) {
  const int G = a.hkv > 0 ? a.hq / a.hkv : 0;
  return a.n_obs == kObs && a.head_dim == kD && (G == 1 || G == 2 || G == 4 || G == 8) && a.hq == G * a.hkv &&
         a.d_model % 64 == 0 && a.d_model >= 64 && a.n_keys >= kObs;
}

template <class T>
hipError_t launch_ckv(const kvc_criticalkv_args& a, void* ws, hipStream_t s) {
  const int G = a.hq / a.hkv, n = a.n_keys, dm = a.d_model, chunks = obs_chunks(a);
  char* w = static_cast<char*>(ws);
  uint16_t* wt = reinterpret_cast<uint16_t*>(w);
  w += al(size_t(a.hq) * dm * kD * 2);
  float* part_ml = reinterpret_cast<float*>(w);
  w += al(size_t(a.hkv) * chunks * G * kObs * 2 * 4);
  float* row_ml = reinterpret_cast<float*>(w);
  const uint16_t* q = static_cast<const uint16_t*>(a.q_obs);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  hipLaunchKernelGGL(wo_transpose, dim3(dm / 64, a.hq * kD / 64), dim3(256), 0, s, static_cast<const uint16_t*>(a.w_o),
                     wt, dm);
  hipLaunchKernelGGL((proj_norm<T>), dim3((n + kTokBlk - 1) / kTokBlk, a.hq), dim3(256), 0, s, v, wt, a.norm, n, G, dm);
  hipLaunchKernelGGL((obs_attn<T, 1>), dim3(chunks, a.hkv), dim3(64 * G), 0, s, q, k, n, G, chunks, part_ml,
                     static_cast<const float*>(nullptr), static_cast<float*>(nullptr));
  hipLaunchKernelGGL(obs_combine, dim3((G * kObs + 3) / 4, a.hkv), dim3(256), 0, s, part_ml, row_ml, G * kObs,
                     chunks);
  hipLaunchKernelGGL((obs_attn<T, 2>), dim3(chunks, a.hkv), dim3(64 * G), 0, s, q, k, n, G, chunks,
                     static_cast<float*>(nullptr), row_ml, a.a_head);
  const int64_t tot = int64_t(n) * a.hkv;
  hipLaunchKernelGGL(group_scores, dim3(unsigned((tot + 255) / 256)), dim3(256), 0, s, a.a_head, a.norm, a.a_group,
                     a.s2_group, n, a.hkv, G);
  return hipGetLastError();
}

hipError_t launch_criticalkv(const kvc_criticalkv_args& a, void* ws, hipStream_t s) {
  return a.kv_dtype == KVC_BF16 ? launch_ckv<BF16>(a, ws, s) : launch_ckv<F16>(a, ws, s);
}

}  // namespace kvc
