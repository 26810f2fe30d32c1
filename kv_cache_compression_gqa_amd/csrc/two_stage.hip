// CriticalKV two-stage budgeted selection (CriticalKV page, "Algoritmo: Seleção Constrainda por Perturbação"):
// per row (KV head), the first budget1 entries in (a desc, index asc), then the first budget - budget1 of the
// remaining entries in (s2 desc, index asc); the union, ascending.
//
// A row is split into 4096-entry chunks handled by separate workgroups (rows x chunks in flight), so the work is
// spread over the GPU instead of one compute unit per row. Keys are the order-preserving 32-bit images of the
// scores, inverted (a smaller key is a larger score; +0 == -0). Four launches:
//   * ts_hist1: a histogram of the top 11 bits of stage 1's keys (2048 bins) per chunk;
//   * ts_classify1: every workgroup sums its row's chunk histograms and picks the bin b holding the budget1-th
//     key and how many entries of b it needs; entries below b are selected, entries of b become candidates
//     (appended to the row's list with their index and their stage-2 bin); stage 2's row histogram is gathered
//     over every entry not selected outright;
//   * ts_stage2: every (row, chunk) workgroup resolves the row's stage-1 candidates itself (the same result in
//     each: the candidates are ranked by (key, index), which is unique, by a radix select on the 21 low key bits
//     and the 16 index bits), takes the selected ones out of stage 2's histogram, picks stage 2's bin, and
//     classifies its chunk for stage 2 as above; it stores its chunk's count of entries selected so far;
//   * ts_finish: every (row, chunk) workgroup resolves the row's stage-2 candidates itself, counts the selected
//     ones per chunk, and writes its chunk's selected indices at the row's running offset, ascending.
// Resolving in every workgroup of a row replaces a one-workgroup-per-row launch and the per-chunk atomics its
// results needed; the workgroups of a row run side by side.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kT = 256;              // threads per workgroup
constexpr int kPer = 16;             // entries per thread and chunk
constexpr int kC = kT * kPer;        // 4096 entries per chunk
constexpr int kBins = 2048;          // top 11 key bits
constexpr int kCandLds = 7168;       // candidates resolved from LDS; more are resolved from global memory
constexpr int kMaxN = 65536;
constexpr int kMaxChunks = kMaxN / kC;  // 16

struct TsWs {
  uint32_t* hist1;      // [rows][chunks][kBins] stage-1 histogram per chunk
  uint32_t* hist2;      // [rows][kBins] stage-2 histogram over the entries stage 1 does not select outright
  int32_t* ncand;       // [2][rows] candidates appended per stage
  int32_t* pick;        // [2][rows][2] bin (-1: none), entries of the bin still to take
  uint32_t* cand_key;   // [2][rows][n] candidate keys, per stage
  int32_t* cand_idx;    // [2][rows][n] candidate indices, per stage
  uint16_t* cand_bin2;  // [rows][n] stage-2 bin of each stage-1 candidate
  uint8_t* cstate;      // [rows * chunks][n] resolve state of candidates beyond LDS, per workgroup
  uint8_t* sel;         // [rows][n16] 1 = selected (either stage)
  int32_t* ccnt;        // [rows][chunks] entries of each chunk selected by stage 1 or outright by stage 2
};

// inverted order-preserving key: smaller key = larger score; -0 folded onto +0 (NaN: undefined order)
__device__ __forceinline__ uint32_t dkey(float s) {
  const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

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
  for (int w = 0; w < kT / kWave; ++w) {
    base += w < wave ? wsum[w] : V(0);
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Thread t holds the counts of bins 8t .. 8t+7 (c); the bin of the need-th smallest key (need >= 1) and how many
// keys of that bin are needed, into pk[0], pk[1] (bin -1, 0 when need <= 0). Contains barriers.
__device__ void pick_bin(const uint32_t (&c)[8], int need, int* pk, int* wsum) {
  if (threadIdx.x == 0) {  // kept if no bin reaches need (more needed than counted: everything is below)
    pk[0] = 1 << 30;
    pk[1] = 0;
  }
  int own = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) own += int(c[k]);
  int tot;
  const int excl = block_excl_scan<int>(own, wsum, &tot);
  if (need <= 0) {
    if (threadIdx.x == 0) {
      pk[0] = -1;
      pk[1] = 0;
    }
  } else if (excl < need && need <= excl + own) {
    int rem = need - excl, b = 0;
    while (b < 7 && rem > int(c[b])) rem -= int(c[b++]);
    pk[0] = 8 * int(threadIdx.x) + b;
    pk[1] = rem;
  }
  __syncthreads();
}

// ---- stage-1 histograms (per chunk; no atomics to global memory, nothing to clear) -----------------------------
__global__ __launch_bounds__(kT) void ts_hist1(const float* __restrict__ a, int n, int chunks, TsWs ws) {
  __shared__ uint32_t h[kT / kWave][kBins];
  const int row = blockIdx.x / chunks, c = blockIdx.x - row * chunks;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < (kT / kWave) * kBins; i += kT) (&h[0][0])[i] = 0u;
  // this row's stage-2 histogram and candidate counters start at zero (they are filled by later kernels)
  for (int i = c * kT + threadIdx.x; i < kBins; i += chunks * kT) ws.hist2[size_t(row) * kBins + i] = 0u;
  if (c == 0 && threadIdx.x < 2) ws.ncand[threadIdx.x * int(gridDim.x / chunks) + row] = 0;
  const float* ar = a + size_t(row) * n;
  float x[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = c * kC + k * kT + threadIdx.x;
    x[k] = ar[min(e, n - 1)];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = c * kC + k * kT + threadIdx.x;
    if (e < n) atomicAdd(&h[wave][dkey(x[k]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* out = ws.hist1 + (size_t(row) * chunks + c) * kBins;
  for (int b = threadIdx.x; b < kBins; b += kT) out[b] = h[0][b] + h[1][b] + h[2][b] + h[3][b];
}

// This chunk's candidates (bit k of is_cand: entry k*kT + t of thread t) appended to the row's list of a stage:
// one slot range per workgroup from the row's counter, then in thread order. Contains barriers.
__device__ __forceinline__ int append_candidates(uint32_t is_cand, int* ncand_row, int* wsum, int* cbase) {
  int total;
  const int pos = block_excl_scan<int>(__popc(is_cand), wsum, &total);
  if (threadIdx.x == 0) *cbase = total > 0 ? atomicAdd(ncand_row, total) : 0;
  __syncthreads();
  return pos + *cbase;
}

// ---- stage 1: pick the row's bin, select the entries below it, collect the bin's entries as candidates ---------
// Stage 2's histogram is gathered over every entry not selected outright (the candidates included).
__global__ __launch_bounds__(kT) void ts_classify1(const float* __restrict__ a, const float* __restrict__ s2, int n,
                                                   int n16, int chunks, int budget1, TsWs ws) {
  __shared__ uint32_t h2[kT / kWave][kBins];
  __shared__ int wsum[kT / kWave];
  __shared__ int pk[2];
  __shared__ int cbase;
  const int row = blockIdx.x / chunks, c = blockIdx.x - row * chunks;
  const int wave = threadIdx.x >> 6;
  uint8_t* sel = ws.sel + size_t(row) * n16;
  // loads first: this chunk's keys and second scores, and every chunk histogram of the row
  float x[kPer], y[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = min(c * kC + k * kT + int(threadIdx.x), n - 1);
    x[k] = a[size_t(row) * n + e];
    y[k] = s2[size_t(row) * n + e];
  }
  // the row's histogram: thread t sums bins 8t .. 8t+7
  uint32_t cnt[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < (kT / kWave) * kBins; i += kT) (&h2[0][0])[i] = 0u;
  {
    uint4 p[kMaxChunks][2];  // every chunk's bins issued at once (clamped to the last chunk, masked below)
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
      const uint4* hp = reinterpret_cast<const uint4*>(ws.hist1 + (size_t(row) * chunks + min(ch, chunks - 1)) * kBins +
                                                       8 * threadIdx.x);
      p[ch][0] = hp[0];
      p[ch][1] = hp[1];
    }
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
      if (ch < chunks) {
        cnt[0] += p[ch][0].x; cnt[1] += p[ch][0].y; cnt[2] += p[ch][0].z; cnt[3] += p[ch][0].w;
        cnt[4] += p[ch][1].x; cnt[5] += p[ch][1].y; cnt[6] += p[ch][1].z; cnt[7] += p[ch][1].w;
      }
    }
  }
  pick_bin(cnt, budget1, pk, wsum);
  const int b = pk[0];
  if (c == 0 && threadIdx.x == 0) {
    ws.pick[row * 2 + 0] = pk[0];
    ws.pick[row * 2 + 1] = pk[1];
  }
  uint32_t key[kPer];
  uint16_t bin2[kPer];
  uint32_t is_cand = 0u;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = c * kC + k * kT + int(threadIdx.x);
    key[k] = dkey(x[k]);
    bin2[k] = uint16_t(dkey(y[k]) >> 21);
    const int d = int(key[k] >> 21);
    const bool take = e < n && d < b;
    const bool cand = e < n && d == b;
    if (e < n) sel[e] = take ? 1 : 0;
    is_cand |= (cand ? 1u : 0u) << k;
    if (e < n && !take) atomicAdd(&h2[wave][bin2[k]], 1u);
  }
  int pos = append_candidates(is_cand, &ws.ncand[row], wsum, &cbase);
  uint32_t* ck = ws.cand_key + size_t(row) * n;
  int32_t* ci = ws.cand_idx + size_t(row) * n;
  uint16_t* cb = ws.cand_bin2 + size_t(row) * n;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if ((is_cand >> k) & 1u) {
      ck[pos] = key[k];
      ci[pos] = c * kC + k * kT + int(threadIdx.x);
      cb[pos] = bin2[k];
      ++pos;
    }
  }
  for (int bin = threadIdx.x; bin < kBins; bin += kT) {
    const uint32_t s = h2[0][bin] + h2[1][bin] + h2[2][bin] + h2[3][bin];
    if (s != 0u) atomicAdd(&ws.hist2[size_t(row) * kBins + bin], s);
  }
}

// ---- resolve: the first `need` candidates of a row in (key, index) order ---------------------------------------
// Candidate state: 2 = still in play, 1 = selected, 0 = out. Radix passes, most significant first, over the 21 low
// key bits (11 + 10) and the 16 index bits (8 + 8); each pass selects the in-play candidates whose digit is below
// the digit holding the need-th one. Stops as soon as nothing is left to decide. Works on LDS copies (ck, ci, cs
// pointing to LDS) or on global memory (generic pointers). Contains barriers and ends with one, so the state is
// complete for every thread and the histogram is free on return.
struct ResolveLds {
  uint32_t hist[kBins];
  int wsum[kT / kWave];
  int pk[2];
};

template <class IdxT>
__device__ void resolve(const uint32_t* ck, const IdxT* ci, uint8_t* cs, int total, int need, ResolveLds& L) {
  for (int i = threadIdx.x; i < total; i += kT) cs[i] = need <= 0 ? 0 : (need >= total ? 1 : 2);
  __syncthreads();
  if (need <= 0 || need >= total) return;
  for (int pass = 0; pass < 4; ++pass) {
    const int bins = pass == 0 ? 2048 : (pass == 1 ? 1024 : 256);
    for (int i = threadIdx.x; i < kBins; i += kT) L.hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < total; i += kT) {
      if (cs[i] == 2) {
        const uint32_t k = ck[i], x = uint32_t(ci[i]);
        const uint32_t d = pass == 0 ? (k >> 10) & 0x7FFu : pass == 1 ? k & 0x3FFu : pass == 2 ? x >> 8 : x & 0xFFu;
        atomicAdd(&L.hist[d], 1u);
      }
    }
    __syncthreads();
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = 8 * int(threadIdx.x) + k < bins ? L.hist[8 * threadIdx.x + k] : 0u;
    pick_bin(c, need, L.pk, L.wsum);
    const int b = L.pk[0];
    if (b < 0 || b >= bins) return;  // cannot happen (need <= candidates in play); keeps every index in range
    const int in_play = int(L.hist[b]);  // the candidates of bin b stay in play; rem of them are needed
    need = L.pk[1];
    for (int i = threadIdx.x; i < total; i += kT) {
      if (cs[i] == 2) {
        const uint32_t k = ck[i], x = uint32_t(ci[i]);
        const int d = int(pass == 0 ? (k >> 10) & 0x7FFu : pass == 1 ? k & 0x3FFu : pass == 2 ? x >> 8 : x & 0xFFu);
        cs[i] = d < b ? 1 : (d == b ? (need == in_play ? 1 : 2) : 0);
      }
    }
    __syncthreads();
    if (need == in_play) return;  // every candidate still in play was taken
  }
  // (key, index) is unique: the index passes leave one candidate in play with need == 1, which returned above
}

// The row's candidates of one stage, resolved in this workgroup: copied to LDS when they fit, else resolved in
// place with this workgroup's own state array in global memory.
struct CandLds {
  uint32_t k[kCandLds];
  uint16_t i[kCandLds];  // indices < 65536
  uint8_t s[kCandLds];
};

struct RowCands {
  const uint32_t* gk;  // the stage's list of the row
  const int32_t* gi;
  uint8_t* gs;         // this workgroup's state array (used when the list does not fit in LDS)
  int total;
  bool in_lds;
  __device__ bool taken(const CandLds& C, int i) const { return (in_lds ? C.s[i] : gs[i]) == 1; }
  __device__ int index(const CandLds& C, int i) const { return in_lds ? int(C.i[i]) : gi[i]; }
};

__device__ RowCands resolve_row(const TsWs& ws, int stage, int row, int rows, int n, int need, CandLds& C,
                                ResolveLds& L) {
  RowCands r;
  const size_t off = (size_t(stage) * rows + row) * n;
  r.gk = ws.cand_key + off;
  r.gi = ws.cand_idx + off;
  r.gs = ws.cstate + size_t(blockIdx.x) * n;
  r.total = min(ws.ncand[stage * rows + row], n);
  r.in_lds = r.total <= kCandLds;
  if (r.in_lds) {
    for (int i = threadIdx.x; i < r.total; i += kT) {
      C.k[i] = r.gk[i];
      C.i[i] = uint16_t(r.gi[i]);
    }
    __syncthreads();
    resolve(C.k, C.i, C.s, r.total, need, L);
  } else {
    resolve(r.gk, r.gi, r.gs, r.total, need, L);
  }
  return r;
}

// ---- stage 2: stage 1's resolution, stage 2's pick, stage-2 classification of this chunk -----------------------
__global__ __launch_bounds__(kT) void ts_stage2(const float* __restrict__ s2, int n, int n16, int chunks, int budget2,
                                                TsWs ws) {
  __shared__ CandLds C;
  __shared__ ResolveLds L;
  __shared__ uint32_t mine[kC / 32];  // entries of this chunk that stage 1's resolution selects
  __shared__ int wsum[kT / kWave];
  __shared__ int cbase;
  const int row = blockIdx.x / chunks, c = blockIdx.x - row * chunks;
  const int rows = int(gridDim.x) / chunks;
  uint8_t* sel = ws.sel + size_t(row) * n16;
  // loads first: this chunk's second scores and stage-1 outright selections, the row's stage-2 histogram
  float x[kPer];
  uint8_t was[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = min(c * kC + k * kT + int(threadIdx.x), n - 1);
    x[k] = s2[size_t(row) * n + e];
    was[k] = sel[e];
  }
  uint32_t cnt[8];
  {
    const uint4* hp = reinterpret_cast<const uint4*>(ws.hist2 + size_t(row) * kBins + 8 * threadIdx.x);
    const uint4 p0 = hp[0], p1 = hp[1];
    cnt[0] = p0.x; cnt[1] = p0.y; cnt[2] = p0.z; cnt[3] = p0.w;
    cnt[4] = p1.x; cnt[5] = p1.y; cnt[6] = p1.z; cnt[7] = p1.w;
  }
  if (threadIdx.x < kC / 32) mine[threadIdx.x] = 0u;
  const RowCands r = resolve_row(ws, 0, row, rows, n, ws.pick[row * 2 + 1], C, L);
  // the selected stage-1 candidates leave stage 2's histogram; the ones in this chunk are marked
#pragma unroll
  for (int k = 0; k < 8; ++k) L.hist[8 * threadIdx.x + k] = cnt[k];
  __syncthreads();
  const uint16_t* cb = ws.cand_bin2 + size_t(row) * n;
  for (int i = threadIdx.x; i < r.total; i += kT) {
    if (r.taken(C, i)) {
      const int e = r.index(C, i);
      atomicSub(&L.hist[cb[i]], 1u);
      if (e / kC == c) atomicOr(&mine[(e - c * kC) >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; ++k) cnt[k] = L.hist[8 * threadIdx.x + k];
  pick_bin(cnt, budget2, L.pk, wsum);
  const int b = L.pk[0];
  if (c == 0 && threadIdx.x == 0) {
    ws.pick[(rows + row) * 2 + 0] = L.pk[0];
    ws.pick[(rows + row) * 2 + 1] = L.pk[1];
  }
  uint32_t key[kPer];
  uint32_t is_cand = 0u;
  int nsel = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int le = k * kT + int(threadIdx.x);
    const int e = c * kC + le;
    const bool m1 = (mine[le >> 5] >> (le & 31)) & 1u;
    const bool prev = was[k] != 0 || m1;
    key[k] = dkey(x[k]);
    const int d = int(key[k] >> 21);
    const bool take = e < n && !prev && d < b;
    const bool cand = e < n && !prev && d == b;
    if (e < n && (m1 || take)) sel[e] = 1;
    nsel += e < n && (prev || take) ? 1 : 0;
    is_cand |= (cand ? 1u : 0u) << k;
  }
  int chunk_sel;
  (void)block_excl_scan<int>(nsel, wsum, &chunk_sel);
  if (threadIdx.x == 0) ws.ccnt[blockIdx.x] = chunk_sel;
  int pos = append_candidates(is_cand, &ws.ncand[rows + row], wsum, &cbase);
  uint32_t* ck = ws.cand_key + (size_t(rows) + row) * n;
  int32_t* ci = ws.cand_idx + (size_t(rows) + row) * n;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if ((is_cand >> k) & 1u) {
      ck[pos] = key[k];
      ci[pos] = c * kC + k * kT + int(threadIdx.x);
      ++pos;
    }
  }
}

// ---- finish: stage 2's resolution, then this chunk's selected indices at the row's running offset --------------
// Thread t writes entries 16t .. 16t+15 of the chunk, in order.
__global__ __launch_bounds__(kT) void ts_finish(int n, int n16, int chunks, int budget, TsWs ws,
                                                int32_t* __restrict__ idx_out) {
  __shared__ CandLds C;
  __shared__ ResolveLds L;
  __shared__ uint32_t mine[kC / 32];  // entries of this chunk that stage 2's resolution selects
  __shared__ int chunk_add[kMaxChunks];
  __shared__ int wsum[kT / kWave];
  const int row = blockIdx.x / chunks, c = blockIdx.x - row * chunks;
  const int rows = int(gridDim.x) / chunks;
  // loads first: the earlier chunks' counts and this thread's 16 selection bytes
  int prev[kMaxChunks];
#pragma unroll
  for (int ch = 0; ch < kMaxChunks; ++ch) prev[ch] = ch < c ? ws.ccnt[row * chunks + ch] : 0;
  const int e0 = c * kC + 16 * int(threadIdx.x);
  uint32_t wv[4] = {0u, 0u, 0u, 0u};
  if (e0 < n16) {
    const uint4 v = *reinterpret_cast<const uint4*>(ws.sel + size_t(row) * n16 + e0);
    wv[0] = v.x; wv[1] = v.y; wv[2] = v.z; wv[3] = v.w;
  }
  if (threadIdx.x < kC / 32) mine[threadIdx.x] = 0u;
  if (threadIdx.x < kMaxChunks) chunk_add[threadIdx.x] = 0;
  const RowCands r = resolve_row(ws, 1, row, rows, n, ws.pick[(rows + row) * 2 + 1], C, L);
  for (int i = threadIdx.x; i < r.total; i += kT) {
    if (r.taken(C, i)) {
      const int e = r.index(C, i);
      atomicAdd(&chunk_add[e / kC], 1);
      if (e / kC == c) atomicOr(&mine[(e - c * kC) >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int ch = 0; ch < kMaxChunks; ++ch) base += ch < c ? prev[ch] + chunk_add[ch] : 0;
  const uint32_t m16 = (mine[(16 * threadIdx.x) >> 5] >> ((16 * threadIdx.x) & 31)) & 0xFFFFu;
  uint32_t bits = 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bool s = ((wv[j >> 2] >> (8 * (j & 3))) & 0xFFu) != 0u || ((m16 >> j) & 1u);
    bits |= (e0 + j < n && s ? 1u : 0u) << j;
  }
  int tot;
  int pos = base + block_excl_scan<int>(__popc(bits), wsum, &tot);
  int32_t* out = idx_out + size_t(row) * budget;
  while (bits) {
    const int j = __builtin_ctz(bits);
    bits &= bits - 1;
    if (pos < budget) out[pos] = e0 + j;
    ++pos;
  }
}

size_t al(size_t x) { return align_up(x, 256); }

struct TsLayout {
  int chunks, n16;
  size_t hist1, hist2, ncand, pick, cand_key, cand_idx, cand_bin2, cstate, sel, ccnt, total;
};

TsLayout ts_layout(const kvc_two_stage_args& a) {
  TsLayout L;
  const size_t rows = size_t(std::max(a.rows, 0)), n = size_t(std::max(a.n, 1));
  L.chunks = int((n + kC - 1) / kC);
  L.n16 = int((n + 15) / 16 * 16);
  size_t o = 0;
  L.hist1 = o;
  o += al(rows * L.chunks * kBins * 4);
  L.hist2 = o;
  o += al(rows * kBins * 4);
  L.ncand = o;
  o += al(2 * rows * 4);
  L.pick = o;
  o += al(2 * rows * 2 * 4);
  L.cand_key = o;
  o += al(2 * rows * n * 4);
  L.cand_idx = o;
  o += al(2 * rows * n * 4);
  L.cand_bin2 = o;
  o += al(rows * n * 2);
  L.cstate = o;
  o += al(rows * L.chunks * n);
  L.sel = o;
  o += al(rows * size_t(L.n16));
  L.ccnt = o;
  o += al(rows * size_t(L.chunks) * 4);
  L.total = o;
  return L;
}

}  // namespace

size_t two_stage_workspace_bytes(const kvc_two_stage_args& a) { return ts_layout(a).total; }

hipError_t launch_two_stage(const kvc_two_stage_args& a, int32_t budget1, void* ws_ptr, hipStream_t s) {
  static_assert(kMaxN <= (1 << 16), "candidate indices are ranked on 16 bits");
  const TsLayout Lo = ts_layout(a);
  char* w = static_cast<char*>(ws_ptr);
  TsWs ws;
  ws.hist1 = reinterpret_cast<uint32_t*>(w + Lo.hist1);
  ws.hist2 = reinterpret_cast<uint32_t*>(w + Lo.hist2);
  ws.ncand = reinterpret_cast<int32_t*>(w + Lo.ncand);
  ws.pick = reinterpret_cast<int32_t*>(w + Lo.pick);
  ws.cand_key = reinterpret_cast<uint32_t*>(w + Lo.cand_key);
  ws.cand_idx = reinterpret_cast<int32_t*>(w + Lo.cand_idx);
  ws.cand_bin2 = reinterpret_cast<uint16_t*>(w + Lo.cand_bin2);
  ws.cstate = reinterpret_cast<uint8_t*>(w + Lo.cstate);
  ws.sel = reinterpret_cast<uint8_t*>(w + Lo.sel);
  ws.ccnt = reinterpret_cast<int32_t*>(w + Lo.ccnt);
  const unsigned grid = unsigned(a.rows) * unsigned(Lo.chunks);
  const int budget2 = a.budget - budget1;
  hipLaunchKernelGGL(ts_hist1, dim3(grid), dim3(kT), 0, s, a.a, a.n, Lo.chunks, ws);
  hipLaunchKernelGGL(ts_classify1, dim3(grid), dim3(kT), 0, s, a.a, a.s2, a.n, Lo.n16, Lo.chunks, budget1, ws);
  hipLaunchKernelGGL(ts_stage2, dim3(grid), dim3(kT), 0, s, a.s2, a.n, Lo.n16, Lo.chunks, budget2, ws);
  hipLaunchKernelGGL(ts_finish, dim3(grid), dim3(kT), 0, s, a.n, Lo.n16, Lo.chunks, a.budget, ws, a.idx);
  return hipGetLastError();
}

}  // namespace kvc
