// C-ABI entry points: host-side validation, workspace sizing, dispatch. No device memory is allocated here and
// no state is kept between calls.
#include <stdint.h>

#include <cmath>

#include "kvc_internal.h"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_cache(const kvc_cache* c) {
  if (c == nullptr) return KVC_E_INVALID;
  if (c->head_dim != kvc::kD || c->window != kvc::kW) return KVC_E_UNSUPPORTED;
  if (!(c->group == 1 || c->group == 2 || c->group == 4 || c->group == 8)) return KVC_E_UNSUPPORTED;
  if (c->kv_dtype != KVC_F16 && c->kv_dtype != KVC_BF16) return KVC_E_UNSUPPORTED;
  if (c->n_units < 1 || c->n_units > 16384 || c->n_windows_max < 1 || c->n_windows_max > 16384 ||
      c->tail_max < 32 || c->tail_max % 32 != 0 || c->reserved != 0) {
    return KVC_E_INVALID;
  }
  if (c->full_slots < 1 || c->ledger_slots < 1 || c->full_slots > c->n_windows_max ||
      c->ledger_slots > c->n_windows_max) {
    return KVC_E_INVALID;
  }
  const void* need16[] = {c->k_full, c->v_full, c->k_tail, c->v_tail, c->k_codes, c->v_codes, c->k_meta, c->v_meta};
  for (const void* p : need16) {
    if (p == nullptr || !aligned(p, 16)) return KVC_E_INVALID;
  }
  const void* need4[] = {c->n_windows, c->tail_len, c->cum, c->res_list, c->res_slot, c->full_slot, c->ledger_slot,
                         c->n_full, c->n_int2, c->status};
  for (const void* p : need4) {
    if (p == nullptr || !aligned(p, 4)) return KVC_E_INVALID;
  }
  if (c->tier == nullptr || c->ledgered == nullptr) return KVC_E_INVALID;
  if (c->reserved2 != 0) return KVC_E_INVALID;
  if (c->k_sum != nullptr) {
    if (c->v_sum == nullptr || c->n_sum == nullptr || !aligned(c->k_sum, 16) || !aligned(c->v_sum, 16) ||
        !aligned(c->n_sum, 4) || c->sum_max < kvc::kW || c->sum_max % kvc::kW != 0) {
      return KVC_E_INVALID;
    }
  } else if (c->sum_max != 0) {
    return KVC_E_INVALID;
  }
  return KVC_OK;
}

int check_decode(const kvc_cache* c, const kvc_decode_args* a, bool need_out) {
  int st = check_cache(c);
  if (st != KVC_OK) return st;
  if (a == nullptr || a->q == nullptr || !aligned(a->q, 16) || a->reserved != 0) return KVC_E_INVALID;
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) return KVC_E_INVALID;
  if (a->k_new != nullptr && (!aligned(a->k_new, 16) || !aligned(a->v_new, 16))) return KVC_E_INVALID;
  if (need_out && a->out == nullptr) return KVC_E_INVALID;
  if (a->accumulate_cum != 0 && a->accumulate_cum != 1) return KVC_E_INVALID;
  if (a->reserved2 != 0 || a->max_summary < 0) return KVC_E_INVALID;
  if (a->max_summary > 0) {
    if (c->k_sum == nullptr || a->max_summary > c->sum_max) return KVC_E_BUDGET;
    if (a->probs != nullptr) return KVC_E_UNSUPPORTED;
  }
  if (a->token_weight != nullptr &&
      (!aligned(a->token_weight, 4) || a->weight_stride < int64_t(c->n_windows_max) * kvc::kW)) {
    return KVC_E_INVALID;
  }
  const int has_new = a->k_new != nullptr ? 1 : 0;
  if (a->max_full < 0 || a->max_int2 < 0 || a->max_tail < 0) return KVC_E_BUDGET;
  if (int64_t(a->max_full) + a->max_int2 > c->n_windows_max) return KVC_E_BUDGET;
  if (int64_t(a->max_tail) + has_new > c->tail_max) return KVC_E_BUDGET;
  if (int64_t(a->max_full) + a->max_int2 + a->max_tail + has_new == 0) return KVC_E_INVALID;
  if (a->probs != nullptr) {
    const int64_t need = int64_t(kvc::kW) * (a->max_full + a->max_int2) + a->max_tail + has_new;
    if (a->probs_stride < need) return KVC_E_INVALID;
  }
  if (!kvc::decode_supported(*c, *a)) return KVC_E_UNSUPPORTED;
  return KVC_OK;
}

int run_decode(const kvc_cache* c, const kvc_decode_args* a, void* ws, size_t ws_bytes, hipStream_t s) {
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < kvc::decode_workspace_bytes(*c, *a)) return KVC_E_WORKSPACE;
  return kvc::launch_decode(*c, *a, ws, s) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int check_list(const kvc_cache* c, const int32_t* list, const int32_t* count, int32_t stride, int64_t max_total) {
  int st = check_cache(c);
  if (st != KVC_OK) return st;
  if (max_total < 0) return KVC_E_BUDGET;
  if (max_total == 0) return KVC_OK;
  if (list == nullptr || count == nullptr || !aligned(list, 4) || !aligned(count, 4)) return KVC_E_INVALID;
  if (stride < 1) return KVC_E_INVALID;
  if (max_total > int64_t(c->n_units) * c->n_windows_max) return KVC_E_BUDGET;
  return KVC_OK;
}

int check_paged(const kvc_paged_decode_args* a) {
  if (a == nullptr || a->reserved != 0) return KVC_E_INVALID;
  if (a->head_dim != kvc::kD) return KVC_E_UNSUPPORTED;
  if (!(a->group == 1 || a->group == 2 || a->group == 4 || a->group == 8)) return KVC_E_UNSUPPORTED;
  if (a->kv_dtype != KVC_F16 && a->kv_dtype != KVC_BF16) return KVC_E_UNSUPPORTED;
  if (a->page < 16 || a->page > 1024 || a->page % 16 != 0) return KVC_E_INVALID;
  if (a->max_pages < 1 || a->page_stride < a->max_pages || int64_t(a->max_pages) * a->page > (int64_t(1) << 24)) {
    return KVC_E_INVALID;
  }
  if (a->n_rows < 0 || a->n_rows > (int64_t(1) << 20) || a->n_pool_pages < 1) return KVC_E_INVALID;
  if (a->n_rows == 0) return KVC_OK;
  const void* need16[] = {a->q, a->k_pool, a->v_pool};
  for (const void* p : need16) {
    if (p == nullptr || !aligned(p, 16)) return KVC_E_INVALID;
  }
  const void* need4[] = {a->page_list, a->lengths, a->out, a->status};
  for (const void* p : need4) {
    if (p == nullptr || !aligned(p, 4)) return KVC_E_INVALID;
  }
  return KVC_OK;
}

int check_retention(const kvc_retention_args* a) {
  if (a == nullptr || a->beta == nullptr || a->score == nullptr) return KVC_E_INVALID;
  if (!aligned(a->beta, 16) || !aligned(a->score, 16)) return KVC_E_INVALID;
  if (a->n_rows < 0 || a->n_tokens <= 0 || a->n_tokens % 4 != 0) return KVC_E_INVALID;
  if (a->n_rows * int64_t(a->n_tokens) >= (int64_t(1) << 31)) return KVC_E_UNSUPPORTED;
  return KVC_OK;
}

int check_topm(const kvc_topm_args* a) {
  if (a == nullptr || a->keep == nullptr || a->row_counts == nullptr || a->status == nullptr || a->reserved != 0 ||
      a->reserved2 != 0) {
    return KVC_E_INVALID;
  }
  const float* src = a->scores != nullptr ? a->scores : a->beta;
  if ((a->scores == nullptr) == (a->beta == nullptr)) return KVC_E_INVALID;  // exactly one input
  if (!aligned(src, 16) || !aligned(a->keep, 16) || !aligned(a->row_counts, 4) || !aligned(a->status, 4)) {
    return KVC_E_INVALID;
  }
  if (a->row_len <= 0 || a->row_len % 16 != 0 || a->n < 0 || a->n % a->row_len != 0) return KVC_E_INVALID;
  // the kernels count blocks per row in int32: (row_len + block - 1) stays below 2^31
  if (a->n > kvc::kTopmMaxN) return KVC_E_UNSUPPORTED;
  if (a->m < 0 || a->m > a->n) return KVC_E_BUDGET;
  return KVC_OK;
}

int check_compact(const kvc_compact_args* a) {
  if (a == nullptr) return KVC_E_INVALID;
  const void* need16[] = {a->keep, a->k_pool, a->v_pool, a->k_out, a->v_out};
  for (const void* p : need16) {
    if (p == nullptr || !aligned(p, 16)) return KVC_E_INVALID;
  }
  const void* need4[] = {a->page_table, a->lengths, a->page_offset, a->n_pages, a->status};
  for (const void* p : need4) {
    if (p == nullptr || !aligned(p, 4)) return KVC_E_INVALID;
  }
  if (a->head_dim != kvc::kD) return KVC_E_UNSUPPORTED;
  if (a->kv_dtype != KVC_F16 && a->kv_dtype != KVC_BF16) return KVC_E_UNSUPPORTED;
  if (a->page <= 0 || a->n_tokens <= 0 || a->n_tokens % 16 != 0 || a->n_tokens % a->page != 0) return KVC_E_INVALID;
  if (a->n_rows < 0 || a->n_src_pages < 1 || a->out_pages_max < 0) return KVC_E_INVALID;
  if (a->n_rows * int64_t(a->n_tokens) >= (int64_t(1) << 31) || a->n_rows > 65535) return KVC_E_UNSUPPORTED;
  return KVC_OK;
}

int check_criticalkv(const kvc_criticalkv_args* a) {
  if (a == nullptr || a->reserved != 0) return KVC_E_INVALID;
  const void* need16[] = {a->q_obs, a->k, a->v, a->w_o, a->a_head, a->norm, a->a_group, a->s2_group};
  for (const void* p : need16) {
    if (p == nullptr || !aligned(p, 16)) return KVC_E_INVALID;
  }
  if (a->kv_dtype != KVC_F16 && a->kv_dtype != KVC_BF16) return KVC_E_UNSUPPORTED;
  if (a->n_keys <= 0 || a->hq <= 0 || a->hkv <= 0 || a->d_model <= 0) return KVC_E_INVALID;
  if (!kvc::criticalkv_supported(*a)) return KVC_E_UNSUPPORTED;
  return KVC_OK;
}

int check_two_stage(const kvc_two_stage_args* a) {
  if (a == nullptr || a->a == nullptr || a->s2 == nullptr || a->idx == nullptr) return KVC_E_INVALID;
  if (!aligned(a->a, 4) || !aligned(a->s2, 4) || !aligned(a->idx, 4)) return KVC_E_INVALID;
  if (a->rows < 0 || a->n < 0) return KVC_E_INVALID;
  if (a->reserved != 0) return KVC_E_INVALID;
  if (a->n > 65536) return KVC_E_UNSUPPORTED;
  if (!(a->alpha >= 0.0 && a->alpha <= 1.0)) return KVC_E_BUDGET;  // NaN fails too
  if (a->budget < 0 || a->budget > a->n) return KVC_E_BUDGET;
  return KVC_OK;
}

}  // namespace

extern "C" {

int kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_str(int status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_E_INVALID: return "invalid argument";
    case KVC_E_UNSUPPORTED: return "unsupported shape, dtype or mode";
    case KVC_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case KVC_E_LEDGER: return "write-once ledger violation";
    case KVC_E_BUDGET: return "budget or bound out of range";
    case KVC_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t kvc_decode_attn_workspace(const kvc_cache* cache, const kvc_decode_args* step) {
  if (check_decode(cache, step, false) != KVC_OK) return 0;
  return kvc::decode_workspace_bytes(*cache, *step);
}

int kvc_decode_attn(const kvc_cache* cache, const kvc_decode_args* step, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  const int st = check_decode(cache, step, true);
  if (st != KVC_OK) return st;
  return run_decode(cache, step, workspace, workspace_bytes, stream);
}

int kvc_decode_attn_static(const kvc_cache* cache, const kvc_decode_args* step, hipStream_t stream) {
  const int st = check_decode(cache, step, true);
  if (st != KVC_OK) return st;
  return kvc::decode_static(*cache, *step, stream);
}

size_t kvc_decode_attn_static_max_bytes(void) { return kvc::kStaticScratchBytes; }

size_t kvc_score_workspace(int32_t mode, const void* args) {
  if (args == nullptr) return 0;
  if (mode == KVC_SCORE_WINDOWS) {
    const kvc_window_score_args* a = static_cast<const kvc_window_score_args*>(args);
    return kvc_decode_attn_workspace(a->cache, a->step);
  }
  if (mode == KVC_SCORE_CRITICALKV) {
    const kvc_criticalkv_args* a = static_cast<const kvc_criticalkv_args*>(args);
    if (check_criticalkv(a) != KVC_OK) return 0;
    return kvc::criticalkv_workspace_bytes(*a);
  }
  return 0;  // KVC_SCORE_RETENTION needs none
}

int kvc_score(int32_t mode, const void* args, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (args == nullptr) return KVC_E_INVALID;
  if (mode == KVC_SCORE_WINDOWS) {
    const kvc_window_score_args* a = static_cast<const kvc_window_score_args*>(args);
    const int st = check_decode(a->cache, a->step, false);
    if (st != KVC_OK) return st;
    kvc_decode_args step = *a->step;
    step.out = nullptr;
    return run_decode(a->cache, &step, workspace, workspace_bytes, stream);
  }
  if (mode == KVC_SCORE_RETENTION) {
    const kvc_retention_args* a = static_cast<const kvc_retention_args*>(args);
    const int st = check_retention(a);
    if (st != KVC_OK) return st;
    return kvc::launch_retention_score(*a, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
  }
  if (mode == KVC_SCORE_CRITICALKV) {
    const kvc_criticalkv_args* a = static_cast<const kvc_criticalkv_args*>(args);
    const int st = check_criticalkv(a);
    if (st != KVC_OK) return st;
    if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < kvc::criticalkv_workspace_bytes(*a)) {
      return KVC_E_WORKSPACE;
    }
    return kvc::launch_criticalkv(*a, workspace, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
  }
  return KVC_E_UNSUPPORTED;
}

size_t kvc_route_workspace(int32_t mode, const void* args) {
  if (mode == KVC_ROUTE_GLOBAL_TOPM) {
    const kvc_topm_args* a = static_cast<const kvc_topm_args*>(args);
    if (check_topm(a) != KVC_OK) return 0;
    return kvc::topm_workspace_bytes(*a);
  }
  if (mode == KVC_ROUTE_TWO_STAGE) {
    const kvc_two_stage_args* a = static_cast<const kvc_two_stage_args*>(args);
    if (check_two_stage(a) != KVC_OK) return 0;
    return kvc::two_stage_workspace_bytes(*a);
  }
  return 0;
}

int kvc_route(int32_t mode, const void* args, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (args == nullptr) return KVC_E_INVALID;
  if (mode == KVC_ROUTE_TIERS) {
    const kvc_tier_route_args* a = static_cast<const kvc_tier_route_args*>(args);
    const int st = check_cache(a->cache);
    if (st != KVC_OK) return st;
    // one workgroup per unit, at most 1024 threads holding at most 4 windows each in registers
    if (a->cache->n_windows_max > kvc::kRouteMaxWindows) return KVC_E_UNSUPPORTED;
    const void* ptrs[] = {a->budget_full, a->budget_int2, a->quant_list, a->n_quant, a->promo_list, a->n_promo};
    for (const void* p : ptrs) {
      if (p == nullptr || !aligned(p, 4)) return KVC_E_INVALID;
    }
    if (a->scores != nullptr && !aligned(a->scores, 4)) return KVC_E_INVALID;
    return kvc::launch_route_tiers(*a, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
  }
  if (mode == KVC_ROUTE_GLOBAL_TOPM) {
    const kvc_topm_args* a = static_cast<const kvc_topm_args*>(args);
    const int st = check_topm(a);
    if (st != KVC_OK) return st;
    if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < kvc::topm_workspace_bytes(*a)) {
      return KVC_E_WORKSPACE;
    }
    return kvc::launch_topm(*a, workspace, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
  }
  if (mode == KVC_ROUTE_TWO_STAGE) {
    const kvc_two_stage_args* a = static_cast<const kvc_two_stage_args*>(args);
    const int st = check_two_stage(a);
    if (st != KVC_OK) return st;
    if (a->rows == 0 || a->budget == 0) return KVC_OK;
    if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < kvc::two_stage_workspace_bytes(*a)) {
      return KVC_E_WORKSPACE;
    }
    // the stage split is CriticalKV's b' = floor(alpha * b), taken here in double precision
    const int32_t budget1 = int32_t(std::floor(a->alpha * double(a->budget)));
    return kvc::launch_two_stage(*a, budget1, workspace, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
  }
  return KVC_E_UNSUPPORTED;
}

size_t kvc_compact_pages_workspace(const kvc_compact_args* args) {
  if (check_compact(args) != KVC_OK) return 0;
  return kvc::compact_workspace_bytes(*args);
}

int kvc_compact_pages(const kvc_compact_args* args, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_compact(args);
  if (st != KVC_OK) return st;
  if (args->n_rows == 0) return KVC_OK;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < kvc::compact_workspace_bytes(*args)) {
    return KVC_E_WORKSPACE;
  }
  return kvc::launch_compact(*args, workspace, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_quantize_int2(const kvc_cache* cache, const int32_t* list, const int32_t* count, int32_t list_stride,
                      int64_t max_total, hipStream_t stream) {
  const int st = check_list(cache, list, count, list_stride, max_total);
  if (st != KVC_OK) return st;
  return kvc::launch_quantize(*cache, list, count, list_stride, max_total, stream) == hipSuccess ? KVC_OK
                                                                                                 : KVC_E_HIP;
}

int kvc_promote(const kvc_cache* cache, const int32_t* list, const int32_t* count, int32_t list_stride,
                int64_t max_total, hipStream_t stream) {
  const int st = check_list(cache, list, count, list_stride, max_total);
  if (st != KVC_OK) return st;
  return kvc::launch_promote(*cache, list, count, list_stride, max_total, stream) == hipSuccess ? KVC_OK
                                                                                                : KVC_E_HIP;
}

size_t kvc_paged_decode_workspace(const kvc_paged_decode_args* args) {
  if (check_paged(args) != KVC_OK) return 0;
  return kvc::paged_workspace_bytes(*args);
}

int kvc_paged_decode_attn(const kvc_paged_decode_args* args, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const int st = check_paged(args);
  if (st != KVC_OK) return st;
  if (args->n_rows == 0) return KVC_OK;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < kvc::paged_workspace_bytes(*args)) {
    return KVC_E_WORKSPACE;
  }
  return kvc::launch_paged_decode(*args, workspace, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_route_diagnostics(const kvc_diag_args* args, hipStream_t stream) {
  if (args == nullptr) return KVC_E_INVALID;
  const kvc_diag_args& a = *args;
  if (a.head_dim != kvc::kD) return KVC_E_UNSUPPORTED;
  if (!(a.group == 1 || a.group == 2 || a.group == 4 || a.group == 8)) return KVC_E_UNSUPPORTED;
  if (a.n_units < 1 || a.n_units > (1 << 20) || a.n_windows_max < 1 || a.n_windows_max > (1 << 20)) {
    return KVC_E_INVALID;
  }
  if (a.tier == nullptr || a.n_windows == nullptr || a.counts == nullptr || a.values == nullptr) return KVC_E_INVALID;
  const void* need4[] = {a.n_windows, a.mass_full, a.o_full, a.o, a.counts, a.values};
  for (const void* p : need4) {
    if (p != nullptr && !aligned(p, 4)) return KVC_E_INVALID;
  }
  return kvc::launch_diagnostics(a, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

size_t kvc_summarize_workspace(const kvc_cache* cache) {
  if (check_cache(cache) != KVC_OK) return 0;
  return kvc::summarize_workspace_bytes(*cache);
}

int kvc_summarize_evicted(const kvc_cache* cache, const int8_t* tier_prev, int32_t max_new, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  const int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (cache->k_sum == nullptr || tier_prev == nullptr) return KVC_E_INVALID;
  if (max_new < 0 || max_new > cache->n_windows_max) return KVC_E_INVALID;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < kvc::summarize_workspace_bytes(*cache)) {
    return KVC_E_WORKSPACE;
  }
  return kvc::launch_summarize(*cache, tier_prev, max_new, workspace, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

size_t kvc_topk_workspace(int64_t n, int64_t k) {
  if (n < 0 || n > kvc::kTopmMaxN || k < 0 || k > n) return 0;
  return kvc::topk_workspace_bytes(n);
}

int kvc_topk(const float* scores, int64_t n, int64_t k, int32_t* idx_out, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
  if (n < 0 || k < 0) return KVC_E_INVALID;
  if (n > kvc::kTopmMaxN) return KVC_E_UNSUPPORTED;
  if (k > n) return KVC_E_BUDGET;
  if (k == 0) return KVC_OK;
  if (scores == nullptr || !aligned(scores, 16) || idx_out == nullptr || !aligned(idx_out, 4)) return KVC_E_INVALID;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < kvc::topk_workspace_bytes(n)) {
    return KVC_E_WORKSPACE;
  }
  return kvc::launch_topk(scores, n, k, idx_out, workspace, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_repack_full(const kvc_cache* cache, void* k_dst, void* v_dst, int32_t dst_slots, hipStream_t stream) {
  const int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (k_dst == nullptr || v_dst == nullptr || !aligned(k_dst, 16) || !aligned(v_dst, 16)) return KVC_E_INVALID;
  if (dst_slots < 1 || dst_slots > cache->n_windows_max) return KVC_E_INVALID;
  return kvc::launch_repack(*cache, k_dst, v_dst, dst_slots, stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

int kvc_read_device_status(const kvc_cache* cache, int32_t* host_status, int32_t clear, hipStream_t stream) {
  if (cache == nullptr || cache->status == nullptr || host_status == nullptr) return KVC_E_INVALID;
  if (hipMemcpyAsync(host_status, cache->status, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess) {
    return KVC_E_HIP;
  }
  if (clear != 0 && hipMemsetAsync(cache->status, 0, sizeof(int32_t), stream) != hipSuccess) return KVC_E_HIP;
  return hipStreamSynchronize(stream) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

}  // extern "C"
