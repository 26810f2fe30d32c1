/* kvc.h — C ABI of the compressed-KV GQA decode library for AMD MI355X (gfx950).
 *
 * One decode step of grouped-query attention over a window-routed, partly INT2-quantised KV cache, as the
 * QEvict page ("Resumo Técnico: QEvict") describes it: contiguous windows, cumulative attention scores,
 * three tiers (full precision / recoverable INT2 / evicted) under a fixed budget, and a write-once quantisation
 * ledger reused by every later promotion and demotion.
 *
 * Conventions for every entry point
 *   - Returns 0 (KVC_OK) or a negative kvc_status. Nothing aborts, nothing throws across the ABI.
 *   - Arguments are validated on the host before any GPU work; an invalid call returns synchronously and
 *     launches nothing.
 *   - All pointers are DEVICE pointers unless a field says "host". The caller allocates and owns every buffer,
 *     workspaces included (sizes from the *_workspace queries). The library allocates no device memory, keeps
 *     no pointer after a call returns and has no global state beyond a per-device cache of the compute-unit
 *     count; buffers must stay valid until the stream has executed the work.
 *   - Work is enqueued on the given stream (0 = the default stream); nothing synchronises and nothing is
 *     copied device->host, so sequences of calls can be captured in a HIP graph.
 *   - Results are bitwise reproducible run to run (no floating-point atomics; fixed combine order).
 *   - Errors found by a kernel (a write-once violation, counts above the host bounds, NaN scores) are OR-ed
 *     into kvc_cache.status as KVC_DEV_* bits; read it with kvc_read_device_status().
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 6

typedef enum {
  KVC_OK = 0,
  KVC_E_INVALID = -1,      /* null pointer, bad size, misaligned buffer, inconsistent arguments */
  KVC_E_UNSUPPORTED = -2,  /* head_dim != 128, window != 32, group not in {1,2,4,8}, unknown dtype or mode */
  KVC_E_WORKSPACE = -3,    /* workspace missing or smaller than the *_workspace query says */
  KVC_E_LEDGER = -4,       /* reserved: no call returns it. Whether a window already has its ledger copy is device
                              state, so a write-once violation is not seen on the host: kvc_quantize_int2 skips
                              such a window and sets KVC_DEV_LEDGER_REWRITE (read with kvc_read_device_status) */
  KVC_E_BUDGET = -5,       /* a budget or bound is negative or larger than the capacity */
  KVC_E_HIP = -6           /* a HIP launch failed */
} kvc_status;

/* Bits OR-ed into *kvc_cache.status by kernels. */
#define KVC_DEV_LEDGER_REWRITE 0x1  /* quantise asked for a window whose ledger copy already exists: skipped */
#define KVC_DEV_BOUND_EXCEEDED 0x2  /* a device count exceeded the host bound given for the launch */
#define KVC_DEV_NAN_SCORE 0x4       /* a routing score was NaN; that unit was not re-routed */

typedef enum { KVC_F16 = 0, KVC_BF16 = 1 } kvc_dtype;
typedef enum { KVC_TIER_FULL = 0, KVC_TIER_INT2 = 1, KVC_TIER_EVICTED = 2 } kvc_tier;

/* The compressed cache of U independent units. A unit is one (batch, layer, KV head); its G query heads share
 * it (grouped-query attention, QEvict page, "Mecanismos Principais"). Window w of a unit holds prefill
 * positions [w*W, (w+1)*W) (QEvict page, "Metodologia": contiguous windows). Window data live in two slot pools
 * whose sizes bound the cache's memory (QEvict page, "Metodologia: QEvict": routing under a fixed memory budget):
 * a window holds a full-precision slot only while it is FULL and a ledger slot from its first demotion to its
 * eviction; tables map windows to slots, so promotion and demotion move no other window's data.
 *
 *   k_full         [U][FS][W][D]   K storage dtype, token-major: full-precision slot s of a unit.
 *   v_full         [U][FS][D][W]   V storage dtype, head_dim-major inside each slot (V^T).
 *   k_codes        [U][LS][W][32]  INT2 ledger slot, K: 32 bytes per token; byte 8*s + 2*g + h holds the codes of
 *                                  head_dim 32g + 8s + 4h + e (e = 0..3) at bits 2e.
 *   k_meta         [U][LS][W][4]   one 32-bit word per (token, 32-element group g): fp16 scale in bits 0..15,
 *                                  fp16 zero in bits 16..31. Dequantised value x = fmaf(code, scale, zero).
 *   v_codes        [U][LS][16][4][8] 16-bit words: word (r, q, dt) holds the codes of tokens 8q + e
 *                                  (e = 0..7) of head_dim 16dt + r at bits 2e.
 *   v_meta         [U][LS][4][4][8] words: word (q, g, e) = scale/zero of token 8q + e, group g.
 *   k_tail         [U][TM][D]      unrouted tail: the partial last prefill window plus every decode-time token,
 *                                  always attended, outside the budgets.
 *   v_tail         [U][TM/32][D][32]  the same tail tokens, head_dim-major inside each 32-token block.
 *   tail_len       [U] int32       valid tail rows (advanced by kvc_decode_attn when it appends a token).
 *   n_windows      [U] int32       routable windows of the unit (<= NW).
 *   tier           [U][NW] int8    kvc_tier of every window (entries >= n_windows unused).
 *   full_slot      [U][NW] int32   the full-precision slot of window w while w is FULL. When an event demotes or
 *                                  evicts w the entry keeps the slot w held until then (the slot is free from then
 *                                  on: see the order of calls below).
 *   ledger_slot    [U][NW] int32   the ledger slot of window w once kvc_route has given it one (at its first
 *                                  demotion); when an event evicts w the entry keeps the slot it held.
 *   ledgered       [U][NW] uint8   1 once the window's INT2 copy has been written (write-once); 0 again at eviction.
 *   cum            [U][NW] float   cumulative window score (sum over steps of the window's attention mass).
 *   res_list       [U][NW] int32   resident windows: the n_full FULL ids ascending, then the n_int2 INT2 ids
 *                                  ascending.
 *   res_slot       [U][NW] int32   the slot of each res_list entry: full-precision slot for the FULL part, ledger
 *                                  slot for the INT2 part (written by kvc_route and kvc_repack_full).
 *   n_full, n_int2 [U] int32       lengths of the two parts of res_list.
 *   status         [1] int32       device error bits (KVC_DEV_*).
 *
 *   k_sum, v_sum, n_sum, sum_max   optional span summaries (SEKV page, "Metodologia" sections 2 and 3: spans that
 *                                  are not expanded enter the attention as summary vectors with a size
 *                                  correction). When a window is evicted, kvc_summarize_evicted appends the means
 *                                  of its 32 keys and values (exact sum, divided by 32, rounded to fp32 and then to
 *                                  the storage dtype) at position n_sum[u]; kvc_decode_attn attends them after the
 *                                  tail with logit q.k/sqrt(D) + ln 32 when step.max_summary > 0. K is token-major,
 *                                  V head_dim-major inside 32-summary blocks (the tail's layouts).
 *
 * Slot pools. A fresh cache has every window FULL: FS >= n_windows with full_slot[w] = w (any distinct slots
 * < FS will do), res_list = res_slot = 0, 1, ..., ledger_slot = -1, ledgered = 0. LS >= b_full + b_int2 holds
 * every ledger copy a unit can have (one per resident window that has been INT2). After the first routing event
 * at most b_full windows are FULL, and kvc_repack_full moves their full-precision copies into a pool of
 * FS' >= b_full slots, so the prefill-sized pool can be released: from then on the cache holds at most
 * (FS' * 16 KiB + LS * 3 KiB) of window data per unit.
 *
 * Order of the calls of one routing event. kvc_route frees the slots of the windows it demotes or evicts and
 * gives the freed slots to the windows it promotes (full-precision slots) or demotes for the first time (ledger
 * slots), lowest free slot first in ascending window order. The calls that read what the event freed must run
 * before the calls that overwrite it: kvc_route, then kvc_summarize_evicted (if summaries are kept; it reads the
 * evicted windows' freed slots), then kvc_quantize_int2 (it reads the freed full-precision slots of the windows
 * demoted for the first time), then kvc_promote (it writes the promoted windows' new full-precision slots).
 *
 * The layouts put, for every MFMA operand the decode kernel builds, one lane's data in one 16-byte load.
 * All K/V rows must be 16-byte aligned (every base pointer 256-byte aligned is sufficient). */
typedef struct kvc_cache {
  int32_t n_units;       /* U >= 1 */
  int32_t group;         /* G query heads per KV head: 1, 2, 4 or 8 */
  int32_t head_dim;      /* D, must be 128 */
  int32_t window;        /* W, must be 32 */
  int32_t n_windows_max; /* NW >= 1 */
  int32_t tail_max;      /* TM >= 32, a multiple of 32 */
  int32_t kv_dtype;      /* kvc_dtype */
  int32_t full_slots;    /* FS >= 1: full-precision slots per unit */
  int32_t ledger_slots;  /* LS >= 1: ledger slots per unit */
  int32_t reserved;      /* must be 0 */
  const int32_t* n_windows;
  void* k_full;
  void* v_full;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint32_t* k_meta;
  uint32_t* v_meta;
  void* k_tail;
  void* v_tail;
  int32_t* tail_len;
  int8_t* tier;
  uint8_t* ledgered;
  int32_t* full_slot;
  int32_t* ledger_slot;
  float* cum;
  int32_t* res_list;
  int32_t* res_slot;
  int32_t* n_full;
  int32_t* n_int2;
  int32_t* status;
  void* k_sum;       /* span summaries (optional, see below): [U][sum_max][D] storage dtype, or NULL */
  void* v_sum;       /* [U][sum_max/32][D][32] storage dtype */
  int32_t* n_sum;    /* [U] summaries written so far */
  int32_t sum_max;   /* capacity per unit, a multiple of 32 (0 with k_sum == NULL) */
  int32_t reserved2; /* must be 0 */
} kvc_cache;

/* One decode step (QEvict page, "Mecanismos Principais": attention is materialised to update the cumulative
 * window scores; GQA supported). Per unit, the resident key set R is: the FULL windows (ascending), the INT2
 * windows (ascending, dequantised in registers), the tail, and — when k_new is given — the new token appended at
 * tail position tail_len. For each query head h of the unit:
 *   s_{h,i} = q_h . k_i / sqrt(D)   p_{h,i} = softmax over R   o_h = sum_i p_{h,i} v_i      (fp32 accumulate)
 *   mass_w  = (1/G) sum_h sum_{i in w} p_{h,i}   for every resident window w;  cum_w += mass_w (if asked).
 *
 *   q        [U][G][D]   storage dtype.
 *   k_new    [U][D]      storage dtype, or NULL (no append). Appended to the tail by this call; tail_len
 *            is incremented at the end of the step. Requires tail_len < tail_max on every unit.
 *   v_new    [U][D]      with k_new.
 *   out      [U][G][D]   float, or NULL (score-only step).
 *   probs    [U][G][probs_stride] float or NULL: per-key probabilities in resident order (FULL keys, INT2 keys,
 *            tail keys, new key). probs_stride >= max over units of W*(n_full+n_int2) + tail_len + (k_new?1:0).
 *   mass     [U][NW] float or NULL: this step's window mass (0 for windows that are not resident).
 *   accumulate_cum  0 or 1.
 *   token_weight   [U][G][weight_stride] float, or NULL. When given, each window key's probability is weighted
 *            per query head in the window score (CriticalKV page, "Algoritmo": the attention weight times the L1
 *            norm of the value projected through W_O, used as a plug-in for an existing accumulation pipeline):
 *            mass_w = (1/G) sum_h sum_{i in w} p_{h,i} token_weight[u][h][i], i the prefill position (w*W + j).
 *            kvc_score(KVC_SCORE_CRITICALKV)'s norm output [hq][n_keys] is this layout for the units = the KV
 *            heads of one layer (weight_stride = n_keys). The outputs o and probs are unchanged.
 *   weight_stride  >= n_windows_max * W when token_weight is given.
 *   max_summary    0, or a HOST bound (<= cache.sum_max) on every unit's n_sum: the unit's summaries are then
 *            attended as keys after the tail (key k_sum[u][j], value v_sum of summary j, logit + ln 32); they
 *            belong to no window (no mass, no cumulative score). Requires cache.k_sum and probs == NULL.
 *   max_full, max_int2, max_tail   HOST upper bounds over units of n_full, n_int2 and tail_len (before the
 *            append). They size the grid; a unit whose device count exceeds them sets KVC_DEV_BOUND_EXCEEDED and
 *            its step is undefined.
 * Workspace: kvc_decode_attn_workspace() bytes, any contents, 256-byte aligned. */
typedef struct kvc_decode_args {
  const void* q;
  const void* k_new;
  const void* v_new;
  float* out;
  float* probs;
  float* mass;
  int32_t probs_stride;
  int32_t accumulate_cum;
  int32_t max_full;
  int32_t max_int2;
  int32_t max_tail;
  int32_t reserved;
  const float* token_weight; /* [U][G][weight_stride] float or NULL; see above */
  int64_t weight_stride;
  int32_t max_summary;       /* HOST bound on n_sum over units; 0 = no summaries attended; see above */
  int32_t reserved2;         /* must be 0 */
} kvc_decode_args;

/* Three-tier routing (QEvict page, "Metodologia: QEvict" and "Mecanismos Principais"). Per unit, the resident
 * windows (tier != EVICTED) are ranked by (score desc, window index asc); ranks [0, budget_full) become FULL,
 * the next budget_int2 become INT2, the rest EVICTED — permanently (evicted windows are never ranked again).
 * Outputs, per unit:
 *   tier, res_list, res_slot, n_full, n_int2 of the cache are rewritten; ledgered is cleared for evicted windows;
 *   slots: a window leaving FULL frees its full-precision slot, an evicted window frees its ledger slot; a window
 *                                 promoted to FULL takes the lowest free full-precision slot and a window demoted
 *                                 for the first time the lowest free ledger slot, in ascending window order
 *                                 (full_slot / ledger_slot updated). A unit whose pools run out (FS < budget_full,
 *                                 or LS below its ledgered windows) sets KVC_DEV_BOUND_EXCEEDED and those windows
 *                                 get slot -1 (never read);
 *   quant_list[u][0..n_quant[u])  windows going FULL -> INT2 with no ledger copy yet (ascending): pass to
 *                                 kvc_quantize_int2 (their first demotion, the only time they are quantised);
 *   promo_list[u][0..n_promo[u])  windows going INT2 -> FULL (ascending): pass to kvc_promote.
 *   A FULL -> INT2 move of a window that already has a ledger copy is a pure index remap.
 *   scores         [U][NW] float, or NULL to rank by cache.cum. Must be finite (NaN: KVC_DEV_NAN_SCORE, the
 *                  unit keeps its tiers).
 *   budget_full, budget_int2   [U] int32 device arrays (>= 0).
 *   n_windows_max <= 4096 (KVC_E_UNSUPPORTED above: one workgroup routes a unit, at most 4 windows per thread).
 *   quant_list, promo_list     [U][NW] int32;  n_quant, n_promo  [U] int32. */
typedef struct kvc_tier_route_args {
  const kvc_cache* cache;
  const float* scores;
  const int32_t* budget_full;
  const int32_t* budget_int2;
  int32_t* quant_list;
  int32_t* n_quant;
  int32_t* promo_list;
  int32_t* n_promo;
} kvc_tier_route_args;

/* Modes of kvc_score / kvc_route. */
#define KVC_SCORE_WINDOWS 0      /* args: const kvc_window_score_args* */
#define KVC_SCORE_RETENTION 1    /* args: const kvc_retention_args*    */
#define KVC_SCORE_CRITICALKV 2   /* args: const kvc_criticalkv_args*   */
#define KVC_ROUTE_TIERS 0        /* args: const kvc_tier_route_args*   */
#define KVC_ROUTE_GLOBAL_TOPM 1  /* args: const kvc_topm_args*         */
#define KVC_ROUTE_TWO_STAGE 2    /* args: const kvc_two_stage_args*    */

/* kvc_score(KVC_SCORE_CRITICALKV): CriticalKV scores of one layer at prefill (CriticalKV page, "Framework
 * Teórico": the output perturbation is bounded through the attention weights and the values projected by W_O;
 * "Algoritmo: Seleção Constrainda por Perturbação": attention weights from the observation window, second-stage
 * score A_i * |V_i W_O|_1 with the projected values). For KV head g and each query head h of its group:
 *   A_{h,i}  = (1/n_obs) sum_j softmax_i(q_{h,j} . k_{g,i} / sqrt(D)), query j at position n_keys - n_obs + j
 *              seeing keys 0 .. n_keys - n_obs + j (causal);
 *   N_{h,i}  = sum_c | sum_d V[g][i][d] * W_O[h*D + d][c] |   (fp32 accumulate);
 *   A_g[i]   = mean_h A_{h,i};   S2_g[i] = mean_h A_{h,i} * N_{h,i}.
 *   q_obs [hq][n_obs][D], k, v [hkv][n_keys][D], w_o [hq*D][d_model] row-major: storage dtype, 16-byte aligned.
 *   a_head, norm [hq][n_keys] float out; a_group, s2_group [hkv][n_keys] float out.
 *   Requires n_obs == 32, D == 128, hq / hkv in {1, 2, 4, 8}, d_model % 64 == 0, n_keys >= 32.
 * Workspace: kvc_score_workspace(KVC_SCORE_CRITICALKV, args) bytes, any contents. */
typedef struct kvc_criticalkv_args {
  const void* q_obs;
  const void* k;
  const void* v;
  const void* w_o;
  float* a_head;
  float* norm;
  float* a_group;
  float* s2_group;
  int32_t n_keys;
  int32_t hq;
  int32_t hkv;
  int32_t n_obs;
  int32_t head_dim;
  int32_t d_model;
  int32_t kv_dtype;
  int32_t reserved;
} kvc_criticalkv_args;

/* kvc_route(KVC_ROUTE_TWO_STAGE): CriticalKV's two-stage budgeted selection (CriticalKV page, "Algoritmo:
 * Seleção Constrainda por Perturbação": a share alpha of the budget goes to the attention weights alone, the rest
 * to the perturbation-aware score), per row (KV head): with budget1 = floor(alpha * budget) (computed by the
 * library in double precision), the first budget1 entries in (a desc, index asc) order, then the first
 * budget - budget1 of the remaining entries in (s2 desc, index asc) order; the union is written ascending.
 *   a, s2  [rows][n] float (finite; a NaN makes the result undefined);  idx [rows][budget] int32 out.
 *   0 <= budget <= n <= 65536;  0 <= alpha <= 1.
 * Workspace: kvc_route_workspace(KVC_ROUTE_TWO_STAGE, args) bytes, any contents, 256-byte aligned. */
typedef struct kvc_two_stage_args {
  const float* a;
  const float* s2;
  int32_t* idx;
  int32_t rows;
  int32_t n;
  int32_t budget;
  int32_t reserved; /* must be 0 */
  double alpha;     /* stage-1 share of the budget */
} kvc_two_stage_args;

/* kvc_score(KVC_SCORE_RETENTION): DBTrimKV retention score (DBTrimKV page, "Metodologia: Evicção Baseada em
 * Retenção Global", section 2: token i's retention weight at step t is beta_i^(t - i)). Written as its logarithm,
 *   score[r][i] = float(t - i) * logf(beta[r][i])      (fp32; the order is that of beta^(t - i))
 * because the power underflows to 0 for most entries of long contexts. Rows r are (layer, KV head) pairs.
 *   beta   [n_rows][n_tokens] float in (0, 1), 16-byte aligned;  score [n_rows][n_tokens] float, 16-byte aligned.
 *   n_tokens % 4 == 0, n_rows * n_tokens < 2^31. No workspace. */
typedef struct kvc_retention_args {
  const float* beta;
  float* score;
  int64_t n_rows;
  int32_t n_tokens;
  int32_t t;
} kvc_retention_args;

/* kvc_route(KVC_ROUTE_GLOBAL_TOPM): one global budget (DBTrimKV page, "Metodologia", section 3: every entry of
 * every layer and head is ranked on one scale and the top M are kept). The kept set is the first m entries in
 * the order (score desc, flat index asc), so it is unique.
 *   scores     [n] float, finite, 16-byte aligned; rows of row_len entries (row_len % 16 == 0, n % row_len == 0,
 *              n <= 2^31 - 8208, larger n: KVC_E_UNSUPPORTED); 0 <= m <= n.
 *   beta, t    instead of scores (scores == NULL): the scores are DBTrimKV's log-retention computed in place,
 *              score[r][i] = float(t - i) * logf(beta[r][i]) with i the position inside row r (the same bits as
 *              kvc_score(KVC_SCORE_RETENTION) writes), so the score array is never written or read. beta in (0, 1),
 *              16-byte aligned, [n] float. Exactly one of scores and beta is given.
 *   keep       [n] uint8 out, 1 = kept (16-byte aligned);  row_counts [n / row_len] int32 out: kept per row.
 *   status     int32 device error bits (KVC_DEV_NAN_SCORE: a NaN score was seen; the result is then undefined).
 * Workspace: kvc_route_workspace(KVC_ROUTE_GLOBAL_TOPM, args) bytes (about 8 n: the entries of the threshold's
 * histogram bin are compacted into it), any contents, 256-byte aligned. */
typedef struct kvc_topm_args {
  const float* scores;
  int64_t n;
  int64_t m;
  int32_t row_len;
  int32_t reserved;
  uint8_t* keep;
  int32_t* row_counts;
  int32_t* status;
  const float* beta; /* fused log-retention input (with scores == NULL), see above */
  int32_t t;
  int32_t reserved2; /* must be 0 */
} kvc_topm_args;

/* kvc_compact_pages: per-row variable-length paged lists (DBTrimKV page, "Metodologia", section 4: paged
 * storage lets every head keep a sequence of its own length). Out of place: for every row r (a (layer, KV head)
 * pair) the kept positions, ascending, are copied into fresh pages of `page` rows; row r owns output pages
 * page_offset[r] .. page_offset[r] + n_pages[r] - 1 (consecutive, rows in order), its last page's unused rows
 * are zeroed.
 *   keep        [n_rows][n_tokens] uint8 (0/1), 16-byte aligned; n_tokens % 16 == 0, n_tokens % page == 0.
 *   page_table  [n_rows][n_tokens / page] int32: source page id of each block of `page` positions.
 *   k_pool, v_pool  [n_src_pages][page][head_dim] storage dtype (fp16/bf16), head_dim == 128, n_src_pages >= 1.
 *   k_out, v_out    [out_pages_max][page][head_dim] storage dtype out.
 *   lengths, page_offset, n_pages   [n_rows] int32 out.
 *   status      int32 device error bits: KVC_DEV_BOUND_EXCEEDED if the pages exceed out_pages_max (the excess is
 *               not written) or a page id is outside [0, n_src_pages) (that row is written as zeros).
 * Workspace: kvc_compact_pages_workspace(args) bytes, any contents. */
typedef struct kvc_compact_args {
  const uint8_t* keep;
  const int32_t* page_table;
  const void* k_pool;
  const void* v_pool;
  void* k_out;
  void* v_out;
  int32_t* lengths;
  int32_t* page_offset;
  int32_t* n_pages;
  int32_t* status;
  int64_t n_rows;
  int64_t n_src_pages;
  int64_t out_pages_max;
  int32_t n_tokens;
  int32_t page;
  int32_t head_dim;
  int32_t kv_dtype;
} kvc_compact_args;

/* kvc_paged_decode_attn: decode attention over per-row variable-length page lists (DBTrimKV page, "Metodologia:
 * Evicção Baseada em Retenção Global", section 4: after the global budget every (layer, KV head) row keeps a
 * sequence of its own length in paged storage; kvc_compact_pages writes such pages). For row r, token i is row
 * i % page of pool page page_list[r * page_stride + i / page]; the row's G query heads attend over its lengths[r]
 * tokens with scaled dot-product attention: out[r][h] = sum_i softmax_i(q[r][h] . k_i / sqrt(128)) v_i (fp32).
 * A row of length 0 gets zeros.
 *   q              [n_rows][group][128] storage dtype, 16-byte aligned.
 *   k_pool, v_pool [n_pool_pages][page][128] storage dtype (token-major pages), 16-byte aligned; rows of a
 *                  listed page past the row's length are read but never weigh in.
 *   page_list      [n_rows][page_stride] int32 pool page ids; entries past a row's page count are never read.
 *   lengths        [n_rows] int32 tokens per row.
 *   out            [n_rows][group][128] float32.
 *   status         int32 device error bits: KVC_DEV_BOUND_EXCEEDED if a length exceeds max_pages * page (tokens
 *                  past the bound are ignored) or a listed page id is outside [0, n_pool_pages) (its tokens are
 *                  ignored).
 *   group in {1, 2, 4, 8}; page a multiple of 16 in [16, 1024]; max_pages = HOST bound on every row's page count
 *   (sizes the grid), 1 <= max_pages <= page_stride, max_pages * page <= 2^24; head_dim 128; n_pool_pages >= 1.
 * Workspace: kvc_paged_decode_workspace(args) bytes, any contents, 256-byte aligned. */
typedef struct kvc_paged_decode_args {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_list;
  const int32_t* lengths;
  float* out;
  int32_t* status;
  int64_t n_rows;
  int64_t n_pool_pages;
  int64_t page_stride;
  int32_t group;
  int32_t page;
  int32_t max_pages;
  int32_t head_dim;
  int32_t kv_dtype;
  int32_t reserved;
} kvc_paged_decode_args;

/* kvc_route_diagnostics: per-unit diagnostics of the routing dynamics and of the output error of the compressed
 * cache. QEvict page, "Principais Contribuições", item 1: future missed mass (the share of later attention on
 * states a policy has already dropped), global latent importance reactivation (windows that left the active set
 * coming back) and selection churn (instability of the assignment between consecutive routing steps); CriticalKV
 * page, "Framework Teórico": the perturbation L = ||o - o^||_1 between the outputs over the full cache and over
 * the kept subset. The active set is the FULL tier. For unit u, over its windows w < n_windows[u]:
 *   counts[u][0] = #{w : tier_prev[w] != tier[w]}                 (churn = counts[0] / n_windows)
 *   counts[u][1] = #{w : tier[w] == FULL and tier_prev[w] != FULL} (re-entries into the active set)
 *   counts[u][2] = #{w : tier[w] == FULL}
 *   counts[u][3] = #{w : tier[w] != EVICTED}
 *   values[u][0] = sum of mass_full[w] over w with tier[w] == EVICTED   (future missed mass; 0 if mass_full NULL)
 *   values[u][1 + h] = sum_d |o_full[u][h][d] - o[u][h][d]|             (0 if o_full or o is NULL)
 *   tier_prev  [U][n_windows_max] int8 tiers before a routing event, or NULL (taken equal to tier).
 *   tier       [U][n_windows_max] int8 tiers after it (or the tiers serving a step).
 *   n_windows  [U] int32 (clamped to [0, n_windows_max]).
 *   mass_full  [U][n_windows_max] float: the window mass of the same step under attention over the full,
 *              uncompressed cache (kvc_decode_attn on a cache whose windows are all FULL), or NULL.
 *   o_full, o  [U][group][128] float: outputs of the step over the full and the compressed cache, or NULL.
 *   counts     [U][4] int32 out; values [U][1 + group] float out (sums in a fixed order: reproducible).
 *   group in {1, 2, 4, 8}; head_dim 128; 1 <= n_units <= 2^20; 1 <= n_windows_max <= 2^20. No workspace. */
typedef struct kvc_diag_args {
  const int8_t* tier_prev;
  const int8_t* tier;
  const int32_t* n_windows;
  const float* mass_full;
  const float* o_full;
  const float* o;
  int32_t* counts;
  float* values;
  int32_t n_units;
  int32_t n_windows_max;
  int32_t group;
  int32_t head_dim;
} kvc_diag_args;

/* kvc_score(KVC_SCORE_WINDOWS): the scoring half of a decode step — the same kernels as kvc_decode_attn with
 * out = NULL: probabilities, window mass and the cumulative score update over the mixed cache. */
typedef struct kvc_window_score_args {
  const kvc_cache* cache;
  const kvc_decode_args* step; /* step->out is ignored */
} kvc_window_score_args;

int kvc_abi_version(void);
const char* kvc_status_str(int status);

/* Bytes of workspace kvc_decode_attn needs for these bounds (0 on invalid arguments). */
size_t kvc_decode_attn_workspace(const kvc_cache* cache, const kvc_decode_args* step);

int kvc_decode_attn(const kvc_cache* cache, const kvc_decode_args* step, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* kvc_decode_attn_static: kvc_decode_attn for callers that cannot allocate device memory (code being captured
 * into a HIP graph, serving loops that must not call hipMalloc, harnesses that forbid allocation). Same arguments,
 * kernels and results as kvc_decode_attn, but no workspace argument: the step's scratch (split-K partials, window
 * exp-sums) lives in a static device array of the library, kvc_decode_attn_static_max_bytes() = 16 MiB, one copy
 * per GPU held until the process ends. A step whose kvc_decode_attn_workspace() exceeds that returns
 * KVC_E_WORKSPACE before any GPU work. It allocates nothing; the first call on a device looks the array up on that
 * device. Every call on one GPU uses the same array: calls that can overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. */
int kvc_decode_attn_static(const kvc_cache* cache, const kvc_decode_args* step, hipStream_t stream);
size_t kvc_decode_attn_static_max_bytes(void);

/* Workspace for kvc_score in the given mode (KVC_SCORE_WINDOWS: same as kvc_decode_attn). */
size_t kvc_score_workspace(int32_t mode, const void* args);
int kvc_score(int32_t mode, const void* args, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Routing in the given mode; KVC_ROUTE_TIERS needs no workspace (pass NULL, 0). */
size_t kvc_route_workspace(int32_t mode, const void* args);
int kvc_route(int32_t mode, const void* args, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Write-once INT2 quantisation (QEvict page, "Mecanismos Principais", write-once quantization ledger): for
 * every listed window w, K and V are quantised from its full-precision copy (slot full_slot[w], the slot it held
 * until the routing event that demoted it: run this before kvc_promote) into ledger slot ledger_slot[w], and the
 * window is marked ledgered. A listed window that is already ledgered is skipped and KVC_DEV_LEDGER_REWRITE is
 * set: the ledger is never rewritten. A slot outside its pool sets KVC_DEV_BOUND_EXCEEDED (window skipped).
 *   list [U][list_stride] int32 window ids; count [U] int32 entries per unit; max_total = HOST bound of
 *   sum(count) (sizes the launch; 0 launches nothing).
 * Quantiser, per token and per 32-element group (INT2 is the width the page names; the rest is this library's
 * format): lo/hi = min/max (fp32); zero z = largest fp16 <= lo; scale s = smallest fp16 >=
 * fl32(fl32(hi - z) / 3), or 0 if hi == z; code = #{k in 0..2 : fl32(x - z) >= (k + 0.5) * s} (0 if s == 0).
 * Precondition: |x| < 65504. */
int kvc_quantize_int2(const kvc_cache* cache, const int32_t* list, const int32_t* count, int32_t list_stride,
                      int64_t max_total, hipStream_t stream);

/* Promotion (QEvict page, "Mecanismos Principais": a quantized window whose cumulative score rises is
 * dequantised and promoted back to full precision): for every listed window w, full-precision slot full_slot[w]
 * is written with round-to-nearest-even(fmaf(code, scale, zero)) in the storage dtype from ledger slot
 * ledger_slot[w]. The ledger copy is kept. Same list conventions as kvc_quantize_int2. */
int kvc_promote(const kvc_cache* cache, const int32_t* list, const int32_t* count, int32_t list_stride,
                int64_t max_total, hipStream_t stream);

size_t kvc_compact_pages_workspace(const kvc_compact_args* args);
int kvc_compact_pages(const kvc_compact_args* args, void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t kvc_paged_decode_workspace(const kvc_paged_decode_args* args);
int kvc_paged_decode_attn(const kvc_paged_decode_args* args, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

int kvc_route_diagnostics(const kvc_diag_args* args, hipStream_t stream);

/* kvc_summarize_evicted: after a routing event, append the summary of every window evicted by it (SEKV page,
 * "Metodologia" sections 2 and 3; see k_sum above). For unit u the windows w < n_windows[u] with
 * tier_prev[u][w] != EVICTED and cache.tier[u][w] == EVICTED, ascending, get summaries n_sum[u], n_sum[u] + 1, ...
 * from the copy the cache held for them: a window evicted from FULL from its full-precision slot full_slot[w], one
 * evicted from INT2 from its ledger slot ledger_slot[w] brought back to the storage dtype (round-to-nearest-even of
 * fmaf(code, scale, zero), what a promotion stores). Both slots were freed by the event: call this right after
 * kvc_route, before kvc_quantize_int2 and kvc_promote. n_sum[u] advances by the count. A unit whose summaries
 * would pass sum_max keeps the first ones and raises KVC_DEV_BOUND_EXCEEDED.
 *   tier_prev  [U][NW] int8: the tiers before the event.
 *   max_new    HOST bound on the windows any unit evicts in this event (sizes the grid; more are an error bit).
 * Workspace: kvc_summarize_workspace(cache) bytes, any contents, 256-byte aligned. */
size_t kvc_summarize_workspace(const kvc_cache* cache);
int kvc_summarize_evicted(const kvc_cache* cache, const int8_t* tier_prev, int32_t max_new, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* kvc_topk: the budgeted selection itself. Every selection on the pages keeps the highest-scoring entries under a
 * fixed budget: QEvict's tiers ("Metodologia: QEvict"), DBTrimKV's global top-M ("Metodologia", section 3),
 * CriticalKV's stages ("Algoritmo: Seleção Constrainda por Perturbação"). Here: the first k entries of scores in
 * the order (score desc, index asc) — a unique set — written as their indices in ascending index order.
 *   scores   [n] float, finite (a NaN makes the order undefined; the output is still k distinct indices in
 *            [0, n)), 16-byte aligned.
 *   idx_out  [k] int32 out, ascending.
 *   0 <= k <= n <= 2^31 - 8208 (larger n: KVC_E_UNSUPPORTED).
 * Workspace: kvc_topk_workspace(n, k) bytes (about 9 n), any contents, 256-byte aligned. */
size_t kvc_topk_workspace(int64_t n, int64_t k);
int kvc_topk(const float* scores, int64_t n, int64_t k, int32_t* idx_out, void* workspace, size_t workspace_bytes,
             hipStream_t stream);

/* kvc_repack_full: move the full-precision copies of every unit's FULL windows into a new pool, so that the
 * prefill-sized pool can be released once routing has cut the FULL tier to its budget (QEvict page, "Metodologia:
 * QEvict": the cache stays within a fixed memory budget). For unit u, FULL window res_list[u][i] (i < n_full[u])
 * is copied from slot res_slot[u][i] of cache.k_full / v_full to slot i of k_dst / v_dst ([U][dst_slots][W][D] and
 * [U][dst_slots][D][W], storage dtype, 16-byte aligned, not overlapping the cache's pools), and full_slot and
 * res_slot are rewritten to i. The caller then points cache.k_full / v_full at the new pool and sets
 * cache.full_slots = dst_slots. Requires n_full[u] <= dst_slots: a unit above it sets KVC_DEV_BOUND_EXCEEDED, and
 * its windows past dst_slots get slot -1. No workspace. */
int kvc_repack_full(const kvc_cache* cache, void* k_dst, void* v_dst, int32_t dst_slots, hipStream_t stream);

/* Reads *cache->status into *host_status (synchronises the stream) and, if clear != 0, zeroes it. */
int kvc_read_device_status(const kvc_cache* cache, int32_t* host_status, int32_t clear, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
