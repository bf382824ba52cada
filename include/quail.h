/*
 * quail.h -- C ABI of the MI355X (gfx950) AI.IF join-prefill library.
 *
 * The library evaluates AI.IF predicates by prefill only: every shared anchor
 * row's KV is computed once per layer, many suffix rows attend to it through
 * cascade attention (suffix->anchor cross-attention plus causal suffix
 * self-attention, merged by LSE rescaling), and the last suffix position emits
 * one token from a head cut to 8 vocabulary columns, which becomes a boolean.
 *
 * Pages this interface follows (cited by title and section):
 *  [pt] "Motor de inferência Quail atinge 1 bilhão de tokens por minuto por
 *       GPU", section "Como funciona": the query-aware KV cache (the plan is
 *       known, so accesses are predictable and eviction has no regret), zero
 *       decode (one token from the final prefill pass), simplified cascade
 *       attention with LSE rescaling, and the output head cut to 8 options.
 *  [fa] "Quail: یک میلیارد توکن در دقیقه روی یک GPU", body and key points:
 *       the AI.IF join example, the engine sees the whole plan, the last
 *       prefill pass predicts one token, the head keeps 8 columns, model
 *       qwen3-4b-fp8 on one GPU.
 *  [it] "Quail, il motore di inferenza che supera il miliardo di token al
 *       minuto su una H100": filter = one model call per row, naive join =
 *       one call per row pair; KV regret.
 *
 * Conventions (all functions):
 *  - "dev" pointers are device (HBM) addresses on the current HIP device;
 *    "host" pointers are ordinary host memory. Tensors are row-major and
 *    contiguous. bf16 is passed as uint16_t bit patterns, fp8 as uint8_t OCP
 *    E4M3 codes (bias 7, max 448, S.1111.111 = NaN).
 *  - The caller owns every device buffer (weights, tokens, outputs, the KV
 *    pool and the workspace). The library never allocates or frees device
 *    memory. It keeps a small pinned host staging area for per-call metadata.
 *  - Host arrays are read before the call returns. Device inputs must stay
 *    valid until the stream reaches the enqueued work.
 *  - Every compute call only enqueues work on `stream` (a hipStream_t; NULL =
 *    the default stream). Nothing waits for the GPU.
 *  - Errors are all-or-nothing: every condition the host can detect (bad
 *    sizes, non-monotone offsets, lengths out of range, a stale handle, a full
 *    pool, an unsupported shape) returns before anything is enqueued, and
 *    quail_last_error() describes it. A failing HIP launch returns
 *    QUAIL_E_HIP; work enqueued before it in the same call may have run.
 *  - A context is not thread-safe and assumes one stream order: use one
 *    context per stream.
 */
#ifndef QUAIL_H
#define QUAIL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t quail_status;
#define QUAIL_OK              0
#define QUAIL_E_INVAL        (-1)   /* malformed argument */
#define QUAIL_E_NOMEM        (-2)   /* KV pool or workspace too small */
#define QUAIL_E_STALE        (-3)   /* anchor handle released or used up */
#define QUAIL_E_HIP          (-4)   /* HIP runtime / launch failure */
#define QUAIL_E_UNSUPPORTED  (-5)   /* shape the kernels do not cover */

/* Guard region size: every anchor slab ends with one, and the last one of
 * the KV pool is one more (see quail_anchor_bytes and quail_ctx_check). */
#define QUAIL_GUARD_BYTES     256

#define QUAIL_DTYPE_F32       0
#define QUAIL_DTYPE_BF16      1
#define QUAIL_DTYPE_FP8_E4M3  2

typedef struct quail_ctx quail_ctx;
typedef void* quail_stream;                      /* hipStream_t */

/* Anchor handle: (generation << 32) | slot. QUAIL_NO_ANCHOR marks a filter
 * row (a suffix with no anchor: anchor length 0). */
typedef int64_t quail_anchor;
#define QUAIL_NO_ANCHOR ((quail_anchor)-1)

/* Model shape. Supported by the kernels: head_dim == 128; hidden a
 * multiple of 128 and intermediate a multiple of 64 (else
 * QUAIL_E_UNSUPPORTED); n_q_heads a multiple of n_kv_heads with
 * group size 1, 2, 4 or 8. kv_dtype is QUAIL_DTYPE_BF16 or
 * QUAIL_DTYPE_FP8_E4M3 (anchor KV stored as E4M3 codes of k/k_scale and
 * v/v_scale, saturating, round-to-nearest-even). RoPE is rotate-half with
 * inverse frequency rope_theta^(-2i/head_dim); RMSNorm is
 * x / sqrt(mean(x^2) + rms_eps) * gamma. Positions: anchor tokens 0..La-1,
 * suffix token j at La + j; La + Ls must not exceed max_anchor_len +
 * max_suffix_len.
 * act_dtype selects what the four projections read ([pt] "Como funciona":
 * the engine's FP8 GEMMs): 0 or QUAIL_DTYPE_BF16 = bf16 activations (W8A16,
 * the default); QUAIL_DTYPE_FP8_E4M3 = per-token E4M3 activations (W8A8: the
 * normed inputs, the attention output and the MLP product are quantised per
 * token as by quail_act_quant_e4m3 and the products run on the fp8 MFMA),
 * which needs hidden a multiple of 256, intermediate of 128 and an even
 * n_q_heads. */
typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
    float rope_theta, rms_eps;
    int32_t kv_dtype;
    float k_scale, v_scale;
    int32_t max_anchor_len, max_suffix_len;
    int32_t act_dtype;
} quail_model_config;

/* One layer's weights (all dev). fp8 matrices are [out, in] E4M3 codes with
 * one bf16 scale per output row: W_eff[o][i] = decode(code[o][i]) * scale[o].
 * w_qkv rows: q (n_q_heads*head_dim), then k, then v (n_kv_heads*head_dim
 * each). w_gate_up rows: gate (intermediate), then up (intermediate). */
typedef struct {
    const uint16_t *attn_norm, *mlp_norm;              /* bf16 [hidden] */
    const uint8_t  *w_qkv, *w_o, *w_gate_up, *w_down;  /* fp8 [out, in] */
    const uint16_t *s_qkv, *s_o, *s_gate_up, *s_down;  /* bf16 [out] */
} quail_layer_weights;

typedef struct {
    const uint16_t *embed;                 /* dev bf16 [vocab, hidden] */
    const quail_layer_weights *layers;     /* host array [n_layers] */
    const uint16_t *final_norm;            /* dev bf16 [hidden] */
    const uint16_t *head8;                 /* dev bf16 [hidden, 8] */
} quail_weights;

/* ---- library ------------------------------------------------------------ */
const char*  quail_version(void);
/* Message of the last failing call on this thread ("" if none). */
const char*  quail_last_error(void);

/* ---- sizing --------------------------------------------------------------- */
/* Pool bytes one anchor of `anchor_len` tokens occupies: layers x {K,V} x
 * kv heads x ceil(anchor_len/64)*64 tokens x head_dim x (2 B bf16 | 1 B fp8),
 * rounded up to 256 B, plus a QUAIL_GUARD_BYTES guard region at its end.
 * Slab layout [layer][K|V][kv_head][token][head_dim], then the guard. */
quail_status quail_anchor_bytes(const quail_model_config* cfg, int32_t anchor_len, size_t* out);

/* Workspace bytes a context needs for batches of up to `max_batch_tokens`
 * tokens (activations, per-batch metadata, the RoPE table). */
quail_status quail_workspace_bytes(const quail_model_config* cfg, int32_t max_batch_tokens,
                                   size_t* out);

/* ---- plan (a1) ------------------------------------------------------------ */
/* Orders pairs for anchor-KV reuse ([pt] "Como funciona", query-aware KV
 * cache bullet; [it] the Modal-blog quote on ordering requests to cache and
 * evict KV): pairs are stably sorted by anchor index (filter rows,
 * pair_anchor < 0, last), then cut greedily into steps that fit both
 * `max_batch_tokens` suffix tokens and `pool_bytes` of distinct anchor slabs.
 * Under prefill-at-first-use and evict-after-last-use, the bytes resident
 * during a step are the slabs of the distinct anchors it touches.
 * Inputs (host): anchor_len[n_anchors], pair_anchor[n_pairs] (-1 = filter
 * row), pair_len[n_pairs]. Outputs (host): pair_order[n_pairs],
 * step_bounds[n_pairs + 1] (step s is pair_order[step_bounds[s] ..
 * step_bounds[s+1]) ), *n_steps, *peak_bytes (largest step residency).
 * E_INVAL for a pair length outside [1, max_batch_tokens] or an anchor index
 * out of range; E_NOMEM if one slab exceeds pool_bytes. Touches no GPU. */
quail_status quail_plan_build(const quail_model_config* cfg, size_t pool_bytes,
                              int32_t max_batch_tokens,
                              int32_t n_anchors, const int32_t* anchor_len,
                              int32_t n_pairs, const int32_t* pair_anchor, const int32_t* pair_len,
                              int32_t* pair_order, int32_t* step_bounds, int32_t* n_steps,
                              size_t* peak_bytes);

/* Plan for several joins over one anchor table, run one after another (a
 * later join may depend on an earlier one's results): [pt] "Como funciona",
 * query-aware KV cache bullet -- with the whole plan known, an anchor's KV is
 * kept for its next use, in whichever join, and evicted when nothing will
 * use it again. Each join is ordered and cut into steps as by
 * quail_plan_build; the steps of all joins form one sequence; an anchor is
 * prefilled before the first step that needs it while not resident, and
 * evicted after its last step in the whole sequence; when a step's new
 * anchors do not fit beside the kept ones, kept anchors are evicted farthest
 * next use first (never used again first; ties: larger slab, lower index).
 * join_offsets: host [n_joins+1], join j owns pairs [join_offsets[j],
 * join_offsets[j+1]) of pair_anchor / pair_len (host; anchor index or -1,
 * suffix tokens).
 * Outputs, host, caller-allocated for P = join_offsets[n_joins] pairs:
 *   pair_order [P]: per join, its pairs' indices within the join in plan
 *     order, joins back to back;
 *   step_info [3*P]: per step (join, lo, hi), positions lo..hi-1 of that
 *     join's plan order; n_steps: the number of steps (<= P);
 *   event_off [3*P+1], event_anchor [2*P]: per step t, three anchor lists:
 *     prefilled before the step event_anchor[event_off[3t] .. event_off[3t+1]),
 *     evicted to make room before it [event_off[3t+1] .. event_off[3t+2]),
 *     evicted after it [event_off[3t+2] .. event_off[3t+3]);
 *   totals [4]: prefills, evictions, regret tokens, peak resident bytes.
 * E_INVAL / E_NOMEM as quail_plan_build. Touches no GPU. */
quail_status quail_multiplan_build(const quail_model_config* cfg, size_t pool_bytes,
                                   int32_t max_batch_tokens, int32_t n_anchors,
                                   const int32_t* anchor_len, int32_t n_joins,
                                   const int32_t* join_offsets, const int32_t* pair_anchor,
                                   const int32_t* pair_len, int32_t* pair_order, int32_t* step_info,
                                   int32_t* n_steps, int32_t* event_off, int32_t* event_anchor,
                                   int64_t* totals);

/* ---- context -------------------------------------------------------------- */
/* Borrows the weights (they must outlive the context), the KV pool (dev,
 * pool_bytes, 256-B aligned; when it holds at least 2 * QUAIL_GUARD_BYTES,
 * its last QUAIL_GUARD_BYTES are a guard region and slabs are carved from
 * the rest) and the workspace (dev, at least quail_workspace_bytes(cfg,
 * max_batch_tokens)). Touches no GPU. */
quail_status quail_ctx_create(const quail_model_config* cfg, const quail_weights* w,
                              void* kv_pool, size_t pool_bytes,
                              void* workspace, size_t ws_bytes, int32_t max_batch_tokens,
                              quail_ctx** out);
quail_status quail_ctx_destroy(quail_ctx* ctx);

/* Debug counters of a context (its guard bytes and token-range check). A
 * slab's guard region is written when the slab is carved and checked when it
 * is evicted (before its memory is written again); this call also checks the
 * guards of every live slab and the pool's tail guard now. guard_errors = the
 * number of guard regions found overwritten since the context was created;
 * bad_tokens = the number of token ids outside [0, vocab) the embedding has
 * met (each such row embeds token 0 instead of reading out of range).
 * Enqueues the checks on `stream` and waits for it. Either pointer may be
 * NULL. Token ids outside [0, vocab) are a caller error: results of a call
 * that met one are undefined, but the GPU never reads outside the table. */
quail_status quail_ctx_check(quail_ctx* ctx, quail_stream stream, int64_t* guard_errors,
                             int64_t* bad_tokens);

/* Per-launch timing of a context's kernels, for measurement: with profiling
 * on, every launch of the model path is bracketed by two HIP events on its
 * stream. Kinds: 0 QKV projection (+ RoPE, KV writer), 1 O projection
 * (+ residual), 2 gate/up projection (+ SwiGLU), 3 down projection
 * (+ residual), 4 cascade attention, 5 RMSNorm (with fp8 activations also
 * the per-token quantiser of the attention output and the MLP product),
 * 6 other (embedding, head, row copies). quail_ctx_profile(enable) switches it and discards what was
 * recorded. quail_ctx_profile_read waits for the recorded launches and
 * returns per kind (host arrays of 7, each nullable): the launch count, the
 * summed launch durations in ms and the summed algorithmic FLOP (GEMMs
 * 2*M*N*K with N the weight rows; attention 4 * n_q_heads * head_dim per
 * visible (query, key) pair), then discards the records. */
#define QUAIL_PROF_KINDS 7
quail_status quail_ctx_profile(quail_ctx* ctx, int32_t enable);
quail_status quail_ctx_profile_read(quail_ctx* ctx, int64_t* launches, double* ms, double* flop);

/* ---- KV-aware join-order search, speed-of-light cost model (host only) ---- */
/* [pt] "Como funciona": the join-order search keeps several candidate plans,
 * drops those that are Pareto-dominated (more tokens, more attention pairs
 * and more cache) and picks among the rest with a "speed-of-light" cost model,
 * a roofline that overstates the hardware's peak on purpose; [fa] (body): the
 * planner chooses the join order with the KV cache in mind.
 *
 * A query is a tree of AI.IF joins over n_tables tables (1..12). Table t has
 * `rows` rows whose prompt field has `field_tokens` tokens. Join k relates
 * tables `left` and `right` (n_tables - 1 joins, no cycle); `anchor_glue` /
 * `suffix_glue` are the template tokens that go with the anchor / suffix
 * part of the prompt; `selectivity` in (0, 1] is the expected fraction of
 * pairs that pass; `symmetric` != 0 lets the search put either table first
 * (else the left table is the anchor). A plan is a left-deep order in which
 * each table joins the earlier ones through one join, plus the anchor side of
 * each symmetric join. Under independence a subset S of tables yields
 * N(S) = prod rows * prod selectivity; table u contributes D_u = min(rows_u,
 * N(S)) distinct rows. Adding table t through join k (other end u in S) runs
 * P = D_u * rows_t pairs with A distinct anchors of La tokens and suffixes of
 * Ls tokens, and adds computed tokens A*La + P*Ls, attention pairs
 * P*(La*Ls + Ls*(Ls+1)/2) + A*La*(La+1)/2 and cache bytes A*La*(KV bytes per
 * token over all layers of cfg). A plan's time is the roofline of its totals,
 * max(FLOP / peak_flops, 2 * cache bytes / peak_bytes_per_s), with FLOP =
 * tokens * GEMM FLOP per token + attention pairs * 4 * Hq * d * layers.
 * The search keeps, for every connected subset of tables, the Pareto set of
 * its partial plans (pruning is exact: extensions add the same amounts to
 * every plan of a subset) and returns the least-time plan of the final set.
 * Outputs (host): order [n_tables]; anchor_right [n_tables - 1] (1 = the
 * right table is join k's anchor); metrics [4] = computed tokens, attention
 * pairs, cache bytes, seconds; frontier [cap][4] (nullable when cap = 0)
 * sorted by the metrics; *n_frontier = the final Pareto set's size. E_INVAL
 * on a bad config, sizes, selectivities, peaks, or joins that are not a tree. */
typedef struct {
  int32_t rows;
  float field_tokens;
} quail_table;
typedef struct {
  int32_t left, right;
  float anchor_glue, suffix_glue, selectivity;
  int32_t symmetric;
} quail_ai_join;
quail_status quail_join_search(const quail_model_config* cfg, int32_t n_tables,
                               const quail_table* tables, int32_t n_joins,
                               const quail_ai_join* joins, double peak_flops,
                               double peak_bytes_per_s, int32_t* order, int32_t* anchor_right,
                               double* metrics, double* frontier, int32_t cap,
                               int32_t* n_frontier);

/* ---- anchor prefill + KV writer (a2, a3, a9) -------------------------------- */
/* Runs the decoder stack over each anchor's tokens (positions 0..La-1) and
 * stores every layer's post-RoPE K and its V in a pool slab carved for the
 * anchor: the anchor's KV is computed once and reused by all of its pairs
 * ([pt] "Como funciona", cascade-attention bullet; [it] ordering requests to
 * reuse KV). Anchor self-attention is causal and reads the stored (for fp8,
 * decoded) K/V.
 * tokens: dev int32, anchors packed back to back; offsets: host [n+1],
 * non-decreasing, anchor a = tokens[offsets[a] .. offsets[a+1]), length in
 * [1, min(max_anchor_len, max_batch_tokens)]. n_uses: host [n], the number of
 * pairs that will read the anchor (0 = never prefilled; its handle is
 * QUAIL_NO_ANCHOR). anchor_ids: host [n] caller row ids or NULL; an id that
 * was prefilled and evicted before counts its tokens as regret.
 * out: host [n] handles. E_NOMEM (nothing enqueued, nothing kept) when the
 * pool cannot hold all n slabs at once. */
quail_status quail_anchor_prefill(quail_ctx* ctx, int32_t n, const int32_t* tokens,
                                  const int32_t* offsets, const int32_t* n_uses,
                                  const int64_t* anchor_ids, quail_anchor* out,
                                  quail_stream stream);

/* Gives up an anchor before its declared uses are spent (its slab is freed;
 * later use returns E_STALE). E_INVAL while prefix nodes of the anchor (see
 * quail_prefix_prefill) are alive. Releasing a prefix node spends the anchor
 * use it holds. */
quail_status quail_anchor_release(quail_ctx* ctx, quail_anchor handle);

/* ---- shared suffix prefixes: two-level cascade ------------------------------ */
/* [pt] "Futuro e método" lists a radix index for prefix sharing as future
 * work, and [fa] (body) names the one workload where vLLM wins: agent traces,
 * whose documents share prefixes the engine cannot exploit. These calls add
 * one shared level between an anchor and its suffixes: anchor -> shared
 * suffix prefix (a "prefix node") -> the rest of each suffix.
 *
 * Groups sequences by shared prefix (host only, no GPU): sequence i =
 * tokens[offsets[i] .. offsets[i+1]) (host int32; offsets host [n+1],
 * non-decreasing, lengths >= 1) with key keys[i] (host [n], e.g. the anchor
 * index; negative = never grouped; NULL = one key for all). Sequences with the
 * same key and the same first min_len tokens (min_len >= 1), at least two of
 * them and each longer than min_len, form one node: the subtrees of the
 * per-key radix tree at depth min_len. The node's prefix is the members'
 * longest common prefix, shortened if needed so every member keeps at least
 * one token: node_len[k] >= min_len, and its tokens are the first node_len[k]
 * tokens of member node_first[k] (its smallest member). Nodes are numbered in
 * increasing node_first. Outputs (host, caller-allocated [n]): group_of[i] =
 * node of sequence i or -1; node_first, node_len; *n_nodes = node count. */
quail_status quail_prefix_groups(int32_t n, const int32_t* tokens, const int32_t* offsets,
                                 const int32_t* keys, int32_t min_len, int32_t* group_of,
                                 int32_t* node_first, int32_t* node_len, int32_t* n_nodes);

/* Nested form of quail_prefix_groups (host only): its nodes are the top
 * level; inside a node that covers tokens [.., end) the members are split by
 * their token at position `end`, and a part of two or more whose common
 * prefix (cut to leave each member a token) reaches end + min_len becomes a
 * child node covering [end, its cut), recursively; every other member stays
 * with the node. Outputs (host, caller-allocated [n]; there are at most n - 1
 * nodes): group_of[i] = the deepest node of sequence i or -1; per node k:
 * node_parent[k] (-1 at the top), node_first[k] (smallest member in its
 * subtree: the node's tokens are tokens [node_start[k], node_end[k]) of that
 * member), node_start[k] (the parent's end, 0 at the top), node_end[k]. Nodes
 * are numbered parents first (each top-level node followed by its subtree,
 * children by smallest member). A child is prefilled with
 * quail_prefix_prefill under its parent's handle. E_INVAL as
 * quail_prefix_groups. */
quail_status quail_prefix_tree(int32_t n, const int32_t* tokens, const int32_t* offsets,
                               const int32_t* keys, int32_t min_len, int32_t* group_of,
                               int32_t* node_parent, int32_t* node_first, int32_t* node_start,
                               int32_t* node_end, int32_t* n_nodes);

/* Prefills prefix nodes: node a = tokens[offsets[a] .. offsets[a+1]) (dev
 * int32; host offsets [n+1], lengths in [1, max_batch_tokens]) continues
 * parent[a] (host handle of a live anchor or node). Under an anchor it sits
 * at positions La.. : it attends to every key of the anchor and causally to
 * itself, and every layer's K/V goes to a slab of its own, as for an anchor.
 * Under a node P (a nested level) it continues P's anchor after P's tokens:
 * its slab starts with a copy of P's rows, its own tokens follow, and it
 * spends one of P's declared uses once its prefill is enqueued (P may then
 * be evicted; the copy precedes any reuse in stream order).
 * n_uses: host [n], the pairs that will name the node (0 = not prefilled,
 * handle QUAIL_NO_ANCHOR). Each node holds one of its anchor's declared uses
 * and spends it when the node is evicted, so the anchor outlives its nodes.
 * A pair naming a node handle in quail_join_prefill runs its tokens at
 * positions La + Lp.. against the anchor's keys, the node's keys (both
 * unmasked) and its own keys (causal): the same result as the full suffix
 * [node tokens ‖ pair tokens] after the anchor. out: host [n] handles.
 * E_STALE: a parent handle is stale, or the anchor (or parent node) has no
 * declared use to spare; E_INVAL: La + (all node rows) + 1 exceeds
 * max_anchor_len + max_suffix_len; E_NOMEM as quail_anchor_prefill. */
quail_status quail_prefix_prefill(quail_ctx* ctx, int32_t n, const quail_anchor* parent,
                                  const int32_t* tokens, const int32_t* offsets,
                                  const int32_t* n_uses, quail_anchor* out, quail_stream stream);

/* Device addresses of an anchor's K and V for one layer ([kv_head][La_pad]
 * [head_dim], bf16 or fp8 per kv_dtype) and its lengths. For tests/tools. */
quail_status quail_anchor_kv(const quail_ctx* ctx, quail_anchor handle, int32_t layer,
                             void** k, void** v, int32_t* anchor_len, int32_t* padded_len);

/* ---- join prefill (a2, a4-a7) --------------------------------------------- */
/* For each pair i: suffix tokens tokens[offsets[i] .. offsets[i+1]) (dev
 * int32; host offsets [n+1], non-decreasing, lengths in [1,
 * min(max_suffix_len, max_batch_tokens)]) at positions La + j after anchor
 * pair_anchor[i] (host handle, or QUAIL_NO_ANCHOR for a filter row). Runs the
 * decoder stack: RMSNorm, W8A16 QKV + RoPE, cascade attention against the
 * anchor's stored KV ([pt] "Como funciona": the suffix attends to the anchor,
 * then to itself, merged by LSE rescaling), O projection + residual,
 * RMSNorm, SwiGLU MLP + residual. Writes the last position's hidden state to
 * h_last (dev bf16 [n, hidden], caller order) and, if h_all is not NULL, every
 * position's final hidden state to h_all (dev bf16 [offsets[n], hidden]).
 * Without h_all only the last positions' states are needed, so the last
 * layer runs its O projection and MLP on those rows alone (their values are
 * the same bit for bit). Pairs may come in any order; each pair spends one use of its anchor and an
 * anchor whose uses reach 0 is evicted (its slab is reused in stream order).
 * A handle may also name a prefix node (quail_prefix_prefill): the pair's
 * tokens then sit at positions La + Lp + j and attend to the anchor's keys,
 * the node's keys and their own. E_STALE if a handle is stale or used more
 * often than declared (an anchor's uses held by live nodes are not
 * available to pairs). */
quail_status quail_join_prefill(quail_ctx* ctx, int32_t n, const quail_anchor* pair_anchor,
                                const int32_t* tokens, const int32_t* offsets,
                                uint16_t* h_last, uint16_t* h_all, quail_stream stream);

/* ---- 8-column head + boolean (a8) ----------------------------------------- */
/* z = bf16(RMSNorm(h_last; final_norm)); logits = z . head8 (fp32 [n, 8]);
 * token = first maximum; decision = (true_mask >> token) & 1 ([pt] "Como
 * funciona", zero-decode bullet and the 8-option head; [fa] key points).
 * h_last dev bf16 [n, hidden]; logits dev f32 [n, 8]; token, decision dev u8
 * [n]. Any output pointer may be NULL except decision. */
quail_status quail_head8(quail_ctx* ctx, int32_t n, const uint16_t* h_last, uint8_t true_mask,
                         float* logits, uint8_t* token, uint8_t* decision, quail_stream stream);

/* Context-free fp32 head without a norm: logits = x . w8 for x dev f32
 * [n, hidden], w8 dev f32 [hidden, 8]. */
quail_status quail_head8_f32(int32_t n, int32_t hidden, const float* x, const float* w8,
                             uint8_t true_mask, float* logits, uint8_t* token,
                             uint8_t* decision, quail_stream stream);

/* ---- whole join (a1-a9 in one call) --------------------------------------- */
/* Runs a join end to end: builds the plan (quail_plan_build order and steps),
 * prefills each anchor just before its first step, runs each step's pairs,
 * evicts each anchor after its last step, and applies the head.
 * a_tokens dev int32 + a_offsets host [n_anchors+1]; pair_anchor host
 * [n_pairs] anchor index or -1; s_tokens dev int32 + s_offsets host
 * [n_pairs+1]. Outputs (dev, caller pair order): logits f32 [n_pairs, 8]
 * (nullable), token u8 (nullable), decision u8 [n_pairs]. */
quail_status quail_join_run(quail_ctx* ctx, int32_t n_anchors, const int32_t* a_tokens,
                            const int32_t* a_offsets, int32_t n_pairs,
                            const int32_t* pair_anchor, const int32_t* s_tokens,
                            const int32_t* s_offsets, uint8_t true_mask, float* logits,
                            uint8_t* token, uint8_t* decision, quail_stream stream);

/* quail_join_run with shared suffix prefixes: within each step of the plan,
 * the pairs of one anchor are grouped by quail_prefix_groups(min_shared) over
 * s_tokens_host (a host copy of s_tokens, same layout); each group's prefix
 * node is prefilled once (quail_prefix_prefill, in chunks that fit half the
 * largest free pool block) and its members run only their remaining tokens.
 * Filter rows (pair_anchor -1) are grouped among themselves; their shared
 * prefix is prefilled as a plain anchor and the rows run after it. The
 * anchor's uses are its ungrouped pairs plus one per node. Plan steps are
 * sized by the tokens each pair computes (its own tokens after its group's
 * prefix plus its share of the prefix). Outputs equal quail_join_run's up to
 * floating-point rounding (the cascade split is exact), except that with an
 * fp8 KV store the shared positions are stored in E4M3 like anchor KV.
 * nested != 0 groups each step with quail_prefix_tree instead: nodes under
 * nodes are prefilled parents first (a child copies its parent's rows, as
 * quail_prefix_prefill under a node does), whole subtrees at a time.
 * The plan is built against the largest free pool block less a reserve that
 * covers one step's largest node subtree (at least the slab of the longest
 * pair), re-planning while the subtrees grow, so nodes fit beside their
 * step's anchors; E_NOMEM, before anything is enqueued, when that leaves
 * nothing. min_shared >= 1; other arguments as quail_join_run. */
quail_status quail_join_run_shared(quail_ctx* ctx, int32_t n_anchors, const int32_t* a_tokens,
                                   const int32_t* a_offsets, int32_t n_pairs,
                                   const int32_t* pair_anchor, const int32_t* s_tokens,
                                   const int32_t* s_offsets, const int32_t* s_tokens_host,
                                   int32_t min_shared, int32_t nested, uint8_t true_mask,
                                   float* logits, uint8_t* token, uint8_t* decision,
                                   quail_stream stream);

/* Runs several joins over one anchor table with the plan of
 * quail_multiplan_build (pool budget: the largest free block of the pool
 * now): per step, prefills its listed anchors, runs its pairs and applies
 * the head. Each prefill declares the pairs the anchor serves until its next
 * prefill, so an anchor the plan evicts early is freed right after its last
 * use before the gap (same prefills and regret, lower peak). Pair indices
 * and outputs are global over the joins (join_offsets as above): a_tokens
 * dev + a_offsets host [n_anchors+1]; pair_anchor host [P]; s_tokens dev +
 * s_offsets host [P+1]; logits f32 [P, 8] (nullable), token u8 (nullable),
 * decision u8 [P], all dev. */
quail_status quail_multijoin_run(quail_ctx* ctx, int32_t n_anchors, const int32_t* a_tokens,
                                 const int32_t* a_offsets, int32_t n_joins,
                                 const int32_t* join_offsets, const int32_t* pair_anchor,
                                 const int32_t* s_tokens, const int32_t* s_offsets,
                                 uint8_t true_mask, float* logits, uint8_t* token,
                                 uint8_t* decision, quail_stream stream);

/* Residency counters: bytes resident now and at peak, anchors prefilled,
 * anchors evicted, regret tokens -- anchor tokens prefilled again after an
 * eviction, the "KV regret" [it] measures for the vLLM baseline on its
 * BIO-4 query (paragraph on the optimistic roofline and KV regret); with the
 * whole plan known it is 0 ([pt] "Como funciona", query-aware KV cache
 * bullet). Any pointer may be NULL. */
quail_status quail_pool_stats(const quail_ctx* ctx, size_t* resident, size_t* peak,
                              int64_t* prefills, int64_t* evictions, int64_t* regret_tokens);

/* ---- cascade attention on given Q/K/V (a5) --------------------------------- */
/* [pt] "Como funciona", cascade-attention bullet: each suffix's queries
 * attend to all of its anchor's keys (cross partial, no mask) and causally to
 * its own keys (self partial, diagonal included); the partials are merged by
 * LSE rescaling. Softmax scale sm_scale; query head h reads KV head
 * h / (hq / hkv).
 * dtype: QUAIL_DTYPE_F32 (head_dim 64 or 128), QUAIL_DTYPE_BF16 (head_dim
 * 128), or QUAIL_DTYPE_FP8_E4M3: bf16 q, k, v and out with the anchor K/V
 * given as OCP E4M3 codes (one byte per element, value = the decoded code,
 * unit scale: the resident-KV format of the multi-join configuration).
 * ak, av: dev [sum La, hkv, d]; a_off: host [n_anchors+1]. q: dev
 * [sum Ls, hq, d]; k, v: dev [sum Ls, hkv, d]; s_off: host [n_suffix+1];
 * s_anchor: host [n_suffix] anchor index or -1 (no anchor). Suffixes of one
 * anchor are processed together; any order is accepted.
 * out: dev [sum Ls, hq, d] (f32 or bf16); lse: dev f32 [sum Ls, hq] natural-log
 * LSE of the merged row, or NULL. workspace: dev, at least
 * quail_cascade_workspace_bytes(...). */
quail_status quail_cascade_workspace_bytes(int32_t n_anchors, const int32_t* a_off,
                                           int32_t n_suffix, const int32_t* s_off,
                                           size_t* out);
quail_status quail_cascade_attn(int32_t dtype, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                int32_t n_anchors, const void* ak, const void* av,
                                const int32_t* a_off, int32_t n_suffix, const int32_t* s_anchor,
                                const void* q, const void* k, const void* v, const int32_t* s_off,
                                void* out, float* lse, void* workspace, size_t ws_bytes,
                                quail_stream stream);

/* quail_cascade_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, without the workspace
 * argument. The per-call metadata (token segments, attention tiles, KV
 * sources) goes to a static scratch array of the library, one per device, of
 * QUAIL_NOALLOC_SCRATCH_BYTES (16 MiB), filled by one hipMemcpyAsync from host
 * memory; nothing is allocated. A call whose metadata
 * (quail_cascade_workspace_bytes) exceeds that returns QUAIL_E_NOMEM before
 * anything is enqueued. Every call on one device shares that device's array:
 * calls in one stream order are safe (each call's copy follows the previous
 * call's kernel), calls that overlap on one device (other streams, other
 * threads) race on it. Other arguments, results and errors as
 * quail_cascade_attn. */
#define QUAIL_NOALLOC_SCRATCH_BYTES (16u << 20)
quail_status quail_cascade_attn_noalloc(int32_t dtype, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                        int32_t n_anchors, const void* ak, const void* av,
                                        const int32_t* a_off, int32_t n_suffix, const int32_t* s_anchor,
                                        const void* q, const void* k, const void* v, const int32_t* s_off,
                                        void* out, float* lse, quail_stream stream);

/* ---- W8A16 GEMM (the projections of a4, a6, a7) ----------------------------- */
/* y[m][n] = bf16( scale[n] * sum_k x[m][k] * decode(w[n][k]) ), fp32
 * accumulation. x dev bf16 [M, K] (row stride K); w dev fp8 [N, K]; scale dev
 * bf16 [N]; y dev bf16 [M, N]. K a multiple of 64, N a multiple of 128 ([it]
 * "Qwen3 4B FP8": FP8 weights, bf16 activations). */
quail_status quail_gemm_w8a16(int32_t M, int32_t N, int32_t K, const uint16_t* x,
                              const uint8_t* w, const uint16_t* scale, uint16_t* y,
                              quail_stream stream);

/* ---- W8A8: E4M3 activations on the fp8 MFMA --------------------------------- */
/* The FP8 GEMM of the engine ([pt] "Como funciona", FP8 GEMM kernels) with
 * both operands in E4M3: one scale per token for the activations, one bf16
 * scale per output row for the weights. Not the contract of
 * quail_join_prefill (whose projections are W8A16): a standalone pair of
 * calls for callers that accept per-token fp8 activations.
 *
 * Per-token quantisation: amax = max_k |x[m][k]|;
 *   codes[m][k] = E4M3(x[m][k] * (448 / amax))  (saturating, round to nearest,
 *                                                ties to the even code)
 *   scale[m]    = amax / 448
 * where 448 / amax, the product and amax / 448 are each one fp32 operation
 * rounded to nearest even. A row of zeros gets codes 0 and scale 0. Every
 * other row must have amax >= 2^-120 so that 448 / amax is finite in fp32
 * (smaller rows give undefined codes). x dev
 * bf16 [M, K] (row stride K, finite values, 16-byte aligned); codes dev u8
 * [M, K]; scale dev f32 [M]. K a multiple of 8. Caller owns every buffer. */
quail_status quail_act_quant_e4m3(int32_t M, int32_t K, const uint16_t* x, uint8_t* codes,
                                  float* scale, quail_stream stream);
/* y[m][n] = bf16( w_scale[n] * x_scale[m] * sum_k decode(xc[m][k]) * decode(wc[n][k]) ),
 * fp32 accumulation of the exact fp8 products. xc dev u8 [M, K]; x_scale dev
 * f32 [M]; wc dev u8 [N, K]; w_scale dev bf16 [N]; y dev bf16 [M, N]. N a
 * multiple of 256, K a multiple of 128, buffers 16-byte aligned (w_scale
 * 8-byte); otherwise QUAIL_E_UNSUPPORTED. */
quail_status quail_gemm_w8a8(int32_t M, int32_t N, int32_t K, const uint8_t* xc, const float* x_scale,
                             const uint8_t* wc, const uint16_t* w_scale, uint16_t* y,
                             quail_stream stream);

/* ---- E4M3 codec of the fp8 KV store -------------------------------------- */
/* codes[i] = E4M3(x[i] / scale): saturate to +-448, round to nearest, ties to
 * the even code (the KV writer's quantiser for anchor K/V held as fp8; the
 * configuration "fp8 KV ~58 GB resident" of the multi-join workload).
 * x dev f32 [n]; codes dev u8 [n]. */
quail_status quail_fp8_e4m3_encode(int64_t n, const float* x, float scale, uint8_t* codes,
                                   quail_stream stream);
/* x[i] = decode(codes[i]) * scale (exact decode; NaN codes give NaN). */
quail_status quail_fp8_e4m3_decode(int64_t n, const uint8_t* codes, float scale, float* x,
                                   quail_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* QUAIL_H */
