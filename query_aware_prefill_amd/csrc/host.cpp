// Host runtime of the AI.IF join-prefill library: argument validation and the
// error model, the plan builders (one join; several joins over one anchor
// table), the radix grouping of suffixes that share a prefix, the anchor-KV
// residency manager (anchors and the prefix nodes that continue them), the
// KV-aware join-order search, per-batch metadata, and the layer loop that
// enqueues the gfx950 kernels.
//
// [pt] "Como funciona": the engine knows the whole plan, so it can predict KV
// accesses and evict with no regret; each anchor's KV is computed once and the
// suffixes reach it through cascade attention; prefill only, one token from
// the final pass through an 8-column head. [it]/[pl]: the vLLM baseline lost
// time to host overhead (the CPU planning while the GPU waited) and to KV
// regret. Hence: plans are built once, in C++, before any launch; each batch
// is a fixed sequence of large launches with no host synchronisation inside
// the layer loop; per-batch metadata goes to the device in one pinned copy.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <numeric>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/quail.h"
#include "quail_internal.h"

using namespace quail;

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
namespace {

thread_local std::string g_err;

quail_status fail(quail_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(QUAIL_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));          \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// pinned staging for host -> device metadata copies (stream ordered)
// ---------------------------------------------------------------------------
class Stager {
 public:
  ~Stager() {
    for (auto& s : slots_) {
      // teardown: nothing to report an error to
      if (s.ev) { (void)hipEventSynchronize(s.ev); (void)hipEventDestroy(s.ev); }
      if (s.buf) (void)hipHostFree(s.buf);
    }
  }
  // Copies `bytes` from host memory `src` to device `dst` on `stream`; `src`
  // may be reused as soon as this returns.
  hipError_t copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    std::lock_guard<std::mutex> lk(mu_);
    if (slots_.empty()) slots_.resize(4);
    Slot& s = slots_[next_];
    next_ = (next_ + 1) % slots_.size();
    hipError_t e;
    if (s.ev) {
      e = hipEventSynchronize(s.ev);       // the previous copy out of this slot is done
      if (e != hipSuccess) return e;
    } else {
      e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    if (s.cap < bytes) {
      if (s.buf) (void)hipHostFree(s.buf);   // its last copy completed (event above)
      s.buf = nullptr;
      s.cap = 0;
      e = hipHostMalloc(&s.buf, align_up(bytes, 1 << 20), hipHostMallocDefault);
      if (e != hipSuccess) return e;
      s.cap = align_up(bytes, 1 << 20);
    }
    std::memcpy(s.buf, src, bytes);
    e = hipMemcpyAsync(dst, s.buf, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return e;
    return hipEventRecord(s.ev, stream);
  }

 private:
  struct Slot { void* buf = nullptr; size_t cap = 0; hipEvent_t ev = nullptr; };
  std::vector<Slot> slots_;
  size_t next_ = 0;
  std::mutex mu_;
};

Stager& stager() {
  static Stager* s = new Stager();   // process lifetime (freed by the runtime at exit)
  return *s;
}

// Host-side blob of device metadata arrays, laid out back to back (256-B
// aligned), copied with one staged copy; returns device pointers.
class Blob {
 public:
  template <typename T>
  size_t add(const std::vector<T>& v) {
    size_t off = align_up(bytes_.size());
    bytes_.resize(off + align_up(v.size() * sizeof(T)));
    if (!v.empty()) std::memcpy(bytes_.data() + off, v.data(), v.size() * sizeof(T));
    return off;
  }
  size_t size() const { return bytes_.size(); }
  const uint8_t* data() const { return bytes_.data(); }
  void clear() { bytes_.clear(); }

 private:
  std::vector<uint8_t> bytes_;
};


bool valid_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

// KV token strides are at most n_kv_heads * 128 elements. The attention
// kernel forms per-lane tile offsets as 24-bit products (row < 64 times the
// stride in bytes), which needs strides below 2^24 bytes; 4096 heads give at
// most 1 MB per token.
constexpr int kMaxKVHeads = 4096;

quail_status check_cfg(const quail_model_config* c) {
  if (!c) return fail(QUAIL_E_INVAL, "config is NULL");
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->intermediate <= 0 || c->vocab <= 0)
    return fail(QUAIL_E_INVAL, "config sizes must be positive");
  if (c->max_anchor_len < 0 || c->max_suffix_len <= 0)
    return fail(QUAIL_E_INVAL, "max_anchor_len >= 0 and max_suffix_len > 0 required");
  if (!(c->rms_eps >= 0.0f) || !(c->rope_theta > 0.0f))
    return fail(QUAIL_E_INVAL, "rms_eps >= 0 and rope_theta > 0 required");
  if (c->head_dim != kHeadDim)
    return fail(QUAIL_E_UNSUPPORTED, "head_dim %d (the kernels take 128)", c->head_dim);
  // hidden is the column count of the O and down projections, whose residual
  // epilogue tiles are 128 columns wide; intermediate is cut into 64-column
  // SwiGLU tiles and 64-deep k-steps of the down projection
  if (c->hidden % 128 || c->intermediate % 64)
    return fail(QUAIL_E_UNSUPPORTED, "hidden must be a multiple of 128 and intermediate of 64");
  if (c->n_q_heads % c->n_kv_heads || !valid_group(c->n_q_heads / c->n_kv_heads))
    return fail(QUAIL_E_UNSUPPORTED, "GQA group size must be 1, 2, 4 or 8");
  if (c->n_kv_heads > kMaxKVHeads)
    return fail(QUAIL_E_UNSUPPORTED, "n_kv_heads %d (at most %d)", c->n_kv_heads, kMaxKVHeads);
  if (c->kv_dtype != QUAIL_DTYPE_BF16 && c->kv_dtype != QUAIL_DTYPE_FP8_E4M3)
    return fail(QUAIL_E_UNSUPPORTED, "kv_dtype must be BF16 or FP8_E4M3");
  if (c->kv_dtype == QUAIL_DTYPE_FP8_E4M3 && !(c->k_scale > 0.0f && c->v_scale > 0.0f))
    return fail(QUAIL_E_INVAL, "fp8 KV needs positive k_scale and v_scale");
  if (c->act_dtype != 0 && c->act_dtype != QUAIL_DTYPE_BF16 && c->act_dtype != QUAIL_DTYPE_FP8_E4M3)
    return fail(QUAIL_E_UNSUPPORTED, "act_dtype must be 0, BF16 or FP8_E4M3");
  // W8A8 tiles: 256 output columns (QKV, O, down), 128 SwiGLU columns,
  // k-steps of 128
  if (c->act_dtype == QUAIL_DTYPE_FP8_E4M3 && (c->hidden % 256 || c->intermediate % 128 || c->n_q_heads % 2))
    return fail(QUAIL_E_UNSUPPORTED,
                "fp8 activations need hidden a multiple of 256, intermediate of 128 and even n_q_heads");
  return QUAIL_OK;
}

bool act_fp8(const quail_model_config& c) { return c.act_dtype == QUAIL_DTYPE_FP8_E4M3; }

size_t kv_elem_bytes(const quail_model_config& c) {
  return c.kv_dtype == QUAIL_DTYPE_FP8_E4M3 ? 1 : 2;
}

int32_t pad_len(int32_t la) { return (la + kKeyTile - 1) / kKeyTile * kKeyTile; }

// Every slab ends with a guard region (a fixed pattern written when the slab
// is carved and checked when it is evicted); the pool's last guard-sized
// block is one more.
constexpr size_t kGuard = QUAIL_GUARD_BYTES;
// guard regions checked or written per launch (device offset table capacity)
constexpr int32_t kGuardCap = 4096;

size_t slab_bytes(const quail_model_config& c, int32_t la) {
  return align_up((size_t)c.n_layers * 2 * c.n_kv_heads * (size_t)pad_len(la) * c.head_dim *
                  kv_elem_bytes(c)) + kGuard;
}

int32_t max_pos(const quail_model_config& c) { return c.max_anchor_len + c.max_suffix_len; }

// Workspace carve for a context.
struct WsLayout {
  size_t rope, h, u, q, k, v, o, m, hlast, xq, xs, meta, status, guard, total;
  size_t meta_cap;
};

// KV-source table entries reserved per batch: the table holds every source
// once per layer, and batches are cut so that it fits (max_batch_srcs).
size_t src_entries(int32_t T, int32_t n_layers) {
  return std::max<size_t>((size_t)T + 2, (size_t)4 * std::max(n_layers, 1));
}

size_t meta_capacity(int32_t T, int32_t n_layers) {
  // tok_src, pos, seg_lo, kv_lapad, last_idx, out_idx (int32), kv_row (int64),
  // tiles (<= T + 64), per-layer source tables, plus alignment slack
  return align_up((size_t)T * 4) * 6 + align_up((size_t)T * 8) +
         align_up((size_t)(T + 64) * sizeof(AttnTile)) + align_up(src_entries(T, n_layers) * sizeof(KVSrc)) +
         16 * kAlign;
}

WsLayout ws_layout(const quail_model_config& c, int32_t T) {
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  const size_t Tt = (size_t)T;
  w.rope = take((size_t)max_pos(c) * (c.head_dim / 2) * sizeof(float2));
  w.h = take(Tt * c.hidden * 4);                  // fp32 residual stream
  w.u = take(Tt * c.hidden * 2);
  w.q = take(Tt * c.n_q_heads * c.head_dim * 2);
  w.k = take(Tt * c.n_kv_heads * c.head_dim * 2);
  w.v = take(Tt * c.n_kv_heads * c.head_dim * 2);
  w.o = take(Tt * c.n_q_heads * c.head_dim * 2);
  w.m = take(Tt * c.intermediate * 2);
  w.hlast = take(Tt * c.hidden * 2);
  if (act_fp8(c)) {
    // per-token E4M3 codes of the widest projection input, and their scales
    const size_t wmax = std::max<size_t>({(size_t)c.hidden, (size_t)c.n_q_heads * c.head_dim,
                                          (size_t)c.intermediate});
    w.xq = take(Tt * wmax);
    w.xs = take(Tt * 4);
  }
  w.meta_cap = meta_capacity(T, c.n_layers);
  w.meta = take(w.meta_cap);
  w.status = take(kAlign);                        // debug counters (uint32): guard errors, bad tokens
  w.guard = take((size_t)kGuardCap * sizeof(int64_t));
  w.total = off;
  return w;
}

// ---------------------------------------------------------------------------
// plan builder (shared by quail_plan_build and quail_join_run)
// ---------------------------------------------------------------------------
struct Plan {
  std::vector<int32_t> order, bounds;
  size_t peak = 0;
};

quail_status build_plan(const std::vector<size_t>& slab, int32_t n_pairs, const int32_t* pair_anchor,
                        const int32_t* pair_len, size_t pool_bytes, int32_t max_batch_tokens,
                        Plan& out) {
  const int32_t na = (int32_t)slab.size();
  for (int32_t i = 0; i < n_pairs; ++i) {
    const int32_t a = pair_anchor[i];
    if (a >= na || a < -1) return fail(QUAIL_E_INVAL, "pair %d: anchor index %d out of range", i, a);
    if (pair_len[i] <= 0 || pair_len[i] > max_batch_tokens)
      return fail(QUAIL_E_INVAL, "pair %d: length %d outside [1, %d]", i, pair_len[i], max_batch_tokens);
    if (a >= 0 && slab[a] > pool_bytes)
      return fail(QUAIL_E_NOMEM, "anchor %d: slab of %zu B exceeds the pool (%zu B)", a, slab[a],
                  pool_bytes);
  }
  out.order.resize(n_pairs);
  std::iota(out.order.begin(), out.order.end(), 0);
  auto key = [&](int32_t i) -> int64_t { return pair_anchor[i] < 0 ? INT64_MAX : pair_anchor[i]; };
  std::stable_sort(out.order.begin(), out.order.end(),
                   [&](int32_t x, int32_t y) { return key(x) < key(y); });
  out.bounds.assign(1, 0);
  out.peak = 0;
  int64_t tokens = 0;
  size_t bytes = 0;
  std::unordered_set<int32_t> anchors;
  for (int32_t pos = 0; pos < n_pairs; ++pos) {
    const int32_t i = out.order[pos];
    const int32_t a = pair_anchor[i];
    const int32_t L = pair_len[i];
    size_t add = (a >= 0 && !anchors.count(a)) ? slab[a] : 0;
    if (pos > out.bounds.back() && (tokens + L > max_batch_tokens || bytes + add > pool_bytes)) {
      out.peak = std::max(out.peak, bytes);
      out.bounds.push_back(pos);
      tokens = 0;
      bytes = 0;
      anchors.clear();
      add = a >= 0 ? slab[a] : 0;
    }
    tokens += L;
    if (a >= 0 && !anchors.count(a)) {
      anchors.insert(a);
      bytes += add;
    }
  }
  if (n_pairs > 0) {
    out.peak = std::max(out.peak, bytes);
    out.bounds.push_back(n_pairs);
  }
  return QUAIL_OK;
}

// ---------------------------------------------------------------------------
// plan-wide residency over several joins that share one anchor table
// ([pt] query-aware KV cache bullet: with the whole plan known, KV is kept
// for its next use and evicted when nothing will need it). Each join keeps
// its own single-join plan (it may depend on an earlier join's results, so
// pairs of different joins are not merged); the steps of all joins form one
// sequence, an anchor's last use is its last step in that sequence, and when
// a step's new anchors do not fit beside the kept ones, kept anchors are
// evicted farthest next use first (never again first; ties: larger slab,
// then lower index).
// ---------------------------------------------------------------------------
struct MultiStep {
  int32_t join = 0, lo = 0, hi = 0;           // positions in that join's plan order
  std::vector<int32_t> prefill, evict_before, evict_after;
};
struct MultiPlan {
  std::vector<Plan> plans;
  std::vector<MultiStep> steps;
  int64_t prefills = 0, evictions = 0, regret = 0;
  size_t peak = 0;
};

quail_status build_multiplan(const std::vector<size_t>& slab, const std::vector<int32_t>& alen,
                             int32_t n_joins, const int32_t* join_off, const int32_t* pair_anchor,
                             const int32_t* pair_len, size_t pool_bytes, int32_t max_batch_tokens,
                             MultiPlan& out) {
  const int32_t na = (int32_t)slab.size();
  out = MultiPlan{};
  out.plans.resize(n_joins);
  std::vector<std::vector<int32_t>> step_anchors;   // per global step, first-use order
  for (int32_t j = 0; j < n_joins; ++j) {
    const int32_t p0 = join_off[j], np = join_off[j + 1] - join_off[j];
    if (quail_status st = build_plan(slab, np, pair_anchor + p0, pair_len + p0, pool_bytes,
                                     max_batch_tokens, out.plans[j]))
      return st;
    const Plan& pl = out.plans[j];
    for (size_t t = 0; t + 1 < pl.bounds.size(); ++t) {
      MultiStep ms;
      ms.join = j;
      ms.lo = pl.bounds[t];
      ms.hi = pl.bounds[t + 1];
      std::vector<int32_t> an;
      for (int32_t k = ms.lo; k < ms.hi; ++k) {
        const int32_t a = pair_anchor[p0 + pl.order[k]];
        if (a >= 0 && std::find(an.begin(), an.end(), a) == an.end()) an.push_back(a);
      }
      out.steps.push_back(std::move(ms));
      step_anchors.push_back(std::move(an));
    }
  }
  const int32_t T = (int32_t)out.steps.size();
  std::vector<std::vector<int32_t>> uses_at(na);
  for (int32_t t = 0; t < T; ++t)
    for (int32_t a : step_anchors[t]) uses_at[a].push_back(t);
  auto next_use = [&](int32_t a, int32_t t) -> int32_t {
    auto it = std::upper_bound(uses_at[a].begin(), uses_at[a].end(), t);
    return it == uses_at[a].end() ? T : *it;
  };
  std::vector<char> resident(na, 0), ever(na, 0);
  size_t bytes = 0;
  for (int32_t t = 0; t < T; ++t) {
    MultiStep& ms = out.steps[t];
    const std::vector<int32_t>& an = step_anchors[t];
    size_t need_b = 0;
    for (int32_t a : an)
      if (!resident[a]) need_b += slab[a];
    while (bytes + need_b > pool_bytes) {
      int32_t best = -1;
      for (int32_t a = 0; a < na; ++a) {
        if (!resident[a] || std::find(an.begin(), an.end(), a) != an.end()) continue;
        if (best < 0) { best = a; continue; }
        const int32_t nu = next_use(a, t), nb = next_use(best, t);
        if (nu > nb || (nu == nb && slab[a] > slab[best])) best = a;   // lower index wins the rest
      }
      if (best < 0) return fail(QUAIL_E_NOMEM, "step %d: its anchors do not fit the pool", t);
      resident[best] = 0;
      bytes -= slab[best];
      out.evictions++;
      ms.evict_before.push_back(best);
    }
    for (int32_t a : an) {
      if (resident[a]) continue;
      if (ever[a]) out.regret += alen[a];
      ever[a] = 1;
      resident[a] = 1;
      bytes += slab[a];
      out.prefills++;
      ms.prefill.push_back(a);
    }
    out.peak = std::max(out.peak, bytes);
    std::vector<int32_t> after;
    for (int32_t a : an)
      if (next_use(a, t) == T) after.push_back(a);
    std::sort(after.begin(), after.end());
    for (int32_t a : after) {
      resident[a] = 0;
      bytes -= slab[a];
      out.evictions++;
    }
    ms.evict_after = std::move(after);
  }
  return QUAIL_OK;
}

// ---------------------------------------------------------------------------
// radix index over suffix token sequences (shared-prefix grouping)
// ---------------------------------------------------------------------------
// Sequence i = tokens[starts[i] .. starts[i] + lens[i]) with key keys[i]
// (the anchor it continues; negative = not grouped). The sequences are sorted
// by (key, tokens); in that order the longest common prefix of a run is the
// minimum of its adjacent LCPs, and the sequences sharing their first
// min_len tokens form one contiguous run -- the subtrees of the per-key radix
// tree at depth min_len. A run of two or more becomes a node whose prefix is
// the run's common prefix, cut so every member keeps at least one token.
// Nodes are numbered by their smallest member. Returns the node count.
int32_t prefix_groups(int32_t n, const int32_t* tokens, const int32_t* starts, const int32_t* lens,
                      const int32_t* keys, int32_t min_len, int32_t* group_of, int32_t* node_first,
                      int32_t* node_len) {
  auto key = [&](int32_t i) { return keys ? keys[i] : 0; };
  std::vector<int32_t> cand;
  for (int32_t i = 0; i < n; ++i) {
    group_of[i] = -1;
    if (key(i) >= 0 && lens[i] > min_len) cand.push_back(i);
  }
  auto lcp = [&](int32_t x, int32_t y) {
    const int32_t m = std::min(lens[x], lens[y]);
    const int32_t* a = tokens + starts[x];
    const int32_t* b = tokens + starts[y];
    int32_t k = 0;
    while (k < m && a[k] == b[k]) ++k;
    return k;
  };
  std::sort(cand.begin(), cand.end(), [&](int32_t x, int32_t y) {
    if (key(x) != key(y)) return key(x) < key(y);
    const int32_t k = lcp(x, y);
    if (k < lens[x] && k < lens[y]) return tokens[starts[x] + k] < tokens[starts[y] + k];
    if (lens[x] != lens[y]) return lens[x] < lens[y];
    return x < y;
  });
  std::vector<std::pair<int32_t, int32_t>> nodes;   // (smallest member, prefix length)
  std::vector<std::vector<int32_t>> members;
  for (size_t i = 0; i < cand.size();) {
    size_t j = i + 1;
    int32_t run_lcp = INT32_MAX;
    while (j < cand.size() && key(cand[j]) == key(cand[i])) {
      const int32_t l = lcp(cand[j - 1], cand[j]);
      if (l < min_len) break;
      run_lcp = std::min(run_lcp, l);
      ++j;
    }
    if (j - i >= 2) {
      int32_t shortest = INT32_MAX, first = INT32_MAX;
      for (size_t k = i; k < j; ++k) {
        shortest = std::min(shortest, lens[cand[k]]);
        first = std::min(first, cand[k]);
      }
      nodes.push_back({first, std::min(run_lcp, shortest - 1)});
      members.emplace_back(cand.begin() + i, cand.begin() + j);
    }
    i = j;
  }
  std::vector<int32_t> idx(nodes.size());
  std::iota(idx.begin(), idx.end(), 0);
  std::sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return nodes[x].first < nodes[y].first; });
  for (size_t r = 0; r < idx.size(); ++r) {
    node_first[r] = nodes[idx[r]].first;
    node_len[r] = nodes[idx[r]].second;
    for (int32_t m : members[idx[r]]) group_of[m] = (int32_t)r;
  }
  return (int32_t)nodes.size();
}

// Nested shared prefixes: prefix_groups' nodes are the top level; inside a
// node that covers tokens up to `end`, its members are split by their token
// at `end`, and a part of two or more whose common prefix (cut so that each
// member keeps a token) reaches end + min_len becomes a child node covering
// [end, its cut), recursively; all other members stay with the node. Nodes
// are numbered parents first: each top-level node (by smallest member)
// followed by its subtree, children by smallest member. group_of[i] = the
// deepest node of sequence i, or -1.
struct TreeNode {
  int32_t parent, first, start, end;
};
void prefix_tree(int32_t n, const int32_t* tokens, const int32_t* starts, const int32_t* lens,
                 const int32_t* keys, int32_t min_len, int32_t* group_of, std::vector<TreeNode>& out) {
  std::vector<int32_t> nf(std::max(n, 1)), nl(std::max(n, 1));
  const int32_t nn = prefix_groups(n, tokens, starts, lens, keys, min_len, group_of, nf.data(), nl.data());
  std::vector<std::vector<int32_t>> top(nn);
  for (int32_t i = 0; i < n; ++i)
    if (group_of[i] >= 0) top[group_of[i]].push_back(i);
  auto tok = [&](int32_t i, int32_t k) { return tokens[starts[i] + k]; };
  auto cut_lcp = [&](const std::vector<int32_t>& m) {
    int32_t common = lens[m[0]], shortest = INT32_MAX;
    for (int32_t i : m) {
      const int32_t lim = std::min(common, lens[i]);
      int32_t k = 0;
      while (k < lim && tok(i, k) == tok(m[0], k)) ++k;
      common = k;
      shortest = std::min(shortest, lens[i]);
    }
    return std::min(common, shortest - 1);
  };
  std::function<void(const std::vector<int32_t>&, int32_t, int32_t)> build =
      [&](const std::vector<int32_t>& m, int32_t parent, int32_t start) {
        const int32_t end = cut_lcp(m);
        const int32_t me = (int32_t)out.size();
        out.push_back({parent, *std::min_element(m.begin(), m.end()), start, end});
        for (int32_t i : m) group_of[i] = me;
        std::map<int32_t, std::vector<int32_t>> parts;
        for (int32_t i : m) parts[tok(i, end)].push_back(i);
        std::vector<std::vector<int32_t>> ps;
        for (auto& kv : parts) ps.push_back(std::move(kv.second));
        std::sort(ps.begin(), ps.end(), [](const std::vector<int32_t>& a, const std::vector<int32_t>& b) {
          return *std::min_element(a.begin(), a.end()) < *std::min_element(b.begin(), b.end());
        });
        for (const auto& part : ps)
          if (part.size() >= 2 && cut_lcp(part) >= end + min_len) build(part, me, end);
      };
  for (int32_t k = 0; k < nn; ++k) build(top[k], -1, 0);
}

}  // namespace

// ---------------------------------------------------------------------------
// context
// ---------------------------------------------------------------------------
struct quail_ctx {
  quail_model_config cfg;
  quail_weights w;
  std::vector<quail_layer_weights> layers;
  uint8_t* pool = nullptr;
  size_t pool_bytes = 0;
  uint8_t* ws = nullptr;
  size_t ws_bytes = 0;
  int32_t T = 0;                      // max batch tokens
  WsLayout L{};
  bool ready = false;                 // RoPE table, debug counters and the pool's tail guard are set
  bool dry = false;                   // placement dry run: bookkeeping only, nothing enqueued
  size_t tail_guard = SIZE_MAX;       // pool offset of the tail guard (none if the pool is too small)
  std::vector<int64_t> pending_checks;   // guard regions of evicted slabs, checked before reuse

  // per-launch timing (quail_ctx_profile): an event before and after each launch
  struct ProfRec { int32_t kind; hipEvent_t e0, e1; double flop; };
  bool prof_on = false;
  std::vector<ProfRec> prof;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_next = 0;

  // residency
  struct Slot {
    bool live = false;
    uint32_t gen = 0;
    size_t off = 0, bytes = 0;
    int32_t len = 0, lapad = 0;
    int64_t uses = 0;
    // two-level cascade: a shared-prefix node continues anchor slot `parent`
    // at positions pos0.. (pos0 = the anchor's length) and holds one of the
    // anchor's uses until it is evicted; `held` counts such holds on an anchor
    int32_t parent = -1, pos0 = 0;
    int64_t held = 0;
    // nested node: its first `copied` slab rows are its parent node's rows
    // (copied at prefill), then its own tokens
    int32_t copied = 0;
  };
  std::vector<Slot> slots;
  std::vector<int32_t> free_slots;
  std::vector<std::pair<size_t, size_t>> free_list;   // (offset, size), sorted by offset
  size_t resident = 0, peak = 0;
  int64_t prefills = 0, evictions = 0, regret = 0;
  std::unordered_set<int64_t> seen_ids;
  int64_t run_serial = 0;            // quail_join_run calls (namespaces their anchor ids)

  Blob blob;

  bool alloc(size_t bytes, size_t& off) {
    for (size_t i = 0; i < free_list.size(); ++i) {
      if (free_list[i].second >= bytes) {
        off = free_list[i].first;
        free_list[i].first += bytes;
        free_list[i].second -= bytes;
        if (free_list[i].second == 0) free_list.erase(free_list.begin() + i);
        return true;
      }
    }
    return false;
  }
  void release(size_t off, size_t bytes) {
    auto it = std::lower_bound(free_list.begin(), free_list.end(), std::make_pair(off, (size_t)0));
    it = free_list.insert(it, {off, bytes});
    size_t i = it - free_list.begin();
    if (i + 1 < free_list.size() && free_list[i].first + free_list[i].second == free_list[i + 1].first) {
      free_list[i].second += free_list[i + 1].second;
      free_list.erase(free_list.begin() + i + 1);
    }
    if (i > 0 && free_list[i - 1].first + free_list[i - 1].second == free_list[i].first) {
      free_list[i - 1].second += free_list[i].second;
      free_list.erase(free_list.begin() + i);
    }
  }
  Slot* lookup(quail_anchor h) {
    if (h < 0) return nullptr;
    const uint32_t slot = (uint32_t)(h & 0xFFFFFFFF);
    const uint32_t gen = (uint32_t)((uint64_t)h >> 32);
    if (slot >= slots.size()) return nullptr;
    Slot& s = slots[slot];
    if (!s.live || s.gen != gen) return nullptr;
    return &s;
  }
  void evict(int32_t slot) {
    Slot& s = slots[slot];
    pending_checks.push_back((int64_t)(s.off + s.bytes - kGuard));
    release(s.off, s.bytes);
    resident -= s.bytes;
    s.live = false;
    s.gen++;
    free_slots.push_back(slot);
    evictions++;
    const int32_t par = s.parent;
    s.parent = -1;
    s.held = 0;
    if (par >= 0) {   // a prefix node spends the anchor use it held
      Slot& ps = slots[par];
      ps.held--;
      if (--ps.uses == 0) evict(par);
    }
  }
};

namespace {

template <typename T>
T* ws_ptr(quail_ctx* c, size_t off) { return reinterpret_cast<T*>(c->ws + off); }

// First enqueueing call of a context: the RoPE table, zeroed debug counters
// and the pool's tail guard.
quail_status ensure_ready(quail_ctx* c, hipStream_t s) {
  if (c->ready || c->dry) return QUAIL_OK;
  const int P = max_pos(c->cfg);
  const int half = c->cfg.head_dim / 2;
  std::vector<float2> tab((size_t)P * half);
  for (int p = 0; p < P; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)c->cfg.rope_theta, -2.0 * i / c->cfg.head_dim);
      const double ang = (double)p * inv;
      tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  HIP_TRY(stager().copy(c->ws + c->L.rope, tab.data(), tab.size() * sizeof(float2), s));
  HIP_TRY(launch_zero_words(ws_ptr<uint32_t>(c, c->L.status), 2, s));
  if (c->tail_guard != SIZE_MAX) {
    const int64_t off = (int64_t)c->tail_guard;
    HIP_TRY(stager().copy(c->ws + c->L.guard, &off, sizeof off, s));
    HIP_TRY(launch_guard(c->pool, ws_ptr<const int64_t>(c, c->L.guard), 1, 1, nullptr, s));
  }
  c->ready = true;
  return QUAIL_OK;
}

// Writes (mode 1) or checks (mode 0) the guard regions at pool offsets offs.
quail_status guard_op(quail_ctx* c, const std::vector<int64_t>& offs, int32_t mode, hipStream_t s) {
  if (c->dry || offs.empty()) return QUAIL_OK;
  if (quail_status st = ensure_ready(c, s)) return st;
  for (size_t i = 0; i < offs.size(); i += kGuardCap) {
    const int32_t n = (int32_t)std::min<size_t>(kGuardCap, offs.size() - i);
    HIP_TRY(stager().copy(c->ws + c->L.guard, offs.data() + i, n * sizeof(int64_t), s));
    HIP_TRY(launch_guard(c->pool, ws_ptr<const int64_t>(c, c->L.guard), n, mode,
                         ws_ptr<uint32_t>(c, c->L.status), s));
  }
  return QUAIL_OK;
}

// Checks the guards of slabs evicted since the last flush. Called before any
// work that may reuse their memory is enqueued.
quail_status flush_guard_checks(quail_ctx* c, hipStream_t s) {
  if (c->dry || c->pending_checks.empty()) return QUAIL_OK;
  if (quail_status st = guard_op(c, c->pending_checks, 0, s)) return st;
  c->pending_checks.clear();
  return QUAIL_OK;
}

// Per-launch timing marks (no-ops unless profiling is on).
enum ProfKind : int32_t { PK_QKV = 0, PK_O = 1, PK_GATE_UP = 2, PK_DOWN = 3, PK_ATTN = 4, PK_NORM = 5,
                          PK_OTHER = 6, PK_COUNT = 7 };

hipError_t prof_mark(quail_ctx* c, hipStream_t s, hipEvent_t* ev) {
  *ev = nullptr;
  if (!c->prof_on) return hipSuccess;
  if (c->ev_next == c->ev_pool.size()) {
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return r;
    c->ev_pool.push_back(e);
  }
  *ev = c->ev_pool[c->ev_next++];
  return hipEventRecord(*ev, s);
}

void prof_add(quail_ctx* c, int32_t kind, hipEvent_t e0, hipEvent_t e1, double flop) {
  if (c->prof_on && e0 && e1) c->prof.push_back({kind, e0, e1, flop});
}

// Launch `expr` between two timing marks of kind `kind` (algorithmic FLOP `flop`).
#define TIMED(kind, flop, expr)                                   \
  do {                                                            \
    hipEvent_t e0_, e1_;                                          \
    HIP_TRY(prof_mark(c, s, &e0_));                               \
    HIP_TRY(expr);                                                \
    HIP_TRY(prof_mark(c, s, &e1_));                               \
    prof_add(c, kind, e0_, e1_, (double)(flop));                  \
  } while (0)

// One batch of token rows through the decoder stack.
struct Batch {
  bool anchor_mode = false;
  bool has_parent = false;                  // anchor_mode: prefix nodes (cross = their anchor's slab)
  bool two_level = false;                   // some tile reads a prefix node as cross2
  int pack = 0;                             // packed attention tiles: waves per tile (0 = unpacked)
  int32_t n_tok = 0;
  std::vector<int32_t> tok_src, pos, seg_lo, kv_lapad;
  std::vector<int64_t> kv_row;
  std::vector<AttnTile> tiles;
  std::vector<KVSrc> srcs;
  std::vector<int64_t> src_layer_stride;   // per src, elements per layer
  // outputs
  std::vector<int32_t> last_row, last_dst;  // h_last: row -> destination row
  std::vector<int32_t> all_dst;             // h_all: internal row -> caller token row
};

// The layer-stride of a KV source is folded in by patching the srcs per layer.
quail_status run_batch(quail_ctx* c, const Batch& b, const int32_t* tokens, uint16_t* h_last,
                       uint16_t* h_all, hipStream_t s) {
  const quail_model_config& cf = c->cfg;
  const int H = cf.hidden, Hq = cf.n_q_heads, Hkv = cf.n_kv_heads, I = cf.intermediate;
  const int G = Hq / Hkv;
  const int n = b.n_tok;
  if (n == 0) return QUAIL_OK;

  // metadata blob: per-layer src tables are laid out back to back
  Blob& bl = c->blob;
  bl.clear();
  const size_t o_tok = bl.add(b.tok_src), o_pos = bl.add(b.pos), o_seg = bl.add(b.seg_lo);
  const size_t o_lap = bl.add(b.kv_lapad), o_row = bl.add(b.kv_row), o_til = bl.add(b.tiles);
  const size_t o_ldst = bl.add(b.last_row), o_ldd = bl.add(b.last_dst), o_all = bl.add(b.all_dst);
  const int nl_attn = b.anchor_mode ? cf.n_layers - 1 : cf.n_layers;
  std::vector<KVSrc> srcs_all;
  srcs_all.reserve((size_t)std::max(nl_attn, 1) * b.srcs.size());
  for (int l = 0; l < std::max(nl_attn, 1); ++l)
    for (size_t i = 0; i < b.srcs.size(); ++i) {
      KVSrc x = b.srcs[i];
      const size_t esz = x.fp8 ? 1 : 2;
      x.k = reinterpret_cast<const uint8_t*>(x.k) + (size_t)l * b.src_layer_stride[i] * esz;
      x.v = reinterpret_cast<const uint8_t*>(x.v) + (size_t)l * b.src_layer_stride[i] * esz;
      srcs_all.push_back(x);
    }
  const size_t o_src = bl.add(srcs_all);
  if (bl.size() > c->L.meta_cap)
    return fail(QUAIL_E_NOMEM, "batch metadata (%zu B) exceeds its workspace region", bl.size());
  if (c->dry) return QUAIL_OK;
  // algorithmic attention FLOP of the batch (per layer): 4 * Hq * d per
  // (query row, visible key) -- every key of the cross sources, the causal
  // self keys from the segment start to the row
  double attn_flop = 0.0;
  if (c->prof_on) {
    double keys = 0.0;
    for (const AttnTile& tl : b.tiles)
      for (int32_t r = 0; r < tl.nq; ++r) {
        if (tl.cross >= 0) keys += b.srcs[tl.cross].len;
        if (tl.cross2 >= 0) keys += b.srcs[tl.cross2].len;
        if (tl.self >= 0) keys += tl.self_qbase + r - std::max(tl.self_k0, b.seg_lo[tl.q0 + r]) + 1;
      }
    attn_flop = 4.0 * Hq * kHeadDim * keys;
  }
  uint8_t* md = c->ws + c->L.meta;
  HIP_TRY(stager().copy(md, bl.data(), bl.size(), s));

  auto dp = [&](size_t off) { return md + off; };
  const int32_t* d_tok = reinterpret_cast<const int32_t*>(dp(o_tok));
  const int32_t* d_pos = reinterpret_cast<const int32_t*>(dp(o_pos));
  const int32_t* d_seg = reinterpret_cast<const int32_t*>(dp(o_seg));
  const int32_t* d_lap = reinterpret_cast<const int32_t*>(dp(o_lap));
  const int64_t* d_row = reinterpret_cast<const int64_t*>(dp(o_row));
  const AttnTile* d_til = reinterpret_cast<const AttnTile*>(dp(o_til));
  const KVSrc* d_src = reinterpret_cast<const KVSrc*>(dp(o_src));

  float* hbuf = ws_ptr<float>(c, c->L.h);
  uint16_t* ubuf = ws_ptr<uint16_t>(c, c->L.u);
  uint16_t* qbuf = ws_ptr<uint16_t>(c, c->L.q);
  uint16_t* kbuf = ws_ptr<uint16_t>(c, c->L.k);
  uint16_t* vbuf = ws_ptr<uint16_t>(c, c->L.v);
  uint16_t* obuf = ws_ptr<uint16_t>(c, c->L.o);
  uint16_t* mbuf = ws_ptr<uint16_t>(c, c->L.m);
  const float2* rope = ws_ptr<const float2>(c, c->L.rope);

  uint32_t* status = ws_ptr<uint32_t>(c, c->L.status);
  // W8A8: each projection reads per-token E4M3 codes (xq) and scales (xs) of
  // its input; the norms write them directly, the attention output and the
  // MLP product go through the quantiser
  const bool a8 = act_fp8(cf);
  uint8_t* xq = a8 ? c->ws + c->L.xq : nullptr;
  float* xs = a8 ? ws_ptr<float>(c, c->L.xs) : nullptr;
  // A join batch whose only output is each pair's last row (h_last, no
  // h_all) needs, at the last layer, every row's K/V and attention (the last
  // rows attend to them) but the O projection, the MLP and their residual
  // adds only for the last rows: those run on the gathered last rows. Each
  // row's arithmetic is the same wherever it sits in a GEMM tile, so the
  // result is bit-identical to running every row.
  const bool prune_tail = !b.anchor_mode && h_all == nullptr && h_last != nullptr && !b.last_row.empty();
  const int32_t* d_last = reinterpret_cast<const int32_t*>(dp(o_ldst));
  const int32_t n_last = (int32_t)b.last_row.size();
  TIMED(PK_OTHER, 0, launch_embed(tokens, d_tok, c->w.embed, hbuf, n, H, cf.vocab, status + 1, s));
  for (int l = 0; l < cf.n_layers; ++l) {
    const quail_layer_weights& lw = c->layers[l];
    NormParams np{};
    np.x = hbuf; np.ldx = H; np.gamma = lw.attn_norm; np.y = ubuf; np.ldy = H;
    np.rows = n; np.H = H; np.eps = cf.rms_eps;
    np.yq = xq; np.ys = xs;
    TIMED(PK_NORM, 0, launch_rmsnorm(np, s));

    GemmParams gp{};
    gp.A = ubuf; gp.lda = H; gp.B = lw.w_qkv; gp.scale = lw.s_qkv;
    gp.A8 = xq; gp.a_scale = xs;
    gp.M = n; gp.N = (Hq + 2 * Hkv) * kHeadDim; gp.K = H;
    gp.hq = Hq; gp.hkv = Hkv; gp.rope = rope; gp.pos = d_pos; gp.q_out = qbuf;
    gp.layer = l;
    if (b.anchor_mode) {
      gp.kv_mode = 1; gp.pool = c->pool; gp.kv_row = d_row; gp.kv_lapad = d_lap;
      gp.kv_fp8 = cf.kv_dtype == QUAIL_DTYPE_FP8_E4M3;
      gp.k_inv_scale = 1.0f / cf.k_scale; gp.v_inv_scale = 1.0f / cf.v_scale;
    } else {
      gp.kv_mode = 0; gp.k_out = kbuf; gp.v_out = vbuf;
    }
    TIMED(PK_QKV, 2.0 * n * gp.N * gp.K, launch_gemm(gp, EPI_QKV, s));
    if (b.anchor_mode && l == cf.n_layers - 1) break;   // last layer: K/V is all an anchor needs

    AttnParams ap{};
    ap.tiles = d_til; ap.n_tiles = (int32_t)b.tiles.size();
    ap.srcs = d_src + (size_t)l * b.srcs.size();
    ap.seg_lo = d_seg; ap.q = qbuf; ap.q_stride = (int64_t)Hq * kHeadDim;
    ap.out = obuf; ap.o_stride = (int64_t)Hq * kHeadDim; ap.lse = nullptr;
    ap.hq = Hq; ap.hkv = Hkv;
    ap.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)kHeadDim));
    ap.k_scale = cf.k_scale; ap.v_scale = cf.v_scale;
    ap.two_level = b.two_level;
    // anchor batches attend over their own slab (self source); join batches
    // read the anchor slab as the cross source and bf16 suffix K/V as self
    const bool slab_fp8 = cf.kv_dtype == QUAIL_DTYPE_FP8_E4M3;
    TIMED(PK_ATTN, attn_flop,
          launch_attn_bf16(ap, G, (!b.anchor_mode || b.has_parent) && slab_fp8, b.anchor_mode && slab_fp8,
                           b.pack, s));

    // rows that go on (the last rows only, gathered, at the last layer of a
    // pruned batch)
    const bool tail = prune_tail && l == cf.n_layers - 1;
    const int32_t m = tail ? n_last : n;
    const int32_t* rmap = tail ? d_last : nullptr;

    if (a8) TIMED(PK_NORM, 0, launch_act_quant_e4m3(n, Hq * kHeadDim, obuf, xq, xs, s));
    GemmParams go{};
    go.A = obuf; go.lda = (int64_t)Hq * kHeadDim; go.B = lw.w_o; go.scale = lw.s_o;
    go.A8 = xq; go.a_scale = xs;
    go.M = m; go.N = H; go.K = Hq * kHeadDim; go.Yf = hbuf; go.ldy = H;
    go.a_map = rmap; go.y_map = rmap;
    TIMED(PK_O, 2.0 * m * go.N * go.K, launch_gemm(go, EPI_RESID, s));

    np.gamma = lw.mlp_norm; np.rows = m; np.row_map = rmap;
    TIMED(PK_NORM, 0, launch_rmsnorm(np, s));

    GemmParams gg{};
    gg.A = ubuf; gg.lda = H; gg.B = lw.w_gate_up; gg.scale = lw.s_gate_up;
    gg.M = m; gg.N = I; gg.K = H; gg.Y = mbuf; gg.ldy = I; gg.inter = I;
    gg.A8 = xq; gg.a_scale = xs;
    TIMED(PK_GATE_UP, 2.0 * m * 2.0 * gg.N * gg.K, launch_gemm(gg, EPI_SWIGLU, s));

    if (a8) TIMED(PK_NORM, 0, launch_act_quant_e4m3(m, I, mbuf, xq, xs, s));
    GemmParams gd{};
    gd.A = mbuf; gd.lda = I; gd.B = lw.w_down; gd.scale = lw.s_down;
    gd.A8 = xq; gd.a_scale = xs;
    gd.M = m; gd.N = H; gd.K = I; gd.Yf = hbuf; gd.ldy = H;
    gd.y_map = rmap;
    TIMED(PK_DOWN, 2.0 * m * gd.N * gd.K, launch_gemm(gd, EPI_RESID, s));
  }
  if (!b.anchor_mode) {
    if (h_last && !b.last_row.empty()) {
      // h_last[last_dst[i]] = h[last_row[i]]
      HIP_TRY(launch_copy_rows(hbuf, H, reinterpret_cast<const int32_t*>(dp(o_ldst)), h_last, H,
                               reinterpret_cast<const int32_t*>(dp(o_ldd)),
                               (int32_t)b.last_row.size(), H, s));
    }
    if (h_all) {
      HIP_TRY(launch_copy_rows(hbuf, H, nullptr, h_all, H,
                               reinterpret_cast<const int32_t*>(dp(o_all)), n, H, s));
    }
  }
  return QUAIL_OK;
}

// Append the KV source of a slab (K and V of layer 0; run_batch adds the
// layer stride).
void push_slab_src(quail_ctx* c, Batch& b, const quail_ctx::Slot& sl) {
  const quail_model_config& cf = c->cfg;
  const size_t esz = kv_elem_bytes(cf);
  KVSrc ks{};
  ks.k = c->pool + sl.off;
  ks.v = c->pool + sl.off + (size_t)cf.n_kv_heads * sl.lapad * kHeadDim * esz;
  ks.tok_stride = kHeadDim;
  ks.head_stride = (int64_t)sl.lapad * kHeadDim;
  ks.len = sl.len;
  ks.fp8 = cf.kv_dtype == QUAIL_DTYPE_FP8_E4M3;
  b.srcs.push_back(ks);
  b.src_layer_stride.push_back((int64_t)2 * cf.n_kv_heads * sl.lapad * kHeadDim);
}

// The batch's source index of slab `slot`, added on first use.
int32_t slab_src(quail_ctx* c, Batch& b, int32_t slot, std::unordered_map<int32_t, int32_t>& src_of) {
  auto it = src_of.find(slot);
  if (it != src_of.end()) return it->second;
  const int32_t idx = (int32_t)b.srcs.size();
  push_slab_src(c, b, c->slots[slot]);
  src_of[slot] = idx;
  return idx;
}

// Sources one batch may read (suffix K/V and slabs) so that its per-layer
// source tables fit the metadata region: at least 4 (suffix K/V, a node and
// its anchor, and one more).
int32_t max_batch_srcs(const quail_ctx* c) {
  return (int32_t)(src_entries(c->T, c->cfg.n_layers) / std::max(c->cfg.n_layers, 1));
}

// Slab sources that reading slot `sl` adds to a batch whose slabs are `in`
// (the slot itself, and a node's anchor), recording them.
int32_t add_slab_srcs(const quail_ctx* c, int32_t sl, std::unordered_set<int32_t>& in, bool commit) {
  int32_t add = 0;
  if (sl < 0) return 0;
  const int32_t par = c->slots[sl].parent;
  if (!in.count(sl)) ++add;
  if (par >= 0 && !in.count(par)) ++add;
  if (commit) {
    in.insert(sl);
    if (par >= 0) in.insert(par);
  }
  return add;
}

quail_status check_offsets(int32_t n, const int32_t* off, int32_t lo, int32_t hi, const char* what) {
  if (n < 0) return fail(QUAIL_E_INVAL, "%s: negative count", what);
  if (n > 0 && !off) return fail(QUAIL_E_INVAL, "%s: offsets are NULL", what);
  if (n > 0 && off[0] < 0) return fail(QUAIL_E_INVAL, "%s: offsets[0] < 0", what);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = (int64_t)off[i + 1] - off[i];
    if (len < lo || len > hi)
      return fail(QUAIL_E_INVAL, "%s %d: length %lld outside [%d, %d]", what, i, (long long)len, lo, hi);
  }
  return QUAIL_OK;
}

hipStream_t as_stream(quail_stream s) { return reinterpret_cast<hipStream_t>(s); }

// Anchor prefill core: anchor a = tokens[starts[a] .. starts[a] + lens[a]).
// With `parents`, entry a with parents[a] >= 0 is a shared-prefix node
// continuing anchor slot parents[a]: its tokens sit at positions La.. and
// attend to the whole anchor (cross) and causally to themselves (its own
// slab); the caller has checked that each parent has a use to spare per node.
// parents[a] = -1 is a plain anchor (the shared prefix of filter rows).
// With copy_from[a] >= 0 (a node slot), entry a is a nested node: its slab
// starts with that node's rows (copied here), and its own lens[a] tokens
// follow at positions La + (copied rows)..
quail_status anchor_core(quail_ctx* c, int32_t n, const int32_t* tokens, const int32_t* starts,
                         const int32_t* lens, const int32_t* n_uses, const int64_t* anchor_ids,
                         quail_anchor* out, hipStream_t s, const int32_t* parents = nullptr,
                         const int32_t* copy_from = nullptr) {
  if (!n_uses || !out) return fail(QUAIL_E_INVAL, "n_uses and out are required");
  if (!tokens) return fail(QUAIL_E_INVAL, "tokens is NULL");
  for (int32_t a = 0; a < n; ++a)
    if (n_uses[a] < 0) return fail(QUAIL_E_INVAL, "anchor %d: negative use count", a);
  // carve all slabs first (all or nothing)
  std::vector<std::pair<size_t, size_t>> got;
  std::vector<int32_t> slot_of(n, -1);
  auto copied_rows = [&](int32_t a) { return copy_from && copy_from[a] >= 0 ? c->slots[copy_from[a]].len : 0; };
  for (int32_t a = 0; a < n; ++a) {
    if (n_uses[a] == 0) continue;
    const size_t bytes = slab_bytes(c->cfg, copied_rows(a) + lens[a]);
    size_t off;
    if (!c->alloc(bytes, off)) {
      for (auto& g : got) c->release(g.first, g.second);
      return fail(QUAIL_E_NOMEM, "KV pool cannot hold the %d new anchor slabs", n);
    }
    got.push_back({off, bytes});
  }
  size_t gi = 0;
  for (int32_t a = 0; a < n; ++a) {
    if (n_uses[a] == 0) { out[a] = QUAIL_NO_ANCHOR; continue; }
    int32_t slot;
    if (!c->free_slots.empty()) { slot = c->free_slots.back(); c->free_slots.pop_back(); }
    else { slot = (int32_t)c->slots.size(); c->slots.emplace_back(); }
    quail_ctx::Slot& sl = c->slots[slot];
    sl.live = true;
    sl.off = got[gi].first;
    sl.bytes = got[gi].second;
    ++gi;
    sl.copied = copied_rows(a);
    sl.len = sl.copied + lens[a];
    sl.lapad = pad_len(sl.len);
    sl.uses = n_uses[a];
    sl.held = 0;
    sl.parent = parents ? parents[a] : -1;
    sl.pos0 = sl.parent >= 0 ? c->slots[sl.parent].len : 0;
    if (sl.parent >= 0) c->slots[sl.parent].held++;
    slot_of[a] = slot;
    out[a] = ((int64_t)sl.gen << 32) | (uint32_t)slot;
    c->resident += sl.bytes;
    c->prefills++;
    if (anchor_ids) {
      if (c->seen_ids.count(anchor_ids[a])) c->regret += sl.len;
      else c->seen_ids.insert(anchor_ids[a]);
    }
  }
  c->peak = std::max(c->peak, c->resident);
  if (c->dry) return QUAIL_OK;

  if (quail_status st = ensure_ready(c, s)) return st;
  // slabs evicted earlier are checked before their memory is written again;
  // then every new slab's guard is set
  if (quail_status st = flush_guard_checks(c, s)) return st;
  {
    std::vector<int64_t> guards;
    for (int32_t a = 0; a < n; ++a)
      if (slot_of[a] >= 0) {
        const quail_ctx::Slot& sl = c->slots[slot_of[a]];
        guards.push_back((int64_t)(sl.off + sl.bytes - kGuard));
      }
    if (quail_status st = guard_op(c, guards, 1, s)) return st;
  }
  const quail_model_config& cf = c->cfg;
  const int G = cf.n_q_heads / cf.n_kv_heads;
  const size_t esz = kv_elem_bytes(cf);
  const bool slab_fp8 = cf.kv_dtype == QUAIL_DTYPE_FP8_E4M3;
  // nested nodes: the parent node's rows, every layer, K and V, every kv head
  for (int32_t a = 0; a < n && copy_from; ++a) {
    if (n_uses[a] == 0 || copy_from[a] < 0) continue;
    const quail_ctx::Slot& from = c->slots[copy_from[a]];
    const quail_ctx::Slot& to = c->slots[slot_of[a]];
    const int32_t row_bytes = (int32_t)(kHeadDim * esz);
    HIP_TRY(launch_copy_slab_rows(c->pool + from.off, (int64_t)from.lapad * row_bytes, c->pool + to.off,
                                  (int64_t)to.lapad * row_bytes, to.copied, row_bytes,
                                  cf.n_layers * 2 * cf.n_kv_heads, s));
  }
  // batches of whole anchors up to T tokens
  int32_t a0 = 0;
  while (a0 < n) {
    Batch b;
    b.anchor_mode = true;
    int32_t a1 = a0;
    int32_t tok = 0, max_len = 0, nsrc = 0;
    std::unordered_set<int32_t> in;
    while (a1 < n && (n_uses[a1] == 0 || tok + lens[a1] <= c->T)) {
      if (n_uses[a1] > 0) {
        const int32_t add = add_slab_srcs(c, slot_of[a1], in, false);
        if (tok > 0 && nsrc + add > max_batch_srcs(c)) break;
        nsrc += add_slab_srcs(c, slot_of[a1], in, true);
        tok += lens[a1];
        max_len = std::max(max_len, lens[a1]);
      }
      ++a1;
    }
    // packed tiles when every anchor is that short (see attn_tile_tokens)
    b.has_parent = false;
    for (int32_t a = a0; a < a1 && parents; ++a) b.has_parent |= n_uses[a] > 0 && parents[a] >= 0;
    b.pack = attn_direct_ok(b.has_parent && slab_fp8, slab_fp8, cf.k_scale, cf.v_scale)
                 ? attn_pack_waves(G, max_len) : 0;
    const int TQ = attn_tile_tokens(G, b.pack);
    std::unordered_map<int32_t, int32_t> parent_src;
    for (int32_t a = a0; a < a1; ++a) {
      if (n_uses[a] == 0) continue;
      const quail_ctx::Slot& sl = c->slots[slot_of[a]];
      const int32_t r0 = b.n_tok;
      const int32_t cross = sl.parent >= 0 ? slab_src(c, b, sl.parent, parent_src) : -1;
      const int32_t src = (int32_t)b.srcs.size();
      push_slab_src(c, b, sl);
      // own tokens: slab rows copied.., positions pos0 + copied..
      const int32_t own = sl.len - sl.copied;
      for (int32_t t = 0; t < own; ++t) {
        b.tok_src.push_back(starts[a] + t);
        b.pos.push_back(sl.pos0 + sl.copied + t);
        b.seg_lo.push_back(0);
        b.kv_row.push_back((int64_t)(sl.off / esz) + (int64_t)(sl.copied + t) * kHeadDim);
        b.kv_lapad.push_back(sl.lapad);
      }
      for (int32_t t0 = 0; t0 < own; t0 += TQ) {
        AttnTile tl{};
        tl.cross2 = -1;
        tl.q0 = r0 + t0;
        tl.nq = std::min(TQ, own - t0);
        tl.cross = cross;
        tl.self = src;
        tl.self_qbase = sl.copied + t0;
        tl.self_k0 = 0;
        b.tiles.push_back(tl);
      }
      b.n_tok += own;
    }
    if (quail_status st = run_batch(c, b, tokens, nullptr, nullptr, s)) return st;
    a0 = a1;
  }
  return QUAIL_OK;
}


}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* quail_version(void) { return "quail-mi355x 0.1 (gfx950)"; }

const char* quail_last_error(void) { return g_err.c_str(); }

quail_status quail_anchor_bytes(const quail_model_config* cfg, int32_t anchor_len, size_t* out) {
  if (quail_status st = check_cfg(cfg)) return st;
  if (!out || anchor_len < 1) return fail(QUAIL_E_INVAL, "anchor_len >= 1 and out required");
  *out = slab_bytes(*cfg, anchor_len);
  return QUAIL_OK;
}

quail_status quail_workspace_bytes(const quail_model_config* cfg, int32_t max_batch_tokens,
                                   size_t* out) {
  if (quail_status st = check_cfg(cfg)) return st;
  if (!out || max_batch_tokens < 1) return fail(QUAIL_E_INVAL, "max_batch_tokens >= 1 and out required");
  *out = ws_layout(*cfg, max_batch_tokens).total;
  return QUAIL_OK;
}

quail_status quail_prefix_groups(int32_t n, const int32_t* tokens, const int32_t* offsets, const int32_t* keys,
                                 int32_t min_len, int32_t* group_of, int32_t* node_first, int32_t* node_len,
                                 int32_t* n_nodes) {
  if (!n_nodes) return fail(QUAIL_E_INVAL, "n_nodes is NULL");
  *n_nodes = 0;
  if (n == 0) return QUAIL_OK;
  if (min_len < 1) return fail(QUAIL_E_INVAL, "min_len must be at least 1");
  if (!tokens || !group_of || !node_first || !node_len)
    return fail(QUAIL_E_INVAL, "tokens, group_of, node_first and node_len are required");
  if (quail_status st = check_offsets(n, offsets, 1, INT32_MAX, "sequence")) return st;
  std::vector<int32_t> starts(offsets, offsets + n), lens(n);
  for (int32_t i = 0; i < n; ++i) lens[i] = offsets[i + 1] - offsets[i];
  *n_nodes = prefix_groups(n, tokens, starts.data(), lens.data(), keys, min_len, group_of, node_first, node_len);
  return QUAIL_OK;
}

// ---- KV-aware join-order search with a speed-of-light cost model ----------
namespace {
// One candidate (partial) plan: metrics (computed tokens, attention pairs,
// cache bytes), the table order so far, and bit k = join k's right table is
// its anchor.
struct JoinPlan {
  double m[3];
  std::vector<int8_t> order;
  uint32_t right = 0;
};

// Adds p to a Pareto set unless a member is <= p in every metric; drops the
// members p now dominates.
void pareto_insert(std::vector<JoinPlan>& set, JoinPlan&& p) {
  for (const JoinPlan& q : set)
    if (q.m[0] <= p.m[0] && q.m[1] <= p.m[1] && q.m[2] <= p.m[2]) return;
  set.erase(std::remove_if(set.begin(), set.end(),
                           [&](const JoinPlan& q) {
                             return p.m[0] <= q.m[0] && p.m[1] <= q.m[1] && p.m[2] <= q.m[2];
                           }),
            set.end());
  set.push_back(std::move(p));
}
}  // namespace

quail_status quail_join_search(const quail_model_config* cfg, int32_t n_tables, const quail_table* tables,
                               int32_t n_joins, const quail_ai_join* joins, double peak_flops,
                               double peak_bytes_per_s, int32_t* order, int32_t* anchor_right, double* metrics,
                               double* frontier, int32_t cap, int32_t* n_frontier) {
  if (quail_status st = check_cfg(cfg)) return st;
  if (n_tables < 1 || n_tables > 12) return fail(QUAIL_E_INVAL, "n_tables must be in [1, 12]");
  if (n_joins != n_tables - 1) return fail(QUAIL_E_INVAL, "a tree of n tables has n - 1 joins");
  if (!tables || (n_joins > 0 && !joins) || !order || (n_joins > 0 && !anchor_right) || !metrics || !n_frontier)
    return fail(QUAIL_E_INVAL, "tables, joins, order, anchor_right, metrics and n_frontier are required");
  if (!(peak_flops > 0) || !(peak_bytes_per_s > 0)) return fail(QUAIL_E_INVAL, "peaks must be positive");
  if (cap < 0 || (cap > 0 && !frontier)) return fail(QUAIL_E_INVAL, "frontier is NULL");
  for (int32_t t = 0; t < n_tables; ++t)
    if (tables[t].rows < 1 || !(tables[t].field_tokens >= 0))
      return fail(QUAIL_E_INVAL, "table %d: rows must be >= 1 and tokens >= 0", t);
  std::vector<int32_t> root(n_tables);
  std::iota(root.begin(), root.end(), 0);
  auto find = [&](int32_t x) { while (root[x] != x) x = root[x] = root[root[x]]; return x; };
  for (int32_t k = 0; k < n_joins; ++k) {
    const quail_ai_join& j = joins[k];
    if (j.left < 0 || j.left >= n_tables || j.right < 0 || j.right >= n_tables || j.left == j.right)
      return fail(QUAIL_E_INVAL, "join %d: tables out of range or equal", k);
    if (!(j.selectivity > 0 && j.selectivity <= 1) || !(j.anchor_glue >= 0) || !(j.suffix_glue >= 0))
      return fail(QUAIL_E_INVAL, "join %d: selectivity must be in (0, 1] and glue >= 0", k);
    const int32_t a = find(j.left), b = find(j.right);
    if (a == b) return fail(QUAIL_E_INVAL, "join %d closes a cycle: the joins must form a tree", k);
    root[a] = b;
  }
  const quail_model_config& c = *cfg;
  const double L = c.n_layers, H = c.hidden, Hq = c.n_q_heads, Hkv = c.n_kv_heads, d = c.head_dim;
  const double gemm = 2.0 * L * (H * (Hq + 2 * Hkv) * d + Hq * d * H + 3.0 * H * c.intermediate);
  const double attn = 4.0 * Hq * d * L;
  const double kv = 2.0 * L * Hkv * d * (double)kv_elem_bytes(c);
  auto seconds = [&](const double* m) {
    return std::max((m[0] * gemm + m[1] * attn) / peak_flops, 2.0 * m[2] / peak_bytes_per_s);
  };
  const uint32_t full = (1u << n_tables) - 1;
  // result cardinality of each subset (independence): rows times the
  // selectivities of the joins inside it
  std::vector<double> card(full + 1, 1.0);
  for (uint32_t S = 1; S <= full; ++S) {
    for (int32_t t = 0; t < n_tables; ++t)
      if (S >> t & 1) card[S] *= tables[t].rows;
    for (int32_t k = 0; k < n_joins; ++k)
      if ((S >> joins[k].left & 1) && (S >> joins[k].right & 1)) card[S] *= joins[k].selectivity;
  }
  std::vector<std::vector<JoinPlan>> dp(full + 1);
  for (int32_t t = 0; t < n_tables; ++t) {
    JoinPlan p{};
    p.order.push_back((int8_t)t);
    dp[1u << t].push_back(std::move(p));
  }
  for (uint32_t S = 1; S < full; ++S) {
    if (dp[S].empty()) continue;
    for (int32_t t = 0; t < n_tables; ++t) {
      if (S >> t & 1) continue;
      int32_t k = -1, cnt = 0;
      for (int32_t q = 0; q < n_joins; ++q)
        if ((joins[q].left == t && (S >> joins[q].right & 1)) || (joins[q].right == t && (S >> joins[q].left & 1))) {
          k = q;
          ++cnt;
        }
      if (cnt != 1) continue;
      const quail_ai_join& j = joins[k];
      const int32_t u = j.left == t ? j.right : j.left;
      const double Du = std::min((double)tables[u].rows, card[S]);
      const double P = Du * tables[t].rows;
      for (int side = 0; side < (j.symmetric ? 2 : 1); ++side) {
        const int32_t x = side ? j.right : j.left, y = side ? j.left : j.right;
        const double A = x == u ? Du : (double)tables[t].rows;
        const double La = tables[x].field_tokens + j.anchor_glue, Ls = tables[y].field_tokens + j.suffix_glue;
        for (const JoinPlan& p : dp[S]) {
          JoinPlan q = p;
          q.m[0] += A * La + P * Ls;
          q.m[1] += P * (La * Ls + Ls * (Ls + 1) / 2.0) + A * La * (La + 1) / 2.0;
          q.m[2] += A * La * kv;
          q.order.push_back((int8_t)t);
          if (side) q.right |= 1u << k;
          pareto_insert(dp[S | (1u << t)], std::move(q));
        }
      }
    }
  }
  std::vector<JoinPlan>& fr = dp[full];
  std::sort(fr.begin(), fr.end(), [](const JoinPlan& a, const JoinPlan& b) {
    return std::lexicographical_compare(a.m, a.m + 3, b.m, b.m + 3);
  });
  size_t best = 0;
  for (size_t i = 1; i < fr.size(); ++i)
    if (seconds(fr[i].m) < seconds(fr[best].m)) best = i;
  for (int32_t t = 0; t < n_tables; ++t) order[t] = fr[best].order[t];
  for (int32_t k = 0; k < n_joins; ++k) anchor_right[k] = (int32_t)(fr[best].right >> k & 1);
  for (int i = 0; i < 3; ++i) metrics[i] = fr[best].m[i];
  metrics[3] = seconds(fr[best].m);
  for (int32_t i = 0; i < std::min<int32_t>(cap, (int32_t)fr.size()); ++i) {
    for (int q = 0; q < 3; ++q) frontier[4 * i + q] = fr[i].m[q];
    frontier[4 * i + 3] = seconds(fr[i].m);
  }
  *n_frontier = (int32_t)fr.size();
  return QUAIL_OK;
}

quail_status quail_prefix_tree(int32_t n, const int32_t* tokens, const int32_t* offsets, const int32_t* keys,
                               int32_t min_len, int32_t* group_of, int32_t* node_parent, int32_t* node_first,
                               int32_t* node_start, int32_t* node_end, int32_t* n_nodes) {
  if (!n_nodes) return fail(QUAIL_E_INVAL, "n_nodes is NULL");
  *n_nodes = 0;
  if (n == 0) return QUAIL_OK;
  if (min_len < 1) return fail(QUAIL_E_INVAL, "min_len must be at least 1");
  if (!tokens || !group_of || !node_parent || !node_first || !node_start || !node_end)
    return fail(QUAIL_E_INVAL, "tokens, group_of and the node arrays are required");
  if (quail_status st = check_offsets(n, offsets, 1, INT32_MAX, "sequence")) return st;
  std::vector<int32_t> starts(offsets, offsets + n), lens(n);
  for (int32_t i = 0; i < n; ++i) lens[i] = offsets[i + 1] - offsets[i];
  std::vector<TreeNode> nodes;
  prefix_tree(n, tokens, starts.data(), lens.data(), keys, min_len, group_of, nodes);
  for (size_t k = 0; k < nodes.size(); ++k) {
    node_parent[k] = nodes[k].parent;
    node_first[k] = nodes[k].first;
    node_start[k] = nodes[k].start;
    node_end[k] = nodes[k].end;
  }
  *n_nodes = (int32_t)nodes.size();
  return QUAIL_OK;
}

quail_status quail_plan_build(const quail_model_config* cfg, size_t pool_bytes, int32_t max_batch_tokens,
                              int32_t n_anchors, const int32_t* anchor_len, int32_t n_pairs,
                              const int32_t* pair_anchor, const int32_t* pair_len, int32_t* pair_order,
                              int32_t* step_bounds, int32_t* n_steps, size_t* peak_bytes) {
  if (quail_status st = check_cfg(cfg)) return st;
  if (n_anchors < 0 || n_pairs < 0 || max_batch_tokens < 1)
    return fail(QUAIL_E_INVAL, "negative count or max_batch_tokens < 1");
  if ((n_anchors > 0 && !anchor_len) || (n_pairs > 0 && (!pair_anchor || !pair_len || !pair_order)) ||
      !step_bounds || !n_steps)
    return fail(QUAIL_E_INVAL, "NULL array");
  std::vector<size_t> slab(n_anchors);
  for (int32_t a = 0; a < n_anchors; ++a) {
    if (anchor_len[a] < 1) return fail(QUAIL_E_INVAL, "anchor %d: length %d < 1", a, anchor_len[a]);
    slab[a] = slab_bytes(*cfg, anchor_len[a]);
  }
  Plan p;
  if (quail_status st = build_plan(slab, n_pairs, pair_anchor, pair_len, pool_bytes, max_batch_tokens, p))
    return st;
  std::copy(p.order.begin(), p.order.end(), pair_order);
  std::copy(p.bounds.begin(), p.bounds.end(), step_bounds);
  *n_steps = (int32_t)p.bounds.size() - 1;
  if (peak_bytes) *peak_bytes = p.peak;
  return QUAIL_OK;
}

quail_status quail_multiplan_build(const quail_model_config* cfg, size_t pool_bytes, int32_t max_batch_tokens,
                                   int32_t n_anchors, const int32_t* anchor_len, int32_t n_joins,
                                   const int32_t* join_offsets, const int32_t* pair_anchor,
                                   const int32_t* pair_len, int32_t* pair_order, int32_t* step_info,
                                   int32_t* n_steps, int32_t* event_off, int32_t* event_anchor,
                                   int64_t* totals) {
  if (quail_status st = check_cfg(cfg)) return st;
  if (n_anchors < 0 || n_joins < 0) return fail(QUAIL_E_INVAL, "negative count");
  if (max_batch_tokens <= 0) return fail(QUAIL_E_INVAL, "max_batch_tokens must be positive");
  if (!join_offsets || (n_anchors > 0 && !anchor_len))
    return fail(QUAIL_E_INVAL, "join_offsets and anchor_len are required");
  if (join_offsets[0] != 0) return fail(QUAIL_E_INVAL, "join_offsets[0] must be 0");
  for (int32_t j = 0; j < n_joins; ++j)
    if (join_offsets[j + 1] < join_offsets[j]) return fail(QUAIL_E_INVAL, "join_offsets must not decrease");
  const int32_t n_pairs = join_offsets[n_joins];
  if (n_pairs > 0 && (!pair_anchor || !pair_len)) return fail(QUAIL_E_INVAL, "pair arrays are required");
  if (!pair_order || !step_info || !n_steps || !event_off || !event_anchor || !totals)
    return fail(QUAIL_E_INVAL, "output arrays are required");
  std::vector<size_t> slab(n_anchors);
  std::vector<int32_t> alen(anchor_len, anchor_len + n_anchors);
  for (int32_t a = 0; a < n_anchors; ++a) {
    if (anchor_len[a] <= 0) return fail(QUAIL_E_INVAL, "anchor %d: length must be positive", a);
    slab[a] = slab_bytes(*cfg, anchor_len[a]);
  }
  MultiPlan mp;
  if (quail_status st = build_multiplan(slab, alen, n_joins, join_offsets, pair_anchor, pair_len, pool_bytes,
                                        max_batch_tokens, mp))
    return st;
  for (int32_t j = 0; j < n_joins; ++j)
    std::copy(mp.plans[j].order.begin(), mp.plans[j].order.end(), pair_order + join_offsets[j]);
  int32_t e = 0;
  event_off[0] = 0;
  for (size_t t = 0; t < mp.steps.size(); ++t) {
    const MultiStep& ms = mp.steps[t];
    step_info[3 * t] = ms.join;
    step_info[3 * t + 1] = ms.lo;
    step_info[3 * t + 2] = ms.hi;
    for (const std::vector<int32_t>* lst : {&ms.prefill, &ms.evict_before, &ms.evict_after}) {
      for (int32_t a : *lst) event_anchor[e++] = a;
      event_off[3 * t + 1 + (lst == &ms.prefill ? 0 : (lst == &ms.evict_before ? 1 : 2))] = e;
    }
  }
  *n_steps = (int32_t)mp.steps.size();
  totals[0] = mp.prefills;
  totals[1] = mp.evictions;
  totals[2] = mp.regret;
  totals[3] = (int64_t)mp.peak;
  return QUAIL_OK;
}

quail_status quail_ctx_create(const quail_model_config* cfg, const quail_weights* w, void* kv_pool,
                              size_t pool_bytes, void* workspace, size_t ws_bytes,
                              int32_t max_batch_tokens, quail_ctx** out) {
  if (quail_status st = check_cfg(cfg)) return st;
  if (!w || !out) return fail(QUAIL_E_INVAL, "weights and out are required");
  if (max_batch_tokens < 1) return fail(QUAIL_E_INVAL, "max_batch_tokens must be >= 1");
  if (!w->embed || !w->layers || !w->head8) return fail(QUAIL_E_INVAL, "weights incomplete");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const quail_layer_weights& x = w->layers[l];
    if (!x.attn_norm || !x.mlp_norm || !x.w_qkv || !x.w_o || !x.w_gate_up || !x.w_down || !x.s_qkv ||
        !x.s_o || !x.s_gate_up || !x.s_down)
      return fail(QUAIL_E_INVAL, "layer %d weights incomplete", l);
  }
  if (pool_bytes > 0 && (!kv_pool || reinterpret_cast<uintptr_t>(kv_pool) % kAlign))
    return fail(QUAIL_E_INVAL, "kv_pool must be non-NULL and 256-B aligned");
  WsLayout L = ws_layout(*cfg, max_batch_tokens);
  if (!workspace || ws_bytes < L.total)
    return fail(QUAIL_E_NOMEM, "workspace of %zu B < %zu B needed", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(QUAIL_E_INVAL, "workspace must be 256-B aligned");
  quail_ctx* c = new quail_ctx();
  c->cfg = *cfg;
  c->w = *w;
  c->layers.assign(w->layers, w->layers + cfg->n_layers);
  c->w.layers = c->layers.data();
  c->pool = static_cast<uint8_t*>(kv_pool);
  c->pool_bytes = pool_bytes / kAlign * kAlign;
  c->ws = static_cast<uint8_t*>(workspace);
  c->ws_bytes = ws_bytes;
  c->T = max_batch_tokens;
  c->L = L;
  // the pool's last guard-sized block is a guard region of its own
  if (c->pool_bytes >= 2 * kGuard) {
    c->tail_guard = c->pool_bytes - kGuard;
    c->free_list.push_back({0, c->pool_bytes - kGuard});
  } else if (c->pool_bytes) {
    c->free_list.push_back({0, c->pool_bytes});
  }
  *out = c;
  return QUAIL_OK;
}

quail_status quail_ctx_destroy(quail_ctx* ctx) {
  if (ctx)
    for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);   // teardown: nothing to report to
  delete ctx;
  return QUAIL_OK;
}

quail_status quail_ctx_check(quail_ctx* c, quail_stream stream, int64_t* guard_errors, int64_t* bad_tokens) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (guard_errors) *guard_errors = 0;
  if (bad_tokens) *bad_tokens = 0;
  if (!c->ready) return QUAIL_OK;                  // nothing has run on this context yet
  hipStream_t s = as_stream(stream);
  if (quail_status st = flush_guard_checks(c, s)) return st;
  std::vector<int64_t> live;
  for (const quail_ctx::Slot& sl : c->slots)
    if (sl.live) live.push_back((int64_t)(sl.off + sl.bytes - kGuard));
  if (c->tail_guard != SIZE_MAX) live.push_back((int64_t)c->tail_guard);
  if (quail_status st = guard_op(c, live, 0, s)) return st;
  uint32_t cnt[2] = {0, 0};
  HIP_TRY(hipMemcpyAsync(cnt, c->ws + c->L.status, sizeof cnt, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (guard_errors) *guard_errors = cnt[0];
  if (bad_tokens) *bad_tokens = cnt[1];
  return QUAIL_OK;
}

quail_status quail_ctx_profile(quail_ctx* c, int32_t enable) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  c->prof_on = enable != 0;
  c->prof.clear();
  c->ev_next = 0;
  return QUAIL_OK;
}

quail_status quail_ctx_profile_read(quail_ctx* c, int64_t* launches, double* ms, double* flop) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  for (int k = 0; k < PK_COUNT; ++k) {
    if (launches) launches[k] = 0;
    if (ms) ms[k] = 0.0;
    if (flop) flop[k] = 0.0;
  }
  if (!c->prof.empty()) HIP_TRY(hipEventSynchronize(c->prof.back().e1));
  for (const quail_ctx::ProfRec& r : c->prof) {
    float t = 0.0f;
    HIP_TRY(hipEventElapsedTime(&t, r.e0, r.e1));
    if (launches) launches[r.kind] += 1;
    if (ms) ms[r.kind] += t;
    if (flop) flop[r.kind] += r.flop;
  }
  c->prof.clear();
  c->ev_next = 0;
  return QUAIL_OK;
}

quail_status quail_pool_stats(const quail_ctx* c, size_t* resident, size_t* peak, int64_t* prefills,
                              int64_t* evictions, int64_t* regret_tokens) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (resident) *resident = c->resident;
  if (peak) *peak = c->peak;
  if (prefills) *prefills = c->prefills;
  if (evictions) *evictions = c->evictions;
  if (regret_tokens) *regret_tokens = c->regret;
  return QUAIL_OK;
}

quail_status quail_anchor_release(quail_ctx* c, quail_anchor h) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  quail_ctx::Slot* s = c->lookup(h);
  if (!s) return fail(QUAIL_E_STALE, "anchor handle %lld is stale", (long long)h);
  if (s->held > 0)
    return fail(QUAIL_E_INVAL, "anchor handle %lld still has %lld live prefix nodes", (long long)h,
                (long long)s->held);
  c->evict((int32_t)(h & 0xFFFFFFFF));
  return QUAIL_OK;
}

quail_status quail_anchor_kv(const quail_ctx* cc, quail_anchor h, int32_t layer, void** k, void** v,
                             int32_t* anchor_len, int32_t* padded_len) {
  quail_ctx* c = const_cast<quail_ctx*>(cc);
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  quail_ctx::Slot* s = c->lookup(h);
  if (!s) return fail(QUAIL_E_STALE, "anchor handle %lld is stale", (long long)h);
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(QUAIL_E_INVAL, "layer %d out of range", layer);
  const size_t esz = kv_elem_bytes(c->cfg);
  const size_t per = (size_t)c->cfg.n_kv_heads * s->lapad * c->cfg.head_dim * esz;
  uint8_t* base = c->pool + s->off + (size_t)layer * 2 * per;
  if (k) *k = base;
  if (v) *v = base + per;
  if (anchor_len) *anchor_len = s->len;
  if (padded_len) *padded_len = s->lapad;
  return QUAIL_OK;
}

quail_status quail_anchor_prefill(quail_ctx* c, int32_t n, const int32_t* tokens, const int32_t* offsets,
                                  const int32_t* n_uses, const int64_t* anchor_ids, quail_anchor* out,
                                  quail_stream stream) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (n == 0) return QUAIL_OK;
  const int32_t maxlen = std::min(c->cfg.max_anchor_len, c->T);
  if (quail_status st = check_offsets(n, offsets, 1, maxlen, "anchor")) return st;
  std::vector<int32_t> starts(offsets, offsets + n), lens(n);
  for (int32_t a = 0; a < n; ++a) lens[a] = offsets[a + 1] - offsets[a];
  return anchor_core(c, n, tokens, starts.data(), lens.data(), n_uses, anchor_ids, out,
                     as_stream(stream));
}

quail_status quail_prefix_prefill(quail_ctx* c, int32_t n, const quail_anchor* parent, const int32_t* tokens,
                                  const int32_t* offsets, const int32_t* n_uses, quail_anchor* out,
                                  quail_stream stream) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (n == 0) return QUAIL_OK;
  if (!parent || !n_uses || !out) return fail(QUAIL_E_INVAL, "parent, n_uses and out are required");
  if (quail_status st = check_offsets(n, offsets, 1, c->T, "prefix node")) return st;
  // a parent that is itself a node: the new node continues it (nested
  // level) -- it copies that node's rows, continues the same anchor, and
  // spends one of the parent node's uses once its prefill is enqueued
  std::vector<int32_t> starts(n), lens(n), par(n), from(n, -1);
  std::unordered_map<int32_t, int64_t> need;
  for (int32_t a = 0; a < n; ++a) {
    starts[a] = offsets[a];
    lens[a] = offsets[a + 1] - offsets[a];
    quail_ctx::Slot* ps = c->lookup(parent[a]);
    if (!ps) return fail(QUAIL_E_STALE, "node %d: parent handle %lld is stale", a, (long long)parent[a]);
    if (n_uses[a] < 0) return fail(QUAIL_E_INVAL, "node %d: negative use count", a);
    const int32_t ps_slot = (int32_t)(parent[a] & 0xFFFFFFFF);
    if (ps->parent >= 0) from[a] = ps_slot;
    par[a] = ps->parent >= 0 ? ps->parent : ps_slot;
    const quail_ctx::Slot& anc = c->slots[par[a]];
    if (n_uses[a] > 0) {
      if (++need[par[a]] > anc.uses - anc.held)
        return fail(QUAIL_E_STALE, "node %d: its anchor has no declared use to spare", a);
      if (from[a] >= 0 && ++need[from[a]] > ps->uses - ps->held)
        return fail(QUAIL_E_STALE, "node %d: its parent node has no declared use to spare", a);
    }
    const int64_t rows = (from[a] >= 0 ? ps->len : 0) + (int64_t)lens[a];
    if ((int64_t)anc.len + rows + 1 > max_pos(c->cfg))
      return fail(QUAIL_E_INVAL, "node %d: anchor + prefix leaves no position for a suffix token", a);
  }
  if (quail_status st = anchor_core(c, n, tokens, starts.data(), lens.data(), n_uses, nullptr, out,
                                    as_stream(stream), par.data(), from.data()))
    return st;
  for (int32_t a = 0; a < n; ++a) {
    if (n_uses[a] == 0 || from[a] < 0) continue;
    quail_ctx::Slot& ps = c->slots[from[a]];
    if (--ps.uses == 0) c->evict(from[a]);
  }
  return QUAIL_OK;
}

}  // extern "C"

namespace {

// Join prefill core: pair i = tokens[starts[i] .. starts[i] + lens[i]) after
// anchor ha[i]; its last hidden row goes to h_last row dst_row[i] (i if NULL);
// with h_all, row (starts[i] + t) of h_all receives position t. Pairs are
// grouped by anchor internally (stable).
quail_status join_core(quail_ctx* c, int32_t n, const quail_anchor* ha, const int32_t* tokens,
                       const int32_t* starts, const int32_t* lens, uint16_t* h_last,
                       const int32_t* dst_row, uint16_t* h_all, hipStream_t s) {
  const quail_model_config& cf = c->cfg;
  if (!ha || !tokens) return fail(QUAIL_E_INVAL, "pair_anchor and tokens are required");
  // validate handles and use counts
  std::unordered_map<int32_t, int64_t> need;
  std::vector<int32_t> slot(n, -1);
  for (int32_t i = 0; i < n; ++i) {
    if (ha[i] == QUAIL_NO_ANCHOR) continue;
    quail_ctx::Slot* sl = c->lookup(ha[i]);
    if (!sl) return fail(QUAIL_E_STALE, "pair %d: anchor handle %lld is stale", i, (long long)ha[i]);
    slot[i] = (int32_t)(ha[i] & 0xFFFFFFFF);
    if (++need[slot[i]] > sl->uses - sl->held)
      return fail(QUAIL_E_STALE, "pair %d: anchor used more often than its declared %lld uses", i,
                  (long long)(sl->uses - sl->held));
    if (sl->pos0 + sl->len + lens[i] > max_pos(cf))
      return fail(QUAIL_E_INVAL, "pair %d: anchor + suffix exceeds the position range", i);
  }
  if (quail_status st = ensure_ready(c, s)) return st;
  if (quail_status st = flush_guard_checks(c, s)) return st;
  std::vector<int32_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    const int64_t kx = slot[x] < 0 ? INT64_MAX : slot[x], ky = slot[y] < 0 ? INT64_MAX : slot[y];
    return kx < ky;
  });
  const int G = cf.n_q_heads / cf.n_kv_heads;
  const bool slab_fp8 = cf.kv_dtype == QUAIL_DTYPE_FP8_E4M3;
  int32_t p0 = c->dry ? n : 0;      // a dry run only spends uses
  while (p0 < n) {
    Batch b;
    b.anchor_mode = false;
    int32_t p1 = p0, tok = 0, nsrc = 1;   // source 0: the batch's suffix K/V
    std::unordered_set<int32_t> in;
    while (p1 < n && tok + lens[order[p1]] <= c->T) {
      const int32_t add = add_slab_srcs(c, slot[order[p1]], in, false);
      if (p1 > p0 && nsrc + add > max_batch_srcs(c)) break;
      nsrc += add_slab_srcs(c, slot[order[p1]], in, true);
      tok += lens[order[p1]];
      ++p1;
    }
    // packed attention tiles when every run of pairs sharing an anchor has
    // that few query tokens (the anchor K/V stream is then the work)
    int32_t max_group = 0;
    for (int32_t i = p0; i < p1;) {
      int32_t j = i, gtok = 0;
      while (j < p1 && slot[order[j]] == slot[order[i]]) gtok += lens[order[j++]];
      max_group = std::max(max_group, gtok);
      i = j;
    }
    b.pack = attn_direct_ok(slab_fp8, false, cf.k_scale, cf.v_scale) ? attn_pack_waves(G, max_group) : 0;
    const int TQ = attn_tile_tokens(G, b.pack);
    // source 0: this batch's suffix K/V (token-major, reused every layer)
    KVSrc self{};
    self.k = ws_ptr<uint16_t>(c, c->L.k);
    self.v = ws_ptr<uint16_t>(c, c->L.v);
    self.tok_stride = (int64_t)cf.n_kv_heads * kHeadDim;
    self.head_stride = kHeadDim;
    self.len = tok;
    self.fp8 = 0;
    b.srcs.push_back(self);
    b.src_layer_stride.push_back(0);
    std::unordered_map<int32_t, int32_t> src_of_slot;
    int32_t i = p0;
    while (i < p1) {
      // a run of pairs with the same anchor
      int32_t j = i;
      while (j < p1 && slot[order[j]] == slot[order[i]]) ++j;
      // cross: the anchor's slab; for a shared-prefix node, the node's
      // anchor and then the node's own slab (cross2)
      int32_t cross = -1, cross2 = -1, la = 0;
      if (slot[order[i]] >= 0) {
        const quail_ctx::Slot& sl = c->slots[slot[order[i]]];
        la = sl.pos0 + sl.len;
        if (sl.parent >= 0) {
          cross = slab_src(c, b, sl.parent, src_of_slot);
          cross2 = slab_src(c, b, slot[order[i]], src_of_slot);
        } else {
          cross = slab_src(c, b, slot[order[i]], src_of_slot);
        }
      }
      const int32_t g0 = b.n_tok;
      for (int32_t k = i; k < j; ++k) {
        const int32_t pi = order[k];
        const int32_t len = lens[pi];
        const int32_t r0 = b.n_tok;
        for (int32_t t = 0; t < len; ++t) {
          b.tok_src.push_back(starts[pi] + t);
          b.pos.push_back(la + t);
          b.seg_lo.push_back(r0);
          b.all_dst.push_back(starts[pi] + t);
        }
        b.last_row.push_back(r0 + len - 1);
        b.last_dst.push_back(dst_row ? dst_row[pi] : pi);
        b.n_tok += len;
      }
      for (int32_t t0 = g0; t0 < b.n_tok; t0 += TQ) {
        AttnTile tl{};
        tl.cross2 = cross2;
        b.two_level |= cross2 >= 0;
        tl.q0 = t0;
        tl.nq = std::min(TQ, b.n_tok - t0);
        tl.cross = cross;
        tl.self = 0;
        tl.self_qbase = t0;
        tl.self_k0 = b.seg_lo[t0];
        b.tiles.push_back(tl);
      }
      i = j;
    }
    if (quail_status st = run_batch(c, b, tokens, h_last, h_all, s)) return st;
    p0 = p1;
  }
  // spend uses; evict anchors at their last use (stream-ordered reuse)
  for (auto& kv : need) {
    quail_ctx::Slot& sl = c->slots[kv.first];
    sl.uses -= kv.second;
    if (sl.uses == 0) c->evict(kv.first);
  }
  return flush_guard_checks(c, s);
}

}  // namespace

extern "C" {

quail_status quail_join_prefill(quail_ctx* c, int32_t n, const quail_anchor* pair_anchor,
                                const int32_t* tokens, const int32_t* offsets, uint16_t* h_last,
                                uint16_t* h_all, quail_stream stream) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (n == 0) return QUAIL_OK;
  if (!h_last) return fail(QUAIL_E_INVAL, "h_last is required");
  const int32_t maxlen = std::min(c->cfg.max_suffix_len, c->T);
  if (quail_status st = check_offsets(n, offsets, 1, maxlen, "pair")) return st;
  std::vector<int32_t> starts(offsets, offsets + n), lens(n);
  for (int32_t i = 0; i < n; ++i) lens[i] = offsets[i + 1] - offsets[i];
  return join_core(c, n, pair_anchor, tokens, starts.data(), lens.data(), h_last, nullptr, h_all,
                   as_stream(stream));
}

quail_status quail_head8(quail_ctx* c, int32_t n, const uint16_t* h_last, uint8_t true_mask,
                         float* logits, uint8_t* token, uint8_t* decision, quail_stream stream) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (n < 0) return fail(QUAIL_E_INVAL, "negative n");
  if (n == 0) return QUAIL_OK;
  if (!h_last || !decision) return fail(QUAIL_E_INVAL, "h_last and decision are required");
  Head8Params p{};
  p.h = h_last; p.ldh = c->cfg.hidden; p.gamma = c->w.final_norm; p.w8 = c->w.head8;
  p.logits = logits; p.token = token; p.decision = decision;
  p.rows = n; p.H = c->cfg.hidden; p.eps = c->cfg.rms_eps; p.true_mask = true_mask;
  HIP_TRY(launch_head8(p, as_stream(stream)));
  return QUAIL_OK;
}

quail_status quail_head8_f32(int32_t n, int32_t hidden, const float* x, const float* w8,
                             uint8_t true_mask, float* logits, uint8_t* token, uint8_t* decision,
                             quail_stream stream) {
  if (n < 0 || hidden <= 0) return fail(QUAIL_E_INVAL, "n >= 0 and hidden > 0 required");
  if (n == 0) return QUAIL_OK;
  if (!x || !w8 || !decision) return fail(QUAIL_E_INVAL, "x, w8 and decision are required");
  HIP_TRY(launch_head8_f32(n, hidden, x, w8, true_mask, logits, token, decision, as_stream(stream)));
  return QUAIL_OK;
}

// One step of a join: its pairs through the decoder stack (join_core), then the
// head on each pair's last row, written to the caller's pair slots outmap[k]
// (the map goes to the metadata region; stream order protects earlier
// readers).
static quail_status run_step_with_head(quail_ctx* c, int32_t np, const quail_anchor* ha,
                                       const int32_t* s_tokens, const int32_t* starts, const int32_t* lens,
                                       const int32_t* outmap, uint8_t true_mask, float* logits, uint8_t* token,
                                       uint8_t* decision, hipStream_t s) {
  uint16_t* hl = ws_ptr<uint16_t>(c, c->L.hlast);
  std::vector<int32_t> dst(np);
  std::iota(dst.begin(), dst.end(), 0);
  if (quail_status r = join_core(c, np, ha, s_tokens, starts, lens, hl, dst.data(), nullptr, s)) return r;
  if (c->dry) return QUAIL_OK;
  Blob& bl = c->blob;
  bl.clear();
  bl.add(std::vector<int32_t>(outmap, outmap + np));
  uint8_t* md = c->ws + c->L.meta;
  HIP_TRY(stager().copy(md, bl.data(), bl.size(), s));
  Head8Params p{};
  p.h = hl; p.ldh = c->cfg.hidden; p.gamma = c->w.final_norm; p.w8 = c->w.head8;
  p.out_map = reinterpret_cast<const int32_t*>(md);
  p.logits = logits; p.token = token; p.decision = decision;
  p.rows = np; p.H = c->cfg.hidden; p.eps = c->cfg.rms_eps; p.true_mask = true_mask;
  TIMED(PK_OTHER, 0, launch_head8(p, s));
  return QUAIL_OK;
}

// Residency state of a context, saved around a placement dry run.
struct ResidencySnapshot {
  std::vector<quail_ctx::Slot> slots;
  std::vector<int32_t> free_slots;
  std::vector<std::pair<size_t, size_t>> free_list;
  size_t resident, peak;
  int64_t prefills, evictions, regret, run_serial;
  std::unordered_set<int64_t> seen_ids;
  std::vector<int64_t> pending_checks;
  explicit ResidencySnapshot(const quail_ctx* c)
      : slots(c->slots), free_slots(c->free_slots), free_list(c->free_list), resident(c->resident),
        peak(c->peak), prefills(c->prefills), evictions(c->evictions), regret(c->regret),
        run_serial(c->run_serial), seen_ids(c->seen_ids), pending_checks(c->pending_checks) {}
  void restore(quail_ctx* c) const {
    c->slots = slots; c->free_slots = free_slots; c->free_list = free_list; c->resident = resident;
    c->peak = peak; c->prefills = prefills; c->evictions = evictions; c->regret = regret;
    c->run_serial = run_serial; c->seen_ids = seen_ids; c->pending_checks = pending_checks;
  }
};

// Runs `schedule(budget)` as a dry run first: slabs are carved first-fit from
// a free list that can fragment, so a plan that fits the pool by its byte
// total may still find no block for a slab. The dry run replays the whole
// schedule's allocations and evictions with nothing enqueued; on E_NOMEM the
// plan is rebuilt against a smaller budget (a step then holds fewer anchors,
// so fewer slabs are live at once). The real run follows only once a dry run
// fits, so a call either enqueues its whole schedule or nothing.
static quail_status run_placed(quail_ctx* c, size_t budget,
                               const std::function<quail_status(size_t, bool)>& schedule) {
  for (int attempt = 0;; ++attempt) {
    ResidencySnapshot snap(c);
    c->dry = true;
    const std::string err0 = g_err;
    quail_status st = schedule(budget, true);
    c->dry = false;
    snap.restore(c);
    if (st == QUAIL_OK) return schedule(budget, false);
    if (st != QUAIL_E_NOMEM || attempt == 8 || budget < 2) return st;
    g_err = err0;
    budget = budget / 4 * 3;
  }
}

// quail_join_run, and with s_tokens_host / min_shared > 0 the same plan with
// the suffixes of each step that share a prefix of at least min_shared tokens
// (under one anchor) grouped into prefix nodes: each node is prefilled once
// after its anchor, and its members run only their remaining tokens against
// anchor + node + themselves (two-level cascade).
static quail_status join_run_core(quail_ctx* c, int32_t n_anchors, const int32_t* a_tokens,
                                  const int32_t* a_offsets, int32_t n_pairs, const int32_t* pair_anchor,
                                  const int32_t* s_tokens, const int32_t* s_offsets,
                                  const int32_t* s_tokens_host, int32_t min_shared, bool nested, uint8_t true_mask,
                                  float* logits, uint8_t* token, uint8_t* decision, quail_stream stream) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (n_pairs == 0) return QUAIL_OK;
  if (!decision) return fail(QUAIL_E_INVAL, "decision is required");
  if (min_shared > 0 && !s_tokens_host) return fail(QUAIL_E_INVAL, "s_tokens_host is required for sharing");
  const int32_t amax = std::min(c->cfg.max_anchor_len, c->T);
  if (quail_status st = check_offsets(n_anchors, a_offsets, 1, amax, "anchor")) return st;
  if (quail_status st = check_offsets(n_pairs, s_offsets, 1, std::min(c->cfg.max_suffix_len, c->T), "pair"))
    return st;
  if (!pair_anchor) return fail(QUAIL_E_INVAL, "pair_anchor is NULL");
  std::vector<size_t> slab(n_anchors);
  std::vector<int32_t> alen(n_anchors), plen(n_pairs);
  for (int32_t a = 0; a < n_anchors; ++a) {
    alen[a] = a_offsets[a + 1] - a_offsets[a];
    slab[a] = slab_bytes(c->cfg, alen[a]);
  }
  for (int32_t i = 0; i < n_pairs; ++i) plen[i] = s_offsets[i + 1] - s_offsets[i];
  // the plan is built against the largest free block of the pool now; with
  // sharing, less the slab of the longest possible prefix node, so that a
  // step's nodes fit beside its anchors
  size_t free_bytes = 0;
  for (auto& f : c->free_list) free_bytes = std::max(free_bytes, f.second);
  // With sharing, steps are sized by the tokens each pair will compute: its
  // own tokens after the prefix it shares, plus its share of that prefix
  // (grouping all pairs of each anchor); steps are regrouped below.
  std::vector<int32_t> step_len(plen);
  if (min_shared > 0) {
    std::vector<int32_t> gof(n_pairs), nf(n_pairs), nl(n_pairs), starts(n_pairs), keys(n_pairs);
    for (int32_t i = 0; i < n_pairs; ++i) {
      starts[i] = s_offsets[i];
      keys[i] = pair_anchor[i] >= 0 ? pair_anchor[i] : n_anchors;   // filter rows group among themselves
    }
    if (!nested) {
      const int32_t nn = prefix_groups(n_pairs, s_tokens_host, starts.data(), plen.data(), keys.data(), min_shared,
                                       gof.data(), nf.data(), nl.data());
      std::vector<int32_t> members(nn, 0);
      for (int32_t i = 0; i < n_pairs; ++i)
        if (gof[i] >= 0) members[gof[i]]++;
      for (int32_t i = 0; i < n_pairs; ++i)
        if (gof[i] >= 0)
          step_len[i] = plen[i] - nl[gof[i]] + (nl[gof[i]] + members[gof[i]] - 1) / members[gof[i]];
    } else {
      // own tokens after the deepest node, plus a share of every node above
      std::vector<TreeNode> tn;
      prefix_tree(n_pairs, s_tokens_host, starts.data(), plen.data(), keys.data(), min_shared, gof.data(), tn);
      std::vector<int32_t> members(tn.size(), 0);
      for (int32_t i = 0; i < n_pairs; ++i)
        for (int32_t v = gof[i]; v >= 0; v = tn[v].parent) members[v]++;
      for (int32_t i = 0; i < n_pairs; ++i) {
        if (gof[i] < 0) continue;
        int32_t len = plen[i] - tn[gof[i]].end;
        for (int32_t v = gof[i]; v >= 0; v = tn[v].parent)
          len += (tn[v].end - tn[v].start + members[v] - 1) / members[v];
        step_len[i] = len;
      }
    }
  }
  // Shared-prefix nodes of each plan step, parents first: one level
  // (prefix_groups) or the nested tree (prefix_tree). A node continues its
  // anchor; in a tree of filter rows the root is a plain anchor that its
  // descendants continue. A node below another node of an anchor (or below a
  // filter tree's second level) copies its parent's rows. Uses: a node's own
  // members, plus one per node that continues it (held until that node is
  // evicted) or copies it (spent when that node is prefilled).
  struct Node {
    int32_t anchor, parent, root, depth, first, start, end, rows, uses;
    std::vector<int32_t> members;   // pairs whose deepest node this is
  };
  Plan plan;
  std::vector<std::vector<Node>> step_nodes;
  std::vector<char> grouped(n_pairs, 0);
  auto group_steps = [&]() -> size_t {   // returns the largest root subtree's slab bytes
    const int32_t n_steps = (int32_t)plan.bounds.size() - 1;
    step_nodes.assign(n_steps, {});
    std::fill(grouped.begin(), grouped.end(), 0);
    size_t need = 0;
    for (int32_t st = 0; st < n_steps; ++st) {
      const int32_t b0 = plan.bounds[st], np = plan.bounds[st + 1] - b0;
      std::vector<int32_t> starts(np), lens(np), keys(np), gof(np);
      for (int32_t k = 0; k < np; ++k) {
        const int32_t pi = plan.order[b0 + k];
        starts[k] = s_offsets[pi];
        lens[k] = plen[pi];
        keys[k] = pair_anchor[pi] >= 0 ? pair_anchor[pi] : n_anchors;
      }
      std::vector<TreeNode> tn;
      if (nested) {
        prefix_tree(np, s_tokens_host, starts.data(), lens.data(), keys.data(), min_shared, gof.data(), tn);
      } else {
        std::vector<int32_t> nf(np), nl(np);
        const int32_t nn = prefix_groups(np, s_tokens_host, starts.data(), lens.data(), keys.data(), min_shared,
                                         gof.data(), nf.data(), nl.data());
        for (int32_t q = 0; q < nn; ++q) tn.push_back({-1, nf[q], 0, nl[q]});
      }
      std::vector<Node>& nodes = step_nodes[st];
      nodes.resize(tn.size());
      for (size_t q = 0; q < tn.size(); ++q) {
        Node& nd = nodes[q];
        nd.anchor = pair_anchor[plan.order[b0 + tn[q].first]];
        nd.parent = tn[q].parent;
        nd.root = nd.parent < 0 ? (int32_t)q : nodes[nd.parent].root;
        nd.depth = nd.parent < 0 ? 0 : nodes[nd.parent].depth + 1;
        nd.first = s_offsets[plan.order[b0 + tn[q].first]];
        nd.start = tn[q].start;
        nd.end = tn[q].end;
        nd.rows = (nd.anchor < 0 && nd.parent >= 0) ? nd.end - nodes[nd.root].end : nd.end;
        nd.uses = 0;
      }
      for (int32_t k = 0; k < np; ++k)
        if (gof[k] >= 0) {
          nodes[gof[k]].members.push_back(plan.order[b0 + k]);
          grouped[plan.order[b0 + k]] = 1;
        }
      std::vector<size_t> sub(nodes.size(), 0);
      for (size_t q = 0; q < nodes.size(); ++q) {
        Node& nd = nodes[q];
        nd.uses += (int32_t)nd.members.size();
        if (nd.parent >= 0) {
          if (nd.anchor < 0) nodes[nd.root].uses++;                      // continues the filter root
          if (nd.anchor >= 0 || nd.parent != nd.root) nodes[nd.parent].uses++;   // copies its parent
        }
        sub[nd.root] += slab_bytes(c->cfg, nd.rows);
      }
      for (size_t q = 0; q < nodes.size(); ++q)
        if (nodes[q].parent < 0) need = std::max(need, sub[q]);
    }
    return need;
  };
  // The plan is built against the largest free pool block less a reserve for
  // one step's largest node subtree, so that it fits beside the step's
  // anchors; the reserve starts at the slab of the longest possible node and
  // grows (re-planning) until it covers the subtrees the plan's steps form.
  auto schedule = [&](size_t budget, bool dry) -> quail_status {
  (void)dry;
  size_t reserve = min_shared > 0 ? slab_bytes(c->cfg, *std::max_element(plen.begin(), plen.end())) : 0;
  for (int32_t it = 0;; ++it) {
    if (min_shared > 0 && budget <= reserve)
      return fail(QUAIL_E_NOMEM, "KV pool (largest free block %zu B) leaves no room for prefix nodes (%zu B)",
                  budget, reserve);
    plan = Plan{};
    if (quail_status st = build_plan(slab, n_pairs, pair_anchor, step_len.data(), budget - reserve, c->T, plan))
      return st;
    if (min_shared <= 0) {
      step_nodes.assign(plan.bounds.size() - 1, {});
      break;
    }
    const size_t need = group_steps();
    if (need <= reserve) break;
    if (it == 3)
      return fail(QUAIL_E_NOMEM, "KV pool cannot hold a step's prefix nodes (%zu B) beside its anchors", need);
    reserve = need;
  }
  // an anchor's uses: its ungrouped pairs plus one per node under it (a
  // node of filter rows, anchor -1, is a plain anchor of its own)
  std::vector<int32_t> uses(n_anchors, 0);
  for (int32_t i = 0; i < n_pairs; ++i)
    if (pair_anchor[i] >= 0 && !grouped[i]) uses[pair_anchor[i]]++;
  for (auto& sn : step_nodes)
    for (auto& nd : sn)
      if (nd.anchor >= 0) uses[nd.anchor]++;
  // anchors in order of first use along the plan
  std::vector<int32_t> first_use;
  {
    std::vector<char> seen(n_anchors, 0);
    for (int32_t k = 0; k < n_pairs; ++k) {
      const int32_t a = pair_anchor[plan.order[k]];
      if (a >= 0 && !seen[a]) { seen[a] = 1; first_use.push_back(a); }
    }
  }
  std::vector<quail_anchor> handle(n_anchors, QUAIL_NO_ANCHOR);
  size_t next_fresh = 0;                      // next anchor (in first-use order) to prefill
  // anchor ids are this call's anchor indices, namespaced by the call, so that
  // regret counts re-prefills within one plan only
  const int64_t id_base = (++c->run_serial) << 32;
  hipStream_t s = as_stream(stream);
  for (size_t st = 0; st + 1 < plan.bounds.size(); ++st) {
    const int32_t b0 = plan.bounds[st], b1 = plan.bounds[st + 1];
    // Prefill the anchors this step needs; batch later steps' anchors with
    // them (up to one batch of tokens and half the free pool) so anchor
    // prefill runs as few, large launches.
    bool need = false;
    for (int32_t k = b0; k < b1 && !need; ++k) {
      const int32_t a = pair_anchor[plan.order[k]];
      need = a >= 0 && handle[a] == QUAIL_NO_ANCHOR;
    }
    if (need) {
      size_t fb = 0;
      for (auto& f : c->free_list) fb = std::max(fb, f.second);
      std::vector<int32_t> batch, st_, ln, nu;
      std::vector<int64_t> ids;
      int64_t tok = 0;
      size_t bytes = 0;
      // every anchor of this step is taken; later ones while they fit
      std::vector<char> in_step(n_anchors, 0);
      for (int32_t k = b0; k < b1; ++k)
        if (pair_anchor[plan.order[k]] >= 0) in_step[pair_anchor[plan.order[k]]] = 1;
      while (next_fresh < first_use.size()) {
        const int32_t a = first_use[next_fresh];
        const bool must = in_step[a];
        if (!must && (tok + alen[a] > c->T || bytes + slab[a] > fb / 2)) break;
        batch.push_back(a);
        st_.push_back(a_offsets[a]);
        ln.push_back(alen[a]);
        nu.push_back(uses[a]);
        ids.push_back(id_base | a);
        tok += alen[a];
        bytes += slab[a];
        ++next_fresh;
      }
      std::vector<quail_anchor> hnd(batch.size());
      if (quail_status r = anchor_core(c, (int32_t)batch.size(), a_tokens, st_.data(), ln.data(), nu.data(),
                                       ids.data(), hnd.data(), s))
        return r;
      for (size_t f = 0; f < batch.size(); ++f) handle[batch[f]] = hnd[f];
    }
    std::vector<quail_anchor> ha;
    std::vector<int32_t> starts, lens, outmap;
    for (int32_t k = b0; k < b1; ++k) {
      const int32_t pi = plan.order[k];
      if (grouped[pi]) continue;
      ha.push_back(pair_anchor[pi] >= 0 ? handle[pair_anchor[pi]] : QUAIL_NO_ANCHOR);
      starts.push_back(s_offsets[pi]);
      lens.push_back(plen[pi]);
      outmap.push_back(pi);
    }
    if (!ha.empty())
      if (quail_status r = run_step_with_head(c, (int32_t)ha.size(), ha.data(), s_tokens, starts.data(),
                                              lens.data(), outmap.data(), true_mask, logits, token, decision, s))
        return r;
    // shared-prefix nodes of this step, whole root subtrees per chunk (chunks
    // fit half the free pool, at least one subtree): prefill the chunk's
    // nodes depth by depth, then run their members' remaining tokens
    std::vector<Node>& nodes = step_nodes[st];
    const size_t nn = nodes.size();
    std::vector<quail_anchor> nh(nn, QUAIL_NO_ANCHOR);
    std::vector<size_t> sub(nn, 0);
    std::vector<int32_t> roots;
    int32_t maxd = 0;
    for (size_t q = 0; q < nn; ++q) {
      sub[nodes[q].root] += slab_bytes(c->cfg, nodes[q].rows);
      if (nodes[q].parent < 0) roots.push_back((int32_t)q);
      maxd = std::max(maxd, nodes[q].depth);
    }
    auto slot_of = [](quail_anchor h) { return (int32_t)(h & 0xFFFFFFFF); };
    for (size_t r0 = 0; r0 < roots.size();) {
      size_t fb = 0;
      for (auto& f : c->free_list) fb = std::max(fb, f.second);
      size_t r1 = r0, bytes = 0;
      while (r1 < roots.size()) {
        if (r1 > r0 && bytes + sub[roots[r1]] > fb / 2) break;
        bytes += sub[roots[r1]];
        ++r1;
      }
      std::vector<char> in_chunk(nn, 0);
      for (size_t r = r0; r < r1; ++r) in_chunk[roots[r]] = 1;
      for (size_t q = 0; q < nn; ++q) in_chunk[q] = in_chunk[nodes[q].root];
      for (int32_t d = 0; d <= maxd; ++d) {
        std::vector<int32_t> idx, nst, nln, nnu, npar, nfrom;
        for (size_t q = 0; q < nn; ++q) {
          if (!in_chunk[q] || nodes[q].depth != d) continue;
          const Node& nd = nodes[q];
          int32_t par = -1, from = -1;
          if (nd.anchor >= 0) {
            par = slot_of(handle[nd.anchor]);
            if (nd.parent >= 0) from = slot_of(nh[nd.parent]);
          } else if (nd.parent >= 0) {
            par = slot_of(nh[nd.root]);
            if (nd.parent != nd.root) from = slot_of(nh[nd.parent]);
          }
          idx.push_back((int32_t)q);
          nst.push_back(nd.first + nd.start);
          nln.push_back(nd.end - nd.start);
          nnu.push_back(nd.uses);
          npar.push_back(par);
          nfrom.push_back(from);
        }
        if (idx.empty()) continue;
        std::vector<quail_anchor> out(idx.size());
        if (quail_status r = anchor_core(c, (int32_t)idx.size(), s_tokens, nst.data(), nln.data(), nnu.data(),
                                         nullptr, out.data(), s, npar.data(), nfrom.data()))
          return r;
        for (size_t k = 0; k < idx.size(); ++k) nh[idx[k]] = out[k];
        for (size_t k = 0; k < idx.size(); ++k)      // a copied parent's use is spent
          if (nfrom[k] >= 0 && --c->slots[nfrom[k]].uses == 0) c->evict(nfrom[k]);
      }
      ha.clear(); starts.clear(); lens.clear(); outmap.clear();
      for (size_t q = 0; q < nn; ++q) {
        if (!in_chunk[q]) continue;
        for (int32_t pi : nodes[q].members) {
          ha.push_back(nh[q]);
          starts.push_back(s_offsets[pi] + nodes[q].end);
          lens.push_back(plen[pi] - nodes[q].end);
          outmap.push_back(pi);
        }
      }
      if (!ha.empty())
        if (quail_status r = run_step_with_head(c, (int32_t)ha.size(), ha.data(), s_tokens, starts.data(),
                                                lens.data(), outmap.data(), true_mask, logits, token, decision, s))
          return r;
      r0 = r1;
    }
  }
  return QUAIL_OK;
  };
  return run_placed(c, free_bytes, schedule);
}

quail_status quail_join_run(quail_ctx* c, int32_t n_anchors, const int32_t* a_tokens,
                            const int32_t* a_offsets, int32_t n_pairs, const int32_t* pair_anchor,
                            const int32_t* s_tokens, const int32_t* s_offsets, uint8_t true_mask,
                            float* logits, uint8_t* token, uint8_t* decision, quail_stream stream) {
  return join_run_core(c, n_anchors, a_tokens, a_offsets, n_pairs, pair_anchor, s_tokens, s_offsets, nullptr, 0,
                       false, true_mask, logits, token, decision, stream);
}

quail_status quail_join_run_shared(quail_ctx* c, int32_t n_anchors, const int32_t* a_tokens,
                                   const int32_t* a_offsets, int32_t n_pairs, const int32_t* pair_anchor,
                                   const int32_t* s_tokens, const int32_t* s_offsets,
                                   const int32_t* s_tokens_host, int32_t min_shared, int32_t nested,
                                   uint8_t true_mask, float* logits, uint8_t* token, uint8_t* decision,
                                   quail_stream stream) {
  if (min_shared < 1) return fail(QUAIL_E_INVAL, "min_shared must be at least 1");
  return join_run_core(c, n_anchors, a_tokens, a_offsets, n_pairs, pair_anchor, s_tokens, s_offsets,
                       s_tokens_host, min_shared, nested != 0, true_mask, logits, token, decision, stream);
}

quail_status quail_multijoin_run(quail_ctx* c, int32_t n_anchors, const int32_t* a_tokens,
                                 const int32_t* a_offsets, int32_t n_joins, const int32_t* join_offsets,
                                 const int32_t* pair_anchor, const int32_t* s_tokens, const int32_t* s_offsets,
                                 uint8_t true_mask, float* logits, uint8_t* token, uint8_t* decision,
                                 quail_stream stream) {
  if (!c) return fail(QUAIL_E_INVAL, "ctx is NULL");
  if (n_joins < 0 || !join_offsets) return fail(QUAIL_E_INVAL, "join_offsets is required");
  if (join_offsets[0] != 0) return fail(QUAIL_E_INVAL, "join_offsets[0] must be 0");
  for (int32_t j = 0; j < n_joins; ++j)
    if (join_offsets[j + 1] < join_offsets[j]) return fail(QUAIL_E_INVAL, "join_offsets must not decrease");
  const int32_t n_pairs = join_offsets[n_joins];
  if (n_pairs == 0) return QUAIL_OK;
  if (!decision) return fail(QUAIL_E_INVAL, "decision is required");
  const int32_t amax = std::min(c->cfg.max_anchor_len, c->T);
  if (quail_status st = check_offsets(n_anchors, a_offsets, 1, amax, "anchor")) return st;
  if (quail_status st = check_offsets(n_pairs, s_offsets, 1, std::min(c->cfg.max_suffix_len, c->T), "pair"))
    return st;
  if (!pair_anchor) return fail(QUAIL_E_INVAL, "pair_anchor is NULL");
  std::vector<size_t> slab(n_anchors);
  std::vector<int32_t> alen(n_anchors), plen(n_pairs);
  for (int32_t a = 0; a < n_anchors; ++a) {
    alen[a] = a_offsets[a + 1] - a_offsets[a];
    slab[a] = slab_bytes(c->cfg, alen[a]);
  }
  for (int32_t i = 0; i < n_pairs; ++i) plen[i] = s_offsets[i + 1] - s_offsets[i];
  // the plan is built against the largest free block of the pool now
  size_t free_bytes = 0;
  for (auto& f : c->free_list) free_bytes = std::max(free_bytes, f.second);
  auto schedule = [&](size_t budget, bool dry) -> quail_status {
  (void)dry;
  MultiPlan mp;
  if (quail_status st = build_multiplan(slab, alen, n_joins, join_offsets, pair_anchor, plen.data(), budget,
                                        c->T, mp))
    return st;
  // Each prefill declares the pairs the anchor serves until its next prefill
  // (or the end), so the residency manager frees it right after the last of
  // them: an anchor the plan evicts early is freed at its last use before
  // the gap, which changes no prefill or regret and only lowers the peak.
  const int32_t T = (int32_t)mp.steps.size();
  std::vector<std::vector<int32_t>> pairs_in(T);   // per step: global pair indices in plan order
  for (int32_t t = 0; t < T; ++t) {
    const MultiStep& ms = mp.steps[t];
    const int32_t p0 = join_offsets[ms.join];
    for (int32_t k = ms.lo; k < ms.hi; ++k) pairs_in[t].push_back(p0 + mp.plans[ms.join].order[k]);
  }
  std::vector<std::vector<int32_t>> prefill_at(n_anchors);
  for (int32_t t = 0; t < T; ++t)
    for (int32_t a : mp.steps[t].prefill) prefill_at[a].push_back(t);
  auto uses_until = [&](int32_t a, int32_t t0) -> int32_t {
    auto it = std::upper_bound(prefill_at[a].begin(), prefill_at[a].end(), t0);
    const int32_t t1 = it == prefill_at[a].end() ? T : *it;
    int32_t u = 0;
    for (int32_t t = t0; t < t1; ++t)
      for (int32_t pi : pairs_in[t]) u += pair_anchor[pi] == a;
    return u;
  };
  std::vector<quail_anchor> handle(n_anchors, QUAIL_NO_ANCHOR);
  const int64_t id_base = (++c->run_serial) << 32;
  hipStream_t s = as_stream(stream);
  for (int32_t t = 0; t < T; ++t) {
    const MultiStep& ms = mp.steps[t];
    if (!ms.prefill.empty()) {
      const int32_t nb = (int32_t)ms.prefill.size();
      std::vector<int32_t> st_(nb), ln(nb), nu(nb);
      std::vector<int64_t> ids(nb);
      for (int32_t f = 0; f < nb; ++f) {
        const int32_t a = ms.prefill[f];
        st_[f] = a_offsets[a];
        ln[f] = alen[a];
        nu[f] = uses_until(a, t);
        ids[f] = id_base | a;
      }
      std::vector<quail_anchor> hnd(nb);
      if (quail_status r = anchor_core(c, nb, a_tokens, st_.data(), ln.data(), nu.data(), ids.data(), hnd.data(), s))
        return r;
      for (int32_t f = 0; f < nb; ++f) handle[ms.prefill[f]] = hnd[f];
    }
    const int32_t np = (int32_t)pairs_in[t].size();
    std::vector<quail_anchor> ha(np);
    std::vector<int32_t> starts(np), lens(np);
    for (int32_t k = 0; k < np; ++k) {
      const int32_t pi = pairs_in[t][k];
      ha[k] = pair_anchor[pi] >= 0 ? handle[pair_anchor[pi]] : QUAIL_NO_ANCHOR;
      starts[k] = s_offsets[pi];
      lens[k] = plen[pi];
    }
    if (quail_status r = run_step_with_head(c, np, ha.data(), s_tokens, starts.data(), lens.data(),
                                            pairs_in[t].data(), true_mask, logits, token, decision, s))
      return r;
  }
  return QUAIL_OK;
  };
  return run_placed(c, free_bytes, schedule);
}

// ---- cascade attention on given Q/K/V ---------------------------------------
quail_status quail_cascade_workspace_bytes(int32_t n_anchors, const int32_t* a_off, int32_t n_suffix,
                                           const int32_t* s_off, size_t* out) {
  if (n_anchors < 0 || n_suffix < 0 || !out) return fail(QUAIL_E_INVAL, "bad arguments");
  if (n_suffix > 0 && !s_off) return fail(QUAIL_E_INVAL, "s_off is NULL");
  if (n_anchors > 0 && !a_off) return fail(QUAIL_E_INVAL, "a_off is NULL");
  const int64_t T = n_suffix > 0 ? s_off[n_suffix] : 0;
  // seg_lo + tok_anchor (int32 per token), a_off copy, tiles (<= T + n_suffix),
  // srcs (n_anchors + 1)
  *out = align_up((size_t)T * 4) * 2 + align_up((size_t)(n_anchors + 1) * 4) +
         align_up((size_t)(T + n_suffix + 1) * sizeof(AttnTile)) +
         align_up((size_t)(n_anchors + 1) * sizeof(KVSrc)) + 8 * kAlign;
  return QUAIL_OK;
}

}  // extern "C"

// Scratch memory of the allocation-free cascade call
// (quail_cascade_attn_noalloc): its per-call metadata, at most 16 MiB. One
// array per device: each GPU the library runs on holds its own copy until the
// process ends. Host code never passes the array's name to a kernel or a
// copy -- on the host the name is only a stand-in -- but the device address
// hipGetSymbolAddress returns, taken once per device (scratch_ptr below).
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Where the cascade call's per-call metadata (token segments, tiles, KV
// sources) goes: a caller workspace, filled through the pinned staging ring,
// or the library's static scratch array, filled by one plain copy from host
// memory (nothing allocated).
struct MetaDest {
  uint8_t* dev;
  size_t bytes;
  bool staged;
};

quail_status meta_copy(const MetaDest& m, const Blob& bl, hipStream_t st) {
  if (bl.size() > m.bytes)
    return fail(QUAIL_E_NOMEM, "cascade metadata of %zu B exceeds the %zu B available", bl.size(), m.bytes);
  if (m.staged) HIP_TRY(stager().copy(m.dev, bl.data(), bl.size(), st));
  else HIP_TRY(hipMemcpyAsync(m.dev, bl.data(), bl.size(), hipMemcpyHostToDevice, st));
  return QUAIL_OK;
}

quail_status cascade_check(int32_t dtype, int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t n_anchors,
                           const void* ak, const void* av, const int32_t* a_off, int32_t n_suffix,
                           const int32_t* s_anchor, const void* q, const void* k, const void* v,
                           const int32_t* s_off, void* out) {
  if (dtype != QUAIL_DTYPE_F32 && dtype != QUAIL_DTYPE_BF16 && dtype != QUAIL_DTYPE_FP8_E4M3)
    return fail(QUAIL_E_UNSUPPORTED, "dtype must be F32, BF16 or FP8_E4M3");
  if (hq <= 0 || hkv <= 0 || hq % hkv) return fail(QUAIL_E_INVAL, "hq must be a positive multiple of hkv");
  if (hkv > kMaxKVHeads) return fail(QUAIL_E_UNSUPPORTED, "hkv %d (at most %d)", hkv, kMaxKVHeads);
  const int G = hq / hkv;
  if (dtype != QUAIL_DTYPE_F32 && (d != kHeadDim || !valid_group(G)))
    return fail(QUAIL_E_UNSUPPORTED, "bf16 / E4M3 path: head_dim 128 and GQA group 1, 2, 4 or 8");
  if (dtype == QUAIL_DTYPE_F32 && d != 64 && d != 128)
    return fail(QUAIL_E_UNSUPPORTED, "fp32 path: head_dim 64 or 128");
  if (!(sm_scale > 0.0f)) return fail(QUAIL_E_INVAL, "sm_scale must be positive");
  if (n_suffix < 0 || n_anchors < 0) return fail(QUAIL_E_INVAL, "negative count");
  if (n_suffix == 0) return QUAIL_OK;
  if (quail_status st = check_offsets(n_suffix, s_off, 1, INT32_MAX, "suffix")) return st;
  if (n_anchors > 0)
    if (quail_status st = check_offsets(n_anchors, a_off, 1, INT32_MAX, "anchor")) return st;
  if (!s_anchor || !q || !k || !v || !out) return fail(QUAIL_E_INVAL, "NULL argument");
  for (int32_t s = 0; s < n_suffix; ++s)
    if (s_anchor[s] < -1 || s_anchor[s] >= n_anchors)
      return fail(QUAIL_E_INVAL, "suffix %d: anchor %d out of range", s, s_anchor[s]);
  if (n_anchors > 0 && (!ak || !av)) return fail(QUAIL_E_INVAL, "anchor K/V are NULL");
  return QUAIL_OK;
}

// The cascade call after validation (n_suffix > 0).
quail_status cascade_core(int32_t dtype, int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t n_anchors,
                          const void* ak, const void* av, const int32_t* a_off, int32_t n_suffix,
                          const int32_t* s_anchor, const void* q, const void* k, const void* v,
                          const int32_t* s_off, void* out, float* lse, const MetaDest& meta, hipStream_t st) {
  const int G = hq / hkv;
  const int32_t T = s_off[n_suffix];
  std::vector<int32_t> seg(T), tok_anchor(T);
  for (int32_t s = 0; s < n_suffix; ++s)
    for (int32_t t = s_off[s]; t < s_off[s + 1]; ++t) { seg[t] = s_off[s]; tok_anchor[t] = s_anchor[s]; }
  Blob bl;
  const size_t o_seg = bl.add(seg);
  if (dtype == QUAIL_DTYPE_F32) {
    const size_t o_ta = bl.add(tok_anchor);
    std::vector<int32_t> ao(a_off, a_off + (n_anchors > 0 ? n_anchors + 1 : 0));
    if (ao.empty()) ao.push_back(0);
    const size_t o_ao = bl.add(ao);
    uint8_t* md = meta.dev;
    if (quail_status r = meta_copy(meta, bl, st)) return r;
    AttnF32Params p{};
    p.ak = static_cast<const float*>(ak); p.av = static_cast<const float*>(av);
    p.a_off = reinterpret_cast<const int32_t*>(md + o_ao);
    p.q = static_cast<const float*>(q); p.k = static_cast<const float*>(k); p.v = static_cast<const float*>(v);
    p.tok_anchor = reinterpret_cast<const int32_t*>(md + o_ta);
    p.tok_seg = reinterpret_cast<const int32_t*>(md + o_seg);
    p.out = static_cast<float*>(out); p.lse = lse;
    p.n_tok = T; p.hq = hq; p.hkv = hkv; p.d = d; p.scale = sm_scale;
    HIP_TRY(launch_attn_f32(p, st));
    return QUAIL_OK;
  }
  std::vector<KVSrc> srcs;
  KVSrc self{};
  self.k = k; self.v = v; self.tok_stride = (int64_t)hkv * d; self.head_stride = d; self.len = T; self.fp8 = 0;
  srcs.push_back(self);
  // anchor K/V: bf16, or E4M3 codes (1 byte per element) for dtype FP8_E4M3
  const bool a_fp8 = dtype == QUAIL_DTYPE_FP8_E4M3;
  const int64_t a_esz = a_fp8 ? 1 : 2;
  for (int32_t a = 0; a < n_anchors; ++a) {
    KVSrc x{};
    x.k = static_cast<const uint8_t*>(ak) + (int64_t)a_off[a] * hkv * d * a_esz;
    x.v = static_cast<const uint8_t*>(av) + (int64_t)a_off[a] * hkv * d * a_esz;
    x.tok_stride = (int64_t)hkv * d; x.head_stride = d; x.len = a_off[a + 1] - a_off[a];
    x.fp8 = a_fp8 ? 1 : 0;
    srcs.push_back(x);
  }
  // packed tiles when every run of suffixes sharing an anchor is that short
  int32_t max_group = 0;
  for (int32_t s0 = 0; s0 < n_suffix;) {
    int32_t s1 = s0 + 1;
    while (s1 < n_suffix && s_anchor[s1] == s_anchor[s0]) ++s1;
    max_group = std::max(max_group, s_off[s1] - s_off[s0]);
    s0 = s1;
  }
  const int pack = attn_pack_waves(G, max_group);
  const int TQ = attn_tile_tokens(G, pack);
  std::vector<AttnTile> tiles;
  int32_t s0 = 0;
  while (s0 < n_suffix) {
    int32_t s1 = s0 + 1;
    while (s1 < n_suffix && s_anchor[s1] == s_anchor[s0]) ++s1;
    const int32_t t_end = s_off[s1];
    for (int32_t t0 = s_off[s0]; t0 < t_end; t0 += TQ) {
      AttnTile tl{};
      tl.cross2 = -1;
      tl.q0 = t0; tl.nq = std::min(TQ, t_end - t0);
      tl.cross = s_anchor[s0] >= 0 ? 1 + s_anchor[s0] : -1;
      tl.self = 0; tl.self_qbase = t0; tl.self_k0 = seg[t0];
      tiles.push_back(tl);
    }
    s0 = s1;
  }
  const size_t o_til = bl.add(tiles);
  const size_t o_src = bl.add(srcs);
  uint8_t* md = meta.dev;
  if (quail_status r = meta_copy(meta, bl, st)) return r;
  AttnParams p{};
  p.tiles = reinterpret_cast<const AttnTile*>(md + o_til);
  p.n_tiles = (int32_t)tiles.size();
  p.srcs = reinterpret_cast<const KVSrc*>(md + o_src);
  p.seg_lo = reinterpret_cast<const int32_t*>(md + o_seg);
  p.q = static_cast<const uint16_t*>(q); p.q_stride = (int64_t)hq * d;
  p.out = static_cast<uint16_t*>(out); p.o_stride = (int64_t)hq * d;
  p.lse = lse; p.hq = hq; p.hkv = hkv;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.k_scale = 1.0f; p.v_scale = 1.0f;
  HIP_TRY(launch_attn_bf16(p, G, a_fp8, false, pack, st));
  return QUAIL_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

quail_status scratch_ptr(uint8_t** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(QUAIL_E_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(QUAIL_E_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
  return QUAIL_OK;
}

}  // namespace

extern "C" {

quail_status quail_cascade_attn(int32_t dtype, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                int32_t n_anchors, const void* ak, const void* av, const int32_t* a_off,
                                int32_t n_suffix, const int32_t* s_anchor, const void* q, const void* k,
                                const void* v, const int32_t* s_off, void* out, float* lse,
                                void* workspace, size_t ws_bytes, quail_stream stream) {
  if (quail_status r = cascade_check(dtype, hq, hkv, d, sm_scale, n_anchors, ak, av, a_off, n_suffix, s_anchor,
                                     q, k, v, s_off, out))
    return r;
  if (n_suffix == 0) return QUAIL_OK;
  size_t need = 0;
  quail_cascade_workspace_bytes(n_anchors, a_off, n_suffix, s_off, &need);
  if (!workspace || ws_bytes < need) return fail(QUAIL_E_NOMEM, "workspace %zu B < %zu B", ws_bytes, need);
  const MetaDest meta{static_cast<uint8_t*>(workspace), ws_bytes, true};
  return cascade_core(dtype, hq, hkv, d, sm_scale, n_anchors, ak, av, a_off, n_suffix, s_anchor, q, k, v, s_off,
                      out, lse, meta, as_stream(stream));
}

quail_status quail_cascade_attn_noalloc(int32_t dtype, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                        int32_t n_anchors, const void* ak, const void* av, const int32_t* a_off,
                                        int32_t n_suffix, const int32_t* s_anchor, const void* q, const void* k,
                                        const void* v, const int32_t* s_off, void* out, float* lse,
                                        quail_stream stream) {
  if (quail_status r = cascade_check(dtype, hq, hkv, d, sm_scale, n_anchors, ak, av, a_off, n_suffix, s_anchor,
                                     q, k, v, s_off, out))
    return r;
  if (n_suffix == 0) return QUAIL_OK;
  size_t need = 0;
  quail_cascade_workspace_bytes(n_anchors, a_off, n_suffix, s_off, &need);
  if (need > kScratchBytes)
    return fail(QUAIL_E_NOMEM, "call needs %zu B of metadata; the allocation-free entry point holds at most %zu B",
                need, kScratchBytes);
  uint8_t* ptr = nullptr;
  if (quail_status r = scratch_ptr(&ptr)) return r;
  const MetaDest meta{ptr, kScratchBytes, false};
  return cascade_core(dtype, hq, hkv, d, sm_scale, n_anchors, ak, av, a_off, n_suffix, s_anchor, q, k, v, s_off,
                      out, lse, meta, as_stream(stream));
}

quail_status quail_gemm_w8a16(int32_t M, int32_t N, int32_t K, const uint16_t* x, const uint8_t* w,
                              const uint16_t* scale, uint16_t* y, quail_stream stream) {
  if (M < 0 || N <= 0 || K <= 0) return fail(QUAIL_E_INVAL, "M >= 0, N > 0, K > 0 required");
  if (K % 64 || N % 128) return fail(QUAIL_E_UNSUPPORTED, "K must be a multiple of 64 and N of 128");
  if (M == 0) return QUAIL_OK;
  if (!x || !w || !scale || !y) return fail(QUAIL_E_INVAL, "NULL argument");
  GemmParams p{};
  p.A = x; p.lda = K; p.B = w; p.scale = scale; p.M = M; p.N = N; p.K = K; p.Y = y; p.ldy = N;
  HIP_TRY(launch_gemm(p, EPI_STORE, as_stream(stream)));
  return QUAIL_OK;
}

static bool aligned_to(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

quail_status quail_act_quant_e4m3(int32_t M, int32_t K, const uint16_t* x, uint8_t* codes, float* scale,
                                  quail_stream stream) {
  if (M < 0 || K <= 0) return fail(QUAIL_E_INVAL, "M >= 0 and K > 0 required");
  if (K % 8) return fail(QUAIL_E_UNSUPPORTED, "K must be a multiple of 8");
  if (M == 0) return QUAIL_OK;
  if (!x || !codes || !scale) return fail(QUAIL_E_INVAL, "NULL argument");
  if (!aligned_to(x, 16) || !aligned_to(codes, 8) || !aligned_to(scale, 4))
    return fail(QUAIL_E_UNSUPPORTED, "x must be 16-byte aligned, codes 8-byte, scale 4-byte");
  HIP_TRY(launch_act_quant_e4m3(M, K, x, codes, scale, as_stream(stream)));
  return QUAIL_OK;
}

quail_status quail_gemm_w8a8(int32_t M, int32_t N, int32_t K, const uint8_t* xc, const float* x_scale,
                             const uint8_t* wc, const uint16_t* w_scale, uint16_t* y, quail_stream stream) {
  if (M < 0 || N <= 0 || K <= 0) return fail(QUAIL_E_INVAL, "M >= 0, N > 0, K > 0 required");
  if (K % 128 || N % 256) return fail(QUAIL_E_UNSUPPORTED, "K must be a multiple of 128 and N of 256");
  if (M == 0) return QUAIL_OK;
  if (!xc || !x_scale || !wc || !w_scale || !y) return fail(QUAIL_E_INVAL, "NULL argument");
  if (!aligned_to(xc, 16) || !aligned_to(wc, 16) || !aligned_to(y, 16) || !aligned_to(w_scale, 8) ||
      !aligned_to(x_scale, 4))
    return fail(QUAIL_E_UNSUPPORTED, "xc, wc and y must be 16-byte aligned, w_scale 8-byte");
  GemmParams p{};
  p.A8 = xc; p.lda = K; p.a_scale = x_scale; p.B = wc; p.scale = w_scale;
  p.M = M; p.N = N; p.K = K; p.Y = y; p.ldy = N;
  HIP_TRY(launch_gemm(p, EPI_STORE, as_stream(stream)));
  return QUAIL_OK;
}

quail_status quail_fp8_e4m3_encode(int64_t n, const float* x, float scale, uint8_t* codes,
                                   quail_stream stream) {
  if (n < 0 || !(scale > 0.0f)) return fail(QUAIL_E_INVAL, "n >= 0 and scale > 0 required");
  if (n == 0) return QUAIL_OK;
  if (!x || !codes) return fail(QUAIL_E_INVAL, "NULL argument");
  HIP_TRY(launch_fp8_encode(n, x, 1.0f / scale, codes, as_stream(stream)));
  return QUAIL_OK;
}

quail_status quail_fp8_e4m3_decode(int64_t n, const uint8_t* codes, float scale, float* x,
                                   quail_stream stream) {
  if (n < 0) return fail(QUAIL_E_INVAL, "n >= 0 required");
  if (n == 0) return QUAIL_OK;
  if (!x || !codes) return fail(QUAIL_E_INVAL, "NULL argument");
  HIP_TRY(launch_fp8_decode(n, codes, scale, x, as_stream(stream)));
  return QUAIL_OK;
}

}  // extern "C"
