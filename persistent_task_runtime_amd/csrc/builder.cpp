// Host task-graph builder: operators -> tiles -> tasks, per-CU queues; graph
// checks; the host form of the start-of-run rule.
//
// Sources (web pages on Mirage Persistent Kernel, "MPK"):
//   P1 "Mirage Persistent Kernel: Fusing Multi-GPU LLM Inference into One
//      Kernel Launch" (hysenlabs.com, English review)
//   P4 "Mirage Persistent Kernel：把 LLM 推理压进单个 GPU 内核" (hysenlabs.com, Chinese review)
//   P5 "Mirage Persistent Kernel kompiliert LLM-Inferenz in einen Persistent
//      Kernel" (hysenlabs.com, German review)
//
// The pages describe a compiler that turns a chain of fused operators into
// tasks which on-GPU schedulers hand to workers (P1 "How MPK Works"; P4
// "工作机制"), and advise that each operator's thread-block count be a multiple
// of the worker count so no worker idles (P1 "The API"; P5 "Grenzen der
// README-Aussagen").  Here each operator is split into at most one tile per
// worker CU (256 on MI355X), tiles become tasks, and each CU gets a static
// queue of its tasks in operator order.  Tasks hand values to each other as
// stamped words (the device runtime): a task waits for exactly the words it
// reads, so the graph needs no event counters; the operator-level edges
// derived here check the graph (producers before consumers, every operator
// an ancestor of the last) and are kept for introspection.
#include <algorithm>
#include <cstring>
#include <memory>
#include <set>

#include "graph.hpp"

static thread_local std::string g_err;

int mpk_fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}
void mpk_clear_error() { g_err.clear(); }

extern "C" const char* mpk_last_error(void) { return g_err.c_str(); }

int mpk_attn_splits(int num_workers, int batch, int nkv, int max_seq) {
  // Enough splits that one split holds at most MPK_ATTN_SPLIT positions at
  // full length, but no more tasks than workers.
  int ns = num_workers / std::max(1, batch * nkv);
  int by_len = (max_seq + MPK_ATTN_SPLIT - 1) / MPK_ATTN_SPLIT;
  ns = std::min(ns, by_len);
  return std::max(1, ns);
}

namespace {

struct Shape {
  int dtype;
  int ndim;
  int64_t d[4];
};

std::string tname(const mpk_graph_s* g, int id) {
  if (id < 0 || id >= (int)g->tensors.size()) return "#" + std::to_string(id);
  const std::string& n = g->names[id];
  return n.empty() ? "#" + std::to_string(id) : n;
}

int check_tensor(const mpk_graph_s* g, int id, int dtype, std::initializer_list<int64_t> dims,
                 const char* what, int op) {
  if (id < 0 || id >= (int)g->tensors.size())
    return mpk_fail(MPK_ERR_INVALID_ARG, "op " + std::to_string(op) + ": " + what + " tensor id " +
                                             std::to_string(id) + " out of range");
  const mpk_tensor& t = g->tensors[id];
  if (t.dtype != dtype)
    return mpk_fail(MPK_ERR_DTYPE, "op " + std::to_string(op) + ": " + what + " (" + tname(g, id) +
                                       ") has the wrong dtype");
  if ((int)dims.size() != t.ndim)
    return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(op) + ": " + what + " (" + tname(g, id) +
                                       ") has " + std::to_string(t.ndim) + " dims, expected " +
                                       std::to_string(dims.size()));
  int i = 0;
  for (int64_t want : dims) {
    if (want >= 0 && t.dims[i] != want)
      return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(op) + ": " + what + " (" + tname(g, id) +
                                         ") dim " + std::to_string(i) + " is " +
                                         std::to_string(t.dims[i]) + ", expected " +
                                         std::to_string(want));
    ++i;
  }
  // bf16 / f32 tensors are read in 16-byte units; int32 meta tensors by element
  const uintptr_t align = t.dtype == MPK_I32 ? 4 : 16;
  if (t.dev_ptr && ((uintptr_t)t.dev_ptr & (align - 1)))
    return mpk_fail(MPK_ERR_ALIGN, "tensor " + tname(g, id) + " is not " + std::to_string(align) + "-byte aligned");
  return MPK_OK;
}

}  // namespace

extern "C" int mpk_build_graph(const mpk_model_cfg* model, const mpk_launch_cfg* launch,
                               const mpk_tensor* tensors, int32_t n_tensors, const mpk_op* ops,
                               int32_t n_ops, const mpk_meta* meta, mpk_graph_t* out) {
  mpk_clear_error();
  if (!model || !launch || !tensors || !ops || !meta || !out || n_tensors <= 0 || n_ops <= 0)
    return mpk_fail(MPK_ERR_INVALID_ARG, "mpk_build_graph: NULL argument or empty table");
  *out = nullptr;
  auto g = new mpk_graph_s();
  std::unique_ptr<mpk_graph_s> guard(g);
  g->model = *model;
  g->launch = *launch;
  g->meta = *meta;
  g->tensors.assign(tensors, tensors + n_tensors);
  for (auto& t : g->tensors) {
    g->names.push_back(t.name ? t.name : "");
    t.name = nullptr;
  }
  g->ops.assign(ops, ops + n_ops);
  const mpk_model_cfg& M = g->model;
  if (M.num_layers <= 0 || M.hidden <= 0 || M.n_q_heads <= 0 || M.n_kv_heads <= 0 ||
      M.head_dim <= 0 || M.ffn <= 0 || M.vocab <= 0 || M.max_seq <= 0 || M.max_batch <= 0 ||
      !(M.rms_eps >= 0.f) || !(M.rope_theta > 0.f))
    return mpk_fail(MPK_ERR_INVALID_ARG, "model config has a non-positive field");
  if (M.n_q_heads % M.n_kv_heads)
    return mpk_fail(MPK_ERR_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  // the attention kernel is specialised for these two head sizes
  if (M.head_dim != 64 && M.head_dim != 128) return mpk_fail(MPK_ERR_SHAPE, "head_dim must be 64 or 128");
  if (M.n_q_heads / M.n_kv_heads > MPK_NW)
    return mpk_fail(MPK_ERR_SHAPE, "more than 8 query heads per kv head");

  // ---- worker / scheduler split (P1 "How MPK Works", restated for CUs) ----
  mpk_launch_cfg& Lc = g->launch;
  if (Lc.num_cus <= 0) return mpk_fail(MPK_ERR_INVALID_ARG, "launch.num_cus must be set (> 0)");
  if (Lc.sched_mode == MPK_SCHED_CORESIDENT) {
    int w = Lc.num_workers ? Lc.num_workers : Lc.num_cus;
    if (w != Lc.num_cus)
      return mpk_fail(MPK_ERR_SPLIT, "co-resident mode needs num_workers == CU count (" +
                                         std::to_string(Lc.num_cus) + ")");
    if (Lc.num_schedulers != 0 && Lc.num_schedulers != w)
      return mpk_fail(MPK_ERR_SPLIT, "co-resident mode carries one scheduler wavefront per worker");
    g->num_workers = w;
  } else if (Lc.sched_mode == MPK_SCHED_DEDICATED) {
    if (Lc.num_workers <= 0 || Lc.num_schedulers <= 0 || Lc.num_schedulers % 4 ||
        Lc.num_workers + Lc.num_schedulers / 4 != Lc.num_cus)
      return mpk_fail(MPK_ERR_SPLIT, "dedicated mode needs num_workers + num_schedulers/4 == "
                                     "CU count with num_schedulers a positive multiple of 4");
    g->num_workers = Lc.num_workers;
  } else {
    return mpk_fail(MPK_ERR_INVALID_ARG, "unknown sched_mode");
  }
  const int W = g->num_workers;
  g->num_queues = Lc.num_cus;

  // ---- meta tensors ----
  // B rows per iteration: R consecutive positions of each of NR requests
  const int NR = meta->num_requests;
  const int R = meta->rows_per_request > 0 ? meta->rows_per_request : 1;
  if (NR <= 0 || meta->rows_per_request < 0 || (int64_t)NR * R > MPK_MAX_BATCH)
    return mpk_fail(MPK_ERR_SHAPE, "num_requests x rows_per_request must be 1, 2 or 8 (and at most max_batch)");
  const int B = NR * R;
  if (B > M.max_batch || (B > 2 && B != MPK_MAX_BATCH))
    return mpk_fail(MPK_ERR_SHAPE, "num_requests x rows_per_request must be 1, 2 or 8 (and at most max_batch)");
  g->rows = B;
  g->rpr = R;
  g->meta.rows_per_request = R;
  int rc;
  if ((rc = check_tensor(g, meta->tokens, MPK_I32, {NR, -1}, "tokens", -1))) return rc;
  if ((rc = check_tensor(g, meta->step, MPK_I32, {NR}, "step", -1))) return rc;
  if ((rc = check_tensor(g, meta->prompt_len, MPK_I32, {NR}, "prompt_len", -1))) return rc;
  for (int id : {meta->tokens, meta->step, meta->prompt_len})
    if (!g->tensors[id].dev_ptr)
      return mpk_fail(MPK_ERR_INVALID_ARG, "meta tensors must be attached caller memory");

  const int H = M.hidden, d = M.head_dim, nq = M.n_q_heads, nkv = M.n_kv_heads;
  const int qkv_w = (nq + 2 * nkv) * d;
  g->producer.assign(n_tensors, -1);
  g->embed_src.assign(n_tensors, -1);
  g->dops.assign(n_ops, mpk_dev_op{});
  std::vector<std::vector<int>> reads(n_ops);  // f32 activations read
  std::vector<int> reads_meta(n_ops, 0);
  int lm_op = -1;

  auto set_producer = [&](int op, int t) -> int {
    if (t < 0 || t >= n_tensors) return mpk_fail(MPK_ERR_INVALID_ARG, "output tensor id out of range");
    if (g->producer[t] != -1)
      return mpk_fail(MPK_ERR_GRAPH, "tensor " + tname(g, t) + " has two producers");
    g->producer[t] = op;
    return MPK_OK;
  };
  auto act_read = [&](int op, int t) {
    if (g->embed_src[t] >= 0) reads_meta[op] = 1;
    else reads[op].push_back(t);
  };

  for (int i = 0; i < n_ops; ++i) {
    const mpk_op& o = g->ops[i];
    mpk_dev_op& D = g->dops[i];
    switch (o.kind) {
      case MPK_OP_EMBED: {
        if ((rc = check_tensor(g, o.in[0], MPK_BF16, {M.vocab, H}, "E", i))) return rc;
        if ((rc = check_tensor(g, o.out[0], MPK_F32, {B, H}, "x", i))) return rc;
        if ((rc = set_producer(i, o.out[0]))) return rc;
        g->embed_src[o.out[0]] = o.in[0];
        D.kind = 0;
        break;
      }
      case MPK_OP_RMSNORM_LINEAR:
      case MPK_OP_LINEAR_RESIDUAL:
      case MPK_OP_RMSNORM_GATEUP:
      case MPK_OP_LMHEAD_ARGMAX: {
        const mpk_tensor& X = g->tensors[o.in[0] >= 0 && o.in[0] < n_tensors ? o.in[0] : 0];
        if (o.in[0] < 0 || o.in[0] >= n_tensors || X.ndim != 2)
          return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) + ": x must be [B, K]");
        const int K = (int)X.dims[1];
        if ((rc = check_tensor(g, o.in[0], MPK_F32, {B, K}, "x", i))) return rc;
        if (K % 8) return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) + ": K must be a multiple of 8");
        const int nseg = (K + MPK_SEG - 1) / MPK_SEG;
        {
          // columns are split over the 8 worker wavefronts in 512-column units
          const int upr = (K + 511) / 512;
          if (!((upr % MPK_NW == 0 && upr / MPK_NW <= 3) || (MPK_NW % upr == 0)))
            return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) + ": K = " + std::to_string(K) +
                                               " must give 1, 2, 4, 8, 16 or 24 units of 512 columns");
        }
        act_read(i, o.in[0]);
        D.kind = MPK_TK_GEMV;
        D.K = K;
        D.nseg = nseg;
        D.x_embed = g->embed_src[o.in[0]] >= 0;
        D.has_norm = o.kind != MPK_OP_LINEAR_RESIDUAL;
        if (D.has_norm && (rc = check_tensor(g, o.in[1], MPK_BF16, {K}, "gain", i))) return rc;
        int N = 0;
        if (o.kind == MPK_OP_RMSNORM_LINEAR) {
          int rows[3] = {0, 0, 0};
          for (int w = 0; w < 3; ++w) {
            int id = o.in[2 + w];
            if (id < 0) {
              if (w == 0) return mpk_fail(MPK_ERR_INVALID_ARG, "rmsnorm_linear needs W0");
              continue;
            }
            if ((rc = check_tensor(g, id, MPK_BF16, {-1, K}, "W", i))) return rc;
            rows[w] = (int)g->tensors[id].dims[0];
          }
          D.N0 = rows[0], D.N1 = rows[1], D.N2 = rows[2];
          N = rows[0] + rows[1] + rows[2];
          if ((rc = check_tensor(g, o.out[0], MPK_F32, {B, N}, "y", i))) return rc;
          D.epi = MPK_EPI_STORE;
        } else if (o.kind == MPK_OP_LINEAR_RESIDUAL) {
          if ((rc = check_tensor(g, o.in[1], MPK_BF16, {-1, K}, "W", i))) return rc;
          N = (int)g->tensors[o.in[1]].dims[0];
          D.N0 = N;
          if ((rc = check_tensor(g, o.in[2], MPK_F32, {B, N}, "residual", i))) return rc;
          if ((rc = check_tensor(g, o.out[0], MPK_F32, {B, N}, "y", i))) return rc;
          act_read(i, o.in[2]);
          D.res_embed = g->embed_src[o.in[2]] >= 0;
          D.epi = MPK_EPI_RESID;
        } else if (o.kind == MPK_OP_RMSNORM_GATEUP) {
          if ((rc = check_tensor(g, o.in[2], MPK_BF16, {-1, K}, "Wg", i))) return rc;
          int F = (int)g->tensors[o.in[2]].dims[0];
          if ((rc = check_tensor(g, o.in[3], MPK_BF16, {F, K}, "Wu", i))) return rc;
          if ((rc = check_tensor(g, o.out[0], MPK_F32, {B, F}, "m", i))) return rc;
          D.N0 = F, D.N1 = F;
          D.pairs = 1;
          N = 2 * F;
          D.epi = MPK_EPI_SILU;
        } else {
          if (lm_op >= 0) return mpk_fail(MPK_ERR_GRAPH, "more than one LM head operator");
          lm_op = i;
          if ((rc = check_tensor(g, o.in[2], MPK_BF16, {M.vocab, K}, "E", i))) return rc;
          N = M.vocab;
          D.N0 = N;
          if (o.out[0] >= 0) {
            if ((rc = check_tensor(g, o.out[0], MPK_F32, {-1, B, M.vocab}, "logits", i))) return rc;
            D.logits_iters = g->tensors[o.out[0]].dims[0];
          }
          D.epi = MPK_EPI_ARGMAX;
          D.kind = MPK_TK_LMHEAD;
          reads_meta[i] = 1;
        }
        if (o.kind != MPK_OP_LMHEAD_ARGMAX || o.out[0] >= 0)
          if ((rc = set_producer(i, o.out[0]))) return rc;
        D.n_out = o.kind == MPK_OP_RMSNORM_GATEUP ? N / 2 : N;
        // tiling: every worker wavefront must get >= 2 weight blocks per tile
        const int a = D.pairs ? 2 : 1;
        const int U = N / a;
        const int per_wave_units = (2 + a * nseg - 1) / (a * nseg);
        const int min_units = MPK_NW * per_wave_units;
        // Rows of one 4096-column group, one request: while a tile's inputs
        // are awaited, its wavefronts also stream assignment units into the
        // LDS beyond the input's landing zone (as many as fit).
        D.lds_pre = K == 4096 && B == 1 ? 1 : 0;
        // A GEMV reading an attention output waits for the whole attention
        // phase, which occupies only the attention tasks' workers: its tiles
        // go to the other workers, which stream ahead meanwhile.
        {
          const int xp = g->producer[o.in[0]];
          if (xp >= 0 && g->dops[xp].kind == MPK_TK_ATTN && g->dops[xp].ntiles <= W / 2 && o.num_tiles <= 0 &&
              !D.pairs && K == 4096 && B == 1 && U / (W - g->dops[xp].ntiles) >= 2 * MPK_NW)
            D.worker_base = g->dops[xp].ntiles;
        }
        const int Wt = W - D.worker_base;  // workers this operator's tiles may use
        // Batch 8, linear + residual over several 4096-column passes (the
        // down projection): split K, one pass per tile, so a CU gathers only
        // its columns of the 8 rows' x (down: 128 KB instead of 384 KB, as
        // much as its weights); each row group's last split merges.
        D.ksplit = B == MPK_MAX_BATCH && o.kind == MPK_OP_LINEAR_RESIDUAL && !D.res_embed && K > 4096 &&
                           K <= 3 * 4096 && K % 4096 == 0 && o.num_tiles <= 0 && !D.worker_base
                       ? K / 4096
                       : 0;
        const int ks = std::max(1, (int)D.ksplit);
        int T = o.num_tiles > 0 ? o.num_tiles : std::max(1, std::min(Wt / ks, U / min_units));
        if (T > Wt || U / T < min_units)
          return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) + ": " + std::to_string(U) +
                                             " rows cannot give " + std::to_string(T) +
                                             " tiles of >= " + std::to_string(min_units) + " rows");
        D.ntiles = T * ks;  // T row groups, ks splits each
        const int tile_rows = ((U + T - 1) / T) * a;  // largest tile, virtual rows
        if (B == MPK_MAX_BATCH) {
          // batch 8 runs the MFMA bodies: x staged in LDS per 4096-column
          // pass, 16-row blocks split over the waves (1 or 2 blocks: all
          // waves split K; up to 6: two row groups; the LM head: up to 40
          // blocks, one row group per wave), 8 x outputs staged in 4 KB
          if (K % 4096)
            return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) + ": at batch 8 the input width K = " +
                                               std::to_string(K) + " must be a multiple of 4096");
          const int nblk = (tile_rows + 15) / 16;
          const int max_blk = D.epi == MPK_EPI_ARGMAX ? 40 : 6;
          if (nblk > max_blk || (D.epi != MPK_EPI_ARGMAX && 8 * (D.pairs ? tile_rows / 2 : tile_rows) > 1024))
            return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) + ": " + std::to_string(tile_rows) +
                                               " rows per tile exceed the batch-8 tile");
        } else if (B > 2) {
          return mpk_fail(MPK_ERR_SHAPE, "num_requests must be 1, 2 or 8");
        } else {
          if (D.kind == MPK_TK_GEMV && (int64_t)B * tile_rows > 512)
            return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) +
                                               ": rows per tile x num_requests exceed 512");
          if ((int64_t)B * tile_rows * 32 > (B == 1 ? 28 * 1024 : 40 * 1024))
            return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) +
                                               ": rows per tile x num_requests exceed the partial-sum buffer");
        }
        break;
      }
      case MPK_OP_ATTENTION: {
        if ((rc = check_tensor(g, o.in[0], MPK_F32, {B, qkv_w}, "qkv", i))) return rc;
        if ((rc = check_tensor(g, o.in[1], MPK_BF16, {d}, "q_norm", i))) return rc;
        if ((rc = check_tensor(g, o.in[2], MPK_BF16, {d}, "k_norm", i))) return rc;
        if ((rc = check_tensor(g, o.in[3], MPK_BF16, {NR, nkv, M.max_seq, d}, "kcache", i))) return rc;
        if ((rc = check_tensor(g, o.in[4], MPK_BF16, {NR, nkv, M.max_seq, d}, "vcache", i))) return rc;
        if (!g->tensors[o.in[3]].dev_ptr || !g->tensors[o.in[4]].dev_ptr)
          return mpk_fail(MPK_ERR_INVALID_ARG, "KV caches must be attached caller memory");
        if ((rc = check_tensor(g, o.out[0], MPK_F32, {B, nq * d}, "o", i))) return rc;
        if ((rc = set_producer(i, o.out[0]))) return rc;
        act_read(i, o.in[0]);
        reads_meta[i] = 1;
        D.kind = MPK_TK_ATTN;
        // one attention task per worker at least per (request, kv head): a
        // split that owns the position gathers the others, so two groups
        // must never share a queue (an owner could wait on a split queued
        // behind it)
        if (B * nkv > W)
          return mpk_fail(MPK_ERR_SHAPE, "op " + std::to_string(i) + ": rows x n_kv_heads = " +
                                             std::to_string(B * nkv) + " exceeds the " + std::to_string(W) +
                                             " workers (one attention task per worker)");
        D.nq = nq, D.nkv = nkv, D.d = d, D.S = M.max_seq;
        D.nsplit = mpk_attn_splits(W, B, nkv, M.max_seq);
        D.ntiles = B * nkv * D.nsplit;
        break;
      }
      default:
        return mpk_fail(MPK_ERR_INVALID_ARG, "op " + std::to_string(i) + ": unknown kind");
    }
  }
  // activations must come from earlier operators
  for (int i = 0; i < n_ops; ++i)
    for (int t : reads[i]) {
      int p = g->producer[t];
      if (p >= i)
        return mpk_fail(MPK_ERR_GRAPH, "op " + std::to_string(i) + " reads " + tname(g, t) +
                                           " before its producer op " + std::to_string(p));
    }
  // ---- internal argmax operator after the LM head ----
  // The LM head's tiles each publish a (max, index) pair; one argmax task
  // reduces them, writes the token and advances step (the iteration's end).
  int NA = n_ops;
  if (lm_op >= 0) {
    mpk_dev_op A{};
    A.kind = MPK_TK_ARGMAX;
    A.ntiles = 1;
    A.N0 = g->dops[lm_op].N0;
    g->dops.push_back(A);
    g->argmax_op = NA;
    reads.emplace_back();
    reads_meta.push_back(1);
    ++NA;
  }
  // ---- events: one flag per producer task (per merge group for attention) ----
  std::vector<int> op_ev(NA, -1);
  for (int i = 0; i < NA; ++i) {
    if (g->dops[i].kind == 0) continue;
    op_ev[i] = (int)g->ev_count.size();
    const mpk_dev_op& D = g->dops[i];
    // tasks that publish the operator's words (attention: one owner split per group)
    int cnt = D.kind == MPK_TK_ATTN ? B * D.nkv : D.ntiles;
    g->ev_count.push_back(cnt);
    g->ev_op.push_back(i);
    g->dops[i].event = op_ev[i];
  }
  int sink = -1;
  for (int i = NA - 1; i >= 0; --i)
    if (g->dops[i].kind) {
      sink = i;
      break;
    }
  if (sink < 0) return mpk_fail(MPK_ERR_GRAPH, "graph has no operator with work");
  if (lm_op >= 0 && lm_op != n_ops - 1)
    return mpk_fail(MPK_ERR_GRAPH, "the LM head operator must be the last operator");
  g->sink = sink;
  // same-iteration ancestors
  std::vector<std::set<int>> direct(NA), anc(NA);
  for (int i = 0; i < NA; ++i) {
    if (!g->dops[i].kind) continue;
    for (int t : reads[i]) {
      int p = g->producer[t];
      if (p >= 0 && g->dops[p].kind) direct[i].insert(p);
    }
    if (i == g->argmax_op) direct[i].insert(lm_op);
    for (int p : direct[i]) {
      anc[i].insert(p);
      anc[i].insert(anc[p].begin(), anc[p].end());
    }
  }
  for (int i = 0; i < NA; ++i)
    if (g->dops[i].kind && i != sink && !anc[sink].count(i))
      return mpk_fail(MPK_ERR_GRAPH, "op " + std::to_string(i) +
                                         " is not an ancestor of the last operator");
  // previous-iteration edge: readers of tokens/step (through the embedding or
  // directly) and every operator without producers wait for the sink.
  std::vector<int> has_prev(NA, 0), needs_prev(NA, 0);
  for (int i = 0; i < NA; ++i) {
    if (!g->dops[i].kind) continue;
    needs_prev[i] = (reads_meta[i] && lm_op >= 0 && i != g->argmax_op) || direct[i].empty();
    has_prev[i] = needs_prev[i];
    for (int p : anc[i]) has_prev[i] |= has_prev[p];
  }
  std::vector<std::vector<std::pair<int, int>>> deps(NA);  // (op, prev)
  for (int i = 0; i < NA; ++i) {
    if (!g->dops[i].kind) continue;
    for (int p : direct[i]) {
      bool implied = false;
      for (int q : direct[i])
        if (q != p && anc[q].count(p)) implied = true;
      if (!implied) deps[i].push_back({p, 0});
    }
    if (needs_prev[i]) {
      bool implied = false;
      for (int q : direct[i])
        if (has_prev[q]) implied = true;
      if (!implied) deps[i].push_back({sink, 1});
    }
    if ((int)deps[i].size() > MPK_MAX_DEPS)
      return mpk_fail(MPK_ERR_GRAPH, "op " + std::to_string(i) + " has more than 3 direct producers");
  }
  // ---- tasks ----
  g->op_first_task.assign(NA, 0);
  g->op_ntasks.assign(NA, 0);
  for (int i = 0; i < NA; ++i) {
    mpk_dev_op& D = g->dops[i];
    g->op_first_task[i] = (int)g->tasks.size();
    if (!D.kind) continue;
    g->op_ntasks[i] = D.ntiles;
    for (int t = 0; t < D.ntiles; ++t) {
      mpk_dev_task T{};
      T.kind = D.kind;
      T.op = i;
      T.tile = t;
      // attention tasks take workers 0, 1, ... (one each); other tiles spread
      // evenly over their workers
      T.worker = D.kind == MPK_TK_ATTN ? t
                                       : D.worker_base + (int)(((int64_t)t * (W - D.worker_base)) / D.ntiles);
      T.split = -1;
      if (D.kind == MPK_TK_ATTN) {
        int per_req = D.nkv * D.nsplit;
        T.row0 = t / per_req;                   // request
        T.nrows = (t % per_req) / D.nsplit;     // kv head
        T.split = t % D.nsplit;
      } else if (D.kind == MPK_TK_ARGMAX) {
        // co-resident mode: worker 0; dedicated mode: the first scheduler CU
        T.worker = g->num_queues > W ? W : 0;
        T.row0 = 0;
        T.nrows = D.N0;
      } else {
        const int a = D.pairs ? 2 : 1;
        const int U = (D.N0 + D.N1 + D.N2) / a;
        const int ks = std::max(1, (int)D.ksplit), ng = D.ntiles / ks, grp = t / ks;
        int u0 = (int)((int64_t)grp * U / ng), u1 = (int)((int64_t)(grp + 1) * U / ng);
        T.row0 = u0 * a;
        T.nrows = (u1 - u0) * a;
        if (D.ksplit > 1) T.split = t % ks;
      }
      mpk_task_info I{};
      for (int k = 0; k < MPK_MAX_DEPS; ++k) I.dep_event[k] = I.dep_count[k] = I.dep_prev[k] = -1;
      for (int k = 0; k < (int)deps[i].size(); ++k) {
        const int e = op_ev[deps[i][k].first];
        I.dep_event[k] = e;
        I.dep_count[k] = g->ev_count[e];
        I.dep_prev[k] = deps[i][k].second;
      }
      g->tasks.push_back(T);
      I.op = i, I.tile = t, I.worker = T.worker, I.row0 = T.row0, I.nrows = T.nrows, I.split = T.split;
      I.out_event = op_ev[i];
      g->info.push_back(I);
    }
  }
  // ---- per-CU queues in operator order (dedicated scheduler CUs hold the
  // argmax task or nothing) ----
  const int NQ = g->num_queues;
  std::vector<std::vector<int>> q(NQ);
  for (size_t k = 0; k < g->tasks.size(); ++k) q[g->tasks[k].worker].push_back((int)k);
  g->qlen.assign(NQ, 0);
  g->max_queue = 1;
  for (int w = 0; w < NQ; ++w) {
    g->qlen[w] = (int)q[w].size();
    g->max_queue = std::max(g->max_queue, g->qlen[w]);
  }
  g->queues.assign((size_t)NQ * g->max_queue, mpk_dev_qentry{-1});
  g->queue_ids.assign((size_t)NQ * g->max_queue, -1);
  for (int w = 0; w < NQ; ++w) {
    const int n = g->qlen[w];
    for (int k = 0; k < n; ++k) {
      g->queues[(size_t)w * g->max_queue + k] = mpk_dev_qentry{q[w][k]};
      g->queue_ids[(size_t)w * g->max_queue + k] = q[w][k];
    }
  }
  *out = guard.release();
  return MPK_OK;
}

extern "C" int mpk_get_graph_info(mpk_graph_t g, mpk_graph_info* info) {
  mpk_clear_error();
  if (!g || !info) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL argument");
  info->num_tasks = (int)g->tasks.size();
  info->num_events = (int)g->ev_count.size();
  info->num_workers = g->num_workers;
  info->num_queues = g->num_queues;
  info->max_queue = g->max_queue;
  info->num_ops = (int)g->dops.size();
  info->sink_op = g->sink;
  info->tasks = g->info.data();
  info->event_count = g->ev_count.data();
  info->event_op = g->ev_op.data();
  info->queue_len = g->qlen.data();
  info->queues = g->queue_ids.data();
  return MPK_OK;
}

extern "C" void mpk_destroy_graph(mpk_graph_t g) { delete g; }

// The start-of-run rule of mpk_begin_run (device) on host copies of the meta
// tensors: positions inside tokens and the KV cache, every id the run reads
// from tokens inside the vocabulary, and with R rows per request (batched
// prompt ingestion) every consumed position followed by a prompt position.
extern "C" int mpk_check_run(mpk_graph_t g, const int32_t* step, const int32_t* tokens,
                             const int32_t* prompt_len, int32_t n_iter) {
  mpk_clear_error();
  if (!g || !step || !tokens || !prompt_len) return mpk_fail(MPK_ERR_INVALID_ARG, "mpk_check_run: NULL argument");
  if (n_iter <= 0) return mpk_fail(MPK_ERR_INVALID_ARG, "num_iterations must be positive");
  const int NR = g->meta.num_requests, R = g->rpr;
  const int64_t width = g->tensors[g->meta.tokens].dims[1];
  const int64_t n_pos = (int64_t)R * n_iter;  // positions each request consumes
  for (int r = 0; r < NR; ++r) {
    const int p0 = step[r];
    if (p0 < 0 || p0 + n_pos >= width || p0 + n_pos > g->model.max_seq)
      return mpk_fail(MPK_ERR_SHAPE, "request " + std::to_string(r) + ": step " + std::to_string(p0) + " + " +
                                         std::to_string(n_pos) +
                                         " positions leaves the tokens tensor or the KV cache");
    if (R > 1 && p0 + n_pos > (int64_t)prompt_len[r] - 1)
      return mpk_fail(MPK_ERR_SHAPE, "request " + std::to_string(r) + ": " + std::to_string(n_pos) +
                                         " positions from step " + std::to_string(p0) +
                                         " reach past the prompt (batched ingestion generates no token)");
    const int q_end = R > 1 ? (int)(p0 + n_pos) : std::min(p0 + n_iter, std::max(prompt_len[r], p0 + 1));
    for (int q = p0; q < q_end; ++q) {
      const int t = tokens[(int64_t)r * width + q];
      if (t < 0 || t >= g->model.vocab)
        return mpk_fail(MPK_ERR_SHAPE, "request " + std::to_string(r) + ": token id " + std::to_string(t) +
                                           " at position " + std::to_string(q) + " is outside the vocabulary");
    }
  }
  return MPK_OK;
}
