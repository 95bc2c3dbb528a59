// Host model of the device's dependency protocol, for tests of the graph
// builder and of the protocol itself (no device code runs here).
//
// Sources (web pages on Mirage Persistent Kernel, "MPK"):
//   P1 "Mirage Persistent Kernel: Fusing Multi-GPU LLM Inference into One
//      Kernel Launch" (hysenlabs.com, English review), "How MPK Works"
//   P4 "Mirage Persistent Kernel：把 LLM 推理压进单个 GPU 内核" (hysenlabs.com,
//      Chinese review), "工作机制"
//
// The pages describe tasks handed to workers once their inputs are ready and
// a step counter advanced after each iteration.  On the device every value one
// task hands to another is a 64-bit word (32-bit payload, 32-bit iteration
// stamp); a task polls exactly the words it reads until they carry the
// iteration's stamp (iter_base + s + 1, iter_base growing across launches),
// K/V rows are plain data stored and drained before the stamped word that
// orders their readers, and the attention split owning the position gathers
// the other splits' partial words.  This file runs that protocol on host
// threads, one per CU queue, over the same operator and task tables the device
// reads, with every task body replaced by a seeded random sleep:
//
//  * word buffers per operator output (and per attention / LM-head operator
//    for split partials and tile maxima) live in a simulation state that
//    persists across mpk_simulate calls, like device buffers across launches;
//  * each accepted word's payload is checked against the value its producer
//    writes in this iteration of this launch (the payload encodes the
//    launch), so a stale word that passes the stamp check is reported;
//  * each K/V row a task reads must have been written (by an earlier
//    iteration's owner split, or prefilled) before it is read;
//  * token words and tokens / step follow the argmax task's rule.
// Planted faults (mpk_sim_cfg.fault) show that each check fires.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstring>
#include <functional>
#include <memory>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "graph.hpp"

namespace {

uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

// The payload a producer writes for element `elem` of buffer `tag` in the
// iteration with stamp `stamp` of simulated launch `epoch`.
uint32_t payload(uint32_t tag, uint64_t elem, uint32_t stamp, uint32_t epoch) {
  return (uint32_t)mix64(mix64(tag + 0x9e3779b97f4a7c15ull) ^ mix64(elem + 0x632be59bd9b4e019ull) ^
                         mix64(((uint64_t)epoch << 32 | stamp) + 0x85ebca77c2b2ae63ull));
}

uint64_t word(uint32_t pay, uint32_t stamp) { return (uint64_t)stamp << 32 | pay; }

struct Words {
  std::unique_ptr<std::atomic<uint64_t>[]> w;
  size_t n = 0;
  void alloc(size_t k) {
    w.reset(new std::atomic<uint64_t>[k]);
    n = k;
    for (size_t i = 0; i < k; ++i) w[i].store(0, std::memory_order_relaxed);
  }
};

constexpr uint32_t KV_PREFILLED = 0xffffffffu;
constexpr uint32_t TAG_OP = 0x10000;  // per-operator buffers: tag TAG_OP + op
constexpr uint32_t NO_TICKET = 0xffffffffu;

}  // namespace

struct mpk_sim_s {
  mpk_graph_t g = nullptr;
  int B = 0;
  int64_t width = 0;
  int S = 0;
  std::unique_ptr<std::atomic<int32_t>[]> tokens;  // [B][width]
  std::unique_ptr<std::atomic<int32_t>[]> step;    // [B]
  std::vector<int32_t> prompt_len;
  std::vector<Words> tensor_words;  // per tensor: stamped words of an operator output (or empty)
  std::vector<Words> op_words;      // per operator: attention split partials, LM-head tile maxima
  std::vector<std::unique_ptr<std::atomic<uint32_t>[]>> kv_ver;  // per attention op: [B][nkv][S] writer stamp
  Words tok;                        // [B] next-token words
  uint32_t epoch = 0;
};

extern "C" int mpk_sim_create(mpk_graph_t g, const int32_t* step, const int32_t* tokens, const int32_t* prompt_len,
                              int32_t kv_filled, mpk_sim_t* out) {
  mpk_clear_error();
  if (!g || !step || !tokens || !prompt_len || !out || kv_filled < 0)
    return mpk_fail(MPK_ERR_INVALID_ARG, "mpk_sim_create: bad argument");
  *out = nullptr;
  std::unique_ptr<mpk_sim_s> s(new mpk_sim_s());
  s->g = g;
  if (g->rpr != 1)
    return mpk_fail(MPK_ERR_SHAPE, "the simulator models decode graphs (one row per request) only");
  s->B = g->meta.num_requests;
  s->width = g->tensors[g->meta.tokens].dims[1];
  s->S = g->model.max_seq;
  if (kv_filled > s->S) return mpk_fail(MPK_ERR_SHAPE, "kv_filled exceeds max_seq");
  s->tokens.reset(new std::atomic<int32_t>[(size_t)s->B * s->width]);
  for (int64_t i = 0; i < (int64_t)s->B * s->width; ++i) s->tokens[i].store(tokens[i], std::memory_order_relaxed);
  s->step.reset(new std::atomic<int32_t>[s->B]);
  for (int r = 0; r < s->B; ++r) s->step[r].store(step[r], std::memory_order_relaxed);
  s->prompt_len.assign(prompt_len, prompt_len + s->B);
  const int NT = (int)g->tensors.size();
  s->tensor_words.resize(NT);
  for (int t = 0; t < NT; ++t) {
    const mpk_tensor& T = g->tensors[t];
    if (g->producer[t] >= 0 && g->embed_src[t] < 0 && T.dtype == MPK_F32 && T.ndim == 2)
      s->tensor_words[t].alloc((size_t)T.dims[0] * T.dims[1]);
  }
  s->op_words.resize(g->dops.size());
  s->kv_ver.resize(g->dops.size());
  for (size_t i = 0; i < g->dops.size(); ++i) {
    const mpk_dev_op& D = g->dops[i];
    if (D.kind == MPK_TK_ATTN) {
      const int G = D.nq / D.nkv;
      s->op_words[i].alloc((size_t)s->B * D.nkv * D.nsplit * G * (D.d + 2));
      const size_t nv = (size_t)s->B * D.nkv * s->S;
      s->kv_ver[i].reset(new std::atomic<uint32_t>[nv]);
      for (size_t k = 0; k < nv; ++k)
        s->kv_ver[i][k].store((int)(k % s->S) < kv_filled ? KV_PREFILLED : 0u, std::memory_order_relaxed);
    } else if (D.kind == MPK_TK_LMHEAD) {
      s->op_words[i].alloc((size_t)D.ntiles * s->B * 2);
    } else if (D.kind == MPK_TK_GEMV && D.ksplit > 1) {
      s->op_words[i].alloc((size_t)(D.ksplit - 1) * s->B * D.n_out);  // split-K partial sums
    }
  }
  s->tok.alloc(s->B);
  *out = s.release();
  return MPK_OK;
}

extern "C" void mpk_sim_destroy(mpk_sim_t s) { delete s; }

extern "C" int mpk_sim_read_meta(mpk_sim_t s, int32_t* step, int32_t* tokens) {
  mpk_clear_error();
  if (!s) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL simulation");
  if (step)
    for (int r = 0; r < s->B; ++r) step[r] = s->step[r].load();
  if (tokens)
    for (int64_t i = 0; i < (int64_t)s->B * s->width; ++i) tokens[i] = s->tokens[i].load();
  return MPK_OK;
}

extern "C" int mpk_simulate(mpk_sim_t sim, const mpk_sim_cfg* cfg, mpk_trace_record* trace) {
  mpk_clear_error();
  if (!sim || !cfg || !trace || cfg->num_iterations <= 0 || cfg->jitter_us < 0 || cfg->timeout_ms <= 0)
    return mpk_fail(MPK_ERR_INVALID_ARG, "mpk_simulate: bad argument");
  mpk_graph_t g = sim->g;
  const int n_iter = cfg->num_iterations, B = sim->B, NT = (int)g->tasks.size(), V = g->model.vocab;
  {
    // the start-of-run rule of the device (mpk_begin_run)
    std::vector<int32_t> st(B), tk((size_t)B * sim->width);
    mpk_sim_read_meta(sim, st.data(), tk.data());
    const int rc = mpk_check_run(g, st.data(), tk.data(), sim->prompt_len.data(), n_iter);
    if (rc) return rc;
  }
  const uint32_t epoch = ++sim->epoch;
  const uint32_t base = cfg->iter_base;
  if ((uint64_t)base + n_iter >= 0xffffffffull) return mpk_fail(MPK_ERR_INVALID_ARG, "iteration stamps exhausted");
  std::vector<int32_t> pos0(B);
  for (int r = 0; r < B; ++r) pos0[r] = sim->step[r].load();
  for (int64_t i = 0; i < (int64_t)n_iter * NT; ++i)
    trace[i] = mpk_trace_record{-1, -1, NO_TICKET, NO_TICKET, ~0ull, ~0ull, ~0u, ~0u, ~0ull};

  std::atomic<uint32_t> ticket{0};
  std::atomic<int> failed{0};
  std::string fail_msg;
  std::atomic<int> fail_owner{0};
  auto fail = [&](int code, const std::string& m) {
    int exp = 0;
    if (fail_owner.compare_exchange_strong(exp, 1)) {
      fail_msg = m;
      failed.store(code);
    }
  };
  const auto t0 = std::chrono::steady_clock::now();
  auto now_ns = [&] {
    return (uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0)
        .count();
  };
  auto stamp = [&](int s) { return base + (uint32_t)s + 1u; };
  auto sleep_us = [](int us) {
    if (us > 0) std::this_thread::sleep_for(std::chrono::microseconds(us));
  };

  auto worker = [&](int q) {
    std::mt19937 rng(cfg->seed * 7919u + (uint32_t)q);
    const int qlen = g->qlen[q];
    // K/V-row stores still in flight (planted fault only): they land at their
    // deadline, or when the queue ends, while the worker goes on
    struct Late {
      std::atomic<uint32_t>* at;
      uint32_t v;
      std::chrono::steady_clock::time_point due;
    };
    std::vector<Late> late;
    auto land = [&](bool all) {
      const auto t = std::chrono::steady_clock::now();
      for (size_t i = 0; i < late.size();)
        if (all || late[i].due <= t) {
          late[i].at->store(late[i].v, std::memory_order_release);
          late[i] = late.back();
          late.pop_back();
        } else {
          ++i;
        }
    };
    struct LandAtExit {
      std::function<void()> f;
      ~LandAtExit() { f(); }
    } land_at_exit{[&] { land(true); }};
    // Wait until word w carries stamp st (acquire); false on a stop.
    auto poll = [&](std::atomic<uint64_t>& w, uint32_t st, uint64_t& val) -> bool {
      const auto start = std::chrono::steady_clock::now();
      for (;;) {
        val = w.load(std::memory_order_acquire);
        if ((uint32_t)(val >> 32) == st) return true;
        if (failed.load(std::memory_order_relaxed)) return false;
        if (std::chrono::steady_clock::now() - start > std::chrono::milliseconds(cfg->timeout_ms)) {
          fail(MPK_ERR_DEVICE_TIMEOUT, "simulated wait timed out (queue " + std::to_string(q) + ")");
          return false;
        }
        std::this_thread::yield();
      }
    };
    // Wait for word i of buffer (tag, W) and check the payload its producer
    // writes in this iteration of this launch.
    auto take = [&](Words& W, uint32_t tag, size_t i, uint32_t st, int task, int s, bool skip_wait) -> bool {
      uint64_t v;
      if (skip_wait) {
        v = W.w[i].load(std::memory_order_acquire);
      } else if (!poll(W.w[i], st, v)) {
        return false;
      }
      if ((uint32_t)(v >> 32) != st || (uint32_t)v != payload(tag, i, st, epoch)) {
        fail(MPK_ERR_GRAPH, "task " + std::to_string(task) + " iteration " + std::to_string(s) +
                                ": accepted a word that is not this iteration's (buffer " + std::to_string(tag) +
                                " element " + std::to_string(i) + ")");
        return false;
      }
      return true;
    };
    auto put = [&](Words& W, uint32_t tag, size_t i, uint32_t st) {
      W.w[i].store(word(payload(tag, i, st, epoch), st), std::memory_order_release);
    };
    // The id request r consumes at position p: from tokens in a launch's
    // first iteration, else from the previous iteration's token word.
    auto token_of = [&](int r, int p, int s, int task) -> bool {
      int32_t t;
      if (s == 0) {
        t = sim->tokens[(int64_t)r * sim->width + p].load(std::memory_order_relaxed);
      } else {
        uint64_t v;
        if (!poll(sim->tok.w[r], stamp(s - 1), v)) return false;
        t = (int32_t)(uint32_t)v;
        if (t != sim->tokens[(int64_t)r * sim->width + p].load(std::memory_order_relaxed)) {
          fail(MPK_ERR_GRAPH, "task " + std::to_string(task) + " iteration " + std::to_string(s) +
                                  ": token word disagrees with tokens at position " + std::to_string(p));
          return false;
        }
      }
      if (t < 0 || t >= V) {
        fail(MPK_ERR_GRAPH, "token id outside the vocabulary reached a task");
        return false;
      }
      return true;
    };

    for (int s = 0; s < n_iter && !failed.load(); ++s) {
      const uint32_t st = stamp(s);
      for (int k = 0; k < qlen && !failed.load(); ++k) {
        const int tid = g->queues[(size_t)q * g->max_queue + k].task;
        const mpk_dev_task& T = g->tasks[tid];
        const mpk_dev_op& D = g->dops[T.op];
        const mpk_op& O = g->ops[T.op < (int)g->ops.size() ? T.op : g->ops.size() - 1];
        land(false);
        mpk_trace_record& R = trace[(int64_t)s * NT + tid];
        R.task = tid, R.iteration = s, R.hw_id = (uint32_t)q, R.xcc_id = 0;
        R.t_start = now_ns();
        const int jit = cfg->jitter_us ? (int)(rng() % (uint32_t)(cfg->jitter_us + 1)) : 0;
        bool ok = true;
        if (T.kind == MPK_TK_GEMV || T.kind == MPK_TK_LMHEAD) {
          // ---- inputs: x (embedding row, stamped words or a plain tensor), residual rows ----
          if (D.x_embed || D.res_embed)
            for (int r = 0; r < B && ok; ++r) ok = token_of(r, pos0[r] + s, s, tid);
          const int xin = O.in[0];
          // split K: the tile reads its own 4096 columns of each row's x
          const bool split = D.ksplit > 1;
          const bool merges = !split || T.split == D.ksplit - 1;
          const size_t c0 = split ? (size_t)T.split * 4096 : 0, c1 = split ? c0 + 4096 : (size_t)D.K;
          if (ok && !D.x_embed && sim->tensor_words[xin].n)
            for (size_t i = 0; i < sim->tensor_words[xin].n && ok; ++i)
              if (i % (size_t)D.K >= c0 && i % (size_t)D.K < c1)
                ok = take(sim->tensor_words[xin], (uint32_t)xin, i, st, tid, s, false);
          if (ok && merges && D.epi == MPK_EPI_RESID && !D.res_embed && sim->tensor_words[O.in[2]].n)
            for (int r = 0; r < B && ok; ++r)
              for (int row = T.row0; row < T.row0 + T.nrows && ok; ++row)
                ok = take(sim->tensor_words[O.in[2]], (uint32_t)O.in[2], (size_t)r * D.n_out + row, st, tid, s,
                          false);
          if (!ok) return;
          R.start_ticket = ticket.fetch_add(1);
          R.t_ready = now_ns();
          sleep_us(jit);
          // ---- outputs ----
          if (cfg->fault == MPK_SIM_FAULT_SKIP_WAIT && D.kind == MPK_TK_GEMV && D.epi == MPK_EPI_STORE && s == 1)
            sleep_us(200000);  // a late QKV producer: a consumer that does not wait reads the old words
          if (split && !merges) {
            // a split that does not merge: its partial sums
            for (int r = 0; r < B; ++r)
              for (int row = T.row0; row < T.row0 + T.nrows; ++row)
                put(sim->op_words[T.op], TAG_OP + T.op, ((size_t)T.split * B + r) * D.n_out + row, st);
          } else if (split) {
            // the merging split: the other splits' partial sums, then the outputs
            for (int c = 0; c < D.ksplit - 1 && ok; ++c)
              for (int r = 0; r < B && ok; ++r)
                for (int row = T.row0; row < T.row0 + T.nrows && ok; ++row)
                  ok = take(sim->op_words[T.op], TAG_OP + T.op, ((size_t)c * B + r) * D.n_out + row, st, tid, s,
                            false);
            if (!ok) return;
            for (int r = 0; r < B; ++r)
              for (int row = T.row0; row < T.row0 + T.nrows; ++row)
                put(sim->tensor_words[O.out[0]], (uint32_t)O.out[0], (size_t)r * D.n_out + row, st);
          } else if (T.kind == MPK_TK_LMHEAD) {
            if (!(cfg->fault == MPK_SIM_FAULT_DROP_PUBLISH && T.tile == 0))
              for (int r = 0; r < B; ++r)
                for (int j = 0; j < 2; ++j)
                  put(sim->op_words[T.op], TAG_OP + T.op, ((size_t)T.tile * B + r) * 2 + j, st);
          } else {
            const int o0 = D.pairs ? T.row0 / 2 : T.row0, on = D.pairs ? T.nrows / 2 : T.nrows;
            for (int r = 0; r < B; ++r)
              for (int row = o0; row < o0 + on; ++row)
                put(sim->tensor_words[O.out[0]], (uint32_t)O.out[0], (size_t)r * D.n_out + row, st);
          }
        } else if (T.kind == MPK_TK_ATTN) {
          const int r = T.row0, j = T.nrows, c = T.split, NS = D.nsplit, d = D.d, G = D.nq / D.nkv;
          // the splits fold positions 0 .. p - 1 from the cache; the owner
          // adds p (the device's split rule)
          const int p = pos0[r] + s, nf = p;
          const int na = std::max(1, std::min(NS, (nf + MPK_ATTN_SPLIT - 1) / MPK_ATTN_SPLIT));
          if (c < na) {
            const int lo = (int)((int64_t)c * nf / na), hi = (int)((int64_t)(c + 1) * nf / na);
            const bool owner = c == na - 1;
            // q of the group's heads, k and v of kv head j
            Words& X = sim->tensor_words[O.in[0]];
            const int qkv_w = (D.nq + 2 * D.nkv) * d;
            const bool skip = cfg->fault == MPK_SIM_FAULT_SKIP_WAIT;
            auto take_span = [&](int off, int len) {
              for (int i = 0; i < len && ok; ++i)
                ok = take(X, (uint32_t)O.in[0], (size_t)r * qkv_w + off + i, st, tid, s, skip);
            };
            take_span(j * G * d, G * d);
            take_span(D.nq * d + j * d, d);
            take_span((D.nq + D.nkv) * d + j * d, d);
            if (!ok) return;
            R.start_ticket = ticket.fetch_add(1);
            R.t_ready = now_ns();
            // K/V rows of this split's positions: written by an earlier
            // iteration's owner split (or pre-filled)
            std::atomic<uint32_t>* ver = sim->kv_ver[T.op].get() + ((size_t)r * D.nkv + j) * sim->S;
            for (int t = lo; t < hi; ++t)
              if (ver[t].load(std::memory_order_acquire) == 0u) {
                fail(MPK_ERR_GRAPH, "task " + std::to_string(tid) + " iteration " + std::to_string(s) +
                                        ": read the K/V row of position " + std::to_string(t) +
                                        " before it was written");
                return;
              }
            sleep_us(jit);
            Words& Pw = sim->op_words[T.op];
            const size_t grp = ((size_t)r * D.nkv + j) * NS;
            const int pw = G * (d + 2);
            Words& Ow = sim->tensor_words[O.out[0]];
            auto publish_o = [&] {
              for (int i = 0; i < G * d; ++i)
                put(Ow, (uint32_t)O.out[0], (size_t)r * D.nq * d + (size_t)j * G * d + i, st);
            };
            if (owner) {
              const bool late_row = cfg->fault == MPK_SIM_FAULT_KV_AFTER_PUBLISH;
              // the K/V row of p, stored and drained before the stamped word
              // that orders its readers
              if (!late_row) ver[p].store(st, std::memory_order_release);
              if (na > 1)
                for (int cc = 0; cc < na - 1 && ok; ++cc)
                  for (int i = 0; i < pw && ok; ++i)
                    ok = take(Pw, TAG_OP + T.op, (grp + cc) * pw + i, st, tid, s, false);
              if (!ok) return;
              publish_o();
              if (late_row)
                late.push_back(Late{&ver[p], st, std::chrono::steady_clock::now() + std::chrono::milliseconds(200)});
            } else {
              for (int i = 0; i < pw; ++i) put(Pw, TAG_OP + T.op, (grp + c) * pw + i, st);
            }
          }
        } else if (T.kind == MPK_TK_ARGMAX) {
          const int lm = g->argmax_op - 1;
          const mpk_dev_op& L = g->dops[lm];
          for (size_t i = 0; i < (size_t)L.ntiles * B * 2 && ok; ++i)
            ok = take(sim->op_words[lm], TAG_OP + lm, i, st, tid, s, false);
          if (!ok) return;
          R.start_ticket = ticket.fetch_add(1);
          R.t_ready = now_ns();
          sleep_us(jit);
          for (int r = 0; r < B; ++r) {
            const int p = pos0[r] + s;
            std::atomic<int32_t>& nx = sim->tokens[(int64_t)r * sim->width + p + 1];
            int32_t next;
            if (p + 1 >= sim->prompt_len[r]) {
              next = (int32_t)(payload(0x30000, (uint64_t)r * sim->width + p, st, 0) % (uint32_t)V);
              nx.store(next, std::memory_order_relaxed);
            } else {
              next = nx.load(std::memory_order_relaxed);  // the prompt's own id
            }
            sim->step[r].store(p + 1, std::memory_order_relaxed);
            sim->tok.w[r].store(word((uint32_t)next, st), std::memory_order_release);
          }
        }
        R.end_ticket = ticket.fetch_add(1);
        R.t_end = now_ns();
      }
    }
  };
  std::vector<std::thread> th;
  for (int q = 0; q < g->num_queues; ++q) th.emplace_back(worker, q);
  for (auto& t : th) t.join();
  if (int code = failed.load()) return mpk_fail(code, fail_msg);
  return MPK_OK;
}
