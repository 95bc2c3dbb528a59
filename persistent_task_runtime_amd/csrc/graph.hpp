// Host-side graph object shared by builder.cpp and runtime.hip.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "mpk_internal.h"

struct mpk_graph_s {
  mpk_model_cfg model{};
  mpk_launch_cfg launch{};
  mpk_meta meta{};
  std::vector<mpk_tensor> tensors;
  std::vector<std::string> names;
  std::vector<mpk_op> ops;

  // derived by the builder
  int rows = 1;          // rows per iteration: num_requests x rows_per_request
  int rpr = 1;           // rows per request (1: decode; > 1: batched prompt ingestion)
  int num_workers = 0;   // CUs that take tiles
  int num_queues = 0;    // CUs of the launch grid (workers + dedicated scheduler CUs)
  int sink = -1;
  std::vector<int> producer;        // per tensor: producing op, -1
  std::vector<int> embed_src;       // per tensor: E tensor id if output of an EMBED op, else -1
  std::vector<mpk_dev_op> dops;     // per op (pointers filled at compile)
  std::vector<int> op_first_task, op_ntasks;
  std::vector<mpk_dev_task> tasks;
  std::vector<mpk_task_info> info;
  std::vector<int> ev_count, ev_op;  // per event (an operator's output words): publishing tasks, operator
  int argmax_op = -1;                           // internal operator appended after the LM head
  std::vector<int> qlen;
  int max_queue = 0;
  std::vector<mpk_dev_qentry> queues;  // [num_queues][max_queue]
  std::vector<int32_t> queue_ids;      // [num_queues][max_queue] task ids (introspection)
};

// Thread-local error reporting shared by both translation units.
int mpk_fail(int code, const std::string& msg);
void mpk_clear_error();

// Attention split count for a graph (tasks per request and kv head).
int mpk_attn_splits(int num_workers, int batch, int nkv, int max_seq);
