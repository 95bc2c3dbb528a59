/*
 * mpk.h -- C ABI of the MI355X persistent decode megakernel.
 *
 * Sources (web pages on Mirage Persistent Kernel, "MPK"):
 *   P1  "Mirage Persistent Kernel: Fusing Multi-GPU LLM Inference into One
 *        Kernel Launch" (hysenlabs.com, English review)
 *   P3  gokawiil.com blog excerpt on MPK, section "Why MPK?", Figure 1
 *   P4  "Mirage Persistent Kernel：把 LLM 推理压进单个 GPU 内核" (hysenlabs.com, Chinese review)
 *   P5  "Mirage Persistent Kernel kompiliert LLM-Inferenz in einen Persistent
 *        Kernel" (hysenlabs.com, German review)
 *
 * The pages describe a Python API: a PersistentKernel object configured with
 * worker and scheduler counts (P1 "How MPK Works"; P5 "Betrieb und
 * Konfiguration"), tensors either attached from PyTorch or allocated by the
 * library (P1 "The API"; P4 "关键 API 与张量管理"), fused operators chained to
 * form a graph such as rmsnorm_linear_layer (P5 "Grenzen der README-Aussagen"),
 * then an explicit compile step followed by execution (P1 "Getting Started").
 * This header is that surface as plain C: a tensor table, an operator list,
 * mpk_build_graph (the task graph), mpk_compile (device resources) and
 * mpk_run_steps (one persistent launch).
 *
 * Conventions for every call:
 *  - Return value: an mpk_status_t (0 = MPK_OK).  On failure nothing is
 *    changed and mpk_last_error() describes the failure.  No call aborts the
 *    process; no C++ exception crosses this boundary.
 *  - Device pointers are plain addresses on the compile-time device (for
 *    example torch.Tensor.data_ptr()).  Tensors attached by the caller stay
 *    owned by the caller, must outlive the executable, and must not be
 *    written by the caller while a run is in flight.  Library-owned tensors
 *    and all runtime buffers are freed by mpk_destroy_exec.
 *  - Streams are hipStream_t values passed as void* (0 = the null stream).
 *    Runs are asynchronous on that stream; device-side failures are visible
 *    through mpk_get_status only after the stream has been synchronised.
 *  - Handles are not thread-safe: one thread at a time per handle.
 */
#ifndef MPK_H
#define MPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mpk_graph_s* mpk_graph_t; /* host task graph (library-owned) */
typedef struct mpk_exec_s* mpk_exec_t;   /* compiled, device-resident graph (library-owned) */

typedef enum {
  MPK_OK = 0,
  MPK_ERR_INVALID_ARG = -1,    /* NULL handle/pointer, bad enum, bad count */
  MPK_ERR_SHAPE = -2,          /* tensor dims disagree with the model or operator */
  MPK_ERR_DTYPE = -3,          /* tensor dtype not the one the operator takes */
  MPK_ERR_ALIGN = -4,          /* device pointer not 16-byte aligned */
  MPK_ERR_SPLIT = -5,          /* worker / scheduler counts break the CU rule */
  MPK_ERR_NOT_CORESIDENT = -6, /* the workers cannot all be resident at once */
  MPK_ERR_HIP = -7,            /* a HIP runtime call failed */
  MPK_ERR_DEVICE_TIMEOUT = -8, /* a dependency wait on the device exceeded spin_timeout_ns */
  MPK_ERR_ABORTED = -9,        /* the run was stopped through mpk_set_abort */
  MPK_ERR_STATE = -10,         /* call out of order (e.g. run before compile) */
  MPK_ERR_GRAPH = -11          /* operator graph malformed (producer order, sink, ...) */
} mpk_status_t;

typedef enum { MPK_BF16 = 1, MPK_F32 = 2, MPK_I32 = 3 } mpk_dtype_t;

/* Decoder shape and the two scalars the pages leave open (see the design
 * notes: RMSNorm eps inside the root, RoPE base). */
typedef struct {
  int32_t num_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;
  float rope_theta;
  int32_t max_batch; /* largest num_requests a graph may use */
  int32_t max_seq;   /* KV-cache capacity in positions */
} mpk_model_cfg;

/* Worker / scheduler split (P1 "How MPK Works": workers plus a quarter of the
 * schedulers must equal the number of SMs; restated here for CUs).
 *   MPK_SCHED_CORESIDENT: every worker workgroup carries one scheduler
 *     wavefront beside its eight worker wavefronts; num_workers must equal
 *     the CU count and num_schedulers must be 0 or num_workers.
 *   MPK_SCHED_DEDICATED: rule num_workers + num_schedulers / 4 == CU count,
 *     num_schedulers a multiple of 4 (four scheduler wavefronts on each
 *     scheduler CU).  Accepted by mpk_build_graph for the rule check only;
 *     mpk_compile rejects it with MPK_ERR_SPLIT (not implemented). */
enum { MPK_SCHED_CORESIDENT = 0, MPK_SCHED_DEDICATED = 1 };

typedef struct {
  int32_t num_cus;         /* CUs of the target device (0 = query device 0 at build time) */
  int32_t num_workers;     /* 0 = num_cus */
  int32_t num_schedulers;  /* see sched_mode */
  int32_t sched_mode;      /* MPK_SCHED_* */
  int32_t trace;           /* 1 = one trace record per executed task, with global ordering
                              tickets; 2 = the same without tickets (timestamps only, lighter) */
  int32_t reserved;
  uint64_t spin_timeout_ns; /* device watchdog per dependency wait; 0 = 2 s */
} mpk_launch_cfg;

/* One entry of the tensor table.  dev_ptr != NULL: attached caller memory
 * (P1 "The API": attach_input); dev_ptr == NULL: allocated, zeroed and owned
 * by the library at mpk_compile (new_tensor).  Row-major, dims[0] outermost,
 * unused dims = 1. */
typedef struct {
  const char* name; /* optional, copied; for error messages */
  int32_t dtype;    /* mpk_dtype_t */
  int32_t ndim;     /* 1..4 */
  int64_t dims[4];
  void* dev_ptr;
} mpk_tensor;

/* Operator kinds and their operands (tensor ids into the table; -1 = none).
 * B = num_requests, K = input width, N = output rows.
 *
 * MPK_OP_EMBED            in  {E[V,H] bf16}
 *                         out {x[B,H] f32}: x[r] = E[tokens[r][step[r]]].  Never
 *                         materialised: consumers gather the row themselves.
 * MPK_OP_RMSNORM_LINEAR   in  {x[B,K] f32, gain[K] bf16, W0[N0,K], W1[N1,K]|-1, W2[N2,K]|-1}
 *                         out {y[B,N0+N1+N2] f32}: y = [W0;W1;W2] . RMSNorm(x; gain)
 *                         (P1 "The API"; P5 "Grenzen der README-Aussagen").
 * MPK_OP_ATTENTION        in  {qkv[B,(nq+2nkv)d] f32, q_norm[d] bf16, k_norm[d] bf16,
 *                              kcache[B,nkv,S,d] bf16, vcache[B,nkv,S,d] bf16}
 *                         out {o[B,nq*d] f32}: per-head RMSNorm of q and k, RoPE at
 *                         step[r], K/V of position step[r] stored in the caches,
 *                         causal grouped-query attention over positions 0..step[r].
 * MPK_OP_LINEAR_RESIDUAL  in  {x[B,K] f32, W[N,K] bf16, residual[B,N] f32}
 *                         out {y[B,N] f32}: y = residual + W . x.
 * MPK_OP_RMSNORM_GATEUP   in  {x[B,K] f32, gain[K] bf16, Wg[F,K] bf16, Wu[F,K] bf16}
 *                         out {m[B,F] f32}: m = silu(Wg z) * (Wu z), z = RMSNorm(x; gain).
 * MPK_OP_LMHEAD_ARGMAX    in  {x[B,H] f32, gain[H] bf16, E[V,H] bf16}
 *                         out {logits[I,B,V] f32 | -1}: logits = E . RMSNorm(x; gain);
 *                         t = argmax (lowest index on ties); when step[r]+1 >=
 *                         prompt_len[r], tokens[r][step[r]+1] = t; then step[r] += 1
 *                         (P1 "How MPK Works": step advances after each iteration).
 *                         With a logits tensor, iteration i of a run stores its
 *                         logits at [i] (I >= iterations per run).
 * Every f32 tensor that is some operator's output must have exactly one
 * producer; an operator may only read outputs of earlier operators, or of
 * MPK_OP_LMHEAD_ARGMAX of the previous iteration (through tokens/step).  The
 * last operator must depend, directly or not, on every other. */
typedef enum {
  MPK_OP_EMBED = 1,
  MPK_OP_RMSNORM_LINEAR = 2,
  MPK_OP_ATTENTION = 3,
  MPK_OP_LINEAR_RESIDUAL = 4,
  MPK_OP_RMSNORM_GATEUP = 5,
  MPK_OP_LMHEAD_ARGMAX = 6
} mpk_op_kind;

typedef struct {
  int32_t kind;      /* mpk_op_kind */
  int32_t layer;     /* decoder layer (informational) */
  int32_t in[5];
  int32_t out[1];
  int32_t num_tiles; /* 0 = the builder's choice; else tiles (GEMV ops) */
} mpk_op;

/* Meta tensors (P1 "How MPK Works"; P4 "工作机制"): tokens[num_requests,
 * seq_length] i32 holding prompts and generated ids, step[num_requests] i32
 * (the position each request consumes next) and prompt_len[num_requests] i32.
 * All three are caller-owned device memory (attached); tokens and step are
 * advanced on the device. */
typedef struct {
  int32_t tokens, step, prompt_len; /* tensor ids */
  int32_t num_requests;
} mpk_meta;

/* Validate the tensors and operators, split each operator into tiles for the
 * worker count, derive dependency events and per-worker task queues, and
 * check the graph (producer order, a single sink, co-residency rule).  Pure
 * host work: no device call is made.  *out receives a new graph handle. */
int mpk_build_graph(const mpk_model_cfg* model, const mpk_launch_cfg* launch,
                    const mpk_tensor* tensors, int32_t n_tensors, const mpk_op* ops,
                    int32_t n_ops, const mpk_meta* meta, mpk_graph_t* out);

/* Allocate the library-owned tensors and runtime buffers on `device`, upload
 * the task, event and queue tables and the RoPE table, and check that all
 * workers can be resident together.  The graph stays owned by the caller. */
int mpk_compile(mpk_graph_t graph, int32_t device, mpk_exec_t* out);

/* Run `num_iterations` decode iterations as ONE persistent cooperative launch
 * on `stream` (preceded by one small kernel that clears the event counters).
 * Requires step[r] + num_iterations < tokens width and < max_seq for every r
 * (checked on the device values at the start of the run after a copy to the
 * host; returns MPK_ERR_SHAPE without launching otherwise). */
int mpk_run_steps(mpk_exec_t exec, int32_t num_iterations, void* stream);

/* The same task bodies launched one kernel per operator per iteration (the
 * comparison the pages make against per-operator kernels, P1 "Alternative").
 * Same tiles, same reduction order: results are bitwise equal to
 * mpk_run_steps. */
int mpk_run_steps_per_op(mpk_exec_t exec, int32_t num_iterations, void* stream);

/* After the stream of the last run is synchronised: device status code
 * (MPK_OK, MPK_ERR_DEVICE_TIMEOUT or MPK_ERR_ABORTED), the iteration and the
 * task id at which it was raised (-1 when OK).  Any pointer may be NULL. */
int mpk_get_status(mpk_exec_t exec, int32_t* code, int32_t* iteration, int32_t* task);

/* Ask a running persistent launch to stop (flag != 0) or clear the request
 * (flag == 0).  Uses an internal stream; waits for the flag write only. */
int mpk_set_abort(mpk_exec_t exec, int32_t flag);

/* Trace of the last run (launch cfg trace = 1 or 2): records of type
 * mpk_trace_record, one per (iteration, task), at index iteration * num_tasks
 * + task; every field of a record no task wrote is all ones (task = -1).
 * Under trace = 2 no tickets are taken: start_ticket stays all ones and
 * end_ticket is 0.  Tickets come from one device-wide atomic counter, so ticket order
 * is consistent with the order in which tasks became visible to each other. */
typedef struct {
  int32_t task;          /* task id, -1 if the slot was never written */
  int32_t iteration;
  uint32_t start_ticket; /* taken after all dependencies were acquired */
  uint32_t end_ticket;   /* taken before the completion signal */
  uint64_t t_start;      /* device constant clock (s_memrealtime) */
  uint64_t t_end;
  uint32_t hw_id;        /* HW_ID hardware register of the scheduler wave */
  uint32_t xcc_id;       /* XCC_ID hardware register */
  uint64_t t_ready;      /* all inputs present (GEMV: staged, weight stream about to be consumed;
                            attention and argmax: their words gathered); all ones when the
                            task had nothing to do (an attention split beyond the context) */
} mpk_trace_record;

int mpk_read_trace(mpk_exec_t exec, void* host_buf, size_t bytes, size_t* written);

/* Introspection of the built graph (host memory, valid until the graph is
 * destroyed).  Arrays follow the layout of mpk_task_info below. */
typedef struct {
  int32_t op;           /* operator index */
  int32_t tile;         /* tile index within the operator */
  int32_t worker;       /* worker (workgroup) whose queue holds the task */
  int32_t row0, nrows;  /* GEMV tiles: virtual rows; attention: request, kv head */
  int32_t split;        /* attention: KV split index; -1 otherwise */
  int32_t dep_event[3]; /* -1 = none */
  int32_t dep_count[3]; /* signals per iteration on that event */
  int32_t dep_prev[3];  /* 1 = wait for the previous iteration's signals */
  int32_t out_event;    /* event signalled when done (-1 = none) */
} mpk_task_info;

typedef struct {
  int32_t num_tasks, num_events, num_workers, max_queue;
  int32_t num_ops;
  int32_t sink_op;
  const mpk_task_info* tasks;
  const int32_t* event_count;  /* [num_events] signals per iteration */
  const int32_t* event_op;     /* [num_events] producing operator */
  const int32_t* queue_len;    /* [num_workers] */
  const int32_t* queues;       /* [num_workers][max_queue] task ids in execution order */
} mpk_graph_info;

int mpk_get_graph_info(mpk_graph_t graph, mpk_graph_info* info);

/* Run the graph's dependency protocol on host threads (one per worker), with
 * every task body replaced by a random sleep of up to jitter_us microseconds
 * (seeded).  Writes one mpk_trace_record per (iteration, task) into
 * host_trace (num_iterations * num_tasks records; times in ns).  Returns
 * MPK_ERR_DEVICE_TIMEOUT if any wait exceeds timeout_ms, which is how a
 * malformed graph shows up as a deadlock.  For tests of the builder. */
int mpk_simulate(mpk_graph_t graph, int32_t num_iterations, uint32_t seed, int32_t jitter_us,
                 int32_t timeout_ms, mpk_trace_record* host_trace);

/* Device address of tensor `tensor_id` (attached or library-owned). */
int mpk_get_tensor_ptr(mpk_exec_t exec, int32_t tensor_id, void** dev_ptr);

void mpk_destroy_exec(mpk_exec_t exec);
void mpk_destroy_graph(mpk_graph_t graph);

/* Message of the last failure on the calling thread (never NULL). */
const char* mpk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MPK_H */
