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
  MPK_ERR_ALIGN = -4,          /* device pointer not 16-byte aligned (int32 tensors: 4-byte) */
  MPK_ERR_SPLIT = -5,          /* worker / scheduler counts break the CU rule */
  MPK_ERR_NOT_CORESIDENT = -6, /* the workers cannot all be resident at once */
  MPK_ERR_HIP = -7,            /* a HIP runtime call failed */
  MPK_ERR_DEVICE_TIMEOUT = -8, /* a dependency wait on the device exceeded spin_timeout_ns */
  MPK_ERR_ABORTED = -9,        /* the run was stopped through mpk_set_abort */
  MPK_ERR_STATE = -10,         /* call out of order (e.g. run before compile) */
  MPK_ERR_GRAPH = -11          /* operator graph malformed (producer order, sink, ...) */
} mpk_status_t;

typedef enum { MPK_BF16 = 1, MPK_F32 = 2, MPK_I32 = 3 } mpk_dtype_t;

/* Decoder shape (head_dim 64 or 128: the attention kernel is specialised
 * for these; MPK_ERR_SHAPE otherwise) and two scalars the pages leave open:
 * the RMSNorm epsilon (added inside the square root) and the RoPE base. */
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
 *     num_schedulers a multiple of 4 (four scheduler wavefronts per
 *     scheduler CU).  Operator tiles go to the num_workers worker CUs only;
 *     the num_schedulers / 4 scheduler CUs hold no tile: the first of them
 *     runs each iteration's argmax / step-advance task, the others idle.
 *     The launch still covers every CU (the pages' split of the chip). */
enum { MPK_SCHED_CORESIDENT = 0, MPK_SCHED_DEDICATED = 1 };

/* Launch parameters.  Three knobs a launch description could carry are fixed
 * by the kernels instead, because the task bodies are written for them: the
 * workgroup is 576 threads (eight worker wavefronts and one scheduler
 * wavefront, one workgroup per CU through 156 KB of dynamic LDS), attention
 * splits hold 64 positions at full use (the split count follows the KV
 * capacity, mpk_graph_info shows the tasks), and timing jitter exists only in
 * the host model of the protocol (mpk_sim_cfg.jitter_us). */
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
 * B = rows = num_requests x rows_per_request (see mpk_meta), K = input width,
 * N = output rows.
 *
 * MPK_OP_EMBED            in  {E[V,H] bf16}
 *                         out {x[B,H] f32}: x[r] = E[tokens[r][step[r]]].  Never
 *                         materialised: consumers gather the row themselves.
 * MPK_OP_RMSNORM_LINEAR   in  {x[B,K] f32, gain[K] bf16, W0[N0,K], W1[N1,K]|-1, W2[N2,K]|-1}
 *                         out {y[B,N0+N1+N2] f32}: y = [W0;W1;W2] . RMSNorm(x; gain)
 *                         (P1 "The API"; P5 "Grenzen der README-Aussagen").
 * MPK_OP_ATTENTION        in  {qkv[B,(nq+2nkv)d] f32, q_norm[d] bf16, k_norm[d] bf16,
 *                              kcache[num_requests,nkv,S,d] bf16, vcache[same] bf16}
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
 * advanced on the device.
 *
 * rows_per_request R (0 or 1: decode): with R > 1 every iteration takes R
 * consecutive prompt positions of each request at once (batched prompt
 * ingestion, the step before decoding the pages' 39-token prompt of P3
 * Figure 1): rows r R .. r R + R - 1 are positions step[r] .. step[r] + R - 1
 * of request r, attention of row r R + i covers positions 0 .. step[r] + i,
 * every row writes its K/V row, and step[r] advances by R per iteration.
 * No token is generated: a run of n iterations needs step[r] + R n <=
 * prompt_len[r] - 1 for every request (MPK_ERR_SHAPE otherwise), so the
 * position after every consumed one is still a prompt position. */
typedef struct {
  int32_t tokens, step, prompt_len; /* tensor ids */
  int32_t num_requests;
  int32_t rows_per_request;         /* R; rows B = num_requests x R must be 1, 2 or 8 */
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
 * on `stream`, preceded by one small kernel (mpk_begin_run) that clears the
 * status word and checks the meta tensors on the device.  Asynchronous: the
 * call makes no host-device round trip and returns once both kernels are
 * queued (the first traced run of a length allocates its trace buffer).
 * Returns MPK_ERR_SHAPE without launching when num_iterations alone exceeds
 * the tokens width or max_seq, or a logits tensor holds fewer iterations.
 * The device check (same rule as mpk_check_run): for every request r,
 * 0 <= step[r], step[r] + num_iterations < tokens width, step[r] +
 * num_iterations <= max_seq, and every token id the run reads from tokens
 * (position step[r], and the prompt positions up to step[r] + num_iterations
 * - 1 below prompt_len[r]) is in [0, vocab).  On failure no iteration runs:
 * after synchronisation mpk_get_status reports MPK_ERR_SHAPE with
 * iteration -1 and the request index as task, and tokens, step and the KV
 * caches are unchanged. */
int mpk_run_steps(mpk_exec_t exec, int32_t num_iterations, void* stream);

/* mpk_run_steps for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same kernels, same results; the call allocates nothing and makes no
 * host-device round trip.  The run scratch (the stamped words between tasks,
 * attention split partials, LM-head tile maxima, token words, status word and
 * positions: mpk_compile sizes it per graph) lives in one static device array
 * of the library per GPU, 64 MiB, held until the process ends; mpk_compile
 * prepares the executable's table into it.  Every call on a GPU shares that
 * GPU's array and leaves its contents behind: runs that overlap on one GPU
 * race (one allocation-free run per GPU at a time).  The packed input words
 * (8-bit stamps) in it are cleared first, by a fill kernel on `stream`,
 * whenever another executable used the array last or their stamps could
 * repeat (no allocation either).  Stop requests stay per
 * executable.  Returns MPK_ERR_SHAPE (nothing launched) when the graph's run
 * scratch exceeds 64 MiB (e.g. batch 1 of the 8B shape at 32768 positions fits;
 * larger batches may not), MPK_ERR_INVALID_ARG for a traced graph (the trace
 * buffer would need an allocation), and otherwise what mpk_run_steps
 * returns; mpk_get_status reports this run's status. */
int mpk_run_steps_static(mpk_exec_t exec, int32_t num_iterations, void* stream);

/* The same task bodies launched one kernel per operator per iteration (the
 * comparison the pages make against per-operator kernels, P1 "Alternative").
 * Same tiles, same reduction order: results are bitwise equal to
 * mpk_run_steps. */
int mpk_run_steps_per_op(mpk_exec_t exec, int32_t num_iterations, void* stream);

/* After the stream of the last run is synchronised: device status code
 * (MPK_OK, MPK_ERR_DEVICE_TIMEOUT, MPK_ERR_ABORTED, or MPK_ERR_SHAPE from
 * the start-of-run check), the iteration and the task id at which it was
 * raised (-1 when OK; for MPK_ERR_SHAPE iteration -1 and the request index).
 * Any pointer may be NULL.  Synchronous (one small device-to-host copy). */
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
  /* Operator-level data edges (introspection; the device waits on the
   * stamped words each task body reads, not on these): an "event" is one
   * operator's output words, published by `count` tasks per iteration. */
  int32_t dep_event[3]; /* producing operator's event, -1 = none */
  int32_t dep_count[3]; /* tasks that publish that operator's words */
  int32_t dep_prev[3];  /* 1 = the previous iteration's words (the token word of the argmax task) */
  int32_t out_event;    /* this operator's event */
} mpk_task_info;

typedef struct {
  int32_t num_tasks, num_events, num_workers, max_queue;
  int32_t num_ops;
  int32_t sink_op;
  int32_t num_queues;          /* CUs of the launch grid: num_workers + dedicated scheduler CUs */
  const mpk_task_info* tasks;
  const int32_t* event_count;  /* [num_events] publishing tasks per iteration */
  const int32_t* event_op;     /* [num_events] producing operator */
  const int32_t* queue_len;    /* [num_queues] */
  const int32_t* queues;       /* [num_queues][max_queue] task ids in execution order */
} mpk_graph_info;

int mpk_get_graph_info(mpk_graph_t graph, mpk_graph_info* info);

/* Host model of the device's dependency protocol (tests of the builder and
 * of the protocol; no device call).  One host thread per CU queue walks the
 * queue's tasks, iteration by iteration, with each task body replaced by a
 * seeded random sleep of up to jitter_us microseconds.  As on the device, a
 * task waits for exactly the stamped 64-bit words it reads (payload + stamp
 * iter_base + s + 1 of iteration s), the attention split owning the
 * position gathers the other splits' partial words, the owner stores the
 * K/V row of the position before it publishes, and the argmax task writes
 * tokens / step and the token word the next iteration's embedding waits for
 * (P1 "How MPK Works").  The word buffers, K/V rows and meta tensors live in
 * a simulation state that persists across mpk_simulate calls, like device
 * buffers across launches.  Checks: every accepted word carries the payload
 * its producer wrote in this iteration of this call (a stale word that
 * passes the stamp check is reported), every K/V row read was written (or
 * pre-filled) before, token words agree with tokens.  Planted faults show
 * that the checks fire. */
typedef struct mpk_sim_s* mpk_sim_t;

enum {
  MPK_SIM_NO_FAULT = 0,
  MPK_SIM_FAULT_KV_AFTER_PUBLISH = 1, /* the owner split publishes before storing the K/V row */
  MPK_SIM_FAULT_SKIP_WAIT = 2,        /* attention reads its q/k/v words without waiting (QKV tiles late) */
  MPK_SIM_FAULT_DROP_PUBLISH = 3      /* LM-head tile 0 never publishes (a wait must time out) */
};

typedef struct {
  int32_t num_iterations;
  uint32_t iter_base;  /* stamp of iteration s is iter_base + s + 1; the caller advances it by
                          num_iterations per call, as the library does per launch */
  uint32_t seed;
  int32_t jitter_us;
  int32_t timeout_ms;  /* per wait; a wait past it ends the call with MPK_ERR_DEVICE_TIMEOUT */
  int32_t fault;       /* MPK_SIM_* */
} mpk_sim_cfg;

/* Simulation state for `graph` from host copies of step[B], tokens[B][width]
 * and prompt_len[B]; K/V rows of positions < kv_filled count as pre-filled.
 * The graph must outlive the state. */
int mpk_sim_create(mpk_graph_t graph, const int32_t* step, const int32_t* tokens,
                   const int32_t* prompt_len, int32_t kv_filled, mpk_sim_t* out);

/* One simulated launch of cfg->num_iterations iterations.  Writes one
 * mpk_trace_record per (iteration, task) into host_trace (times in ns since
 * the call's start; hw_id = the queue; start_ticket is taken once every word
 * the task reads is present, before it writes any; attention splits with
 * nothing to do keep start_ticket all ones).  Returns MPK_OK,
 * MPK_ERR_SHAPE (the start-of-run rule of mpk_run_steps),
 * MPK_ERR_DEVICE_TIMEOUT (a wait exceeded timeout_ms) or MPK_ERR_GRAPH (a
 * protocol check failed; mpk_last_error says which). */
int mpk_simulate(mpk_sim_t sim, const mpk_sim_cfg* cfg, mpk_trace_record* host_trace);

/* Current step[B] and tokens[B][width] of the simulation (either may be NULL). */
int mpk_sim_read_meta(mpk_sim_t sim, int32_t* step, int32_t* tokens);

void mpk_sim_destroy(mpk_sim_t sim);

/* The start-of-run rule of mpk_run_steps applied on the host to host copies
 * of the meta tensors (step[B], tokens[B][width], prompt_len[B] with the
 * graph's shapes), for callers that keep them: MPK_OK, or MPK_ERR_SHAPE
 * naming the first request and position that break it.  Pure host work. */
int mpk_check_run(mpk_graph_t graph, const int32_t* step, const int32_t* tokens,
                  const int32_t* prompt_len, int32_t num_iterations);

/* Device address of tensor `tensor_id` (attached or library-owned). */
int mpk_get_tensor_ptr(mpk_exec_t exec, int32_t tensor_id, void** dev_ptr);

void mpk_destroy_exec(mpk_exec_t exec);
void mpk_destroy_graph(mpk_graph_t graph);

/* Measured HBM read ceiling (a measurement utility, not part of the decode
 * path).  The decode step is bound by streaming its weights once per
 * iteration (P3 "Why MPK?", Figure 1: weight bytes over memory bandwidth);
 * this reads `bytes` at device address `src` once, asynchronously on
 * `stream`, with the load form of the weight streams (16-byte nontemporal
 * loads, 8 wavefronts per workgroup, 16 loads in flight per lane), on
 * `workgroups` workgroups striding over 128 KiB units.  The
 * caller times it (events on the same stream) to get the stream-read rate
 * that a roofline fraction can also be stated against.  `sink` is one
 * caller-owned device word that is written only if the XOR of all the data
 * read equals a fixed constant (it keeps the loads live).  Errors:
 * MPK_ERR_INVALID_ARG (NULL pointer, workgroups < 1), MPK_ERR_SHAPE (bytes
 * not a positive multiple of 131072), MPK_ERR_ALIGN (src not 16-byte or sink
 * not 4-byte aligned), MPK_ERR_HIP (launch failure). */
int mpk_stream_read(const void* src, uint64_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

/* Message of the last failure on the calling thread (never NULL). */
const char* mpk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MPK_H */
