/*
 * Internal tables shared by the host graph builder (builder.cpp) and the
 * device runtime (runtime.hip).  Plain structs, identical layout on both
 * sides.
 */
#ifndef MPK_INTERNAL_H
#define MPK_INTERNAL_H

#include <stdint.h>

#include "mpk.h"

#define MPK_NW 8                        /* worker wavefronts per workgroup */
#define MPK_THREADS (64 * (MPK_NW + 1)) /* + one scheduler wavefront */
#define MPK_SEG 4096                    /* columns of one weight block */
#define MPK_BU 8                        /* 16-byte-per-lane units per block */
#define MPK_MAX_DEPS 3
#define MPK_ATTN_SPLIT 64              /* positions per attention split (at full use) */
#define MPK_LDS_BYTES (96 * 1024)       /* dynamic LDS per workgroup (forces one per CU) */
#define MPK_MAX_BATCH 8

enum { MPK_TK_GEMV = 1, MPK_TK_ATTN = 2, MPK_TK_LMHEAD = 3, MPK_TK_ARGMAX = 4 };
enum { MPK_EPI_STORE = 0, MPK_EPI_RESID = 1, MPK_EPI_SILU = 2, MPK_EPI_ARGMAX = 3 };

/* One operator as the device sees it. */
typedef struct {
  int32_t kind;      /* MPK_TK_* */
  int32_t epi;       /* MPK_EPI_* for GEMV / LMHEAD */
  int32_t K;         /* input width */
  int32_t nseg;      /* ceil(K / MPK_SEG) */
  int32_t N0, N1, N2;/* rows of W0, W1, W2 */
  int32_t pairs;     /* 1: virtual rows interleave (gate, up) */
  int32_t x_embed;   /* 1: x[r] is E[tokens[r][step[r]]] */
  int32_t res_embed; /* 1: residual[r] is E[tokens[r][step[r]]] */
  int32_t has_norm;  /* 1: x is RMS-normalised with `gain` */
  int32_t event;     /* event this operator's tasks signal */
  int32_t n_out;     /* width of y (per request) */
  int32_t ntiles;    /* tasks of this operator */
  /* attention */
  int32_t nq, nkv, d, nsplit, S;
  /* worker_base: a GEMV whose input is an attention output runs its tiles on
   * workers [worker_base, W) (the attention tasks on [0, worker_base)).
   * lds_pre = 1: rows of one 4096-column group and one request, so while a
   * tile's inputs are awaited its wavefronts also stream assignment units of
   * the tile into LDS (as many as fit beyond the input's landing zone) */
  int32_t worker_base;
  int32_t lds_pre;
  /* ksplit > 1 (batch-8 linear + residual with K = ksplit * 4096): tile t is
   * row group t / ksplit over columns [4096 k, 4096 k + 4096), k = its split
   * (t % ksplit); splits k < ksplit - 1 publish their partial sums as
   * stamped words in pll [ksplit - 1][B][n_out], split ksplit - 1 adds them
   * (in split order) to its own and applies the epilogue.  0: no split. */
  int32_t ksplit;
  const float* x;         /* plain input (a graph input tensor), or NULL */
  const uint64_t* xll;    /* stamped input words (output of another operator), or NULL */
  const uint16_t* gain;
  const uint16_t* W0;
  const uint16_t* W1;
  const uint16_t* W2;
  const float* resid;     /* plain residual input, or NULL */
  const uint64_t* rll;    /* stamped residual words, or NULL */
  float* y;               /* plain output (tensor attached by the caller), or NULL */
  uint64_t* yll;          /* stamped output words */
  /* Packed words (one per element: value rounded to 24 bits, 8-bit stamp)
   * beside the stamped ones, for the input gathers of GEMV tasks: xpk, when
   * set, holds the same input as xll; ypk receives the outputs also written
   * to yll.  NULL when unused. */
  const uint32_t* xpk;
  uint32_t* ypk;
  const uint16_t* E; /* embedding rows for x_embed / res_embed */
  const uint16_t* qn;
  const uint16_t* kn;
  uint16_t* kc;
  uint16_t* vc;
  uint64_t* pll;     /* stamped attention split partials [B][nkv][nsplit][G][d + 2];
                        LM head: per tile and request (value, row);
                        split-K linear: partial sums [ksplit - 1][B][n_out] */
  float* logits;     /* LM head: optional [iters][B][V] */
  int64_t logits_iters;
} mpk_dev_op;

/* One task (a tile of an operator).  A task carries no dependency fields: it
 * waits for exactly the stamped words its body reads. */
typedef struct {
  int32_t kind;
  int32_t op;
  int32_t tile;
  int32_t worker;
  int32_t row0, nrows; /* GEMV: virtual rows; ATTN: request, kv head */
  int32_t split;       /* ATTN split */
  int32_t pad;
} mpk_dev_task;

/* Per queue entry: the task id. */
typedef struct {
  int32_t task;
} mpk_dev_qentry;

typedef struct {
  int32_t code;      /* mpk_status_t of the device side */
  int32_t iteration;
  int32_t task;
  int32_t abort_req; /* host-written stop request */
} mpk_dev_status;

typedef struct {
  const mpk_dev_task* tasks;
  const mpk_dev_op* ops;
  const mpk_dev_qentry* queues; /* [num_workers][qstride] */
  const int32_t* qlen;          /* [num_workers] */
  uint64_t* tok_ll;              /* [B] stamped next token, written by the argmax task */
  int32_t* tokens;
  int32_t* step;
  const int32_t* prompt_len;
  const float* rope_cos;        /* [max_seq][d/2] */
  const float* rope_sin;
  mpk_dev_status* status;       /* code / iteration / task of the run */
  int32_t* abort_req;           /* the executable's stop request (mpk_set_abort) */
  mpk_trace_record* trace;      /* NULL = off */
  int32_t trace_tickets;        /* 1: also take global tickets (slower) */
  uint32_t* ticket_ctr;
  uint64_t timeout_ticks;       /* s_memrealtime ticks (100 MHz) */
  int32_t qstride;
  int32_t n_iter;
  int32_t n_tasks;
  int32_t B;                    /* rows per iteration */
  int32_t rpr;                  /* rows per request: row b is position pos0[b / rpr] + rpr s + b % rpr */
  int32_t tokens_width;
  int32_t rope_half;
  float rms_eps;
  int32_t vocab;
  int32_t max_seq;
  int32_t* pos0;                /* [requests] step[r] at launch, written by the run's first kernel */
  uint32_t iter_base;           /* stamp of iteration s is iter_base + s + 1 */
} mpk_kparams;

#endif
