// Device runtime of the persistent decode megakernel (gfx950 / CDNA4) and
// the host side of the C ABI (compile, run, status, trace).
//
// Sources (web pages on Mirage Persistent Kernel, "MPK"):
//   P1 "Mirage Persistent Kernel: Fusing Multi-GPU LLM Inference into One
//      Kernel Launch" (hysenlabs.com, English review)
//   P3 gokawiil.com blog excerpt on MPK, section "Why MPK?" and Figure 1
//   P4 "Mirage Persistent Kernel：把 LLM 推理压进单个 GPU 内核" (hysenlabs.com, Chinese review)
//
// One cooperative launch keeps one workgroup resident on every CU for the
// whole decode loop (P1 "How MPK Works"; P4 "工作机制").  A workgroup is eight
// worker wavefronts plus one scheduler wavefront and walks the CU's static
// task queue.  Tasks hand values to each other as stamped 64-bit words
// (payload + iteration stamp, see st_ll): a task waits for exactly the words
// it reads, and a producer publishes each output word as soon as it is
// computed - there is no per-task completion flag, fence or store drain on
// the path between two tasks.
//
// Weights stream through an eight-deep register ring per wavefront
// (16-byte nontemporal loads).  A task issues its first eight units before
// it waits for its inputs, so the weights of the next operator are already
// in flight while the current one's outputs are still being produced: the
// "load the next layer while computing this one" overlap of P3 "Why MPK?",
// done per CU with the queue known at compile time.
//
// The iteration's last task picks the argmax token, writes it into tokens,
// advances step (P1 "How MPK Works") and publishes the token word the next
// iteration's embedding reads wait for.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "graph.hpp"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

#define DEV __device__ __forceinline__
#define CAS __attribute__((address_space(4)))

// Read-only tables are read through the constant address space so that
// uniform reads become scalar loads (they must not wait on vector-memory
// counters, which also count the weight stream's loads).
typedef const CAS mpk_dev_task ctask;
typedef const CAS mpk_dev_op cop;
typedef const CAS mpk_dev_qentry cqent;
typedef float __attribute__((address_space(1))) gfloat;
typedef uint16_t __attribute__((address_space(1))) gu16;
typedef int32_t __attribute__((address_space(1))) gi32;

// Wave-uniform copies (the compiler cannot always prove uniformity of
// loop-carried scheduling state; uniform values live in SGPRs and their
// table reads become scalar loads).
DEV int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
DEV T* unip(T* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
DEV ctask* unip(ctask* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (ctask*)(((uint64_t)hi << 32) | lo);
}
DEV cop* unip(cop* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (cop*)(((uint64_t)hi << 32) | lo);
}

DEV ctask* tasks_of(const mpk_kparams& P) { return (ctask*)(const void*)P.tasks; }
DEV cop* ops_of(const mpk_kparams& P) { return (cop*)(const void*)P.ops; }

// Plain global stores/loads (not flat): a flat access would also hold the LDS
// counter and stall the ring's LDS reads until it completes.
DEV void gst(float* p, float v) { *(gfloat*)(void*)p = v; }
DEV void gst16(uint16_t* p, uint16_t v) { *(gu16*)(void*)p = v; }
DEV float gld(const float* p) { return *(const gfloat*)(const void*)p; }
DEV int gldi(const int32_t* p) { return *(const gi32*)(const void*)p; }
DEV uint16_t gld16(const uint16_t* p) { return *(const gu16*)(const void*)p; }
DEV uint32_t gld32(const uint32_t* p) { return *(const __attribute__((address_space(1))) uint32_t*)(const void*)p; }
template <typename T>
DEV T gldv(const void* p) { return *(const T __attribute__((address_space(1)))*)p; }

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
DEV float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (NaN stays NaN): the hardware
// conversion v_cvt_pk_bf16_f32, two values per instruction in f2bf2 (low
// half a, high half b)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
DEV uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
DEV uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

template <int CTRL>
DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes of a wavefront in a fixed order; the result is uniform.
DEV float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

DEV float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

DEV uint64_t clock_now() { return __builtin_amdgcn_s_memrealtime(); }

DEV uint32_t hwreg_hw_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(v));
  return v;
}
DEV uint32_t hwreg_xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}

// LDS pointer from an LDS byte address (no generic-pointer conversion)
DEV lptr_t lds_ptr(uint32_t a) { return (lptr_t)(uintptr_t)a; }

// LDS traffic inside the weight stream is written in asm, each block waiting
// for its own reads (with a memory clobber): it pins each unit's x reads and
// FMAs between the ring's refills, which keeps the compiler from reordering
// the stream into a shape whose waits drain the whole ring.
DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lptr_t)(void*)p; }

// Volatile LDS words (control flags, counters, wait slots) through an LDS
// pointer: through a generic pointer a volatile access stays a FLAT access,
// which also counts as a vector-memory operation, and the compiler follows
// each with a full vmcnt drain (the weight ring included).
typedef volatile __attribute__((address_space(3))) int lds_vi;
DEV lds_vi* lvi(const void* smem, int off) { return (lds_vi*)lds_ptr(lds_addr(smem) + (uint32_t)off); }

DEV u32x4 lds_read_u32x4(uint32_t a) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
DEV void lds_write_u32x4(uint32_t a, u32x4 v) { asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory"); }
DEV void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Two float4 at byte address a and a + 1024.  The outputs are early-clobber:
// the first read may land before the second has read its address operand, so
// neither output may share a register with the address.
DEV void lds_read_2f4(uint32_t a, f32x4& x0, f32x4& x1) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x0), "=&v"(x1)
               : "v"(a)
               : "memory");
}

// Two float4 at byte address a and a + 16 (early-clobber outputs, see
// lds_read_2f4).
DEV void lds_read_2f4_near(uint32_t a, f32x4& x0, f32x4& x1) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x0), "=&v"(x1)
               : "v"(a)
               : "memory");
}

DEV float lds_read_f32(uint32_t a) {
  float v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}

// Wait until at most N vector-memory operations of this wavefront are in
// flight (opaque to the compiler's own wait insertion).
template <int N>
DEV void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// s_waitcnt vmcnt(0) that the compiler's wait insertion sees (the asm form
// above is opaque to it): afterwards it knows nothing is in flight, so its
// own waits on a register ring stay exact instead of falling back to full
// drains when stores or atomics of earlier code might still be pending.
// Also used as a precaution between loads of different kinds (plain,
// nontemporal, device-scope): the compiler's count-based waits assume that
// all of a wavefront's loads return in issue order; the code does not rely
// on that across kinds where the fence costs nothing.
DEV void vm_drain_known() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt 0, expcnt 7, lgkmcnt 15
// The same with N vector-memory operations left in flight (the N issued
// last: loads complete in issue order).
template <int N>
DEV void vm_wait_known() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}


// Device-scope ("sc1") accesses.  Every value one task hands to another task
// on another CU (stamped words, K/V rows, tokens, step) is written with
// device-scope stores and read with device-scope loads: these go to the point
// of coherence shared by all XCDs, so no L2 write-back or invalidate is needed
// to pass data between CUs.  Data that is not itself stamped (a K/V row) is
// stored and its stores waited for (s_waitcnt vmcnt(0)) before the stamped
// word that orders its readers is published.
DEV float ld_dev(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV int ld_devi(const int32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV uint32_t ld_devu(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void st_devi(int32_t* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void st_devu(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Cache-policy bits of a load (global->LDS DMA, buffer load): sc1 makes it
// device scope (coherent with device-scope stores of other CUs on any XCD),
// nt marks data read once.  Streams of data read once reach a higher HBM
// rate with nt (about 6.8 against 6.0 TB/s in a 256-CU streaming test of
// 8 KB steps), also together with sc1.
#define CPOL_NT 2
#define CPOL_SC1 16

// all vector-memory operations of this wavefront complete (the scheduler
// wavefront issues no weight loads, so this waits only for its own stores)
DEV void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// LDS layout (bytes)
//   [0, 2048)                 control words, reductions, 1/rms, tile argmax,
//                             positions and tokens of the iteration
//   [LDS_OUT, +4096)          attention: split partial / output, new K/V row
//   [LDS_X, +XS)              staged activations x (or attention scratch)
//   [RES, +2048)              staged residual rows of the tile
// x is staged permuted so each 16-byte LDS read is lane-contiguous:
//   column k -> unit u = k / 512, lane l = (k % 512) / 8, half h = (k % 8) / 4
//   offset (floats) = u * 512 + h * 256 + l * 4 + (k % 4)
// ---------------------------------------------------------------------------
#define LDS_CTL 0
#define LDS_RED 256                      // [16][8] floats: per-wave partials
#define LDS_INV (LDS_RED + 16 * 8 * 4)   // [8] floats (spare)
#define LDS_BEST (LDS_INV + 64)          // [8 waves][8] (float) + [8][8] (int)
#define LDS_POS (LDS_BEST + 512)         // [8] int: position of request r in the current iteration
#define LDS_TOK (LDS_POS + 32)           // [8] int: token of request r in the current iteration
#define LDS_SYNCED (LDS_TOK + 32)        // int: a task of this iteration has received inputs of it
#define LDS_POS0 (LDS_SYNCED + 32)       // [8] int: position of request r in the launch's first iteration
// control words: [0] stop flag, [8, 40) wait-round slots, [40] row claims
#define LDS_OUT 2048
#define LDS_OUT_FLOATS 1024
#define LDS_X (LDS_OUT + LDS_OUT_FLOATS * 4)
#define LDS_RES_BYTES 2048

template <int NB>
struct Lay {
  static constexpr int XS = 49152 * NB;             // staged x bytes
  static constexpr int RES = LDS_X + XS;            // residual rows
  // attention uses [LDS_X, TOTAL) as scratch (position-group partials and
  // the gathered split partials); one workgroup per CU, so the whole LDS
  static constexpr int TOTAL = 156 * 1024;
};
// batch 8: linear tasks stage x per 4096-column pass (gemv8_body)
template <>
struct Lay<8> {
  static constexpr int XS = 0;
  static constexpr int RES = LDS_X;
  static constexpr int TOTAL = 156 * 1024;
};
static_assert(Lay<1>::RES + LDS_RES_BYTES <= Lay<1>::TOTAL, "LDS budget");
static_assert(Lay<2>::RES + LDS_RES_BYTES <= Lay<2>::TOTAL, "LDS budget");

DEV void lds_write_f32(uint32_t a, float v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(v) : "memory");
}
DEV void lds_write_f32x2(uint32_t a, float2 v) {
  asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(v) : "memory");
}
DEV void lds_write_f32x4(uint32_t a, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(v) : "memory");
}

DEV int xperm(int k) { return (k & ~511) + ((k & 4) << 6) + (((k & 511) >> 3) << 2) + (k & 3); }

// Position of row b in the current iteration (written into LDS_POS by the
// scheduler wavefront at the start of each iteration).
DEV int cur_pos(const char* smem, int b) {
  return __builtin_amdgcn_readfirstlane(lvi(smem, LDS_POS)[b]);
}

// Scheduler wavefront, once per launch: the positions of the launch's first
// iteration (written by mpk_begin_run ahead of the launch) into LDS_POS0.
DEV void load_positions(const mpk_kparams& P, char* smem, int lane) {
  if (lane < P.B / P.rpr) lvi(smem, LDS_POS0)[lane] = ld_devi(P.pos0 + lane);
}

// Scheduler wavefront: positions of iteration s into LDS_POS.  Row b is
// position pos0[r] + rpr s + i of request r = b / rpr, i = b % rpr (rpr = 1:
// one position per request and iteration).
DEV void set_positions(const mpk_kparams& P, char* smem, int s, int lane) {
  if (lane == 0)
    for (int b = 0; b < P.B; ++b)
      lvi(smem, LDS_POS)[b] = lvi(smem, LDS_POS0)[b / P.rpr] + P.rpr * s + b % P.rpr;
}

// Per-lane forms: the position of request b (b may differ between lanes), and
// the token id it consumes in this iteration (resolved into LDS_TOK by
// resolve_tokens before a task reads embedding rows).
DEV int cur_pos_v(const char* smem, int b) { return lvi(smem, LDS_POS)[b]; }
DEV int cur_token_v(const char* smem, int b) { return lvi(smem, LDS_TOK)[b]; }

// ---------------------------------------------------------------------------
// Stamped words.  Every value one task hands to another (an activation
// element, an attention split's partial, an LM-head tile's maximum, the next
// token) travels as one 64-bit word: the 32-bit payload in the low half and
// the stamp of the iteration that wrote it in the high half.  A 64-bit
// device-scope store is single-copy atomic, so a reader that sees the
// expected stamp also sees the payload: consumers spin on exactly the words
// they read, and producers publish with plain device-scope stores - no
// completion flag, no store drain, no fence between them.
// The stamp of iteration s is iter_base + s + 1, with iter_base taken from a
// process-wide counter that grows by the iteration count of every launch, so
// words left by an earlier launch (an aborted one, or another executable
// whose memory was reused) never carry a current stamp.  Buffers are zeroed
// (stamp 0) before an executable is returned.
// ---------------------------------------------------------------------------
DEV uint32_t stamp_of(const mpk_kparams& P, int s) { return P.iter_base + (uint32_t)s + 1u; }
DEV void st_ll(uint64_t* p, float v, uint32_t st) {
  __hip_atomic_store(p, ((uint64_t)st << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_lli(uint64_t* p, int v, uint32_t st) {
  __hip_atomic_store(p, ((uint64_t)st << 32) | (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint64_t ld_ll(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV bool ll_ok(uint64_t w, uint32_t st) { return (uint32_t)(w >> 32) == st; }
DEV float ll_f(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Packed words: one 32-bit word per element, the fp32 value rounded to
// nearest (ties to even) at 15 mantissa bits in the upper 24 bits and an
// 8-bit stamp in the low byte, so an input gather moves half the bytes.  A
// 32-bit device-scope store is single-copy atomic like the 64-bit one.  The
// 8-bit stamp of iteration stamp st is st mod 255 + 1 (never 0: zeroed
// buffers hold no current word).  Within a run it is enough: a consumer
// reads its words every iteration, so a word it reads holds this
// iteration's value or the previous one's (it saw that one, and every word
// is rewritten once per iteration after all of the previous iteration's
// reads of it), and consecutive stamps differ.  Across runs the host
// clears the packed buffers before a run whenever a stale word could be 255
// or more stamps old (see prepare_run).
DEV uint32_t stamp8(uint32_t st) { return st % 255u + 1u; }
DEV uint32_t pk_word(float v, uint32_t s8) {
  const uint32_t u = __float_as_uint(v);
  return ((u + 0x7fu + ((u >> 8) & 1u)) & 0xffffff00u) | s8;
}
DEV float pk_f(uint32_t w) { return __uint_as_float(w & 0xffffff00u); }
DEV void st_pk(uint32_t* p, float v, uint32_t s8) {
  __hip_atomic_store(p, pk_word(v, s8), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint32_t ld_pk(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier over LDS data only: this wavefront's LDS operations are
// complete first, its vector-memory loads need not be (the barrier that
// __syncthreads compiles to also drains vmcnt, which would wait out a weight
// ring just issued).
DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup-wide wait.  Every thread of the workgroup calls wait_round once
// per round with `pending` = this thread still misses words; the result is
// uniform: 0 = nobody waits any more, 1 = poll again, -1 = stop (watchdog
// expired, stop requested by the host, or an error recorded by another
// workgroup).  Thread 0 runs the watchdog; the first workgroup to fail
// records the status.
// The watchdog's clock starts when a wait first polls again (t0 = 0 until
// then): a wait satisfied at first look reads no clock (s_memrealtime is a
// scalar-memory operation, and every later lgkmcnt wait of the wavefront,
// LDS waits included, would wait for it).
struct Waiter {
  uint64_t t0;
  int rounds;
};

DEV Waiter waiter_start() { return Waiter{0, 0}; }

DEV int wait_round(const mpk_kparams& P, Waiter& Wt, bool pending, int s, int task_id, char* smem, int tid) {
  lds_vi* ctl = lvi(smem, LDS_CTL);
  const int wave = tid >> 6;
  ++Wt.rounds;
  // (not on the first round: a wait satisfied at first look costs no status reads)
  if (tid == 0 && (Wt.rounds & 7) == 2) {
    int mine = 0;
    const int code = __hip_atomic_load(&P.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int abort_req = __hip_atomic_load(P.abort_req, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (abort_req) mine = MPK_ERR_ABORTED;
    else if (Wt.t0 != 0 && clock_now() - Wt.t0 > P.timeout_ticks) mine = MPK_ERR_DEVICE_TIMEOUT;
    if (mine) {
      int expected = 0;
      if (__hip_atomic_compare_exchange_strong(&P.status->code, &expected, mine, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        __hip_atomic_store(&P.status->iteration, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&P.status->task, task_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (mine || code) ctl[0] = 1;
  }
  // per-wave "still waiting" bits, double-buffered by round parity so a
  // wavefront entering the next round never overwrites a slot still read
  lds_vi* slot = ctl + 8 + (Wt.rounds & 1) * 16;
  const bool any_wave = __ballot(pending) != 0;
  if ((tid & 63) == 0) slot[wave] = any_wave ? 1 : 0;
  lds_barrier();
  int any = 0;
  for (int w = 0; w <= MPK_NW; ++w) any |= slot[w];
  if (ctl[0]) return -1;
  if (!any) return 0;
  if (tid == 0 && Wt.t0 == 0) Wt.t0 = clock_now();
  __builtin_amdgcn_s_sleep(1);
  return 1;
}

// A wavefront's own watchdog for per-wavefront polling (the rules of
// wait_round: a stop requested by the host, an error recorded by another
// workgroup, or this wait past the timeout, whose clock starts at the first
// repeated poll).  Called once per repeated poll; true = the workgroup stops
// (its stop flag is set).
DEV bool wave_watch(const mpk_kparams& P, Waiter& Wt, int s, int task_id, char* smem, int lane) {
  lds_vi* ctl = lvi(smem, LDS_CTL);
  ++Wt.rounds;
  if (Wt.t0 == 0) {
    Wt.t0 = clock_now();
  } else if ((Wt.rounds & 7) == 0) {
    const int code = __hip_atomic_load(&P.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int abort_req = __hip_atomic_load(P.abort_req, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int mine = abort_req ? MPK_ERR_ABORTED
                               : (clock_now() - Wt.t0 > P.timeout_ticks ? MPK_ERR_DEVICE_TIMEOUT : 0);
    if (mine && lane == 0) {
      int expected = 0;
      if (__hip_atomic_compare_exchange_strong(&P.status->code, &expected, mine, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        __hip_atomic_store(&P.status->iteration, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&P.status->task, task_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if ((mine || code) && lane == 0) ctl[0] = 1;
  }
  return ctl[0] != 0;
}

// Trace hook: the task's inputs are all present.  With tickets on, the
// ticket is taken (and returned) before any output of the task is stored.
DEV void mark_ready(const mpk_kparams& P, int s, int task_id, int tid) {
  if (!P.trace) return;
  if (tid == MPK_NW * 64) {
    mpk_trace_record& Rr = P.trace[(int64_t)s * P.n_tasks + task_id];
    Rr.t_ready = clock_now();
    if (P.trace_tickets)
      Rr.start_ticket = __hip_atomic_fetch_add(P.ticket_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (P.trace_tickets) __syncthreads();
}

// Tokens of this iteration into LDS_TOK.  In the first iteration of a launch
// the token at the request's position is in `tokens` (prompt, or written by
// the previous launch); later iterations take the previous iteration's
// argmax task word (which also carries teacher-forced prompt tokens).
DEV int resolve_tokens(const mpk_kparams& P, char* smem, int tid, int s, int task_id, Waiter& Wt) {
  lds_vi* tok = lvi(smem, LDS_TOK);
  bool need = false;
  if (tid < P.B) {
    if (s == 0) {
      tok[tid] = ld_devi(P.tokens + (int64_t)(tid / P.rpr) * P.tokens_width + cur_pos_v(smem, tid));
    } else {
      need = true;
    }
  }
  const uint32_t want = stamp_of(P, s - 1);
  for (;;) {
    if (need) {
      const uint64_t w = ld_ll(P.tok_ll + tid);
      if (ll_ok(w, want)) tok[tid] = (int)(uint32_t)w, need = false;
    }
    const int rc = wait_round(P, Wt, need, s, task_id, smem, tid);
    if (rc <= 0) {
      if (rc == 0 && tid < P.B) {
        // every id a run consumes is checked by mpk_begin_run before the
        // run starts (a failed check stops the run); the clamp only keeps an
        // id that the caller changed during the run inside the table
        const int t = tok[tid];
        tok[tid] = t < 0 ? 0 : (t >= P.vocab ? P.vocab - 1 : t);
      }
      __syncthreads();
      return rc;
    }
  }
}

// Collective gather of n stamped words src[0, n) into LDS dst[0, n) (their
// 32-bit payloads).  CH words per thread are in flight per round; each
// wavefront polls its own words (wave_watch), the workgroup meets once at
// the end.
template <int CH>
DEV int gather_ll(const mpk_kparams& P, const uint64_t* src, int n, uint32_t* dst, uint32_t st, Waiter& Wt, int s,
                  int task_id, char* smem, int tid) {
  const int lane = tid & 63;
  bool stop = false;
  for (int base = 0; base < n && !stop; base += CH * MPK_THREADS) {
    uint32_t need = 0;
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (base + tid + j * MPK_THREADS < n) need |= 1u << j;
    for (;;) {
      uint64_t v[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j)
        if ((need >> j) & 1u) v[j] = ld_ll(src + base + tid + j * MPK_THREADS);
#pragma unroll
      for (int j = 0; j < CH; ++j)
        if (((need >> j) & 1u) && ll_ok(v[j], st)) {
          dst[base + tid + j * MPK_THREADS] = (uint32_t)v[j];
          need &= ~(1u << j);
        }
      if (__ballot(need != 0) == 0) break;
      if (wave_watch(P, Wt, s, task_id, smem, lane)) {
        stop = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  lds_barrier();
  return *lvi(smem, LDS_CTL) ? -1 : 0;
}

// Stamped words src[0, n) (n even, src 16 bytes aligned) into LDS at byte
// address dst, 8 bytes per word, by global->LDS DMA (device scope): 1 KB
// chunks (whole chunks are written: ceil(8 n / 1 KB) KB must be free at dst),
// chunk k taken by wavefront k % 9.  Each wavefront checks the stamps of its
// own chunks and fetches the stale ones again, so all chunks are in flight at
// once and nothing is held in registers.  Every thread of the workgroup
// calls it; returns -1 on stop.
DEV int gather_ll_dma(const mpk_kparams& P, const uint64_t* src, int n, uint32_t dst, uint32_t st, Waiter& Wt,
                      int s, int task_id, char* smem, int tid) {
  constexpr int NWAVES = MPK_THREADS / 64, MAXC = 16;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nch = (n * 8 + 1023) >> 10, npiece = n >> 1;
  uint32_t need = 0;  // bit k: chunk wave + 9 k is still to fetch
#pragma unroll
  for (int k = 0; k < MAXC; ++k)
    if (wave + NWAVES * k < nch) need |= 1u << k;
  while (need) {
#pragma unroll
    for (int k = 0; k < MAXC; ++k)
      if ((need >> k) & 1u) {
        const int pc = min((wave + NWAVES * k) * 64 + lane, npiece - 1);  // lanes past the end repeat the last piece
        __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(src + 2 * pc),
                                         lds_ptr(dst + (uint32_t)(wave + NWAVES * k) * 1024u), 16, 0,
                                         CPOL_SC1);
      }
    vm_drain_known();
    uint32_t stale = 0;
#pragma unroll
    for (int k = 0; k < MAXC; ++k)
      if ((need >> k) & 1u) {
        const int piece = (wave + NWAVES * k) * 64 + lane;
        const u32x4 v = lds_read_u32x4(dst + (uint32_t)(wave + NWAVES * k) * 1024u + lane * 16u);
        if (__ballot(piece < npiece && (v.y != st || v.w != st)) != 0) stale |= 1u << k;
      }
    need = stale;
    if (!need) break;
    if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  lds_barrier();
  return *lvi(smem, LDS_CTL) ? -1 : 0;
}

// ---------------------------------------------------------------------------
// weight units (GEMV and LM-head tiles)
//   A tile covers virtual rows [row0, row0 + nrows).  Rows go to the worker
//   wavefronts in assignment units of `a` rows (a = 2 for gate/up pairs):
//   wave w takes units w, w + 8, w + 16, ...  A row is read as ceil(K/512)
//   units of 512 bf16 (1 KB, 16 bytes per lane); a wavefront's sequence is
//   its rows in order, each row's units in order, padded with repeat reads
//   to a whole number of groups of 8 units (at least one group).
//   Units travel in an eight-deep register ring per wavefront: eight
//   16-byte loads in flight, each refilled as the unit eight places earlier
//   is consumed.  A task's first eight are issued before its inputs are
//   awaited.
// ---------------------------------------------------------------------------
#define MPK_RING 8  // units in flight per wavefront

DEV int units_per_row(cop& D) { return (D.K + 511) >> 9; }

DEV int wave_units(cop& D, ctask& T, int wave) {
  const int a = D.pairs ? 2 : 1;
  const int au = T.nrows / a;
  const int mine = au > wave ? (au - wave + MPK_NW - 1) / MPK_NW : 0;
  return mine * a * units_per_row(D);
}

DEV int padded_units(int n) { return n <= MPK_RING ? MPK_RING : ((n + MPK_RING - 1) / MPK_RING) * MPK_RING; }

// Walks one task's units for one wavefront.  Everything is copied out of the
// descriptors into wave-uniform scalars, so stepping performs no memory read.
struct Cursor {
  const uint16_t* W0;
  const uint16_t* W1;
  const uint16_t* W2;
  const uint16_t* row;  // current row (lane offset not included)
  int N0, N1, K, pairs, row0, a, upr;
  int au, rr, u;  // assignment unit (a rows) of the tile, row within it, unit within row
  int i, n;       // next unit index, real units
};

DEV void cursor_row(Cursor& C, int wave) {
  // Select among loaded pointer values (not among field addresses: a
  // variable-index field access would keep the cursor in scratch memory).
  const uint16_t* w0 = unip(C.W0);
  const uint16_t* w1 = unip(C.W1);
  const uint16_t* w2 = unip(C.W2);
  const int vrow = C.row0 + C.au * C.a + C.rr;
  const uint16_t* base;
  int r;
  if (C.pairs) {
    base = (vrow & 1) ? w1 : w0;
    r = vrow >> 1;
  } else if (vrow < C.N0) {
    base = w0;
    r = vrow;
  } else if (vrow - C.N0 < C.N1) {
    base = w1;
    r = vrow - C.N0;
  } else {
    base = w2;
    r = vrow - C.N0 - C.N1;
  }
  C.row = unip(base + (int64_t)r * C.K);
}

DEV void cursor_init(Cursor& C, cop& D, ctask& T, int wave) {
  C.W0 = unip(D.W0), C.W1 = unip(D.W1), C.W2 = unip(D.W2);
  C.N0 = uni(D.N0), C.N1 = uni(D.N1), C.K = uni(D.K), C.pairs = uni(D.pairs);
  C.row0 = uni(T.row0);
  C.a = C.pairs ? 2 : 1;
  C.upr = uni(units_per_row(D));
  C.au = wave, C.rr = 0, C.u = 0, C.i = 0;
  C.n = uni(wave_units(D, T, wave));
  if (C.n > 0) cursor_row(C, wave);
  else C.row = unip(C.W0);  // padding only: re-read the first unit of W0
}

// Global address of the cursor's current unit for this lane (padding units
// re-read the last real unit; lanes past the end of a row re-read its start).
DEV gptr_t cursor_addr(const Cursor& C, int lane) {
  const int kleft = C.K - C.u * 512;
  const int col = lane * 8 < kleft ? C.u * 512 + lane * 8 : 0;
  return (gptr_t)(const void*)(C.row + col);
}

// Point the cursor at unit u of row rr of assignment unit au; the caller
// bounds the walk from there (no padding).
DEV void cursor_goto(Cursor& C, int au, int rr, int u, int wave) {
  C.au = au, C.rr = rr, C.u = u;
  C.i = 0, C.n = 1 << 30;
  cursor_row(C, wave);
}

DEV void cursor_step(Cursor& C, int wave) {
  C.i = uni(C.i + 1);
  if (C.i >= C.n) return;  // padding: stay on the last real unit
  C.u = uni(C.u + 1);
  if (C.u == C.upr) {
    C.u = 0;
    C.rr = uni(C.rr + 1);
    if (C.rr == C.a) {
      C.rr = 0;
      C.au = uni(C.au + MPK_NW);
    }
    cursor_row(C, wave);
  }
}

// Stage the GEMV input into LDS: x (gathered from its producers' packed or
// stamped words, an embedding row, or a plain input tensor), times the RMSNorm gain
// when the operator normalises, and the tile's residual rows; inv receives
// 1 / rms per request (1 without a norm) in every thread.  Every thread of
// the workgroup takes part.  The calling wavefront's first weight loads
// (ring_ops vector-memory operations: 8, 16 or 24) go out while the inputs
// are awaited: issue_ring() issues the register ring's first group
// (MPK_RING loads) with the first poll round; issue_step(i), i >= 1, issues
// PF_STEP more (the rows of an LDS assignment unit), one step per later
// round, the rest after the inputs arrive.  Returns -1 on stop.
//
// Why in steps: every request a CU sends waits behind the requests already
// queued to memory, its own and its XCD's.  Issuing the whole prefetch at
// once (up to 192 KB per CU) made the polls of the tasks that start last
// (their inputs all present at the first round) wait behind it; in steps
// of 4 KB per wavefront the last inputs of an operator are staged about
// 1 us earlier (2 to 8 KB steps measured the same).
#define PF_STEP 4
#define XCH 8    // input words per thread per gather pass (register path)
#define XGMAX 4  // chunks per wavefront whose gains and sums of squares stay in registers (DMA path)

// DMA staging: the landing zone beyond the residual rows (1 KB per chunk:
// 128 stamped words, or 256 packed words when the input has them) and, with
// a norm, the gains of each chunk's columns (2 bytes per column), which go
// into the staged-x area beyond x when they fit there (they are read before
// x is complete) and after the landing zone otherwise.
DEV int chunk_cols(cop& D) { return D.xpk ? 256 : 128; }
template <int NB>
DEV int n_chunks(cop& D) {
  return (NB * D.K + chunk_cols(D) - 1) / chunk_cols(D);
}
template <int NB>
DEV bool gains_in_xs(cop& D) {
  const int Kpad = ((D.K + 511) / 512) * 512;
  return LDS_X + NB * Kpad * 4 + n_chunks<NB>(D) * chunk_cols(D) * 2 <= Lay<NB>::RES;
}
// bytes the DMA staging occupies from the landing zone's start
template <int NB>
DEV int land_bytes(cop& D) {
  const int nchunk = n_chunks<NB>(D);
  return nchunk * 1024 + (D.has_norm && !gains_in_xs<NB>(D) ? nchunk * chunk_cols(D) * 2 : 0);
}

// Chunks in which the task's x arrives by global->LDS DMA, or 0 when it
// takes the register path.
template <int NB>
DEV int dma_chunks(cop& D) {
  const int land = Lay<NB>::RES + LDS_RES_BYTES;
  const int nchunk = n_chunks<NB>(D);
  const bool ok = D.xll && (D.K % chunk_cols(D)) == 0 && land + land_bytes<NB>(D) <= Lay<NB>::TOTAL &&
                  nchunk <= 32 * MPK_NW && (!D.has_norm || nchunk <= XGMAX * MPK_NW);
  return ok ? nchunk : 0;
}

DEV uint32_t lds_read_u32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
template <int NB, class Ring, class Step>
DEV int stage_inputs(const mpk_kparams& P, cop& D, ctask& T, char* smem, int tid, int s, int task_id,
                     float (&inv)[NB], int ring_ops, Ring&& issue_ring, Step&& issue_step) {
  float* xs = reinterpret_cast<float*>(smem + LDS_X);
  float* res = reinterpret_cast<float*>(smem + Lay<NB>::RES);
  float* red = reinterpret_cast<float*>(smem + LDS_RED);
  const int K = D.K;
  const int Kpad = ((K + 511) / 512) * 512;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool worker = tid < MPK_NW * 64;
  const uint32_t st = stamp_of(P, s);
  Waiter Wt = waiter_start();
  if (D.x_embed || D.res_embed) {
    const int rc = resolve_tokens(P, smem, tid, s, task_id, Wt);
    if (rc) return rc;
  }
  const int NE = NB * K;
  // Stamped x words that fit the free LDS beyond the residual rows come by
  // global->LDS DMA, 1 KB chunks (128 words, 2 per lane) per wavefront
  // instruction: wavefront w owns chunks w + 8 i, all in flight at once, and
  // a chunk with a stale word is fetched again in the wavefront's next round.
  // Each wavefront polls on its own (one barrier at the end): a round then
  // lasts one chunk's round trip, not the slowest of the workgroup's.  The first
  // round is issued ahead of the weight loads, so it is not queued behind
  // them.  Each wavefront applies the gain to its chunks as they arrive and
  // publishes its RMS partial sums once all of them are in; the sums run in
  // a fixed order whatever the arrival order (deterministic).
  const int land = Lay<NB>::RES + LDS_RES_BYTES;
  const int nchunk = n_chunks<NB>(D);
  const int nres = D.epi == MPK_EPI_RESID ? NB * T.nrows : 0;
  // (the DMA path leaves the residual rows to the scheduler wavefront)
  const bool dma = dma_chunks<NB>(D) > 0 && nres <= 64;
  // zero padding columns of x (K not a multiple of 512); no gather writes them
  for (int i = K + (worker ? tid : Kpad); i < Kpad; i += MPK_NW * 64)
#pragma unroll
    for (int b = 0; b < NB; ++b) xs[b * Kpad + xperm(i)] = 0.f;
  // Residual element rt of the tile (request rb, row rrow).  With the DMA
  // path the scheduler wavefront's lanes take them: it streams no weights,
  // so waiting for a residual word (its count of loads in flight unknown to
  // the compiler: a full drain) waits behind no weight ring.
  const bool rsched = dma;
  const int rt = rsched ? tid - MPK_NW * 64 : tid;
  bool need_r = false;
  float rv = 0.f;
  int rb = 0, rrow = 0;
  if (rt >= 0 && rt < nres) {
    rb = rt / T.nrows;
    rrow = T.row0 + rt - rb * T.nrows;
    if (D.res_embed) rv = bf16f(gld16(D.E + (int64_t)cur_token_v(smem, rb) * D.n_out + rrow));
    else if (D.rll) need_r = true;
    else rv = gld(D.resid + (int64_t)rb * D.n_out + rrow);
  }
  if (dma) {
    const uint32_t lb = lds_addr(smem);
    uint32_t need = 0;  // chunks c = wave + 8 i of this wavefront, bit i
    if (worker)
      for (int i = 0; wave + MPK_NW * i < nchunk; ++i) need |= 1u << i;
    need = __builtin_amdgcn_readfirstlane(need);
    const uint32_t mine = need;
    // A chunk is 1 KB: 128 stamped words (2 per lane), or with packed
    // words 256 of them (4 per lane).
    const bool pk = D.xpk != nullptr;
    const int cc = pk ? 256 : 128;  // columns per chunk
    const uint32_t s8 = stamp8(st);
    // Gains of this lane's columns in chunks i < XGMAX (packed bf16 pairs:
    // one, or two with packed words at +256 bytes), by DMA into LDS after the
    // landing zone: as loads into registers the compiler would wait for them
    // with a full drain (the ring behind them has a path-dependent length).
    const uint32_t gla = lb + (gains_in_xs<NB>(D) ? LDS_X + NB * Kpad * 4 : land + nchunk * 1024);
    uint32_t gp[XGMAX], gq[XGMAX];
    float sq[XGMAX];  // a chunk's sum of squares (the RMS partials, in chunk order)
#pragma unroll
    for (int i = 0; i < XGMAX; ++i) {
      const int c = wave + MPK_NW * i;
      const int k = (c * cc) % K;
      if (D.has_norm && ((mine >> i) & 1u)) {
        const uint32_t gd = gla + c * cc * 2;
        if (pk) {
          __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(D.gain + k + lane * 4), lds_ptr(gd), 4, 0, 0);
          __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(D.gain + k + lane * 4 + 2), lds_ptr(gd + 256), 4, 0,
                                           0);
        } else {
          __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(D.gain + k + lane * 2), lds_ptr(gd), 4, 0, 0);
        }
      }
      gp[i] = 0u;
      gq[i] = 0u;
      sq[i] = 0.f;
    }
    // Chunks of this wavefront in LDS (mask m): take each whose words are
    // all current.
    auto take = [&](uint32_t m) {
      for (; m; m &= m - 1) {
        const int i = __builtin_ctz(m), c = wave + MPK_NW * i;
        const u32x4 w = lds_read_u32x4(lb + land + c * 1024 + lane * 16);
        const bool stale = pk ? ((w.x & 0xffu) != s8) | ((w.y & 0xffu) != s8) | ((w.z & 0xffu) != s8) |
                                    ((w.w & 0xffu) != s8)
                              : (w.y != st) | (w.w != st);
        if (__ballot(stale) == 0) {
          need &= ~(1u << i);
          const int e = c * cc + lane * (pk ? 4 : 2);
          const int b = e / K, k = e - b * K;
          const uint32_t xa = lb + LDS_X + (uint32_t)(b * Kpad + xperm(k)) * 4u;
          // (LDS stores written in asm: after a global->LDS DMA the
          // compiler puts a full vmcnt drain before its own LDS stores)
          if (pk) {
            f32x4 x = f32x4{pk_f(w.x), pk_f(w.y), pk_f(w.z), pk_f(w.w)};
            if (D.has_norm) {
              // i < XGMAX here (checked with dma)
              const float q = fmaf(x.x, x.x, x.y * x.y) + fmaf(x.z, x.z, x.w * x.w);
#pragma unroll
              for (int j = 0; j < XGMAX; ++j)
                if (j == i)
                  sq[j] = q, x = f32x4{x.x * bf16lo(gp[j]), x.y * bf16hi(gp[j]), x.z * bf16lo(gq[j]),
                                       x.w * bf16hi(gq[j])};
            }
            lds_write_f32x4(xa, x);
          } else {
            float2 x{__uint_as_float(w.x), __uint_as_float(w.z)};
            if (D.has_norm) {
              const float q = fmaf(x.x, x.x, x.y * x.y);
#pragma unroll
              for (int j = 0; j < XGMAX; ++j)
                if (j == i) sq[j] = q, x = float2{x.x * bf16lo(gp[j]), x.y * bf16hi(gp[j])};
            }
            lds_write_f32x2(xa, x);
          }
        }
      }
      need = __builtin_amdgcn_readfirstlane(need);
    };
    // Every round fetches all of the wavefront's chunks still missing.
    // (Probing one missing chunk per round and fetching the rest once it is
    // current measured 0.6 % slower: the last inputs then take an extra
    // round.)
    const int nsteps = worker ? 1 + (ring_ops - MPK_RING) / PF_STEP : 0;
    int step = 0;
    bool first = true, published = false;
    if (worker) {
      for (;;) {
        if (first) {
          // stale landing data must not pass the stamp check before the
          // first round's DMA has landed: clear the landing stamps first
          for (uint32_t m = need; m; m &= m - 1)
            lds_write_u32x4(lb + land + (wave + MPK_NW * __builtin_ctz(m)) * 1024 + lane * 16, u32x4{0u, 0u, 0u, 0u});
          lds_wait();
        }
        const uint32_t fetch = need;
        for (uint32_t m = fetch; m; m &= m - 1) {
          const int c = wave + MPK_NW * __builtin_ctz(m);
          const void* src = pk ? (const void*)(D.xpk + c * 256 + lane * 4) : (const void*)(D.xll + c * 128 + lane * 2);
          __builtin_amdgcn_global_load_lds((gptr_t)src, lds_ptr(lb + land + c * 1024), 16, 0, CPOL_SC1);
        }
        // the next prefetch step goes out behind this round's words; wait
        // for the words only (loads complete in issue order)
        if (first) {
          issue_ring();
          step = 1;
          vm_wait_known<MPK_RING>();
        } else if (step < nsteps) {
          issue_step(step);
          ++step;
          vm_wait_known<PF_STEP>();
        } else {
          vm_drain_known();
        }
        if (first && D.has_norm) {
          // the gains are in LDS
#pragma unroll
          for (int i = 0; i < XGMAX; ++i) {
            if ((mine >> i) & 1u) {
              const uint32_t gd = gla + (wave + MPK_NW * i) * cc * 2 + lane * 4;
              gp[i] = lds_read_u32(gd);
              if (pk) gq[i] = lds_read_u32(gd + 256);
            }
          }
        }
        take(fetch);
        if (D.has_norm && need == 0 && !published) {
          published = true;
          // this wavefront's chunks are all in: its RMS partials, in chunk order
          float ss[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) ss[b] = 0.f;
#pragma unroll
          for (int i = 0; i < XGMAX; ++i) {
            if ((mine >> i) & 1u) {
              const int b = (wave + MPK_NW * i) * cc / K;
#pragma unroll
              for (int bb = 0; bb < NB; ++bb) ss[bb] += bb == b ? sq[i] : 0.f;
            }
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const float t = wave_sum(ss[b]);
            if (lane == 0) lds_write_f32(lb + LDS_RED + (uint32_t)(wave * 8 + b) * 4u, t);
          }
        }
        first = false;
        if (need == 0) break;
        if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
        __builtin_amdgcn_s_sleep(1);
      }
      // the prefetch steps not issued during the wait
      for (step = max(step, 1); step < nsteps; ++step) issue_step(step);
    } else {
      // the scheduler wavefront: the tile's residual rows (its loads share
      // no register with a worker's, so no wait of theirs covers them)
      if (rt >= 0 && rt < nres && !D.rll) res[rt] = rv;
      for (;;) {
        if (need_r) {
          const uint64_t wr = ld_ll(D.rll + (int64_t)rb * D.n_out + rrow);
          if (ll_ok(wr, st)) res[rt] = ll_f(wr), need_r = false;
        }
        if (__ballot(need_r) == 0) break;
        if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    // every wavefront's inputs are in, or the workgroup stops
    lds_barrier();
    if (*lvi(smem, LDS_CTL)) return -1;
  } else {
    if (worker) issue_ring();
    for (int i = 1; worker && i < 1 + (ring_ops - MPK_RING) / PF_STEP; ++i) issue_step(i);
    // RMSNorm gains of this thread's columns (k = tid + 512 j), loaded before
    // the inputs are awaited when K fits one gather pass
    const bool gains_early = K <= XCH * MPK_NW * 64;
    float gk[XCH];
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int k = tid + j * MPK_NW * 64;
      gk[j] = D.has_norm && gains_early && worker && k < K ? bf16f(gld16(D.gain + k)) : 0.f;
    }
    float ss[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) ss[b] = 0.f;
    // x element e = b * K + k, per thread e = base + tid + 512 j.  Raw values
    // land in LDS as they arrive; the RMS sums and the gain are applied
    // afterwards in a fixed order (deterministic).
    for (int base = 0; base < NE; base += XCH * MPK_NW * 64) {
      uint32_t need = 0;
#pragma unroll
      for (int j = 0; j < XCH; ++j)
        if (worker && base + tid + j * MPK_NW * 64 < NE) need |= 1u << j;
      if (D.xll) {
        // packed words when the input has them (the same values the DMA
        // path of a smaller batch reads)
        const bool pk = D.xpk != nullptr;
        const uint32_t s8 = stamp8(st);
        for (;;) {
          uint64_t v[XCH];
#pragma unroll
          for (int j = 0; j < XCH; ++j) {
            const int e = base + tid + j * MPK_NW * 64;
            if ((need >> j) & 1u) v[j] = pk ? (uint64_t)ld_pk(D.xpk + e) : ld_ll(D.xll + e);
          }
          uint64_t wr = 0;
          if (need_r) wr = ld_ll(D.rll + (int64_t)rb * D.n_out + rrow);
          // (request, column) of element j, stepped from j = 0 without divisions
          int eb = (base + tid) / K, ek = base + tid - eb * K;
#pragma unroll
          for (int j = 0; j < XCH; ++j) {
            const bool cur = pk ? ((uint32_t)v[j] & 0xffu) == s8 : ll_ok(v[j], st);
            if (((need >> j) & 1u) && cur) {
              xs[eb * Kpad + xperm(ek)] = pk ? pk_f((uint32_t)v[j]) : ll_f(v[j]);
              need &= ~(1u << j);
            }
            ek += MPK_NW * 64;
            while (ek >= K) ek -= K, ++eb;
          }
          if (need_r && ll_ok(wr, st)) rv = ll_f(wr), need_r = false;
          const int rc = wait_round(P, Wt, need != 0 || need_r, s, task_id, smem, tid);
          if (rc < 0) return rc;
          if (rc == 0) break;
        }
      } else {
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
          if ((need >> j) & 1u) {
            const int e = base + tid + j * MPK_NW * 64;
            const int b = e / K, k = e - b * K;
            xs[b * Kpad + xperm(k)] =
                D.x_embed ? bf16f(gld16(D.E + (int64_t)cur_token_v(smem, b) * K + k)) : gld(D.x + e);
          }
        }
      }
    }
    // the residual element may have been a plain load issued before the
    // device-scope polls: see vm_drain_known
    vm_drain_known();
    // RMS sums and gain, each thread over its own columns in a fixed order
    if (D.has_norm && gains_early) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float xr[XCH];
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
          const int k = tid + j * MPK_NW * 64;
          xr[j] = worker && k < K ? xs[b * Kpad + xperm(k)] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
          const int k = tid + j * MPK_NW * 64;
          ss[b] = fmaf(xr[j], xr[j], ss[b]);
          if (worker && k < K) xs[b * Kpad + xperm(k)] = xr[j] * gk[j];
        }
      }
    } else if (D.has_norm) {
      for (int e = worker ? tid : NE; e < NE; e += MPK_NW * 64) {
        const int b = e / K, k = e - b * K;
        float* px = xs + b * Kpad + xperm(k);
        const float x = *px;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) ss[bb] = fmaf(bb == b ? x : 0.f, x, ss[bb]);
        *px = x * bf16f(gld16(D.gain + k));
      }
    }
    // a residual not gathered with x (x did not come from stamped words)
    if (D.rll && !D.xll) {
      for (;;) {
        if (need_r) {
          const uint64_t wr = ld_ll(D.rll + (int64_t)rb * D.n_out + rrow);
          if (ll_ok(wr, st)) rv = ll_f(wr), need_r = false;
        }
        const int rc = wait_round(P, Wt, need_r, s, task_id, smem, tid);
        if (rc < 0) return rc;
        if (rc == 0) break;
      }
    }
    if (rt >= 0 && rt < nres) res[rt] = rv;
    if (D.has_norm && worker) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float t = wave_sum(ss[b]);
        if (lane == 0) red[wave * 8 + b] = t;
      }
    }
    __syncthreads();
  }
  // every wavefront's partials are in (the last barrier above, or the final
  // wait round): each thread forms 1 / rms itself, in the same order
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (D.has_norm) {
      float t = 0.f;
      for (int w = 0; w < MPK_NW; ++w) t += lds_read_f32(lds_addr(smem) + LDS_RED + (uint32_t)(w * 8 + b) * 4u);
      inv[b] = 1.0f / sqrtf(t / (float)K + P.rms_eps);
    } else {
      inv[b] = 1.0f;
    }
  }
  if (tid == 0) *lvi(smem, LDS_SYNCED) = 1;
  return 0;
}

DEV float silu(float g) { return g / (1.0f + expf(-g)); }

DEV void unpack8(const u32x4 w, float (&f)[8]) {
  f[0] = bf16lo(w.x), f[1] = bf16hi(w.x), f[2] = bf16lo(w.y), f[3] = bf16hi(w.y);
  f[4] = bf16lo(w.z), f[5] = bf16hi(w.z), f[6] = bf16lo(w.w), f[7] = bf16hi(w.w);
}

// Publish one output element: its stamped word for consumer tasks, and the
// plain value when the tensor is attached by the caller.
DEV void put_out(cop& D, int64_t i, float v, uint32_t st, uint32_t s8) {
  st_ll(D.yll + i, v, st);
  if (D.ypk) st_pk(D.ypk + i, v, s8);
  if (D.y) gst(D.y + i, v);
}

// ---------------------------------------------------------------------------
// GEMV-type task: rmsnorm_linear (EPI_STORE), linear + residual (EPI_RESID),
// rmsnorm + gate/up + SiLU-mul (EPI_SILU), final norm + LM head + tile argmax
// (EPI_ARGMAX).  Each wavefront publishes its rows' output words after its
// stream (see row_done).  Returns -1 on stop.
// ---------------------------------------------------------------------------
// LDS address of a logit of the LM-head tile: after the staged x of the NB
// requests.
DEV uint32_t lds_logits(uint32_t lb, int nb, cop& D, ctask& T, int b, int lrow) {
  const int Kpad = ((D.K + 511) / 512) * 512;
  return lb + LDS_X + (uint32_t)(nb * Kpad + b * T.nrows + lrow) * 4u;
}

template <int NB>
struct GemvState {
  float acc[NB], gate[NB], best_v[NB];
  int best_i[NB];
  int u, rr, kk;  // unit within the row, row within the assignment unit, static assignment count
};

template <int NB>
DEV void unit_fma(const u32x4 w, uint32_t xaddr, int Kpad, float (&acc)[NB]) {
  const float wf[8] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                       bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    f32x4 x0, x1;
    lds_read_2f4(xaddr + (uint32_t)(b * Kpad) * 4u, x0, x1);
    float sacc = acc[b];
    sacc = fmaf(wf[0], x0.x, sacc);
    sacc = fmaf(wf[1], x0.y, sacc);
    sacc = fmaf(wf[2], x0.z, sacc);
    sacc = fmaf(wf[3], x0.w, sacc);
    sacc = fmaf(wf[4], x1.x, sacc);
    sacc = fmaf(wf[5], x1.y, sacc);
    sacc = fmaf(wf[6], x1.z, sacc);
    sacc = fmaf(wf[7], x1.w, sacc);
    acc[b] = sacc;
  }
  // The unit is consumed here, before the next load into its register is
  // issued: without this the compiler sinks the FMAs below the refills and
  // must then wait for every load in flight to copy the old values out.
#pragma unroll
  for (int b = 0; b < NB; ++b) asm volatile("" : "+v"(acc[b])::"memory");
}

// A row of the tile is complete: reduce and apply the epilogue into LDS
// (outputs, or logits and the running maximum for the LM head).  Nothing is
// stored to memory inside the weight stream: a store pending among the
// stream's loads would make every wait on them a full drain.
template <int NB>
DEV void row_done(cop& D, ctask& T, GemvState<NB>& G, uint32_t lb, const float (&inv)[NB], int a, int au,
                  int lane) {
  const int EPI = D.epi;
  const int lrow = au * a + G.rr;  // row within the tile
  const int vrow = T.row0 + lrow;
  const uint32_t ob = lb + LDS_OUT;
  const int n_out_tile = D.pairs ? T.nrows / 2 : T.nrows;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float sum = wave_sum(G.acc[b]);
    G.acc[b] = 0.f;
    // LDS traffic inside the weight stream stays in asm (see lds_addr)
    if (EPI == MPK_EPI_STORE) {
      if (lane == 0) lds_write_f32(ob + (uint32_t)(b * n_out_tile + lrow) * 4u, sum * inv[b]);
    } else if (EPI == MPK_EPI_RESID) {
      const float rv = lds_read_f32(lb + Lay<NB>::RES + (uint32_t)(b * T.nrows + lrow) * 4u);
      if (lane == 0) lds_write_f32(ob + (uint32_t)(b * n_out_tile + lrow) * 4u, rv + sum);
    } else if (EPI == MPK_EPI_SILU) {
      if (G.rr == 0) {
        G.gate[b] = sum * inv[b];
      } else if (lane == 0) {
        lds_write_f32(ob + (uint32_t)(b * n_out_tile + (lrow >> 1)) * 4u, silu(G.gate[b]) * (sum * inv[b]));
      }
    } else {  // ARGMAX
      const float logit = sum * inv[b];
      if (D.logits && lane == 0) lds_write_f32(lds_logits(lb, NB, D, T, b, lrow), logit);
      if (logit > G.best_v[b]) G.best_v[b] = logit, G.best_i[b] = vrow;
    }
  }
  if (++G.rr == a) {
    G.rr = 0;
    ++G.kk;
  }
}

// Publish the tile's outputs from LDS (stamped output words, the plain
// output when attached, LM-head logits when requested), every thread of the
// workgroup taking a share.  Called after a barrier that follows the
// stream.
template <int NB>
DEV void publish_tile(const mpk_kparams& P, cop& D, ctask& T, uint32_t lb, int s, uint32_t st, int tid) {
  const uint32_t ob = lb + LDS_OUT;
  if (D.epi == MPK_EPI_ARGMAX) {
    if (D.logits && s < D.logits_iters)
      for (int i = tid; i < NB * T.nrows; i += MPK_THREADS) {
        const int b = i / T.nrows, lrow = i - b * T.nrows;
        gst(D.logits + ((int64_t)s * P.B + b) * D.N0 + T.row0 + lrow, lds_read_f32(lds_logits(lb, NB, D, T, b, lrow)));
      }
    return;
  }
  const int n_out_tile = D.pairs ? T.nrows / 2 : T.nrows;
  const int orow0 = D.pairs ? T.row0 / 2 : T.row0;
  const uint32_t s8 = stamp8(st);
  for (int i = tid; i < NB * n_out_tile; i += MPK_THREADS) {
    const int b = i / n_out_tile, ol = i - b * n_out_tile;
    put_out(D, (int64_t)b * D.n_out + orow0 + ol, lds_read_f32(ob + (uint32_t)(b * n_out_tile + ol) * 4u), st, s8);
  }
}

// Generic consumer step (rows of any length): one unit, then the row's
// epilogue when the unit ends a row.  Padding units are skipped.
template <int NB>
DEV void gemv_consume(ctask& T, cop& D, GemvState<NB>& G, const u32x4 w, int unit, int n, uint32_t lb,
                      const float (&inv)[NB], int Kpad, int upr, int a, int wave, int lane) {
  if (unit >= n) return;  // padding unit (uniform)
  unit_fma<NB>(w, lb + LDS_X + (uint32_t)(G.u * 512 + lane * 4) * 4u, Kpad, G.acc);
  if (++G.u == upr) {
    G.u = 0;
    row_done<NB>(D, T, G, lb, inv, a, wave + MPK_NW * G.kk, lane);
  }
}

DEV u32x4 load_unit(const Cursor& C, int lane) {
  return __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1)))*)cursor_addr(C, lane));
}

// This lane's 16 bytes of unit u of the cursor's current row, unit u + j
// at p[64 j] (rows of whole groups: no clamping, no row change)
typedef const u32x4 __attribute__((address_space(1))) gu32x4;
DEV const gu32x4* unit_ptr(const Cursor& C, int u, int lane) {
  return (const gu32x4*)(const void*)(C.row + u * 512) + lane;
}

// Next free assignment unit of the tile (workgroup counter in LDS, reset to
// MPK_NW at task start: units 0 .. MPK_NW - 1 go to the wavefronts of the
// same index).
#define LDS_CLAIM (LDS_CTL + 40 * 4)
DEV int claim_unit(char* smem, int lane) {
  int v = 0;
  if (lane == 0)
    v = __hip_atomic_fetch_add(reinterpret_cast<int*>(smem + LDS_CLAIM), 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
}

// One assignment unit (a rows of one group of eight units each) whose
// weights are in LDS at pf (row rr at pf + 8 KB rr, 1 KB per unit, 16 bytes
// per lane), with the epilogue of each row; same arithmetic as the register
// path.  Called between assignment units (G.rr == 0).
template <int NB>
DEV void lds_au(cop& D, ctask& T, GemvState<NB>& G, uint32_t lb, uint32_t pf, uint32_t xl, int Kpad,
                const float (&inv)[NB], int a, int au, int lane) {
  for (int rr = 0; rr < a; ++rr) {
#pragma unroll
    for (int u = 0; u < MPK_RING; ++u)
      unit_fma<NB>(lds_read_u32x4(pf + (rr * MPK_RING + u) * 1024 + lane * 16), xl + u * 2048, Kpad, G.acc);
    row_done<NB>(D, T, G, lb, inv, a, au, lane);
  }
}

// Pull the next task's descriptors into the scalar cache while this task
// streams.  A task's first table reads form a chain (queue entry, task,
// operator); each miss would wait out the memory system's latency under the
// weight stream.
DEV void warm_tables(const mpk_kparams& P, int next) {
  const CAS uint32_t* t = (const CAS uint32_t*)(const CAS void*)unip(tasks_of(P) + next);
  const int op = uni((int)t[offsetof(mpk_dev_task, op) / 4]);
  const CAS uint32_t* d = (const CAS uint32_t*)(const CAS void*)unip(ops_of(P) + op);
  uint32_t acc = t[sizeof(mpk_dev_task) / 4 - 1];
  for (int i = 0; i < (int)(sizeof(mpk_dev_op) / 4); i += 16) acc ^= d[i];
  acc ^= d[sizeof(mpk_dev_op) / 4 - 1];
  asm volatile("" ::"s"(acc));
}

template <int NB>
DEV int gemv_task(const mpk_kparams& P, ctask& T, cop& D, int s, int task_id, char* smem, int tid, bool sched,
                  int next) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint32_t lb = lds_addr(smem);  // LDS byte address of the workgroup's area
  // LDS assignment units: with lds_pre (rows of one 4096-column group, one
  // request), wavefront w < npre also prefetches assignment unit MPK_NW + w
  // of the tile (a rows of 8 KB) into the LDS beyond the input's landing
  // zone while the inputs are awaited, and computes it after its first one:
  // up to twice the weights in flight during the wait.
  const int a_pre = D.pairs ? 2 : 1;
  const int land_end = Lay<NB>::RES + LDS_RES_BYTES + land_bytes<NB>(D);
  const int pre_cap = D.lds_pre && NB == 1 && D.K == MPK_RING * 512
                          ? min(MPK_NW, max(0, Lay<NB>::TOTAL - land_end) / (a_pre * MPK_RING * 1024))
                          : 0;
  const int nau_all = D.pairs ? T.nrows / 2 : T.nrows;
  const int npre = uni(min(pre_cap, max(0, nau_all - MPK_NW)));  // LDS assignment units of the tile
  bool lds_pending = !sched && wave < npre;
  const uint32_t pf = lb + land_end + wave * a_pre * MPK_RING * 1024;  // this wavefront's LDS unit
  // claims start after the staging's barriers
  if (tid == 0) *lvi(smem, LDS_CLAIM) = MPK_NW + npre;
  // The ring's first group (units 0..7) is issued before the inputs are
  // awaited: these weights do not depend on them, and the wait is what
  // they hide.
  Cursor I;  // issue side: runs MPK_RING units ahead of consumption
  u32x4 b[MPK_RING];
  // rows are whole groups of eight full units (K a multiple of 4096): a
  // group's units are consecutive in one row
  const bool whole = D.K % (MPK_RING * 512) == 0;
  int n = 0, npad = MPK_RING;
  if (!sched) {
    cursor_init(I, D, T, wave);
    n = I.n;
    npad = uni(padded_units(n));
  }
  float inv[NB];
  {
    const int ring_ops = MPK_RING + (lds_pending ? a_pre * MPK_RING : 0);
    // First weight loads: the ring's first group, then (steps 1, 2, ...)
    // the rows of the LDS assignment unit, PF_STEP units per step.
    static_assert(MPK_RING % PF_STEP == 0, "LDS unit steps");
    Cursor C2;  // the LDS assignment unit's rows
    const int rc = stage_inputs<NB>(P, D, T, smem, tid, s, task_id, inv, ring_ops, [&]() {
      if (sched) return;
      if (whole) {
        // units 0..7 of the wavefront's first row (of W0 when it has none)
        const gu32x4* wp = unit_ptr(I, 0, lane);
#pragma unroll
        for (int j = 0; j < MPK_RING; ++j) b[j] = __builtin_nontemporal_load(wp + j * 64);
      } else {
#pragma unroll
        for (int j = 0; j < MPK_RING; ++j) {
          b[j] = load_unit(I, lane);
          cursor_step(I, wave);
        }
      }
    }, [&](int step) {
      if (sched) return;
      const int q = (step - 1) * PF_STEP;  // first unit of the step within the LDS assignment unit
      if (q % MPK_RING == 0) {
        C2 = I;
        cursor_goto(C2, MPK_NW + wave, q / MPK_RING, 0, wave);
      }
      const gu32x4* wp = unit_ptr(C2, 0, lane);
#pragma unroll
      for (int u = 0; u < PF_STEP; ++u)
        __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(wp + (q % MPK_RING + u) * 64),
                                         lds_ptr(pf + (q + u) * 1024), 16, 0, CPOL_NT);
    });
    if (rc) return rc;
  }
  mark_ready(P, s, task_id, tid);
  const uint32_t st = stamp_of(P, s);
  const int Kpad = ((D.K + 511) / 512) * 512;
  GemvState<NB> G;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
    G.acc[bb] = 0.f, G.gate[bb] = 0.f, G.best_v[bb] = -INFINITY, G.best_i[bb] = 0x7fffffff;
  G.u = 0, G.rr = 0, G.kk = 0;
  if (!sched) {
    const int a = D.pairs ? 2 : 1;
    const int upr = uni(units_per_row(D));
    // everything issued so far (the first group, the staging's loads) is
    // complete here, and the compiler knows it: its waits on the ring stay
    // exact
    vm_drain_known();
    if (whole) {
      // Rows are whole groups of eight units (K a multiple of 4096 bf16 per
      // group): the epilogue runs between groups only, which keeps the
      // register ring's waits exact inside the unrolled group.  Assignment
      // units (a rows) are handed out dynamically within the workgroup:
      // wavefront w starts on unit w and claims the next free one from an
      // LDS counter when its issue side finishes one, so wavefronts that
      // stream slower take fewer rows and all end together.
      const int nau = T.nrows / a;
      const int gpa = a * upr / MPK_RING;  // groups per assignment unit
      const uint32_t xl = lb + LDS_X + lane * 16;
      int au_c = wave, gc = 0;  // the group in the ring: its assignment unit, group within it
      for (;;) {
        int au_n = au_c, gn = gc + 1;  // the group to issue next
        if (gn == gpa) {
          au_n = claim_unit(smem, lane);
          gn = 0;
        }
        if (au_n >= nau || au_c >= nau) break;
        {
          const int q = gn * MPK_RING;  // first unit of the group within the assignment unit
          const int rr = q / upr;
          cursor_goto(I, au_n, rr, q - rr * upr, wave);
        }
        const uint32_t xg = xl + G.u * 2048;
        const gu32x4* wp = unit_ptr(I, I.u, lane);
#pragma unroll
        for (int j = 0; j < MPK_RING; ++j) {
          unit_fma<NB>(b[j], xg + j * 2048, Kpad, G.acc);
          b[j] = __builtin_nontemporal_load(wp + j * 64);
        }
        G.u += MPK_RING;
        if (G.u == upr) {
          G.u = 0;
          row_done<NB>(D, T, G, lb, inv, a, au_c, lane);
        }
        if (lds_pending && G.rr == 0 && G.u == 0) {
          // the first assignment unit is done and the next one's loads are
          // in flight: compute the unit waiting in LDS meanwhile
          lds_au<NB>(D, T, G, lb, pf, xl, Kpad, inv, a, MPK_NW + wave, lane);
          lds_pending = false;
        }
        au_c = au_n, gc = gn;
      }
      // last group (none when this wavefront had no assignment unit)
      if (au_c < nau) {
        const uint32_t xg = xl + G.u * 2048;
#pragma unroll
        for (int j = 0; j < MPK_RING; ++j) unit_fma<NB>(b[j], xg + j * 2048, Kpad, G.acc);
        G.u += MPK_RING;
        if (G.u == upr) {
          G.u = 0;
          row_done<NB>(D, T, G, lb, inv, a, au_c, lane);
        }
      }
      if (lds_pending) lds_au<NB>(D, T, G, lb, pf, xl, Kpad, inv, a, MPK_NW + wave, lane);
    } else {
      // generic rows (short K): static assignment units, per-unit
      // bookkeeping, padding skipped
      const int ng = npad / MPK_RING;  // group g holds units 8g .. 8g + 7
      for (int g = 0; g < ng - 1; ++g) {
#pragma unroll
        for (int j = 0; j < MPK_RING; ++j) {
          gemv_consume<NB>(T, D, G, b[j], g * MPK_RING + j, n, lb, inv, Kpad, upr, a, wave, lane);
          b[j] = load_unit(I, lane);
          cursor_step(I, wave);
        }
      }
      const int g = ng - 1;
#pragma unroll
      for (int j = 0; j < MPK_RING; ++j)
        gemv_consume<NB>(T, D, G, b[j], g * MPK_RING + j, n, lb, inv, Kpad, upr, a, wave, lane);
    }
  } else if (next >= 0) {
    warm_tables(P, next);
  }
  __syncthreads();  // every row of the tile is in LDS
  publish_tile<NB>(P, D, T, lb, s, st, tid);
  if (D.epi == MPK_EPI_ARGMAX) {
    // tile argmax over the waves (lowest row among equal maxima), published
    // as two stamped words (value, row) per request
    float* bv = reinterpret_cast<float*>(smem + LDS_BEST);
    int* bi = reinterpret_cast<int*>(smem + LDS_BEST + MPK_NW * 8 * 4);
    if (!sched && lane == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) bv[wave * 8 + b] = G.best_v[b], bi[wave * 8 + b] = G.best_i[b];
    }
    __syncthreads();
    if (tid < NB) {
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int w = 0; w < MPK_NW; ++w) {
        const float vv = bv[w * 8 + tid];
        const int ii = bi[w * 8 + tid];
        if (vv > v || (vv == v && ii < ix)) v = vv, ix = ii;
      }
      uint64_t* pw = D.pll + ((int64_t)T.tile * NB + tid) * 2;
      st_ll(pw, v, st);
      st_lli(pw + 1, ix, st);
    }
  }
  return 0;
}

// Argmax task: the LM head's per-tile maxima -> next token per request.
// Writes tokens[r][p + 1] when generating (the prompt's own token otherwise
// stays), advances step, and publishes the token word that the next
// iteration's embedding reads wait for.
template <int NB>
DEV int argmax_task(const mpk_kparams& P, cop& D, char* smem, int tid, int s, int task_id) {
  const uint32_t st = stamp_of(P, s);
  uint32_t* raw = reinterpret_cast<uint32_t*>(smem + LDS_X);  // [N1 * NB][2]
  const int nw = D.N1 * NB * 2;                                // N1: LM-head tiles
  Waiter Wt = waiter_start();
  {
    const int rc = gather_ll<4>(P, D.pll, nw, raw, st, Wt, s, task_id, smem, tid);
    if (rc) return rc;
  }
  mark_ready(P, s, task_id, tid);
  const int wave = tid >> 6, lane = tid & 63;
  if (wave == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int t = lane; t < D.N1; t += 64) {
        const float vv = __uint_as_float(raw[(t * NB + b) * 2]);
        const int ii = (int)raw[(t * NB + b) * 2 + 1];
        if (vv > v || (vv == v && ii < ix)) v = vv, ix = ii;
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off);
        const int oi = __shfl_xor(ix, off);
        if (ov > v || (ov == v && oi < ix)) v = ov, ix = oi;
      }
      if (lane == 0) {
        const int p = cur_pos(smem, b);
        int next = ix;
        if (P.rpr == 1) {
          if (p + 1 >= ld_devi(P.prompt_len + b)) {
            st_devi(P.tokens + (int64_t)b * P.tokens_width + p + 1, ix);
          } else {
            next = ld_devi(P.tokens + (int64_t)b * P.tokens_width + p + 1);  // teacher-forced prompt token
          }
          st_devi(P.step + b, p + 1);
        } else {
          // batched prompt ingestion: the row's next position p + rpr is a
          // prompt position in every iteration of the run (checked at its
          // start); the request's last row advances its step past the chunk
          const int r = b / P.rpr;
          next = s + 1 < P.n_iter ? ld_devi(P.tokens + (int64_t)r * P.tokens_width + p + P.rpr) : 0;
          if (b % P.rpr == P.rpr - 1) st_devi(P.step + r, p + 1);
        }
        st_lli(P.tok_ll + b, next, st);
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Attention task (request r, kv head j, split c of nsplit): per-head RMSNorm
// of q and k, RoPE at the request's position p, K/V of p into the caches
// (by the split that owns p), then softmax(q K^T) V over this split's
// positions on MFMA, and one merge across the wavefronts.  The context
// [0, p] is cut into na = min(nsplit, ceil((p + 1) / 64)) splits; splits
// c >= na have nothing to do this iteration.  With one split the task writes
// the attention output of the group's query heads; with several, splits
// publish stamped partials (m, l, acc) and the split that owns p merges them
// into the output.  Returns -1 on stop.
//
// The split's positions go in steps of 16 (wave w of the eight worker waves
// takes steps w, w + 8, ...):
//   S = K q on v_mfma_f32_16x16x32_bf16: the step's K rows are the A operand
//     (16 positions x 32 dims per instruction), q the B operand: columns 0..3 the bf16 (hi) parts of the group's heads,
//     columns 4..7 the bf16 parts of what hi leaves (lo), so q keeps about 16
//     bits; S = column h + column h + 4.  Scores are in base 2 (q carries
//     log2(e) / sqrt(d)).
//   An online softmax per head: the reference maximum moves only when a
//     score exceeds it by 8 (weights stay below 2^8, most steps skip the
//     rescale); any reference gives the same softmax once l and acc share
//     it.
//   O^T += V^T P on v_mfma_f32_16x16x16_bf16: the step's V rows land in LDS
//     by global->LDS DMA (1 KB = 512 / d rows per instruction, 32 bytes of
//     padding between instructions) and are read transposed, 4 positions of
//     one dim per lane, as the A operand; P (hi / lo columns again) is the B
//     operand, taken from the score layout with one exchange.
//   K and V of a step land in LDS by global->LDS DMA (device scope): K as
//     whole rows (each DMA reads whole lines), its 16-byte segments placed by
//     an XOR of segment and row so the A operand's reads (one row per lane
//     column) are conflict-free, V as rows (above).  at_ring(DH)
//     steps per wave are in flight.  With no loads into registers in the
//     fold, every wait on them is explicit (the compiler's own waits on a
//     register ring fall back to full drains across this loop).
// Position p itself is not read from the cache: its K/V are in LDS; the
// scheduler wavefront scores it and it joins the merge as a ninth partial.
// Idle positions (past the split, or p) read row lo and score -inf.
// ---------------------------------------------------------------------------
#define ATT_MAXG 4
#define AT_VRING (LDS_X + 3 * 1024)    // after q [4][128] and the k / v row of p
// one step's K (DH / 32 KB) and V (16 rows in 1 KB DMA chunks + 32 bytes of
// padding each) in the ring, and the steps in flight per wave
constexpr int at_slot(int dh) { return dh * 32 + (dh / 32) * 1056; }
constexpr int at_ring(int dh) { return dh == 128 ? 2 : 3; }
static_assert(AT_VRING + MPK_NW * at_ring(128) * at_slot(128) <= 156 * 1024, "attention ring exceeds the LDS");
static_assert(AT_VRING + MPK_NW * at_ring(64) * at_slot(64) <= 156 * 1024, "attention ring exceeds the LDS");
// the merge area ([9][G][128] partial sums, [9][G] maxima, [9][G] sums) over
// the ring, then the split partials gathered by DMA (whole KB chunks, at most
// 9 x 16 of them)
#define AT_GATH (AT_VRING + (9 * ATT_MAXG * 128 + 2 * 9 * ATT_MAXG) * 4)
static_assert(AT_GATH % 16 == 0 && AT_GATH + 64 * 1024 <= 156 * 1024 && (156 * 1024 - AT_GATH) / 1024 <= 9 * 16,
              "attention merge area and partial gather do not fit the LDS");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// hi and lo bf16 parts (round to nearest even) of 8 values, 16 bytes each
DEV void split_hilo8(const float (&v)[8], u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = f2bf2(v[2 * e], v[2 * e + 1]);
    l[e] = f2bf2(v[2 * e] - __uint_as_float(h[e] << 16), v[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u));
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}


// bf16 hi part of 4 values (packed pairs) and of what hi leaves (lo)
DEV void split_hilo4(const float (&v)[4], u32x2& hi, u32x2& lo) {
  const uint32_t h0 = f2bf2(v[0], v[1]), h1 = f2bf2(v[2], v[3]);
  hi = u32x2{h0, h1};
  lo = u32x2{f2bf2(v[0] - __uint_as_float(h0 << 16), v[1] - __uint_as_float(h0 & 0xffff0000u)),
             f2bf2(v[2] - __uint_as_float(h1 << 16), v[3] - __uint_as_float(h1 & 0xffff0000u))};
}

// The transposed A operand of V^T P for two 16-dim blocks: 4 positions of one
// dim each, at a (block b0: rows a, a + RS, a + 2 RS, a + 3 RS) and a + 32.
// Zero-extending 16-bit reads, packed in pairs afterwards (the d16 forms do
// not keep the other half of the register when SRAM ECC is on).  asm LDS
// reads: a compiler-visible LDS read after the DMAs would wait for every DMA
// in flight.
template <int RS>
DEV void lds_read_vt2(uint32_t a, u32x2& x, u32x2& y) {
  uint32_t v[8];
  asm volatile(
      "ds_read_u16 %0, %8\n\tds_read_u16 %1, %8 offset:%9\n\t"
      "ds_read_u16 %2, %8 offset:%10\n\tds_read_u16 %3, %8 offset:%11\n\t"
      "ds_read_u16 %4, %8 offset:32\n\tds_read_u16 %5, %8 offset:%12\n\t"
      "ds_read_u16 %6, %8 offset:%13\n\tds_read_u16 %7, %8 offset:%14\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a), "n"(RS), "n"(2 * RS), "n"(3 * RS), "n"(32 + RS), "n"(32 + 2 * RS), "n"(32 + 3 * RS)
      : "memory");
  x = u32x2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
  y = u32x2{v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
}

// The A operand of a step's scores: KS 16-byte reads at a[0 .. KS-1]
// (early-clobber outputs, see lds_read_2f4)
template <int KS>
DEV void lds_read_k(const uint32_t (&a)[KS], u32x4 (&k)[KS]) {
  static_assert(KS == 2 || KS == 4, "head_dim 64 or 128");
  if constexpr (KS == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(k[0]), "=&v"(k[1])
                 : "v"(a[0]), "v"(a[1])
                 : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
}

template <int DH>
DEV int attn_task(const mpk_kparams& P, ctask& T, cop& D, char* smem, int tid, bool sched, int s, int task_id) {
  constexpr int KS = DH / 32;    // k-steps of a score MFMA
  constexpr int DB = DH / 16;    // 16-dim blocks of V
  constexpr int PPI = 512 / DH;  // V rows per 1 KB DMA chunk
  constexpr int LPR = DH / 8;    // lanes per V row (16 bytes each)
  constexpr int OPS = KS + 16 / PPI;  // vector-memory operations per step (K and V DMAs)
  constexpr int AT_R = at_ring(DH), SLOT = at_slot(DH), KBYTES = DH * 32;
  constexpr int KSEG = DH / 8, KRPC = 64 / KSEG;  // K: 16-byte segments per row, rows per 1 KB chunk
  static_assert(DB % 2 == 0, "V^T blocks are read in pairs");
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g4 = lane >> 4, cn = lane & 15;  // MFMA lane: row group, column
  const int r = T.row0, j = T.nrows, c = T.split, NS = D.nsplit;
  const int G = D.nq / D.nkv, half = DH >> 1;
  // row r is position p of request rq, the off-th row of the request in this
  // iteration: rows r - off .. r are positions p - off .. p, taken from this
  // iteration's q/k/v words; the splits fold the cache positions before them
  const int rq = r / P.rpr, off = r % P.rpr;
  const int p = cur_pos(smem, r);
  const int nf = p - off;
  const int na = max(1, min(NS, (nf + MPK_ATTN_SPLIT - 1) / MPK_ATTN_SPLIT));
  if (c >= na) return 0;  // uniform over the workgroup: nothing to do this iteration
  const int lo = (int)(((int64_t)c * nf) / na), hi = (int)(((int64_t)(c + 1) * nf) / na);
  const bool owner = c == na - 1;  // the split that adds positions p - off .. p and merges
  const uint32_t st = stamp_of(P, s);
  const uint32_t lb = lds_addr(smem);
  float* qs = reinterpret_cast<float*>(smem + LDS_X);  // [G][DH], scaled for base-2 scores
  float* kv = qs + ATT_MAXG * 128;                      // k [DH], v [DH] of p (bf16-rounded)
  float* mo = reinterpret_cast<float*>(smem + AT_VRING);  // merge: [9][G][DH] (over the ring)
  float* mm = mo + 9 * ATT_MAXG * 128;                    // [9][G] maxima
  float* ml = mm + 9 * ATT_MAXG;                          // [9][G] sums
  uint32_t* gath = reinterpret_cast<uint32_t*>(smem + AT_GATH);        // gathered split partials
  float* outs = reinterpret_cast<float*>(smem + LDS_OUT);               // partial, then o
  uint32_t* kvrow = reinterpret_cast<uint32_t*>(smem + LDS_OUT) + 640;  // bf16 K row, then V row
  const int qkv_w = (D.nq + 2 * D.nkv) * DH;
  uint16_t* kc = D.kc + ((int64_t)(rq * D.nkv + j) * D.S) * DH;
  uint16_t* vc = D.vc + ((int64_t)(rq * D.nkv + j) * D.S) * DH;
  // base-2 scores: log2(e) / sqrt(d) is applied to q once, when it is staged
  const float scale = 1.4426950408889634f / sqrtf((float)DH);

  // ---- the fold's steps of 16 positions: wave w starts with steps w, w + 8,
  // ... (AT_R - 1 of them), then claims the next free step from a workgroup
  // counter each time it frees a ring slot (waves whose data arrives sooner
  // take more steps) ----
  const int nst = (hi - lo + 15) >> 4;
  if (tid == 0) *lvi(smem, LDS_CLAIM) = MPK_NW * (AT_R - 1);  // read only after the barriers below
  const uint32_t ring = lb + AT_VRING + (uint32_t)wave * (AT_R * SLOT);
  // step k: positions t0 .. t0 + 15, t0 = lo + 16 k, into ring slot `slot`
  // (K, then V)
  auto issue = [&](int k, uint32_t slot) {
    const int t0 = lo + 16 * k;
    // K: chunk j holds rows KRPC j .. + KRPC - 1 whole (coalesced lines);
    // lane l takes row KRPC j + l / KSEG, segment (l % KSEG) ^ (row % KSEG)
#pragma unroll
    for (int kj = 0; kj < KS; ++kj) {
      const int rr = KRPC * kj + lane / KSEG;
      const int tk = t0 + rr;
      const int rk = tk < hi ? tk : lo;
      const int seg = (lane % KSEG) ^ (rr % KSEG);
      __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(kc + (int64_t)rk * DH + 8 * seg),
                                       lds_ptr(slot + kj * 1024), 16, 0, CPOL_SC1 | CPOL_NT);
    }
#pragma unroll
    for (int c4 = 0; c4 < 16 / PPI; ++c4) {
      const int tv = t0 + c4 * PPI + lane / LPR;
      const int rv = tv < hi ? tv : lo;
      __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(vc + (int64_t)rv * DH + 8 * (lane % LPR)),
                                       lds_ptr(slot + KBYTES + c4 * 1056), 16, 0, CPOL_SC1 | CPOL_NT);
    }
  };
  // The cache rows below p were written by earlier iterations, all ended once
  // any input of this iteration has arrived.  If an earlier task of this
  // iteration on this CU has already waited for one, the first steps are
  // issued before this task's own wait; otherwise after it.
  // (Whatever earlier tasks left in flight is waited for first: the
  // compiler's waits would otherwise drain these loads as well, at once.)
  vm_drain_known();
  int sq[AT_R];  // the step in each ring slot, -1: none (steps are taken in slot order)
#pragma unroll
  for (int i = 0; i < AT_R; ++i) sq[i] = i < AT_R - 1 && wave + MPK_NW * i < nst ? wave + MPK_NW * i : -1;
  const bool early = !sched && uni(*lvi(smem, LDS_SYNCED)) != 0;
  if (early) {
#pragma unroll
    for (int i = 0; i < AT_R - 1; ++i)
      if (sq[i] >= 0) issue(sq[i], ring + i * SLOT);
  }

  // ---- q / k / v words of the group: wave hh < G + 2 takes one head vector ----
  const int hh = wave;
  // RoPE factors and norm gains do not depend on this iteration's words:
  // loaded before the wait
  float cs = 0.f, sn = 0.f, ga = 0.f, gb = 0.f;
  if (!sched && hh <= G && lane < half) {
    cs = gld(P.rope_cos + (int64_t)p * half + lane);
    sn = gld(P.rope_sin + (int64_t)p * half + lane);
    const uint16_t* gsrc = hh < G ? D.qn : D.kn;
    ga = bf16f(gld16(gsrc + lane));
    gb = bf16f(gld16(gsrc + lane + half));
  }
  Waiter Wt = waiter_start();
  const bool mine = !sched && hh < G + 2 && lane < half;
  const uint64_t* src = D.xll + (int64_t)r * qkv_w +
                        (hh < G ? (j * G + hh) * DH : (hh == G ? D.nq * DH + j * DH : (D.nq + D.nkv) * DH + j * DH));
  uint64_t wa = 0, wb = 0;
  {
    // each wavefront polls its own head vector; the workgroup meets once
    bool need = mine;
    for (;;) {
      if (need) {
        wa = ld_ll(src + lane);
        wb = ld_ll(src + lane + half);
        need = !(ll_ok(wa, st) && ll_ok(wb, st));
      }
      if (__ballot(need) == 0) break;
      if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
      __builtin_amdgcn_s_sleep(1);
    }
    lds_barrier();
    if (*lvi(smem, LDS_CTL)) return -1;
  }
  if (tid == 0) *lvi(smem, LDS_SYNCED) = 1;
  // the K/V steps, RoPE factors and gains above are loads issued before the
  // device-scope polls: complete them here (see vm_drain_known; they were
  // issued first, so this costs little)
  vm_drain_known();
  mark_ready(P, s, task_id, tid);

  // ---- RMSNorm + RoPE (waves 0..G+1) ----
  if (!sched && hh < G + 2) {
    const float a = lane < half ? ll_f(wa) : 0.f;
    const float b = lane < half ? ll_f(wb) : 0.f;
    if (hh <= G) {
      const float ss = wave_sum(a * a + b * b);
      const float inv = 1.0f / sqrtf(ss / (float)DH + P.rms_eps);
      if (lane < half) {
        const float ya = ga * (a * inv);
        const float yb = gb * (b * inv);
        const float ra = ya * cs - yb * sn;
        const float rb = yb * cs + ya * sn;
        if (hh < G) {
          qs[hh * DH + lane] = ra * scale;
          qs[hh * DH + lane + half] = rb * scale;
        } else {
          const uint16_t ka = f2bf(ra), kb = f2bf(rb);
          kv[lane] = bf16f(ka);
          kv[lane + half] = bf16f(kb);
          reinterpret_cast<uint16_t*>(kvrow)[lane] = ka;
          reinterpret_cast<uint16_t*>(kvrow)[lane + half] = kb;
        }
      }
    } else if (lane < half) {
      const uint16_t va = f2bf(a), vb = f2bf(b);
      kv[DH + lane] = bf16f(va);
      kv[DH + lane + half] = bf16f(vb);
      reinterpret_cast<uint16_t*>(kvrow)[DH + lane] = va;
      reinterpret_cast<uint16_t*>(kvrow)[DH + lane + half] = vb;
    }
  }
  __syncthreads();

  float m = -INFINITY, l = 0.f;  // workers, head cn (lanes cn < G): running reference and this lane's sum
  f32x4 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Scheduler wave of the owner: positions p - off .. p, the merge's ninth
  // partial, as a running maximum cm, sum cl and weighted V co per head (a
  // lane holds dims lane and lane + half of co; lanes < half).
  float cm[ATT_MAXG], cl[ATT_MAXG], co[ATT_MAXG][2];
#pragma unroll
  for (int h = 0; h < ATT_MAXG; ++h) cm[h] = -INFINITY, cl[h] = 0.f, co[h][0] = co[h][1] = 0.f;
  if (sched && owner) {
    // K/V of p into the caches.  The stores complete before the output is
    // published (next iteration's readers are ordered after that output):
    // this wavefront waits for them after the merge area is written, before
    // the barrier that precedes the publish, so the wait overlaps the fold.
    uint32_t* kdst = reinterpret_cast<uint32_t*>(kc + (int64_t)p * DH);
    uint32_t* vdst = reinterpret_cast<uint32_t*>(vc + (int64_t)p * DH);
    for (int i = lane; i < DH / 2; i += 64) {
      st_devu(kdst + i, kvrow[i]);
      st_devu(vdst + i, kvrow[DH / 2 + i]);
    }
    const bool pl = lane < half;
    auto fold_pos = [&](float ka, float kb, float va, float vb) {
#pragma unroll
      for (int h = 0; h < ATT_MAXG; ++h) {
        if (h < G) {
          const float sc = wave_sum(pl ? fmaf(qs[h * DH + lane], ka, qs[h * DH + lane + half] * kb) : 0.f);
          const float mn = fmaxf(cm[h], sc);
          const float a1 = cm[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(cm[h] - mn);
          const float a2 = __builtin_amdgcn_exp2f(sc - mn);
          cl[h] = fmaf(cl[h], a1, a2);
          co[h][0] = fmaf(co[h][0], a1, va * a2);
          co[h][1] = fmaf(co[h][1], a1, vb * a2);
          cm[h] = mn;
        }
      }
    };
    // the request's earlier rows in this iteration (positions p - off ..
    // p - 1): K and V from their q/k/v words, K normalised and rotated as the
    // rows' own tasks do, both rounded to bf16 as the cache holds them
    for (int bb = r - off; bb < r; ++bb) {
      const uint64_t* kw = D.xll + (int64_t)bb * qkv_w + (D.nq + j) * DH;
      const uint64_t* vw = kw + D.nkv * DH;
      uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
      bool need = pl;
      for (;;) {
        if (need) {
          w0 = ld_ll(kw + lane), w1 = ld_ll(kw + lane + half);
          w2 = ld_ll(vw + lane), w3 = ld_ll(vw + lane + half);
          need = !(ll_ok(w0, st) && ll_ok(w1, st) && ll_ok(w2, st) && ll_ok(w3, st));
        }
        if (__ballot(need) == 0) break;
        if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
        __builtin_amdgcn_s_sleep(1);
      }
      const float a = pl ? ll_f(w0) : 0.f, b = pl ? ll_f(w1) : 0.f;
      const float ss = wave_sum(a * a + b * b);
      const float inv = 1.0f / sqrtf(ss / (float)DH + P.rms_eps);
      float ka = 0.f, kb = 0.f, va = 0.f, vb = 0.f;
      if (pl) {
        const int pb = cur_pos(smem, bb);
        const float cs = gld(P.rope_cos + (int64_t)pb * half + lane);
        const float sn = gld(P.rope_sin + (int64_t)pb * half + lane);
        const float ya = bf16f(gld16(D.kn + lane)) * (a * inv);
        const float yb = bf16f(gld16(D.kn + lane + half)) * (b * inv);
        ka = bf16f(f2bf(ya * cs - yb * sn));
        kb = bf16f(f2bf(yb * cs + ya * sn));
        va = bf16f(f2bf(ll_f(w2)));
        vb = bf16f(f2bf(ll_f(w3)));
      }
      fold_pos(ka, kb, va, vb);
    }
    // position p (its K/V in LDS)
    fold_pos(pl ? kv[lane] : 0.f, pl ? kv[lane + half] : 0.f, pl ? kv[DH + lane] : 0.f,
             pl ? kv[DH + lane + half] : 0.f);
  } else if (!sched) {
    // ---- the MFMA fold over this wave's steps ----
    // q as the B operand of the scores, per 32-dim k-step
    u32x4 qb[KS];
    {
      const int h = cn & 3;
      const bool has = cn < 8 && h < G;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        float qv[8];
        f32x4 q0, q1;
        lds_read_2f4_near(lb + LDS_X + (uint32_t)(h * DH + 32 * kk + 8 * g4) * 4u, q0, q1);
        qv[0] = q0.x, qv[1] = q0.y, qv[2] = q0.z, qv[3] = q0.w;
        qv[4] = q1.x, qv[5] = q1.y, qv[6] = q1.z, qv[7] = q1.w;
        u32x4 hi8, lo8;
        split_hilo8(qv, hi8, lo8);
        qb[kk] = !has ? u32x4{0u, 0u, 0u, 0u} : (cn < 4 ? hi8 : lo8);
      }
    }
    if (!early) {
#pragma unroll
      for (int i = 0; i < AT_R - 1; ++i)
        if (sq[i] >= 0) issue(sq[i], ring + i * SLOT);
    }
    for (bool more = sq[0] >= 0; more;) {
#pragma unroll
      for (int sl = 0; sl < AT_R; ++sl) {
        if (sq[sl] < 0) {
          more = false;
          break;
        }
        // the slot freed by the previous step takes the next free step
        // (none once a claim has come back empty: the last slot filled is -1)
        const int nx = (sl + AT_R - 1) % AT_R;
        int k = -1;
        if (sq[(sl + AT_R - 2) % AT_R] >= 0) {
          k = claim_unit(smem, lane);
          if (k >= nst) k = -1;
        }
        sq[nx] = k;
        if (k >= 0) issue(k, ring + nx * SLOT);
        // this step has landed (loads complete in issue order: only the
        // later steps' operations may still be in flight)
        int later = 0;
#pragma unroll
        for (int q = 1; q < AT_R; ++q) later += sq[(sl + q) % AT_R] >= 0;
        if (later >= 2) vm_wait_known<2 * OPS>();
        else if (later == 1) vm_wait_known<OPS>();
        else vm_wait_known<0>();
        const int t0 = lo + 16 * sq[sl];
        // scores of the step's 16 positions: lane (g4, cn) holds positions
        // t0 + 4 g4 + e of column cn; hi + lo columns
        const uint32_t slot = ring + sl * SLOT;
        u32x4 kr[KS];
        // row cn, segment 4 kk + g4: chunk cn / KRPC, slot KSEG (cn % KRPC) +
        // (segment ^ (cn % KSEG)) (the XOR keeps a 16-lane read conflict-free)
        uint32_t ka[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          ka[kk] = slot + (uint32_t)(cn / KRPC) * 1024u +
                   (uint32_t)(KSEG * (cn % KRPC) + ((4 * kk + g4) ^ (cn % KSEG))) * 16u;
        lds_read_k<KS>(ka, kr);
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]),
                                                       __builtin_bit_cast(bf16x8, qb[kk]), sa, 0, 0, 0);
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = sa[e] + __shfl_xor(sa[e], 4);
          const int t = t0 + 4 * g4 + e;
          sv[e] = cn < G && t < hi ? v : -INFINITY;
          mx = fmaxf(mx, sv[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool mv = mx > m + 8.f;  // (always for the first score: m = -inf)
        if (__ballot(mv) != 0) {
          const float mn = mv ? mx : m;
          const float co = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
          l *= co;
          m = mn;
          // columns cn and cn + 4 belong to head cn & 3
          const float cc = __shfl(co, (lane & 0x30) | (lane & 3));
#pragma unroll
          for (int b = 0; b < DB; ++b) acc[b] *= cc;
        }
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = sv[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[e] - m);
          l += pv[e];
        }
        // P as the B operand: lane (g4, cn) takes positions 4 g4 .. + 3 of
        // column cn: the hi parts for cn < 4, the lo parts (from lane - 4) for
        // cn in 4..7, zero beyond
        u32x2 ph, pl;
        split_hilo4(pv, ph, pl);
        const int srcl = cn >= 4 && cn < 8 ? lane - 4 : lane;
        const uint32_t l0 = __shfl(pl.x, srcl), l1 = __shfl(pl.y, srcl);
        const u32x2 pb = cn < 4 ? ph : (cn < 8 ? u32x2{l0, l1} : u32x2{0u, 0u});
        // O^T += V^T P: the A operand of block b is V[4 g4 .. + 3][16 b + cn]
        const uint32_t va = slot + KBYTES + (uint32_t)((4 * g4) / PPI) * 1056u +
                            (uint32_t)((4 * g4) % PPI) * (2 * DH) + (uint32_t)cn * 2u;
#pragma unroll
        for (int b = 0; b < DB; b += 2) {
          u32x2 x0, x1;
          lds_read_vt2<2 * DH>(va + b * 32, x0, x1);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, x0),
                                                             __builtin_bit_cast(bf16x4, pb), acc[b], 0, 0, 0);
          acc[b + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, x1),
                                                                 __builtin_bit_cast(bf16x4, pb), acc[b + 1], 0, 0,
                                                                 0);
        }
      }
    }
    // O[h][d] = column h + column h + 4; this wave's sums per head
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[b][e] += __shfl_xor(acc[b][e], 4);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
  }
  // every worker wave's ring is drained before the merge area over it is
  // written (the scheduler wave's K/V stores are waited for further down)
  if (!sched) vm_drain_known();
  lds_barrier();
  if (*lvi(smem, LDS_CTL)) return -1;  // (a wait above ended the run)
  if (sched) {
#pragma unroll
    for (int h = 0; h < ATT_MAXG; ++h) {
      if (h < G) {
        if (lane < half) {
          mo[(MPK_NW * ATT_MAXG + h) * 128 + lane] = co[h][0];
          mo[(MPK_NW * ATT_MAXG + h) * 128 + lane + half] = co[h][1];
        }
        if (lane == 0) {
          mm[MPK_NW * ATT_MAXG + h] = cm[h];
          ml[MPK_NW * ATT_MAXG + h] = cl[h];
        }
      }
    }
  } else if (cn < G) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
      *reinterpret_cast<float4*>(mo + (wave * ATT_MAXG + cn) * 128 + 16 * b + 4 * g4) =
          float4{acc[b][0], acc[b][1], acc[b][2], acc[b][3]};
    if (g4 == 0) {
      mm[wave * ATT_MAXG + cn] = m;
      ml[wave * ATT_MAXG + cn] = l;
    }
  }
  if (sched) vm_drain();  // the owner's K/V stores, before any output is published
  __syncthreads();
  // ---- merge the nine partials (eight waves, position p) per head ----
  const int stride = DH + 2;
  const int64_t o_base = (int64_t)r * D.nq * DH + (int64_t)j * G * DH;
  for (int idx = tid; idx < G * DH && !sched; idx += MPK_NW * 64) {
    const int h = idx / DH, i = idx - h * DH;
    float M = -INFINITY;
    for (int w = 0; w <= MPK_NW; ++w) M = fmaxf(M, mm[w * ATT_MAXG + h]);
    float A = 0.f, L = 0.f;
    for (int w = 0; w <= MPK_NW; ++w) {
      const float mw = mm[w * ATT_MAXG + h];
      const float cw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      A = fmaf(mo[(w * ATT_MAXG + h) * 128 + i], cw, A);
      L = fmaf(ml[w * ATT_MAXG + h], cw, L);
    }
    if (na == 1) {
      put_out(D, o_base + idx, A / L, st, stamp8(st));  // the whole context in one split
    } else {
      outs[h * stride + 2 + i] = A;
      if (i == 0) {
        outs[h * stride] = M;
        outs[h * stride + 1] = L;
      }
    }
  }
  if (na == 1) return 0;
  __syncthreads();
  uint64_t* pgrp = D.pll + (int64_t)((r * D.nkv + j) * NS) * G * stride;
  if (!owner) {
    // publish this split's partial for the owner
    for (int i = tid; i < G * stride; i += MPK_THREADS) st_ll(pgrp + (int64_t)c * G * stride + i, outs[i], st);
    return 0;
  }
  // owner: merge the other splits' partials into its own, as many per round
  // as the LDS holds (gathered by DMA): o = sum_c acc_c 2^(m_c - M) /
  // sum_c l_c 2^(m_c - M), with M the largest m_c; a round's weights
  // 2^(m_c - M) are computed once per head and partial
  const int idx = tid;
  const bool mine_o = !sched && idx < G * DH;
  const int h = mine_o ? idx / DH : 0, i = mine_o ? idx - h * DH : 0;
  float L = mine_o ? outs[h * stride + 1] : 0.f;
  float O = mine_o ? outs[h * stride + 2 + i] : 0.f;
  float* mrun = mm;  // [G] running reference per head (the merge area is free now)
  float* wt = mo;    // [chunk + 1][G]: the partials' weights, then the running sums' rescale
  if (tid < G) mrun[tid] = outs[tid * stride];  // (read after the gather's barrier)
  const float* gf = reinterpret_cast<const float*>(gath);  // word w's payload at gf[2 w]
  const int avail = (Lay<1>::TOTAL - (int)((char*)gath - smem)) & ~1023;
  const int chunk = avail / (G * stride * 8);
  for (int c0 = 0; c0 < na - 1; c0 += chunk) {
    const int nc = min(chunk, na - 1 - c0);
    const int rc = gather_ll_dma(P, pgrp + (int64_t)c0 * G * stride, nc * G * stride, lds_addr(gath), st, Wt, s,
                                 task_id, smem, tid);
    if (rc) return rc;
    if (!sched && wave < G) {
      // worker wave hh: head hh, one lane per partial
      const int hh = wave;
      const float Mo = mrun[hh];
      float Mn = Mo;
      for (int cc = lane; cc < nc; cc += 64)
        if (gf[2 * ((cc * G + hh) * stride + 1)] > 0.f) Mn = fmaxf(Mn, gf[2 * (cc * G + hh) * stride]);
      Mn = wave_max(Mn);
      for (int cc = lane; cc < nc; cc += 64) {
        const float mc = gf[2 * (cc * G + hh) * stride], lc = gf[2 * ((cc * G + hh) * stride + 1)];
        wt[cc * G + hh] = lc > 0.f ? exp2f(mc - Mn) : 0.f;
      }
      if (lane == 0) {
        wt[nc * G + hh] = exp2f(Mo - Mn);
        mrun[hh] = Mn;
      }
    }
    __syncthreads();
    if (mine_o) {
      const float ca = wt[nc * G + h];
      L *= ca;
      O *= ca;
      for (int cc = 0; cc < nc; ++cc) {
        const float w = wt[cc * G + h];
        L = fmaf(gf[2 * ((cc * G + h) * stride + 1)], w, L);
        O = fmaf(gf[2 * ((cc * G + h) * stride + 2 + i)], w, O);
      }
    }
    __syncthreads();  // the gather area and the weights are reused by the next round
  }
  if (mine_o) put_out(D, o_base + idx, O / L, st, stamp8(st));
  return 0;
}

// ---------------------------------------------------------------------------
// Batch-8 linear tasks on MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// y[r][row] = W[row] . x[r] for the 8 requests as steps of [16 rows] x [32
// columns of W] x [16 MFMA columns].  The 16 MFMA columns carry each
// request's input twice: its bf16 value (hi) and the bf16 value of what hi
// leaves (lo = x - hi), so an input keeps about 16 significant bits while
// the MFMA forms the hi and lo products in one instruction (padding 8
// requests to 16 columns would otherwise waste them); y = D[row][r] +
// D[row][r + 8].  The products of bf16 pairs are exact in fp32.
//
// A tile's rows form 16-row blocks; rows past the tile repeat its last row
// (the same cache lines as a real row: no extra HBM traffic; discarded).  x
// is staged in LDS in passes of 4096 columns as MFMA B operands: 1 KB per
// 32-column k-step, lane l's 16 bytes at 16 l holding request l % 8 (hi for
// l % 16 < 8, lo otherwise), columns 8 (l / 16) .. + 7 of the step; with a
// norm, times the gain, and 1 / rms is applied to the sums.  Worker wave w
// takes the blocks w / WK + (8 / WK) j (j < NBW) and the k-steps
// [(w % WK) KS, (w % WK + 1) KS) of every pass, KS = 128 / WK; each lane loads
// 16 bytes of weights per (block, k-step) straight into the A operand (row
// l % 16 of the block, columns 8 (l / 16) .. + 7 of the step: 16 rows x 64
// bytes per load, and the next k-step continues the same rows), RG k-steps
// of loads in flight, the first RG issued before the inputs are awaited.
// With WK > 1 the waves' partial sums meet in LDS and are added in wave
// order: the result does not depend on timing (bitwise reproducible).
// ---------------------------------------------------------------------------
#define G8_PASS 4096               // columns of x staged per pass
#define G8_KSTEPS (G8_PASS / 32)   // MFMA k-steps per pass
#define G8_ITEMS (8 * G8_PASS / 8) // (request, 8-column group) staging items per pass
#define G8_NI ((G8_ITEMS + MPK_THREADS - 1) / MPK_THREADS)
static_assert(MPK_THREADS % 8 == 0, "a thread's staging items share one request");
static_assert(LDS_X + G8_KSTEPS * 1024 <= 156 * 1024, "a staged pass must fit the LDS");

// Weight row of virtual row vr (rows of W0, W1, W2 in order; gate/up pairs
// interleaved).
DEV const uint16_t* vrow_ptr(cop& D, int vr) {
  if (D.pairs) return ((vr & 1) ? D.W1 : D.W0) + (int64_t)(vr >> 1) * D.K;
  if (vr < D.N0) return D.W0 + (int64_t)vr * D.K;
  if (vr < D.N0 + D.N1) return D.W1 + (int64_t)(vr - D.N0) * D.K;
  return D.W2 + (int64_t)(vr - D.N0 - D.N1) * D.K;
}

// Stage pass p of the 8 rows' x into LDS as B operands, every thread of the
// workgroup taking part.  The B operand of k-step t holds, in the 16 bytes of
// lane 16 (q & 3) + r (hi) and lane 16 (q & 3) + r + 8 (lo), the 8 columns of
// item q = 4 t + (q & 3) of row r.  With a norm, each item's sum of squares
// of the raw values goes to LDS at G8_SQ, [row][item].  Returns -1 on stop.
#define G8_SQ (LDS_X + G8_KSTEPS * 1024)  // [8][512] floats
static_assert(G8_SQ + 8 * 512 * 4 <= 156 * 1024, "staging sums exceed the LDS");

DEV void lds_write_u32_nw(uint32_t a, uint32_t v) { asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory"); }

// Stamped x: 1 KB units, unit u = row u % 8, columns 128 (u / 8) .. + 127 of
// the pass: one coalesced 16-byte device-scope load per lane (two words:
// columns 2 l, 2 l + 1 of the unit); four lanes cover an item and write 4
// bytes each of its hi and lo slots.  Wavefront w polls units w + 9 k, up to
// IG of them in flight together, and fetches a unit again while any of its
// words is stale; the workgroup meets at the end.
DEV int stage_pass8_ll(const mpk_kparams& P, cop& D, int p, char* smem, int tid, int s, int task_id, Waiter& Wt,
                       uint32_t st) {
  constexpr int NWAVES = MPK_THREADS / 64;
  constexpr int NU = 8 * G8_PASS / 128;           // units per pass
  constexpr int UPW = (NU + NWAVES - 1) / NWAVES;  // units per wavefront
  constexpr int IG = 8;                            // units in flight per wavefront
  static_assert(UPW <= 32, "a wavefront's units fit one mask");
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int pc = lane & 3, qi = lane >> 2;  // this lane's piece of its item, the item within the unit
  const uint32_t xb = lds_addr(smem) + LDS_X, sqb = lds_addr(smem) + G8_SQ;
  const int K = D.K;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(D.xll), (short)0, 8 * K * 8, 0x00020000);
  uint32_t need = 0;
  for (int k = 0; k < UPW; ++k)
    if (wave + NWAVES * k < NU) need |= 1u << k;
  for (;;) {
    uint32_t left = need;
    while (left) {
      int ks[IG];
#pragma unroll
      for (int i = 0; i < IG; ++i) {
        ks[i] = left ? __builtin_ctz(left) : -1;
        left &= left - 1;
      }
      u32x4 v[IG];
      uint32_t g[IG];
#pragma unroll
      for (int i = 0; i < IG; ++i) {
        if (ks[i] >= 0) {
          const int u = wave + NWAVES * ks[i];
          const int col = p * G8_PASS + (u >> 3) * 128 + 2 * lane;
          v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((u & 7) * K + col) * 8, 0, CPOL_SC1);
          g[i] = D.has_norm ? gldv<uint32_t>(D.gain + col) : 0u;
        }
      }
#pragma unroll
      for (int i = 0; i < IG; ++i) {
        if (ks[i] < 0) continue;
        if (__ballot(v[i].y != st || v[i].w != st) != 0) continue;  // fetched again next round
        need &= ~(1u << ks[i]);
        const int u = wave + NWAVES * ks[i];
        const int r = u & 7, q = (u >> 3) * 16 + qi;
        float x0 = __uint_as_float(v[i].x), x1 = __uint_as_float(v[i].z);
        if (D.has_norm) {
          float ssq = fmaf(x0, x0, x1 * x1);
          ssq += __shfl_xor(ssq, 1);
          ssq += __shfl_xor(ssq, 2);
          if (pc == 0) lds_write_u32_nw(sqb + (uint32_t)(r * 512 + q) * 4u, __float_as_uint(ssq));
          x0 *= bf16lo(g[i]);
          x1 *= bf16hi(g[i]);
        }
        const uint32_t hi = f2bf2(x0, x1);
        const uint32_t lo = f2bf2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
        const uint32_t a = xb + (uint32_t)(q >> 2) * 1024u + (uint32_t)(16 * (q & 3) + r) * 16u + 4u * pc;
        lds_write_u32_nw(a, hi);
        lds_write_u32_nw(a + 128u, lo);
      }
    }
    if (need == 0) break;
    if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  lds_barrier();
  return *lvi(smem, LDS_CTL) ? -1 : 0;
}
// Packed x (mpk_dev_op::xpk): 1 KB units of 256 columns, unit u = row u % 8,
// columns 256 (u / 8) .. + 255 of the pass; a lane's 16 bytes are four
// packed words (columns 4 l .. 4 l + 3), two lanes cover an item and write 8
// bytes each of its hi and lo slots.  Same polling and the same sums of
// squares (in the same association) as with stamped words.
DEV void lds_write_u32x2_nw(uint32_t a, uint32_t v0, uint32_t v1) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(u32x2_t{v0, v1}) : "memory");
}
DEV int stage_pass8_pk(const mpk_kparams& P, cop& D, int p, char* smem, int tid, int s, int task_id, Waiter& Wt,
                       uint32_t st) {
  constexpr int NWAVES = MPK_THREADS / 64;
  constexpr int NU = 8 * G8_PASS / 256;           // units per pass
  constexpr int UPW = (NU + NWAVES - 1) / NWAVES;  // units per wavefront
  constexpr int IG = 4;                            // units in flight per wavefront (8 measured 1.6 % slower)
  static_assert(UPW <= 32, "a wavefront's units fit one mask");
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int ph = lane & 1, qi = lane >> 1;  // this lane's half of its item, the item within the unit
  const uint32_t xb = lds_addr(smem) + LDS_X, sqb = lds_addr(smem) + G8_SQ;
  const int K = D.K;
  const uint32_t s8 = stamp8(st);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(D.xpk), (short)0, 8 * K * 4, 0x00020000);
  uint32_t need = 0;
  for (int k = 0; k < UPW; ++k)
    if (wave + NWAVES * k < NU) need |= 1u << k;
  for (;;) {
    uint32_t left = need;
    while (left) {
      int ks[IG];
#pragma unroll
      for (int i = 0; i < IG; ++i) {
        ks[i] = left ? __builtin_ctz(left) : -1;
        left &= left - 1;
      }
      u32x4 v[IG];
      uint32_t g0[IG], g1[IG];
#pragma unroll
      for (int i = 0; i < IG; ++i) {
        if (ks[i] >= 0) {
          const int u = wave + NWAVES * ks[i];
          const int col = p * G8_PASS + (u >> 3) * 256 + 4 * lane;
          v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((u & 7) * K + col) * 4, 0, CPOL_SC1);
          g0[i] = D.has_norm ? gldv<uint32_t>(D.gain + col) : 0u;
          g1[i] = D.has_norm ? gldv<uint32_t>(D.gain + col + 2) : 0u;
        }
      }
#pragma unroll
      for (int i = 0; i < IG; ++i) {
        if (ks[i] < 0) continue;
        const bool stale = ((v[i].x & 0xffu) != s8) | ((v[i].y & 0xffu) != s8) | ((v[i].z & 0xffu) != s8) |
                           ((v[i].w & 0xffu) != s8);
        if (__ballot(stale) != 0) continue;  // fetched again next round
        need &= ~(1u << ks[i]);
        const int u = wave + NWAVES * ks[i];
        const int r = u & 7, q = (u >> 3) * 32 + qi;
        float x0 = pk_f(v[i].x), x1 = pk_f(v[i].y), x2 = pk_f(v[i].z), x3 = pk_f(v[i].w);
        if (D.has_norm) {
          float ssq = fmaf(x0, x0, x1 * x1) + fmaf(x2, x2, x3 * x3);
          ssq += __shfl_xor(ssq, 1);
          if (ph == 0) lds_write_u32_nw(sqb + (uint32_t)(r * 512 + q) * 4u, __float_as_uint(ssq));
          x0 *= bf16lo(g0[i]);
          x1 *= bf16hi(g0[i]);
          x2 *= bf16lo(g1[i]);
          x3 *= bf16hi(g1[i]);
        }
        const uint32_t h0 = f2bf2(x0, x1), h1 = f2bf2(x2, x3);
        const uint32_t l0 = f2bf2(x0 - __uint_as_float(h0 << 16), x1 - __uint_as_float(h0 & 0xffff0000u));
        const uint32_t l1 = f2bf2(x2 - __uint_as_float(h1 << 16), x3 - __uint_as_float(h1 & 0xffff0000u));
        const uint32_t a = xb + (uint32_t)(q >> 2) * 1024u + (uint32_t)(16 * (q & 3) + r) * 16u + 8u * ph;
        lds_write_u32x2_nw(a, h0, h1);
        lds_write_u32x2_nw(a + 128u, l0, l1);
      }
    }
    if (need == 0) break;
    if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  lds_barrier();
  return *lvi(smem, LDS_CTL) ? -1 : 0;
}


// Unstamped x (an embedding row, or a plain input tensor): item i = tid +
// MPK_THREADS j covers row i % 8 and columns 8 (i / 8) .. + 7 of the pass.
// PK = false leaves the packed staging out of the caller: inlined into the
// LM head's body it made that body's stream 25 % slower (the LM head at
// batch 8 reads the stamped words).
template <bool PK>
DEV int stage_pass8(const mpk_kparams& P, cop& D, int p, char* smem, int tid, int s, int task_id, Waiter& Wt,
                    uint32_t st) {
  if (PK && D.xpk) return stage_pass8_pk(P, D, p, smem, tid, s, task_id, Wt, st);
  if (D.xll) return stage_pass8_ll(P, D, p, smem, tid, s, task_id, Wt, st);
  const uint32_t xb = lds_addr(smem) + LDS_X;
  const uint32_t sqb = lds_addr(smem) + G8_SQ;
  const int b = tid & 7;
  const int64_t xrow = (int64_t)b * D.K + (int64_t)p * G8_PASS;
  const uint16_t* erow = D.x_embed ? D.E + (int64_t)cur_token_v(smem, b) * D.K + (int64_t)p * G8_PASS : nullptr;
#pragma unroll 1
  for (int j = 0; j < G8_NI; ++j) {
    if (tid + MPK_THREADS * j >= G8_ITEMS) continue;
    const int q = (tid + MPK_THREADS * j) >> 3;  // 8-column group within the pass
    float v[8];
    if (erow) {
      unpack8(gldv<u32x4>(erow + 8 * q), v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = gld(D.x + xrow + 8 * q + e);
    }
    if (D.has_norm) {
      float ssq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ssq = fmaf(v[e], v[e], ssq);
      lds_write_f32(sqb + (uint32_t)(b * 512 + q) * 4u, ssq);
      float gf[8];
      unpack8(gldv<u32x4>(D.gain + p * G8_PASS + 8 * q), gf);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= gf[e];
    }
    u32x4 hi, lo;
    split_hilo8(v, hi, lo);
    const uint32_t a = xb + (uint32_t)(q >> 2) * 1024u + (uint32_t)(16 * (q & 3) + b) * 16u;
    lds_write_u32x4(a, hi);
    lds_write_u32x4(a + 128u, lo);
  }
  (void)s, (void)task_id, (void)Wt, (void)st;
  lds_barrier();
  return *lvi(smem, LDS_CTL) ? -1 : 0;
}

DEV void rms8(const mpk_kparams& P, cop& D, char* smem, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  float* inv = reinterpret_cast<float*>(smem + LDS_INV);
  if (D.has_norm && wave < 8) {
    const float* sq = reinterpret_cast<const float*>(smem + G8_SQ) + wave * 512 + lane * 8;
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t += sq[e];
    t = wave_sum(t);
    if (lane == 0) inv[wave] = 1.0f / sqrtf(t / (float)D.K + P.rms_eps);
  } else if (!D.has_norm && tid < 8) {
    inv[tid] = 1.0f;
  }
  __syncthreads();
}

// Residuals of an EPI_RESID tile into LDS_OUT ([request][output row], the
// layout the epilogue then overwrites with the outputs): polled stamped
// words, embedding rows, or a plain tensor.  Element idx goes to thread
// idx % MPK_THREADS (the thread that later adds its sum); each wavefront polls
// its own words with the watchdog.  Returns -1 on stop.
DEV int gather_resid8(const mpk_kparams& P, cop& D, ctask& T, char* smem, int tid, int s, int task_id, Waiter& Wt,
                      uint32_t st, int n_out_tile) {
  const int lane = tid & 63;
  const uint32_t ob = lds_addr(smem) + LDS_OUT;
  constexpr int PER = (8 * 128 + MPK_THREADS - 1) / MPK_THREADS;  // outputs per thread at most
  uint32_t need = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = tid + k * MPK_THREADS;
    if (idx >= 8 * n_out_tile) continue;
    const int r = idx / n_out_tile, row = T.row0 + idx - r * n_out_tile;
    if (D.res_embed) {
      lds_write_f32(ob + (uint32_t)idx * 4u, bf16f(gld16(D.E + (int64_t)cur_token_v(smem, r) * D.n_out + row)));
    } else if (!D.rll) {
      lds_write_f32(ob + (uint32_t)idx * 4u, gld(D.resid + (int64_t)r * D.n_out + row));
    } else {
      need |= 1u << k;
    }
  }
  for (;;) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (!((need >> k) & 1u)) continue;
      const int idx = tid + k * MPK_THREADS;
      const int r = idx / n_out_tile, row = T.row0 + idx - r * n_out_tile;
      const uint64_t w = ld_ll(D.rll + (int64_t)r * D.n_out + row);
      if (ll_ok(w, st)) {
        lds_write_f32(ob + (uint32_t)idx * 4u, ll_f(w));
        need &= ~(1u << k);
      }
    }
    if (__ballot(need != 0) == 0) break;
    if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  lds_barrier();
  return *lvi(smem, LDS_CTL) ? -1 : 0;
}

// Split K, the merging split: the other splits' partial sums of the outputs
// this thread holds in LDS_OUT (the residuals gather_resid8 left there, same
// element-to-thread map), polled as stamped words, then added to them as
// resid + (p_0 + p_1 + ...) in split order.  Returns -1 on stop.
#define G8_MAXPARTS 2  // splits that publish partials (ksplit <= 3)
DEV int gather_parts8(const mpk_kparams& P, cop& D, ctask& T, char* smem, int tid, int s, int task_id, Waiter& Wt,
                      uint32_t st, int n_out_tile) {
  const int lane = tid & 63;
  const uint32_t ob = lds_addr(smem) + LDS_OUT;
  constexpr int PER = (8 * 128 + MPK_THREADS - 1) / MPK_THREADS;  // outputs per thread at most
  const int np = D.ksplit - 1;
  float pv[PER][G8_MAXPARTS];
  uint32_t need = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
#pragma unroll
    for (int c = 0; c < G8_MAXPARTS; ++c) {
      pv[k][c] = 0.f;
      if (tid + k * MPK_THREADS < 8 * n_out_tile && c < np) need |= 1u << (k * G8_MAXPARTS + c);
    }
  }
  for (;;) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = tid + k * MPK_THREADS;
      const int r = idx / n_out_tile, row = T.row0 + idx - r * n_out_tile;
#pragma unroll
      for (int c = 0; c < G8_MAXPARTS; ++c) {
        if (!((need >> (k * G8_MAXPARTS + c)) & 1u)) continue;
        const uint64_t w = ld_ll(D.pll + ((int64_t)(c * 8 + r) * D.n_out + row));
        if (ll_ok(w, st)) {
          pv[k][c] = ll_f(w);
          need &= ~(1u << (k * G8_MAXPARTS + c));
        }
      }
    }
    if (__ballot(need != 0) == 0) break;
    if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = tid + k * MPK_THREADS;
    if (idx >= 8 * n_out_tile) continue;
    float sum = pv[k][0];
#pragma unroll
    for (int c = 1; c < G8_MAXPARTS; ++c)
      if (c < np) sum += pv[k][c];
    const uint32_t a = ob + (uint32_t)idx * 4u;
    lds_write_f32(a, lds_read_f32(a) + sum);
  }
  lds_barrier();
  return *lvi(smem, LDS_CTL) ? -1 : 0;
}

template <int NBW, int WK>
DEV int gemv8_body(const mpk_kparams& P, ctask& T, cop& D, int s, int task_id, char* smem, int tid, bool sched) {
  constexpr int WR = MPK_NW / WK;       // row groups of waves
  constexpr int KSW = G8_KSTEPS / WK;   // k-steps per wave per pass
  // k-steps of weight loads in flight: the stream rate is set by the bytes in
  // flight, the ring by the registers (168 per lane with three wavefronts on
  // a SIMD, no spills): 16 loads of 1 KB per wave for one block, 8 for two,
  // 12 for three, 10 for five.  Half of them are issued before the inputs
  // are staged (registers for the staging), the rest after.
  constexpr int RG = NBW == 1 ? 16 : (NBW == 2 ? 4 : (NBW == 3 ? 4 : 2));
  static_assert(KSW % RG == 0, "passes hold whole ring rounds");
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int wr = wave / WK, wk = wave % WK;
  const int nrows = uni(T.nrows), row0 = uni(T.row0);
  const int nblk = (nrows + 15) >> 4;
  // split K: this tile's one pass is pass kc of the row (kc = 0: all passes;
  // never in the LM head's body, NBW = 5, which keeps its plain addressing)
  const int kc = NBW != 5 && D.ksplit > 1 ? uni(T.split) : 0;
  const int npass = NBW != 5 && D.ksplit > 1 ? 1 : uni(D.K / G8_PASS);
  const int U = npass * KSW;  // this wave's k-steps over the task
  const uint32_t st = stamp_of(P, s);
  const uint32_t lb = lds_addr(smem);
  const uint32_t xb = lb + LDS_X;
  // weight row of each of this wave's blocks for this lane, at its first column
  const gu32x4* wrow[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    int lr = (wr + WR * j) * 16 + (lane & 15);
    lr = lr < nrows ? lr : nrows - 1;
    wrow[j] = (const gu32x4*)(const void*)(vrow_ptr(D, row0 + lr) + kc * G8_PASS + 8 * (lane >> 4) + wk * KSW * 32);
  }
  // the ring: k-step u of this wave reads columns (u / KSW) G8_PASS + (u % KSW) 32 past wrow.
  // Plain loads, not nontemporal: a row's 128-byte line is read as two 64-byte
  // halves by consecutive k-steps, and the cache has to keep it in between
  // (nontemporal measured 5.50 against 5.18 ms per batch-8 iteration).
  u32x4 ring[RG][NBW];
  auto issue = [&](int u, u32x4(&r)[NBW]) {
    const int pp = u / KSW, t = u - pp * KSW;
    const int off = (pp * G8_PASS + t * 32) / 8;  // in 16-byte units
#pragma unroll
    for (int j = 0; j < NBW; ++j) r[j] = wrow[j][off];
  };
  if (!sched) {
#pragma unroll
    for (int g = 0; g < RG / 2; ++g) issue(g, ring[g]);
  }
  Waiter Wt = waiter_start();
  if (D.x_embed || D.res_embed) {
    const int rc = resolve_tokens(P, smem, tid, s, task_id, Wt);
    if (rc) return rc;
  }
  {
    const int rc = stage_pass8<(NBW != 5)>(P, D, kc, smem, tid, s, task_id, Wt, st);
    if (rc) return rc;
  }
  if (!sched) {
#pragma unroll
    for (int g = RG / 2; g < RG; ++g)
      if (g < U) issue(g, ring[g]);
  }
  rms8(P, D, smem, tid);
  const float* inv = reinterpret_cast<const float*>(smem + LDS_INV);
  mark_ready(P, s, task_id, tid);
  if (tid == 0) *lvi(smem, LDS_SYNCED) = 1;
  f32x4 acc[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int u0 = 0; u0 < U; u0 += RG) {
    if (u0 > 0 && u0 % KSW == 0) {
      // next pass: every wave is done with the staged one
      lds_barrier();
      const int rc = stage_pass8<(NBW != 5)>(P, D, kc + u0 / KSW, smem, tid, s, task_id, Wt, st);
      if (rc) {
        vm_wait<0>();
        return rc;
      }
    }
    if (!sched) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const int ks = wk * KSW + (u0 + g) % KSW;
        const u32x4 B = lds_read_u32x4(xb + (uint32_t)ks * 1024u + (uint32_t)lane * 16u);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ring[g][j]),
                                                           __builtin_bit_cast(bf16x8, B), acc[j], 0, 0, 0);
        if (u0 + g + RG < U) issue(u0 + g + RG, ring[g]);
      }
    }
  }
  // hi + lo: lanes with l % 16 < 8 hold request l % 16, rows 4 (l / 16) + i of each block
#pragma unroll
  for (int j = 0; j < NBW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] += __shfl_xor(acc[j][i], 8);
  const int n = lane & 15, g4 = lane >> 4;
  const uint32_t ob = lb + LDS_OUT;
  if (D.epi == MPK_EPI_ARGMAX) {
    // ---- LM head (WK = 1): logits, this wave's best row per request ----
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (!sched && n < 8) {
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int blk = wr + WR * j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lr = blk * 16 + 4 * g4 + i;
          if (lr < nrows) {
            const float logit = acc[j][i] * inv[n];
            if (D.logits && s < D.logits_iters) gst(D.logits + ((int64_t)s * P.B + n) * D.N0 + row0 + lr, logit);
            if (logit > bv || (logit == bv && row0 + lr < bi)) bv = logit, bi = row0 + lr;
          }
        }
      }
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) bv = ov, bi = oi;
    }
    float* bvs = reinterpret_cast<float*>(smem + LDS_BEST);
    int* bis = reinterpret_cast<int*>(smem + LDS_BEST + MPK_NW * 8 * 4);
    if (!sched && lane < 8) bvs[wave * 8 + lane] = bv, bis[wave * 8 + lane] = bi;
    __syncthreads();
    if (tid < 8) {
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int w = 0; w < MPK_NW; ++w) {
        const float vv = bvs[w * 8 + tid];
        const int ii = bis[w * 8 + tid];
        if (vv > v || (vv == v && ii < ix)) v = vv, ix = ii;
      }
      uint64_t* pw = D.pll + ((int64_t)T.tile * 8 + tid) * 2;
      st_ll(pw, v, st);
      st_lli(pw + 1, ix, st);
    }
    return 0;
  }
  // ---- cross-wave sums (in wave order) into LDS, then the epilogue ----
  lds_barrier();  // every wave is done with the staged x: its area takes the partial sums
  float* red = reinterpret_cast<float*>(smem + LDS_X);  // [WK][nblk][16 rows][8 requests]
  if (!sched && n < 8) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int blk = wr + WR * j;
      if (blk < nblk)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wk * nblk + blk) * 16 + 4 * g4 + i) * 8 + n] = acc[j][i];
    }
  }
  __syncthreads();
  const int n_out_tile = D.pairs ? nrows / 2 : nrows;
  // output o of the tile, request r: its rows' sums over the waves
  auto rowsum = [&](int lr, int r) {
    float v = 0.f;
    for (int k = 0; k < WK; ++k) v += red[((k * nblk + (lr >> 4)) * 16 + (lr & 15)) * 8 + r];
    return v;
  };
  if (D.ksplit > 1 && kc < D.ksplit - 1) {
    // a split that does not merge: its partial sums for the merging split
    for (int idx = tid; idx < 8 * n_out_tile; idx += MPK_THREADS) {
      const int r = idx / n_out_tile, o = idx - r * n_out_tile;
      st_ll(D.pll + ((int64_t)(kc * 8 + r) * D.n_out + row0 + o), rowsum(o, r), st);
    }
    return 0;
  }
  if (D.epi == MPK_EPI_RESID) {
    int rc = gather_resid8(P, D, T, smem, tid, s, task_id, Wt, st, n_out_tile);
    if (!rc && D.ksplit > 1) rc = gather_parts8(P, D, T, smem, tid, s, task_id, Wt, st, n_out_tile);
    if (rc) return rc;
  }
  for (int idx = tid; idx < 8 * n_out_tile; idx += MPK_THREADS) {
    const int r = idx / n_out_tile, o = idx - r * n_out_tile;
    const uint32_t a = ob + (uint32_t)idx * 4u;
    float y;
    if (D.epi == MPK_EPI_SILU) {
      y = silu(rowsum(2 * o, r) * inv[r]) * (rowsum(2 * o + 1, r) * inv[r]);
    } else if (D.epi == MPK_EPI_RESID) {
      y = lds_read_f32(a) + rowsum(o, r);  // this thread's own residual (gather_resid8)
    } else {
      y = rowsum(o, r) * inv[r];
    }
    lds_write_f32(a, y);
  }
  __syncthreads();
  publish_tile<8>(P, D, T, lb, s, st, tid);
  return 0;
}

// Batch-8 linear task: the work split for the tile's blocks.
DEV int gemv8_task(const mpk_kparams& P, ctask& T, cop& D, int s, int task_id, char* smem, int tid, bool sched) {
  const int nblk = (uni(T.nrows) + 15) >> 4;
  if (D.epi == MPK_EPI_ARGMAX) return gemv8_body<5, 1>(P, T, D, s, task_id, smem, tid, sched);
  if (nblk == 1) return gemv8_body<1, 8>(P, T, D, s, task_id, smem, tid, sched);
  if (nblk == 2) return gemv8_body<2, 8>(P, T, D, s, task_id, smem, tid, sched);
  return gemv8_body<3, 4>(P, T, D, s, task_id, smem, tid, sched);
}

// ---------------------------------------------------------------------------
// dispatch of one task body; returns -1 when the run must stop
// ---------------------------------------------------------------------------
template <int NB>
DEV int run_task(const mpk_kparams& P, ctask& T, int task_id, int s, char* smem, int tid, bool sched, int next) {
  cop& D = ops_of(P)[T.op];
  if (T.kind == MPK_TK_ATTN)
    return D.d == 128 ? attn_task<128>(P, T, D, smem, tid, sched, s, task_id)
                      : attn_task<64>(P, T, D, smem, tid, sched, s, task_id);
  if (T.kind == MPK_TK_ARGMAX) return argmax_task<NB>(P, D, smem, tid, s, task_id);
  if constexpr (NB == 8) {
    (void)next;
    return gemv8_task(P, T, D, s, task_id, smem, tid, sched);
  } else {
    return gemv_task<NB>(P, T, D, s, task_id, smem, tid, sched, next);
  }
}

// ---------------------------------------------------------------------------
// the persistent kernel
// ---------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(MPK_THREADS, 1) void mpk_persistent(mpk_kparams P) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool sched = wave == MPK_NW;
  cqent* Q = (cqent*)(const void*)P.queues + (int64_t)blockIdx.x * P.qstride;
  const int qlen = ((const CAS int32_t*)(const void*)P.qlen)[blockIdx.x];
  // a failed start-of-run check (or a stop already recorded): no work at all
  if (uni(__hip_atomic_load(&P.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0) return;
  lds_vi* ctl = lvi(smem, LDS_CTL);
  if (tid == 0) ctl[0] = 0;
  if (sched) load_positions(P, smem, lane);
  for (int s = 0; s < P.n_iter; ++s) {
    for (int k = 0; k < qlen; ++k) {
      const int task_id = Q[k].task;
      ctask& T = tasks_of(P)[task_id];
      if (k == 0) {
        if (sched) set_positions(P, smem, s, lane);
        if (tid == 0) *lvi(smem, LDS_SYNCED) = 0;
        __syncthreads();
      }
      if (sched && lane == 0 && P.trace) {
        mpk_trace_record& Rr = P.trace[(int64_t)s * P.n_tasks + task_id];
        Rr.task = task_id;
        Rr.iteration = s;
        Rr.t_start = clock_now();
        Rr.hw_id = hwreg_hw_id();
        Rr.xcc_id = hwreg_xcc_id();
      }
      // An opaque copy of the thread id per task keeps the compiler from
      // hoisting per-lane address arithmetic of every body out of the task
      // loop (it would stay live, and spill, across all bodies).
      int tid_o = tid;
      asm volatile("" : "+v"(tid_o));
      const int rc = run_task<NB>(P, T, task_id, s, smem, tid_o, sched, k + 1 < qlen ? Q[k + 1].task : -1);
      if (rc < 0) {
        vm_wait<0>();  // leave no load in flight
        return;
      }
      __syncthreads();
      if (sched && lane == 0 && P.trace) {
        mpk_trace_record& Rr = P.trace[(int64_t)s * P.n_tasks + task_id];
        Rr.end_ticket = P.trace_tickets ? __hip_atomic_fetch_add(P.ticket_ctr, 1u, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT) : 0u;
        Rr.t_end = clock_now();
      }
    }
  }
  vm_wait<0>();
}

// One operator's tasks as one ordinary launch (grid = the operator's tiles),
// for the one-launch-per-operator comparison.  Same bodies, same tiles.
template <int NB>
__global__ __launch_bounds__(MPK_THREADS, 1) void mpk_op_kernel(mpk_kparams P, int first_task, int s) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool sched = wave == MPK_NW;
  const int task_id = first_task + blockIdx.x;
  ctask& T = tasks_of(P)[task_id];
  if (uni(__hip_atomic_load(&P.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0) return;
  lds_vi* ctl = lvi(smem, LDS_CTL);
  if (tid == 0) ctl[0] = 0;
  // every earlier launch (every earlier iteration) has ended
  if (tid == 0) *lvi(smem, LDS_SYNCED) = 1;
  if (sched) load_positions(P, smem, lane);
  if (sched) set_positions(P, smem, s, lane);
  __syncthreads();
  run_task<NB>(P, T, task_id, s, smem, tid, sched, -1);
  vm_wait<0>();
}

// First kernel of every run, on the run's stream: clears the status word
// (not the host's stop request) and the trace ticket counter, records each
// request's position at launch (pos0) for the run's kernels, and checks what
// the run will consume: 0 <= step[r], step[r] + n < tokens width,
// step[r] + n <= max_seq, and every token id read from `tokens` (position
// step[r], and the prompt ids at step[r] + 1 .. step[r] + n - 1 that the
// iterations feed forward) inside [0, vocab).  A failed check records
// MPK_ERR_SHAPE with iteration -1 and the request as the task; every kernel
// of the run then returns at once.  Same rule as mpk_check_run on the host.
// One workgroup of 64 threads.
__global__ void mpk_begin_run(mpk_kparams P, int n_iter) {
  const int lane = threadIdx.x;
  if (lane == 0) {
    P.status->code = 0;
    P.status->iteration = 0;
    P.status->task = 0;
    *P.ticket_ctr = 0u;
  }
  __syncthreads();
  const int64_t n_pos = (int64_t)P.rpr * n_iter;  // positions each request consumes
  for (int r = 0; r < P.B / P.rpr; ++r) {
    const int p0 = P.step[r];
    const int plen = P.prompt_len[r];
    bool bad = p0 < 0 || p0 + n_pos >= P.tokens_width || p0 + n_pos > P.max_seq ||
               (P.rpr > 1 && p0 + n_pos > plen - 1);
    if (!bad) {
      // ids read from tokens: position p0, and q in (p0, p0 + n) below the
      // prompt's end; batched ingestion reads every consumed position
      const int q_end = P.rpr > 1 ? (int)(p0 + n_pos) : min(p0 + n_iter, max(plen, p0 + 1));
      for (int q = p0 + lane; q < q_end; q += 64) {
        const int t = P.tokens[(int64_t)r * P.tokens_width + q];
        bad |= t < 0 || t >= P.vocab;
      }
    }
    if (__ballot(bad) != 0) {
      if (lane == 0) {
        P.status->code = MPK_ERR_SHAPE;
        P.status->iteration = -1;
        P.status->task = r;
      }
      return;
    }
    if (lane == 0) P.pos0[r] = p0;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct mpk_exec_s {
  int device = 0;
  mpk_graph_t g = nullptr;
  int B = 1;
  std::vector<void*> owned;     // library allocations
  std::vector<void*> tensor_ptr;
  mpk_dev_task* d_tasks = nullptr;
  mpk_dev_op* d_ops = nullptr;
  mpk_dev_qentry* d_queues = nullptr;
  int32_t* d_qlen = nullptr;
  uint32_t* d_ticket_ctr = nullptr;  // trace ticket counter
  uint64_t* d_tok_ll = nullptr;      // [B] stamped next token
  std::vector<uint64_t*> ll_ptr;     // per tensor: stamped words of an operator output, or NULL
  std::vector<uint32_t*> pk_ptr;     // per tensor: packed twin of ll_ptr, or NULL
  std::pair<void*, size_t> pk_buf{nullptr, 0};  // the packed twins (one allocation; run scratch)
  void* pk_buf_static = nullptr;     // the same in the static array
  uint64_t pk_clear_base = 0;        // stamp counter when the own packed twins were last cleared
  float* d_rope = nullptr;
  mpk_dev_status* d_status = nullptr;
  int32_t* d_pos0 = nullptr;         // [MPK_MAX_BATCH] positions at launch (mpk_begin_run)
  mpk_trace_record* d_trace = nullptr;
  int64_t trace_cap = 0;  // records
  int last_iters = 0;
  hipStream_t side = nullptr;
  const void* kernel_persistent = nullptr;
  const void* kernel_op = nullptr;
  int lds_bytes = 0;
  mpk_kparams kp{};
  // Run scratch: every buffer the run's kernels write besides the caller's
  // tensors (stamped words, split partials, tile maxima, token words,
  // status, ticket, positions), in allocation order; mpk_run_steps_static
  // places the same buffers at the same offsets in the static array.
  std::vector<std::pair<void*, size_t>> scratch;
  size_t scratch_bytes = 0;           // their total, each rounded up to 256 bytes
  mpk_dev_op* d_ops_static = nullptr; // operator table pointing into the static array (NULL: does not fit)
  mpk_kparams kp_static{};
  mpk_dev_status* last_status = nullptr;  // status word of the last run (own or static)
};

#define HIPCHK(x)                                                                          \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess)                                                                  \
      return mpk_fail(MPK_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_));        \
  } while (0)

template <int NB>
static void kernels_for(const void** pers, const void** op, int* lds) {
  *pers = reinterpret_cast<const void*>(&mpk_persistent<NB>);
  *op = reinterpret_cast<const void*>(&mpk_op_kernel<NB>);
  *lds = Lay<NB>::TOTAL;
}

static int select_kernels(int B, const void** pers, const void** op, int* lds) {
  switch (B) {
    case 1: kernels_for<1>(pers, op, lds); return MPK_OK;
    case 2: kernels_for<2>(pers, op, lds); return MPK_OK;
    case 8: kernels_for<8>(pers, op, lds); return MPK_OK;
    default:
      return mpk_fail(MPK_ERR_SHAPE, "this build runs num_requests in {1, 2, 8}");
  }
}

template <typename T>
static int dalloc(mpk_exec_s* x, T** p, size_t bytes) {
  void* q = nullptr;
  HIPCHK(hipMalloc(&q, bytes ? bytes : 16));
  HIPCHK(hipMemset(q, 0, bytes ? bytes : 16));
  x->owned.push_back(q);
  *p = reinterpret_cast<T*>(q);
  return MPK_OK;
}

// A buffer the run's kernels write (see mpk_exec_s::scratch).
template <typename T>
static int salloc(mpk_exec_s* x, T** p, size_t bytes) {
  const int rc = dalloc(x, p, bytes);
  if (rc) return rc;
  x->scratch.emplace_back((void*)*p, bytes);
  x->scratch_bytes += (bytes + 255) & ~(size_t)255;
  return MPK_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free runs (mpk_run_steps_static).  The run scratch lives in one
// file-scope device array per GPU, held until the process ends.  Host code
// never uses the array's name as an address: its device address is taken
// once per device with hipGetSymbolAddress (at the first mpk_compile on that
// device, with the device current) and kept per device.
// ---------------------------------------------------------------------------
#define MPK_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
#define MPK_MAX_DEVICES 64
static __device__ __align__(256) unsigned char scratch[MPK_STATIC_SCRATCH_BYTES];

__global__ void mpk_fill_zero(uint4* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[MPK_MAX_DEVICES];
// Per device: the executable whose allocation-free run used the static
// array last, and the stamp counter when its packed twins there were
// cleared (see prepare_run).
static const void* g_static_owner[MPK_MAX_DEVICES];
static uint64_t g_static_pk_base[MPK_MAX_DEVICES];

// Device address of the static array on `device` (current), cleared once:
// stamped words left in it by earlier runs of this process carry stamps no
// later run uses, but the array's first contents are unknown.
static int static_scratch(int device, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (device < 0 || device >= MPK_MAX_DEVICES) return mpk_fail(MPK_ERR_INVALID_ARG, "device ordinal out of range");
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    hipLaunchKernelGGL(mpk_fill_zero, dim3(1024), dim3(256), 0, 0, (uint4*)p,
                       (int64_t)(MPK_STATIC_SCRATCH_BYTES / sizeof(uint4)));
    HIPCHK(hipGetLastError());
    HIPCHK(hipDeviceSynchronize());
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return MPK_OK;
}

// The static operator table and kernel parameters of x: the same buffers at
// the same offsets in the static array.  Left unset when they do not fit.
static int build_static_tables(mpk_exec_s* x, const std::vector<mpk_dev_op>& dops) {
  if (x->scratch_bytes > MPK_STATIC_SCRATCH_BYTES) return MPK_OK;
  void* base = nullptr;
  int rc = static_scratch(x->device, &base);
  if (rc) return rc;
  struct span {
    const char* own;
    size_t bytes;
    char* at;  // static address
  };
  std::vector<span> map;  // own buffer -> static address
  size_t off = 0;
  for (const auto& b : x->scratch) {
    map.push_back({(const char*)b.first, b.second, (char*)base + off});
    off += (b.second + 255) & ~(size_t)255;
  }
  // a pointer into a scratch buffer (its start or inside it, as the packed
  // twins that share one allocation) moves with the buffer
  auto remap = [&](auto* p) -> decltype(p) {
    if (!p) return p;
    const char* c = (const char*)(const void*)p;
    for (const auto& m : map)
      if (c >= m.own && c < m.own + m.bytes) return reinterpret_cast<decltype(p)>(m.at + (c - m.own));
    return p;  // caller memory (attached tensors) is not scratch
  };
  std::vector<mpk_dev_op> sops = dops;
  for (mpk_dev_op& D : sops) {
    D.xll = remap(D.xll);
    D.rll = remap(D.rll);
    D.yll = remap(D.yll);
    D.pll = remap(D.pll);
    D.xpk = remap(D.xpk);
    D.ypk = remap(D.ypk);
  }
  if ((rc = dalloc(x, &x->d_ops_static, sops.size() * sizeof(mpk_dev_op)))) return rc;
  HIPCHK(hipMemcpy(x->d_ops_static, sops.data(), sops.size() * sizeof(mpk_dev_op), hipMemcpyHostToDevice));
  mpk_kparams& K = x->kp_static;
  K = x->kp;
  K.ops = x->d_ops_static;
  K.tok_ll = remap(x->kp.tok_ll);
  K.status = remap(x->kp.status);
  K.ticket_ctr = remap(x->kp.ticket_ctr);
  K.pos0 = remap(x->kp.pos0);
  x->pk_buf_static = remap(x->pk_buf.first);
  return MPK_OK;
}

// Iteration stamps handed out so far in this process (see prepare_run).
static std::atomic<uint64_t> g_stamps{0};

static int64_t tensor_bytes(const mpk_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.dims[i];
  return n * (t.dtype == MPK_BF16 ? 2 : 4);
}

extern "C" int mpk_compile(mpk_graph_t g, int32_t device, mpk_exec_t* out) {
  mpk_clear_error();
  if (!g || !out) return mpk_fail(MPK_ERR_INVALID_ARG, "mpk_compile: NULL argument");
  *out = nullptr;
  HIPCHK(hipSetDevice(device));
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, device));
  if (prop.multiProcessorCount != g->num_queues)
    return mpk_fail(MPK_ERR_SPLIT, "graph built for " + std::to_string(g->num_queues) +
                                       " CUs, device has " +
                                       std::to_string(prop.multiProcessorCount));
  int coop = 0;
  HIPCHK(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device));
  if (!coop) return mpk_fail(MPK_ERR_NOT_CORESIDENT, "device has no cooperative launch");

  std::unique_ptr<mpk_exec_s, void (*)(mpk_exec_s*)> x(new mpk_exec_s(), [](mpk_exec_s* e) {
    mpk_destroy_exec(e);
  });
  x->device = device;
  x->g = g;
  x->B = g->rows;
  int rc = select_kernels(x->B, &x->kernel_persistent, &x->kernel_op, &x->lds_bytes);
  if (rc) return rc;
  HIPCHK(hipFuncSetAttribute(x->kernel_persistent, hipFuncAttributeMaxDynamicSharedMemorySize, x->lds_bytes));
  HIPCHK(hipFuncSetAttribute(x->kernel_op, hipFuncAttributeMaxDynamicSharedMemorySize, x->lds_bytes));
  int per_cu = 0;
  HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, x->kernel_persistent, MPK_THREADS, x->lds_bytes));
  if (per_cu < 1)
    return mpk_fail(MPK_ERR_NOT_CORESIDENT, "persistent kernel cannot be resident (occupancy 0)");

  // tensors
  const int NTEN = (int)g->tensors.size();
  x->tensor_ptr.assign(NTEN, nullptr);
  // Operator outputs in f32 are handed between tasks as stamped words (one
  // 64-bit word per element); an attached output is also written plainly.
  x->ll_ptr.assign(NTEN, nullptr);
  for (int i = 0; i < NTEN; ++i) {
    const mpk_tensor& t = g->tensors[i];
    const bool produced = g->producer[i] >= 0 && g->embed_src[i] < 0;
    if (produced && t.dtype == MPK_F32) {
      const int64_t n = tensor_bytes(t) / 4;
      if ((rc = salloc(x.get(), &x->ll_ptr[i], (size_t)n * 8))) return rc;
    }
    if (t.dev_ptr) {
      x->tensor_ptr[i] = t.dev_ptr;
    } else if (x->ll_ptr[i]) {
      x->tensor_ptr[i] = x->ll_ptr[i];
    } else if (g->embed_src[i] < 0) {
      if ((rc = dalloc(x.get(), &x->tensor_ptr[i], (size_t)tensor_bytes(t)))) return rc;
    }
  }
  auto P = [&](int id) -> void* { return id >= 0 ? x->tensor_ptr[id] : nullptr; };
  // plain pointer of an attached tensor (NULL for library-owned stamped ones)
  auto PA = [&](int id) -> void* { return id >= 0 && g->tensors[id].dev_ptr ? x->tensor_ptr[id] : nullptr; };
  auto PL = [&](int id) -> uint64_t* { return id >= 0 ? x->ll_ptr[id] : nullptr; };
  // Packed twins (mpk_dev_op::xpk) of the stamped outputs that GEMV tasks
  // gather as their input x: the outputs of attention, linear + residual and
  // gate/up operators, when the consumer's K is a multiple of 256.
  // All twins share one allocation (cleared in one pass, see prepare_run).
  x->pk_ptr.assign(NTEN, nullptr);
  {
    std::vector<size_t> off(NTEN, SIZE_MAX);
    size_t total = 0;
    for (size_t i = 0; i < g->ops.size(); ++i) {
      const mpk_op& o = g->ops[i];
      const bool gemv_in = o.kind == MPK_OP_RMSNORM_LINEAR || o.kind == MPK_OP_LINEAR_RESIDUAL ||
                           o.kind == MPK_OP_RMSNORM_GATEUP || o.kind == MPK_OP_LMHEAD_ARGMAX;
      if (!gemv_in || o.in[0] < 0 || !x->ll_ptr[o.in[0]] || g->dops[i].K % 256 != 0) continue;
      const int src = o.in[0];
      const int prod = g->producer[src];
      if (prod < 0) continue;
      const int pkind = g->ops[prod].kind;
      if (pkind != MPK_OP_ATTENTION && pkind != MPK_OP_LINEAR_RESIDUAL && pkind != MPK_OP_RMSNORM_GATEUP) continue;
      if (off[src] == SIZE_MAX) {
        off[src] = total;
        total += ((size_t)tensor_bytes(g->tensors[src]) + 255) & ~(size_t)255;  // one 32-bit word per f32
      }
    }
    if (total) {
      uint32_t* blk = nullptr;
      if ((rc = salloc(x.get(), &blk, total))) return rc;
      for (int t = 0; t < NTEN; ++t)
        if (off[t] != SIZE_MAX) x->pk_ptr[t] = (uint32_t*)((char*)blk + off[t]);
      x->pk_buf = {(void*)blk, total};
    }
  }
  x->pk_clear_base = g_stamps.load();
  auto PK = [&](int id) -> uint32_t* { return id >= 0 ? x->pk_ptr[id] : nullptr; };
  const mpk_model_cfg& M = g->model;
  const int B = x->B;

  std::vector<mpk_dev_op> dops = g->dops;
  if ((rc = salloc(x.get(), &x->d_ticket_ctr, 4))) return rc;
  if ((rc = salloc(x.get(), &x->d_tok_ll, (size_t)B * 8))) return rc;

  for (size_t i = 0; i < dops.size(); ++i) {
    mpk_dev_op& D = dops[i];
    if (!D.kind || D.kind == MPK_TK_ARGMAX) continue;
    const mpk_op& o = g->ops[i];
    if (D.kind == MPK_TK_ATTN) {
      D.xll = PL(o.in[0]);
      if (!D.xll) return mpk_fail(MPK_ERR_GRAPH, "attention input must be the output of an operator");
      D.qn = (const uint16_t*)P(o.in[1]);
      D.kn = (const uint16_t*)P(o.in[2]);
      D.kc = (uint16_t*)P(o.in[3]);
      D.vc = (uint16_t*)P(o.in[4]);
      D.y = (float*)PA(o.out[0]);
      D.yll = PL(o.out[0]);
      D.ypk = PK(o.out[0]);
      const int G = D.nq / D.nkv;
      if (G > ATT_MAXG) return mpk_fail(MPK_ERR_SHAPE, "more than 4 query heads per kv head");
      if (D.d != 64 && D.d != 128) return mpk_fail(MPK_ERR_SHAPE, "head_dim must be 64 or 128");
      if ((rc = salloc(x.get(), &D.pll, (size_t)B * D.nkv * D.nsplit * G * (D.d + 2) * 8))) return rc;
      continue;
    }
    const int e_in = o.in[0];
    D.xll = D.x_embed ? nullptr : PL(e_in);
    // (the batch-8 LM head stages the stamped words: see stage_pass8)
    D.xpk = D.x_embed || (B == 8 && o.kind == MPK_OP_LMHEAD_ARGMAX) ? nullptr : PK(e_in);
    D.x = D.x_embed || D.xll ? nullptr : (const float*)P(e_in);
    if (D.x_embed) D.E = (const uint16_t*)P(g->embed_src[e_in]);
    D.gain = D.has_norm ? (const uint16_t*)P(o.in[1]) : nullptr;
    if (o.kind == MPK_OP_RMSNORM_LINEAR) {
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.W1 = (const uint16_t*)P(o.in[3]);
      D.W2 = (const uint16_t*)P(o.in[4]);
      D.y = (float*)PA(o.out[0]);
      D.yll = PL(o.out[0]);
    } else if (o.kind == MPK_OP_LINEAR_RESIDUAL) {
      D.W0 = (const uint16_t*)P(o.in[1]);
      if (D.res_embed) {
        D.E = (const uint16_t*)P(g->embed_src[o.in[2]]);
      } else {
        D.rll = PL(o.in[2]);
        D.resid = D.rll ? nullptr : (const float*)P(o.in[2]);
      }
      D.y = (float*)PA(o.out[0]);
      D.yll = PL(o.out[0]);
      D.ypk = PK(o.out[0]);
      if (D.ksplit > 1) {
        if (D.ksplit - 1 > G8_MAXPARTS || B != 8) return mpk_fail(MPK_ERR_SHAPE, "split K beyond its limits");
        if ((rc = salloc(x.get(), &D.pll, (size_t)(D.ksplit - 1) * B * D.n_out * 8))) return rc;
      }
    } else if (o.kind == MPK_OP_RMSNORM_GATEUP) {
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.W1 = (const uint16_t*)P(o.in[3]);
      D.y = (float*)PA(o.out[0]);
      D.yll = PL(o.out[0]);
      D.ypk = PK(o.out[0]);
    } else {  // LM head
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.logits = o.out[0] >= 0 ? (float*)P(o.out[0]) : nullptr;
      if ((rc = salloc(x.get(), &D.pll, (size_t)D.ntiles * B * 2 * 8))) return rc;
    }
  }
  if (g->argmax_op >= 0) {
    // the argmax task reads the LM head's per-tile (max, index) pairs
    const int lm = g->argmax_op - 1;
    dops[g->argmax_op].pll = dops[lm].pll;
    dops[g->argmax_op].N1 = dops[lm].ntiles;
  }
  if ((rc = dalloc(x.get(), &x->d_ops, dops.size() * sizeof(mpk_dev_op)))) return rc;
  HIPCHK(hipMemcpy(x->d_ops, dops.data(), dops.size() * sizeof(mpk_dev_op), hipMemcpyHostToDevice));
  if ((rc = dalloc(x.get(), &x->d_tasks, g->tasks.size() * sizeof(mpk_dev_task)))) return rc;
  HIPCHK(hipMemcpy(x->d_tasks, g->tasks.data(), g->tasks.size() * sizeof(mpk_dev_task), hipMemcpyHostToDevice));
  if ((rc = dalloc(x.get(), &x->d_queues, g->queues.size() * sizeof(mpk_dev_qentry)))) return rc;
  HIPCHK(hipMemcpy(x->d_queues, g->queues.data(), g->queues.size() * sizeof(mpk_dev_qentry), hipMemcpyHostToDevice));
  if ((rc = dalloc(x.get(), &x->d_qlen, g->qlen.size() * 4))) return rc;
  HIPCHK(hipMemcpy(x->d_qlen, g->qlen.data(), g->qlen.size() * 4, hipMemcpyHostToDevice));
  if ((rc = salloc(x.get(), &x->d_status, sizeof(mpk_dev_status)))) return rc;
  if ((rc = salloc(x.get(), &x->d_pos0, MPK_MAX_BATCH * sizeof(int32_t)))) return rc;

  // RoPE table, fp64 angles rounded to fp32 (pair i of a head: angle p * theta^(-2i/d))
  const int half = M.head_dim / 2;
  std::vector<float> rope((size_t)2 * M.max_seq * half);
  for (int p = 0; p < M.max_seq; ++p)
    for (int i = 0; i < half; ++i) {
      double ang = (double)p * std::pow((double)M.rope_theta, -2.0 * i / (double)M.head_dim);
      rope[(size_t)p * half + i] = (float)std::cos(ang);
      rope[(size_t)M.max_seq * half + (size_t)p * half + i] = (float)std::sin(ang);
    }
  if ((rc = dalloc(x.get(), &x->d_rope, rope.size() * 4))) return rc;
  HIPCHK(hipMemcpy(x->d_rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(hipStreamCreateWithFlags(&x->side, hipStreamNonBlocking));

  mpk_kparams& K = x->kp;
  K.tasks = x->d_tasks;
  K.ops = x->d_ops;
  K.queues = x->d_queues;
  K.qlen = x->d_qlen;
  K.tok_ll = x->d_tok_ll;
  K.tokens = (int32_t*)P(g->meta.tokens);
  K.step = (int32_t*)P(g->meta.step);
  K.prompt_len = (const int32_t*)P(g->meta.prompt_len);
  K.rope_cos = x->d_rope;
  K.rope_sin = x->d_rope + (size_t)M.max_seq * half;
  K.status = x->d_status;
  K.abort_req = &x->d_status->abort_req;
  K.trace = nullptr;
  K.ticket_ctr = x->d_ticket_ctr;
  uint64_t ns = g->launch.spin_timeout_ns ? g->launch.spin_timeout_ns : 2000000000ull;
  K.timeout_ticks = ns / 10;  // s_memrealtime runs at 100 MHz
  K.qstride = g->max_queue;
  K.n_tasks = (int)g->tasks.size();
  K.B = B;
  K.rpr = g->rpr;
  K.tokens_width = (int)g->tensors[g->meta.tokens].dims[1];
  K.rope_half = half;
  K.rms_eps = M.rms_eps;
  K.vocab = M.vocab;
  K.max_seq = M.max_seq;
  K.pos0 = x->d_pos0;
  // The zero fills above (hipMemset) are ordered on the null stream only;
  // a run on another stream must never see a buffer before it is zeroed (a
  // reused allocation could still hold words stamped by an earlier
  // executable).
  x->last_status = x->d_status;
  if ((rc = build_static_tables(x.get(), dops))) return rc;
  HIPCHK(hipDeviceSynchronize());
  *out = x.release();
  return MPK_OK;
}


// Host checks, stamps and the start-of-run kernel of a run with parameters
// K (x->kp, or x->kp_static for an allocation-free run).
static int prepare_run(mpk_exec_t x, int32_t n_iter, hipStream_t st, mpk_kparams& K) {
  if (n_iter <= 0) return mpk_fail(MPK_ERR_INVALID_ARG, "num_iterations must be positive");
  // Checks that need no device value; positions and token ids are checked
  // on the device by mpk_begin_run (no host round trip per launch).
  if ((int64_t)K.rpr * n_iter >= K.tokens_width || (int64_t)K.rpr * n_iter > x->g->model.max_seq)
    return mpk_fail(MPK_ERR_SHAPE, std::to_string(n_iter) + " iterations leave the tokens tensor or the KV cache");
  for (size_t i = 0; i < x->g->dops.size(); ++i) {
    const mpk_dev_op& D = x->g->dops[i];
    if (D.kind == MPK_TK_LMHEAD && x->g->ops[i].out[0] >= 0 && D.logits_iters < n_iter)
      return mpk_fail(MPK_ERR_SHAPE, "logits tensor holds fewer iterations than requested");
  }
  HIPCHK(hipSetDevice(x->device));
  // trace buffer (allocated by the first traced run that needs more room)
  K.trace = nullptr;
  if (x->g->launch.trace) {
    int64_t need = (int64_t)n_iter * K.n_tasks;
    if (need > x->trace_cap) {
      void* p = nullptr;
      HIPCHK(hipMalloc(&p, (size_t)need * sizeof(mpk_trace_record)));
      x->owned.push_back(p);
      x->d_trace = (mpk_trace_record*)p;
      x->trace_cap = need;
    }
    HIPCHK(hipMemsetAsync(x->d_trace, 0xff, (size_t)need * sizeof(mpk_trace_record), st));
    K.trace = x->d_trace;
    K.trace_tickets = x->g->launch.trace == 1;
  }
  K.n_iter = n_iter;
  x->last_iters = n_iter;
  // stamps of this run: base + 1 .. base + n_iter, taken from a counter
  // shared by every executable of the process, so no two runs (of this or
  // any other executable) ever use the same stamp
  const uint64_t base = g_stamps.fetch_add((uint64_t)n_iter);
  if (base + (uint64_t)n_iter >= 0xffffffffull)
    return mpk_fail(MPK_ERR_STATE, "iteration stamps exhausted (2^32 iterations per process)");
  K.iter_base = (uint32_t)base;
  // Packed twins carry 8-bit stamps (st mod 255 + 1).  A word left from an
  // earlier run was written with a stamp in (clear base, base]; the first
  // iteration's stamp base + 1 could match it only if it is 255 or more
  // stamps old, so the twins are cleared (to stamp 0, never current) first
  // when the counter has moved 255 or more since they were last cleared, and
  // in the static array also when another executable used it last.
  if (x->pk_buf.second) {
    const bool stat = &K == &x->kp_static;
    void* p = stat ? x->pk_buf_static : x->pk_buf.first;
    bool clear;
    if (stat) {
      std::lock_guard<std::mutex> lk(g_scratch_mu);
      clear = g_static_owner[x->device] != (const void*)x || base - g_static_pk_base[x->device] >= 255;
      if (clear) g_static_owner[x->device] = x, g_static_pk_base[x->device] = base;
    } else {
      clear = base - x->pk_clear_base >= 255;
      if (clear) x->pk_clear_base = base;
    }
    if (clear) {
      const int64_t n16 = (int64_t)(x->pk_buf.second / 16);
      hipLaunchKernelGGL(mpk_fill_zero, dim3((unsigned)std::min<int64_t>(1024, (n16 + 255) / 256)), dim3(256), 0, st,
                         (uint4*)p, n16);
      HIPCHK(hipGetLastError());
    }
  }
  // status, trace ticket, positions at launch, checks of step / tokens
  hipLaunchKernelGGL(mpk_begin_run, dim3(1), dim3(64), 0, st, K, (int)n_iter);
  HIPCHK(hipGetLastError());
  x->last_status = K.status == x->kp.status ? x->d_status : x->kp_static.status;
  return MPK_OK;
}

extern "C" int mpk_run_steps(mpk_exec_t x, int32_t n_iter, void* stream) {
  mpk_clear_error();
  if (!x) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL exec");
  hipStream_t st = (hipStream_t)stream;
  int rc = prepare_run(x, n_iter, st, x->kp);
  if (rc) return rc;
  void* args[] = {&x->kp};
  HIPCHK(hipLaunchCooperativeKernel(x->kernel_persistent, dim3(x->g->num_queues), dim3(MPK_THREADS), args,
                                    x->lds_bytes, st));
  return MPK_OK;
}

extern "C" int mpk_run_steps_static(mpk_exec_t x, int32_t n_iter, void* stream) {
  mpk_clear_error();
  if (!x) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL exec");
  if (!x->d_ops_static)
    return mpk_fail(MPK_ERR_SHAPE, "the run scratch of this graph needs " + std::to_string(x->scratch_bytes) +
                                       " bytes; the static array holds " +
                                       std::to_string(MPK_STATIC_SCRATCH_BYTES));
  if (x->g->launch.trace)
    return mpk_fail(MPK_ERR_INVALID_ARG, "a traced graph needs a trace buffer; the allocation-free run has none");
  hipStream_t st = (hipStream_t)stream;
  int rc = prepare_run(x, n_iter, st, x->kp_static);
  if (rc) return rc;
  void* args[] = {&x->kp_static};
  HIPCHK(hipLaunchCooperativeKernel(x->kernel_persistent, dim3(x->g->num_queues), dim3(MPK_THREADS), args,
                                    x->lds_bytes, st));
  return MPK_OK;
}

extern "C" int mpk_run_steps_per_op(mpk_exec_t x, int32_t n_iter, void* stream) {
  mpk_clear_error();
  if (!x) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL exec");
  hipStream_t st = (hipStream_t)stream;
  int rc = prepare_run(x, n_iter, st, x->kp);
  if (rc) return rc;
  x->kp.trace = nullptr;
  const mpk_graph_s* g = x->g;
  for (int s = 0; s < n_iter; ++s)
    for (size_t i = 0; i < g->dops.size(); ++i) {
      if (!g->op_ntasks[i]) continue;
      int first = g->op_first_task[i];
      void* args[] = {&x->kp, &first, &s};
      HIPCHK(hipLaunchKernel(x->kernel_op, dim3(g->op_ntasks[i]), dim3(MPK_THREADS), args, x->lds_bytes, st));
    }
  return MPK_OK;
}

extern "C" int mpk_get_status(mpk_exec_t x, int32_t* code, int32_t* iteration, int32_t* task) {
  mpk_clear_error();
  if (!x) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL exec");
  mpk_dev_status s{};
  HIPCHK(hipSetDevice(x->device));
  HIPCHK(hipMemcpy(&s, x->last_status, sizeof(s), hipMemcpyDeviceToHost));
  if (code) *code = s.code;
  if (iteration) *iteration = s.code ? s.iteration : -1;
  if (task) *task = s.code ? s.task : -1;
  return MPK_OK;
}

extern "C" int mpk_set_abort(mpk_exec_t x, int32_t flag) {
  mpk_clear_error();
  if (!x) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL exec");
  HIPCHK(hipSetDevice(x->device));
  int32_t v = flag ? 1 : 0;
  HIPCHK(hipMemcpyAsync(&x->d_status->abort_req, &v, 4, hipMemcpyHostToDevice, x->side));
  HIPCHK(hipStreamSynchronize(x->side));
  return MPK_OK;
}

extern "C" int mpk_read_trace(mpk_exec_t x, void* host_buf, size_t bytes, size_t* written) {
  mpk_clear_error();
  if (!x || !host_buf) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL argument");
  if (!x->d_trace || !x->last_iters) return mpk_fail(MPK_ERR_STATE, "no trace recorded");
  size_t have = (size_t)x->last_iters * x->kp.n_tasks * sizeof(mpk_trace_record);
  size_t n = std::min(bytes, have);
  n -= n % sizeof(mpk_trace_record);
  HIPCHK(hipSetDevice(x->device));
  HIPCHK(hipMemcpy(host_buf, x->d_trace, n, hipMemcpyDeviceToHost));
  if (written) *written = n;
  return MPK_OK;
}

extern "C" int mpk_get_tensor_ptr(mpk_exec_t x, int32_t id, void** p) {
  mpk_clear_error();
  if (!x || !p || id < 0 || id >= (int)x->tensor_ptr.size())
    return mpk_fail(MPK_ERR_INVALID_ARG, "bad tensor id");
  *p = x->tensor_ptr[id];
  return MPK_OK;
}

extern "C" void mpk_destroy_exec(mpk_exec_t x) {
  if (!x) return;
  (void)hipSetDevice(x->device);
  for (void* p : x->owned) (void)hipFree(p);
  if (x->side) (void)hipStreamDestroy(x->side);
  delete x;
}
