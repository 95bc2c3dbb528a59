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
#include <string>
#include <vector>

#include "graph.hpp"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// float -> bf16 bits, round to nearest even
DEV uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
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

// K and V of two position rounds from an LDS ring slot: [K0][K1][V0][V1],
// 1 KB each, this lane's 16 bytes at a (early-clobber outputs, see
// lds_read_2f4).
DEV void lds_read_kv2(uint32_t a, u32x4 (&K)[2], u32x4 (&V)[2]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(K[0]), "=&v"(K[1]), "=&v"(V[0]), "=&v"(V[1])
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
// 16 bytes written earlier in the launch by another CU, possibly on another
// XCD (the K/V rows of earlier positions): device-scope loads, since a plain
// load may hit a line of this XCD's L2 that predates the write.
DEV u32x4 ld_dev16(const void* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<void*>(p));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
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
static_assert(Lay<1>::RES + LDS_RES_BYTES <= Lay<1>::TOTAL, "LDS budget");
static_assert(Lay<2>::RES + LDS_RES_BYTES <= Lay<2>::TOTAL, "LDS budget");

DEV void lds_write_f32(uint32_t a, float v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(v) : "memory");
}
DEV void lds_write_f32x2(uint32_t a, float2 v) {
  asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(v) : "memory");
}

DEV int xperm(int k) { return (k & ~511) + ((k & 4) << 6) + (((k & 511) >> 3) << 2) + (k & 3); }

// Position of request b in the current iteration (written into LDS_POS by the
// scheduler wavefront at the start of each iteration).
DEV int cur_pos(const char* smem, int b) {
  return __builtin_amdgcn_readfirstlane(lvi(smem, LDS_POS)[b]);
}

// Scheduler wavefront: positions of iteration s into LDS_POS (uniform
// indices into the kernel-argument array).
DEV void set_positions(const mpk_kparams& P, char* smem, int s, int lane) {
  if (lane == 0)
    for (int b = 0; b < P.B; ++b) lvi(smem, LDS_POS)[b] = P.pos0[b] + s;
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
    const int abort_req = __hip_atomic_load(&P.status->abort_req, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
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
    const int abort_req = __hip_atomic_load(&P.status->abort_req, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
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
      tok[tid] = ld_devi(P.tokens + (int64_t)tid * P.tokens_width + cur_pos_v(smem, tid));
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
        const int t = tok[tid];
        tok[tid] = t < 0 ? 0 : (t >= P.vocab ? P.vocab - 1 : t);  // ids are checked on the host; stay in bounds
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

// Stage the GEMV input into LDS: x (gathered from its producers' stamped
// words, an embedding row, or a plain input tensor), times the RMSNorm gain
// when the operator normalises, and the tile's residual rows; inv receives
// 1 / rms per request (1 without a norm) in every thread.  Every thread of
// the workgroup takes part.  issue_ring() issues the calling wavefront's
// first weight loads (ring_ops vector-memory operations: 8, 16 or 24): it is
// called once, as early as the input wait allows.  Returns -1 on stop.
#define XCH 8    // stamped x words per thread per gather pass (register path)
#define XGMAX 4  // chunks per wavefront whose gains and values stay in registers (DMA path)

// DMA staging: the landing zone beyond the residual rows (1 KB per chunk of
// 128 stamped words) and, with a norm, the gains of each chunk's columns
// (256 bytes per chunk), which go into the staged-x area beyond x when they
// fit there (they are read before x is complete) and after the landing zone
// otherwise.
template <int NB>
DEV bool gains_in_xs(cop& D) {
  const int Kpad = ((D.K + 511) / 512) * 512;
  const int nchunk = (NB * D.K + 127) >> 7;
  return LDS_X + NB * Kpad * 4 + nchunk * 256 <= Lay<NB>::RES;
}
// bytes the DMA staging occupies from the landing zone's start
template <int NB>
DEV int land_bytes(cop& D) {
  const int nchunk = (NB * D.K + 127) >> 7;
  return nchunk * 1024 + (D.has_norm && !gains_in_xs<NB>(D) ? nchunk * 256 : 0);
}

// Chunks in which the task's x arrives by global->LDS DMA, or 0 when it
// takes the register path.
template <int NB>
DEV int dma_chunks(cop& D) {
  const int land = Lay<NB>::RES + LDS_RES_BYTES;
  const int nchunk = (NB * D.K + 127) >> 7;
  const bool ok = D.xll && (D.K & 127) == 0 && land + land_bytes<NB>(D) <= Lay<NB>::TOTAL &&
                  nchunk <= 32 * MPK_NW && (!D.has_norm || nchunk <= XGMAX * MPK_NW);
  return ok ? nchunk : 0;
}

DEV uint32_t lds_read_u32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
template <int NB, class Ring>
DEV int stage_inputs(const mpk_kparams& P, cop& D, ctask& T, char* smem, int tid, int s, int task_id,
                     float (&inv)[NB], int ring_ops, Ring&& issue_ring) {
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
  const int nchunk = (NE + 127) >> 7;
  const int nres = D.epi == MPK_EPI_RESID ? NB * T.nrows : 0;
  const bool dma = dma_chunks<NB>(D) > 0;
  // zero padding columns of x (K not a multiple of 512); no gather writes them
  for (int i = K + (worker ? tid : Kpad); i < Kpad; i += MPK_NW * 64)
#pragma unroll
    for (int b = 0; b < NB; ++b) xs[b * Kpad + xperm(i)] = 0.f;
  // Residual element rt of the tile (request rb, row rrow).  With the DMA
  // path the scheduler wavefront's lanes take them: it streams no weights,
  // so waiting for a residual word (its count of loads in flight unknown to
  // the compiler: a full drain) waits behind no weight ring.
  const bool rsched = dma && nres <= 64;
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
    // Gains of this lane's two columns in chunks i < XGMAX (packed bf16
    // pair), by DMA into LDS after the landing zone: as loads into registers
    // the compiler would wait for them with a full drain (the ring behind
    // them has a path-dependent length).
    const uint32_t gla = lb + (gains_in_xs<NB>(D) ? LDS_X + NB * Kpad * 4 : land + nchunk * 1024);
    uint32_t gp[XGMAX];
    float2 xv[XGMAX];
#pragma unroll
    for (int i = 0; i < XGMAX; ++i) {
      const int c = wave + MPK_NW * i;
      const int k = (c * 128) % K;
      if (D.has_norm && ((mine >> i) & 1u))
        __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(D.gain + k + lane * 2), lds_ptr(gla + c * 256), 4, 0, 0);
      gp[i] = 0u;
      xv[i] = float2{0.f, 0.f};
    }
    // Chunks of this wavefront in LDS (mask m): take each whose words are
    // all current (with a norm the raw values also stay in registers for
    // the RMS sums).
    auto take = [&](uint32_t m) {
      for (; m; m &= m - 1) {
        const int i = __builtin_ctz(m), c = wave + MPK_NW * i;
        const u32x4 w = lds_read_u32x4(lb + land + c * 1024 + lane * 16);
        if (__ballot(w.y != st || w.w != st) == 0) {
          need &= ~(1u << i);
          const int e = c * 128 + lane * 2;
          const int b = e / K, k = e - b * K;
          float2 x{__uint_as_float(w.x), __uint_as_float(w.z)};
          if (D.has_norm) {
            // i < XGMAX here (checked with dma)
#pragma unroll
            for (int j = 0; j < XGMAX; ++j)
              if (j == i) xv[j] = x, x = float2{x.x * bf16lo(gp[j]), x.y * bf16hi(gp[j])};
          }
          // (LDS stores written in asm: after a global->LDS DMA the
          // compiler puts a full vmcnt drain before its own LDS stores)
          lds_write_f32x2(lb + LDS_X + (uint32_t)(b * Kpad + xperm(k)) * 4u, x);
        }
      }
      need = __builtin_amdgcn_readfirstlane(need);
    };
    bool first = true, published = false;
    for (;;) {
      if (first) {
        // stale landing data must not pass the stamp check before the first
        // round's DMA has landed: clear the landing stamps first
        for (uint32_t m = need; m; m &= m - 1)
          lds_write_u32x4(lb + land + (wave + MPK_NW * __builtin_ctz(m)) * 1024 + lane * 16, u32x4{0u, 0u, 0u, 0u});
        lds_wait();
      }
      for (uint32_t m = need; m; m &= m - 1) {
        const int c = wave + MPK_NW * __builtin_ctz(m);
        __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(D.xll + c * 128 + lane * 2), lds_ptr(lb + land + c * 1024),
                                         16, 0, 16 /* sc1: device scope */);
      }
      uint64_t wr = 0;
      if (need_r) wr = ld_ll(D.rll + (int64_t)rb * D.n_out + rrow);
      if (first) {
        // the weights go out behind this round's words; wait for the words
        // only (loads complete in issue order)
        issue_ring();
        // (ring group, and the rows of an LDS assignment unit)
        if (worker && ring_ops == 3 * MPK_RING) vm_wait_known<3 * MPK_RING>();
        else if (worker && ring_ops == 2 * MPK_RING) vm_wait_known<2 * MPK_RING>();
        else if (worker) vm_wait_known<MPK_RING>();
        // the gains are in LDS
        if (D.has_norm) {
#pragma unroll
          for (int i = 0; i < XGMAX; ++i)
            if ((mine >> i) & 1u) gp[i] = lds_read_u32(gla + (wave + MPK_NW * i) * 256 + lane * 4);
        }
      } else if (worker) {
        vm_drain_known();
      }
      take(need);
      if (D.has_norm && worker && need == 0 && !published) {
        published = true;
        // this wavefront's chunks are all in: its RMS partials, in chunk order
        float ss[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) ss[b] = 0.f;
#pragma unroll
        for (int i = 0; i < XGMAX; ++i) {
          if ((mine >> i) & 1u) {
            const int b = (wave + MPK_NW * i) * 128 / K;
            const float q = fmaf(xv[i].x, xv[i].x, xv[i].y * xv[i].y);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) ss[bb] += bb == b ? q : 0.f;
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float t = wave_sum(ss[b]);
          if (lane == 0) lds_write_f32(lb + LDS_RED + (uint32_t)(wave * 8 + b) * 4u, t);
        }
      }
      if (need_r && ll_ok(wr, st)) res[rt] = ll_f(wr), need_r = false;
      if (first && rt >= 0 && rt < nres && !D.rll) res[rt] = rv;
      first = false;
      if (need == 0 && __ballot(need_r) == 0) break;
      if (wave_watch(P, Wt, s, task_id, smem, lane)) break;
      __builtin_amdgcn_s_sleep(1);
    }
    // every wavefront's inputs are in, or the workgroup stops
    lds_barrier();
    if (*lvi(smem, LDS_CTL)) return -1;
  } else {
    issue_ring();
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
        for (;;) {
          uint64_t v[XCH];
#pragma unroll
          for (int j = 0; j < XCH; ++j)
            if ((need >> j) & 1u) v[j] = ld_ll(D.xll + base + tid + j * MPK_NW * 64);
          uint64_t wr = 0;
          if (need_r) wr = ld_ll(D.rll + (int64_t)rb * D.n_out + rrow);
          // (request, column) of element j, stepped from j = 0 without divisions
          int eb = (base + tid) / K, ek = base + tid - eb * K;
#pragma unroll
          for (int j = 0; j < XCH; ++j) {
            if (((need >> j) & 1u) && ll_ok(v[j], st)) {
              xs[eb * Kpad + xperm(ek)] = ll_f(v[j]);
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
DEV void put_out(cop& D, int64_t i, float v, uint32_t st) {
  st_ll(D.yll + i, v, st);
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
  for (int i = tid; i < NB * n_out_tile; i += MPK_THREADS) {
    const int b = i / n_out_tile, ol = i - b * n_out_tile;
    put_out(D, (int64_t)b * D.n_out + orow0 + ol, lds_read_f32(ob + (uint32_t)(b * n_out_tile + ol) * 4u), st);
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
    const int rc = stage_inputs<NB>(P, D, T, smem, tid, s, task_id, inv, ring_ops, [&]() {
      if (!sched && whole) {
        // units 0..7 of the wavefront's first row (of W0 when it has none)
        const gu32x4* wp = unit_ptr(I, 0, lane);
#pragma unroll
        for (int j = 0; j < MPK_RING; ++j) b[j] = __builtin_nontemporal_load(wp + j * 64);
      } else if (!sched) {
#pragma unroll
        for (int j = 0; j < MPK_RING; ++j) {
          b[j] = load_unit(I, lane);
          cursor_step(I, wave);
        }
      }
      if (!sched) {
        if (lds_pending) {
          Cursor C2 = I;
          for (int rr = 0; rr < a_pre; ++rr) {
            cursor_goto(C2, MPK_NW + wave, rr, 0, wave);
            const gu32x4* wp = unit_ptr(C2, 0, lane);
#pragma unroll
            for (int u = 0; u < MPK_RING; ++u)
              __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(wp + u * 64),
                                               lds_ptr(pf + (rr * MPK_RING + u) * 1024), 16, 0, 0);
          }
        }
      }
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
        if (p + 1 >= ld_devi(P.prompt_len + b)) {
          st_devi(P.tokens + (int64_t)b * P.tokens_width + p + 1, ix);
        } else {
          next = ld_devi(P.tokens + (int64_t)b * P.tokens_width + p + 1);  // teacher-forced prompt token
        }
        st_devi(P.step + b, p + 1);
        st_lli(P.tok_ll + b, next, st);
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Attention task (request r, kv head j, split c of nsplit): per-head RMSNorm
// of q and k, RoPE at the request's position p, K/V of p into the caches
// (by the split that owns p), an online softmax over this split's positions
// kept per lane group in registers, and one merge across the wavefronts.
// The context [0, p] is cut into na = min(nsplit, ceil((p + 1) / 64))
// splits; splits c >= na have nothing to do this iteration.  With one split
// the task writes the attention output of the group's query heads; with
// several, splits publish stamped partials (m, l, acc) and the split that
// owns p merges them into the output.  Returns -1 on stop.
// ---------------------------------------------------------------------------
#define ATT_MAXG 4
#define ATT_ROUNDS 2    // position rounds per wavefront whose K/V rows are loaded together
#define ATT_GROUPS 64   // position groups per workgroup at most (NW waves x 64 / LP, d >= 64)
#define ATT_RING 2      // LDS ring slots (steps of K/V rows) per wavefront, multi-step splits
#define ATT_SLOT (2 * ATT_ROUNDS * 1024)  // one ring slot: K and V of a step, 1 KB per round each
static_assert(ATT_ROUNDS == 2, "lds_read_kv2 reads two rounds");
static_assert((ATT_RING & (ATT_RING - 1)) == 0 && ATT_RING >= 2, "ring slots are indexed with i & (ATT_RING - 1)");
// the ring overlays the group accumulators and what follows them
static_assert(LDS_X + (ATT_MAXG * 128 + 256 + 2 * ATT_GROUPS * ATT_MAXG) * 4 + MPK_NW * ATT_RING * ATT_SLOT <=
                  Lay<1>::TOTAL,
              "attention K/V ring exceeds the LDS");

// Sum over the LP lanes of a position group (lanes [g*LP, (g+1)*LP)), every
// lane of the group receiving the same value (quad swaps, then half-row and
// row mirrors: DPP, no LDS round trip).
DEV float group_sum(float v, int LP) {
  v += dpp<0xB1>(v);                  // quad_perm [1,0,3,2]
  if (LP >= 4) v += dpp<0x4E>(v);     // quad_perm [2,3,0,1]
  if (LP >= 8) v += dpp<0x141>(v);    // row_half_mirror
  if (LP >= 16) v += dpp<0x140>(v);   // row_mirror
  return v;
}

struct SoftState {
  float m[ATT_MAXG], l[ATT_MAXG], acc[ATT_MAXG][8];
};

DEV int attn_task(const mpk_kparams& P, ctask& T, cop& D, char* smem, int tid, bool sched, int s, int task_id) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = T.row0, j = T.nrows, c = T.split, NS = D.nsplit;
  const int d = D.d, G = D.nq / D.nkv, half = d >> 1, LP = d >> 3, PPR = 64 / LP;
  const int step = MPK_NW * PPR * ATT_ROUNDS;  // positions per step of all wavefronts
  const int p = cur_pos(smem, r);
  const int n = p + 1;
  const int na = min(NS, (n + MPK_ATTN_SPLIT - 1) / MPK_ATTN_SPLIT);
  if (c >= na) return 0;  // uniform over the workgroup: nothing to do this iteration
  const int lo = (int)(((int64_t)c * n) / na), hi = (int)(((int64_t)(c + 1) * n) / na);
  const bool owner = c == na - 1;  // the split holding position p
  const uint32_t st = stamp_of(P, s);
  // position groups: lanes [g*LP, (g+1)*LP) of a wavefront take one position
  // (LP lanes x 8 dims); NG = NW * PPR groups per workgroup
  const int NG = MPK_NW * PPR;
  float* qs = reinterpret_cast<float*>(smem + LDS_X);  // [G][d]
  float* kv = qs + ATT_MAXG * 128;                      // k [d], v [d] (bf16-rounded)
  float* wm = kv + 256;                                 // [NG][G] group maxima
  float* wl = wm + ATT_GROUPS * ATT_MAXG;               // [NG][G] group sums
  float* wacc = wl + ATT_GROUPS * ATT_MAXG;             // [NG][G][d] group accumulators
  uint32_t* gath = reinterpret_cast<uint32_t*>(wacc + ATT_GROUPS * ATT_MAXG * 64);  // gathered partials
  float* outs = reinterpret_cast<float*>(smem + LDS_OUT);               // partial, then o
  uint32_t* kvrow = reinterpret_cast<uint32_t*>(smem + LDS_OUT) + 640;  // bf16 K row, then V row
  const int qkv_w = (D.nq + 2 * D.nkv) * d;
  uint16_t* kc = D.kc + ((int64_t)(r * D.nkv + j) * D.S) * d;
  uint16_t* vc = D.vc + ((int64_t)(r * D.nkv + j) * D.S) * d;
  const int dim0 = (lane % LP) * 8;
  const int pg = lane / LP;
  // scores are kept in base-2 units, s * log2(e) / sqrt(d): every
  // exponential below is one exp2.  The factor is applied to q once, when
  // q is staged, rather than to every score.
  const float scale = 1.4426950408889634f / sqrtf((float)d);

  SoftState sm;
#pragma unroll
  for (int h = 0; h < ATT_MAXG; ++h) {
    sm.m[h] = -INFINITY, sm.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.acc[h][e] = 0.f;
  }
  // K/V rows of this wave's first rounds.  The cache rows below p were
  // written by earlier iterations, all ended once any input of this
  // iteration has arrived.  If an earlier task of this iteration on this CU
  // has already waited for one (LDS_SYNCED), the rows are loaded before
  // this task's own wait; otherwise (nothing before it on this queue, or only
  // tasks with nothing to do) after it.
  // (Splits of more than one step stream their rows through an LDS ring
  // instead, below.)
  const bool multi = hi - lo > step;
  u32x4 kr[ATT_ROUNDS], vr[ATT_ROUNDS];
  auto load_into = [&](u32x4(&K)[ATT_ROUNDS], u32x4(&V)[ATT_ROUNDS], int base) {
#pragma unroll
    for (int q = 0; q < ATT_ROUNDS; ++q) {
      const int t = base + (wave + MPK_NW * q) * PPR + pg;
      const int tc = t < hi && t != p ? t : lo;  // in-bounds row for idle lanes
      K[q] = ld_dev16(kc + (int64_t)tc * d + dim0);
      V[q] = ld_dev16(vc + (int64_t)tc * d + dim0);
    }
  };
  auto load_rounds = [&](int base) { load_into(kr, vr, base); };
  const bool early = uni(*lvi(smem, LDS_SYNCED)) != 0;
  if (!sched && lo < hi && !multi && early) load_rounds(lo);

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
                        (hh < G ? (j * G + hh) * d : (hh == G ? D.nq * d + j * d : (D.nq + D.nkv) * d + j * d));
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
  if (!sched && lo < hi && !multi && !early) load_rounds(lo);
  // The K/V rows, RoPE factors and gains above are loads issued before the
  // device-scope polls: complete them here (see vm_drain_known; they were
  // issued first, so this costs little).
  vm_drain_known();
  mark_ready(P, s, task_id, tid);

  // ---- RMSNorm + RoPE (waves 0..G+1) ----
  if (!sched && hh < G + 2) {
    const float a = lane < half ? ll_f(wa) : 0.f;
    const float b = lane < half ? ll_f(wb) : 0.f;
    if (hh <= G) {
      const float ss = wave_sum(a * a + b * b);
      const float inv = 1.0f / sqrtf(ss / (float)d + P.rms_eps);
      if (lane < half) {
        const float ya = ga * (a * inv);
        const float yb = gb * (b * inv);
        const float ra = ya * cs - yb * sn;
        const float rb = yb * cs + ya * sn;
        if (hh < G) {
          qs[hh * d + lane] = ra * scale;
          qs[hh * d + lane + half] = rb * scale;
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
      kv[d + lane] = bf16f(va);
      kv[d + lane + half] = bf16f(vb);
      reinterpret_cast<uint16_t*>(kvrow)[d + lane] = va;
      reinterpret_cast<uint16_t*>(kvrow)[d + lane + half] = vb;
    }
  }
  __syncthreads();
  // the owner's scheduler wavefront writes K/V of p into the caches while the
  // workers score; its stores complete before the output is published (next
  // iteration's readers are ordered after that output)
  if (sched && owner) {
    uint32_t* kdst = reinterpret_cast<uint32_t*>(kc + (int64_t)p * d);
    uint32_t* vdst = reinterpret_cast<uint32_t*>(vc + (int64_t)p * d);
    for (int i = lane; i < d / 2; i += 64) {
      st_devu(kdst + i, kvrow[i]);
      st_devu(vdst + i, kvrow[d / 2 + i]);
    }
    vm_drain();
  }

  // ---- scores and online softmax over this wave's positions ----
  if (!sched) {
    // q is read from LDS in each step (asm reads: not hoisted into 32 more
    // live registers across the loop)
    const uint32_t qa = lds_addr(qs) + (uint32_t)dim0 * 4u;
    const uint32_t kva = lds_addr(kv) + (uint32_t)dim0 * 4u;
    // one base step: its positions folded into the running (m, l, acc)
    auto fold = [&](u32x4(&K)[ATT_ROUNDS], u32x4(&V)[ATT_ROUNDS], int base) {
      // this round's ATT_ROUNDS positions per lane group are folded into the
      // running (m, l, acc) together: one rescale per head per base step
      float kf[ATT_ROUNDS][8], vf[ATT_ROUNDS][8];
      bool valid[ATT_ROUNDS];
#pragma unroll
      for (int q = 0; q < ATT_ROUNDS; ++q) {
        const int t = base + (wave + MPK_NW * q) * PPR + pg;
        valid[q] = t < hi;
        // The loaded rows are unpacked on every lane (the wait for them is
        // then in straight-line code, not in a branch that all lanes may
        // skip, which would leave them outstanding into the next step's
        // loads).  Row p comes from LDS; an idle lane (its row is not this
        // split's) takes it too, so no value outside the rows in [lo, p)
        // reaches the sums, whatever the cache holds there.
        unpack8(K[q], kf[q]);
        unpack8(V[q], vf[q]);
        if (t == p || !valid[q]) {
          // (asm reads: a compiler-visible LDS read here would wait for
          // every K/V ring DMA in flight)
          f32x4 k0, k1, v0, v1;
          lds_read_2f4_near(kva, k0, k1);
          lds_read_2f4_near(kva + (uint32_t)d * 4u, v0, v1);
          kf[q][0] = k0.x, kf[q][1] = k0.y, kf[q][2] = k0.z, kf[q][3] = k0.w;
          kf[q][4] = k1.x, kf[q][5] = k1.y, kf[q][6] = k1.z, kf[q][7] = k1.w;
          vf[q][0] = v0.x, vf[q][1] = v0.y, vf[q][2] = v0.z, vf[q][3] = v0.w;
          vf[q][4] = v1.x, vf[q][5] = v1.y, vf[q][6] = v1.z, vf[q][7] = v1.w;
        }
      }
#pragma unroll
      for (int h = 0; h < ATT_MAXG; ++h) {
        if (h < G) {
          f32x4 q0, q1;  // q of head h, dims dim0 .. dim0 + 7
          lds_read_2f4_near(qa + (uint32_t)(h * d) * 4u, q0, q1);
          const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
          float sc[ATT_ROUNDS];
          float Mx = -INFINITY;
#pragma unroll
          for (int q = 0; q < ATT_ROUNDS; ++q) {
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(qv[e], kf[q][e], part);
            part = group_sum(part, LP);  // all lanes of a group share valid[q]
            sc[q] = valid[q] ? part : -INFINITY;
            Mx = fmaxf(Mx, sc[q]);
          }
          // (m, l, acc) hold the sums relative to a reference m that moves
          // only when a score exceeds it by more than 8 (base 2; always for
          // the first score, m = -inf): weights stay below 2^8, and most
          // steps skip the rescale.  Any reference gives the same softmax
          // once l and acc share it, which the merges below rely on.
          // (exponentials: the hardware's v_exp_f32, which maps -inf to 0;
          // no weight here needs a denormal result)
          if (Mx > sm.m[h] + 8.f) {
            const float co = __builtin_amdgcn_exp2f(sm.m[h] - Mx);  // 0 for m = -inf
            sm.l[h] *= co;
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.acc[h][e] *= co;
            sm.m[h] = Mx;
          }
          if (Mx != -INFINITY) {
            float L = sm.l[h];
#pragma unroll
            for (int q = 0; q < ATT_ROUNDS; ++q) {
              const float w = __builtin_amdgcn_exp2f(sc[q] - sm.m[h]);  // 0 for an idle position
              L += w;
#pragma unroll
              for (int e = 0; e < 8; ++e) sm.acc[h][e] = fmaf(w, vf[q][e], sm.acc[h][e]);
            }
            sm.l[h] = L;
          }
        }
      }
    };
    if (!multi) {
      fold(kr, vr, lo);
    } else {
      // K/V rows through a ring of ATT_RING steps per wavefront in LDS,
      // filled by global->LDS DMA: ATT_RING - 1 steps stay in flight while
      // one is folded, and no registers are held by loads in flight.  The
      // ring overlays the group accumulators (written below, after every
      // wavefront has left this loop) and the gathered partials.  Past the
      // end, steps re-read row lo (folded with weight 0).  Waits are exact
      // counts: the loop issues no other vector-memory operation, and its
      // LDS reads are asm, which the compiler does not hold for the DMAs.
      const uint32_t ring = lds_addr(wacc) + (uint32_t)wave * (ATT_RING * ATT_SLOT);
      auto dma_step = [&](int i) {
        const int base = lo + i * step;
        const uint32_t slot = ring + (uint32_t)(i & (ATT_RING - 1)) * ATT_SLOT;
#pragma unroll
        for (int q = 0; q < ATT_ROUNDS; ++q) {
          const int t = base + (wave + MPK_NW * q) * PPR + pg;
          const int tc = t < hi && t != p ? t : lo;  // in-bounds row for idle lanes
          __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(kc + (int64_t)tc * d + dim0),
                                           lds_ptr(slot + q * 1024), 16, 0, 16 /* sc1: device scope */);
          __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(vc + (int64_t)tc * d + dim0),
                                           lds_ptr(slot + (ATT_ROUNDS + q) * 1024), 16, 0, 16);
        }
      };
      const int nst = (hi - lo + step - 1) / step;
#pragma unroll
      for (int i = 0; i < ATT_RING - 1; ++i) dma_step(i);
      for (int i = 0; i < nst; ++i) {
        dma_step(i + ATT_RING - 1);
        vm_wait_known<(ATT_RING - 1) * 2 * ATT_ROUNDS>();  // step i has landed
        u32x4 K[ATT_ROUNDS], V[ATT_ROUNDS];
        lds_read_kv2(ring + (uint32_t)(i & (ATT_RING - 1)) * ATT_SLOT + (uint32_t)lane * 16u, K, V);
        fold(K, V, lo + i * step);
      }
      vm_drain_known();
    }
  }
  // every wavefront is done with the ring before the accumulators over it
  // are written
  if (multi) __syncthreads();
  if (!sched) {
    // each position group's (m, l, acc) to LDS: merged across groups and
    // wavefronts below in one pass
    const int grp = wave * PPR + pg;
#pragma unroll
    for (int h = 0; h < ATT_MAXG; ++h) {
      if (h < G) {
        if ((lane % LP) == 0) {
          wm[grp * ATT_MAXG + h] = sm.m[h];
          wl[grp * ATT_MAXG + h] = sm.l[h];
        }
        float* dst = wacc + (grp * ATT_MAXG + h) * d + dim0;
        *reinterpret_cast<float4*>(dst) = float4{sm.acc[h][0], sm.acc[h][1], sm.acc[h][2], sm.acc[h][3]};
        *reinterpret_cast<float4*>(dst + 4) = float4{sm.acc[h][4], sm.acc[h][5], sm.acc[h][6], sm.acc[h][7]};
      }
    }
  }
  __syncthreads();
  // ---- merge the position groups: this split's (m, l, acc) per head ----
  // wave h (< G) turns the groups' maxima into per-group weights once
  float* hML = reinterpret_cast<float*>(smem + LDS_RED);  // [G][2]: M, L per head
  if (!sched && wave < G) {
    const int h = wave;
    float mg = -INFINITY, lg = 0.f;
    float M = -INFINITY;
    for (int g0 = 0; g0 < NG; g0 += 64) {
      const int g = g0 + lane;
      M = fmaxf(M, g < NG ? wm[g * ATT_MAXG + h] : -INFINITY);
    }
    M = wave_max(M);
    float L = 0.f;
    for (int g0 = 0; g0 < NG; g0 += 64) {
      const int g = g0 + lane;
      if (g < NG) {
        mg = wm[g * ATT_MAXG + h];
        lg = wl[g * ATT_MAXG + h];
      }
      const float cg = g < NG && mg != -INFINITY ? exp2f(mg - M) : 0.f;
      L += lg * cg;
      if (g < NG) wm[g * ATT_MAXG + h] = cg;  // the group's weight replaces its reference m
    }
    L = wave_sum(L);
    if (lane == 0) hML[2 * h] = M, hML[2 * h + 1] = L;
  }
  __syncthreads();
  const int stride = d + 2;
  const int64_t o_base = (int64_t)r * D.nq * d + (int64_t)j * G * d;
  for (int idx = tid; idx < G * d && !sched; idx += MPK_NW * 64) {
    const int h = idx / d, i = idx - h * d;
    float A = 0.f;
    for (int g = 0; g < NG; ++g) A = fmaf(wacc[(g * ATT_MAXG + h) * d + i], wm[g * ATT_MAXG + h], A);
    const float M = hML[2 * h], L = hML[2 * h + 1];
    if (na == 1) {
      put_out(D, o_base + idx, A / L, st);  // the whole context in one split
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
  // owner: merge the other splits' partials (gathered in chunks) into its own,
  // in split order: o = sum_c acc_c e^(m_c - M) / sum_c l_c e^(m_c - M)
  const int idx = tid;
  const bool mine_o = !sched && idx < G * d;
  const int h = mine_o ? idx / d : 0, i = mine_o ? idx - h * d : 0;
  float M = mine_o ? outs[h * stride] : 0.f;
  float L = mine_o ? outs[h * stride + 1] : 0.f;
  float O = mine_o ? outs[h * stride + 2 + i] : 0.f;
  const int chunk = (Lay<1>::TOTAL - (int)((char*)gath - smem)) / 4 / (G * stride);
  for (int c0 = 0; c0 < na - 1; c0 += chunk) {
    const int nc = min(chunk, na - 1 - c0);
    const int rc =
        gather_ll<16>(P, pgrp + (int64_t)c0 * G * stride, nc * G * stride, gath, st, Wt, s, task_id, smem, tid);
    if (rc) return rc;
    if (mine_o) {
      for (int cc = 0; cc < nc; ++cc) {
        const float mc = __uint_as_float(gath[(cc * G + h) * stride]);
        const float lc = __uint_as_float(gath[(cc * G + h) * stride + 1]);
        const float ac = __uint_as_float(gath[(cc * G + h) * stride + 2 + i]);
        if (lc > 0.f) {
          const float Mn = fmaxf(M, mc);
          const float ca = M == -INFINITY ? 0.f : exp2f(M - Mn);
          const float cb = exp2f(mc - Mn);
          L = L * ca + lc * cb;
          O = O * ca + ac * cb;
          M = Mn;
        }
      }
    }
    __syncthreads();  // the gather area is reused by the next chunk
  }
  if (mine_o) put_out(D, o_base + idx, O / L, st);
  return 0;
}

// ---------------------------------------------------------------------------
// dispatch of one task body; returns -1 when the run must stop
// ---------------------------------------------------------------------------
template <int NB>
DEV int run_task(const mpk_kparams& P, ctask& T, int task_id, int s, char* smem, int tid, bool sched, int next) {
  cop& D = ops_of(P)[T.op];
  if (T.kind == MPK_TK_ATTN) return attn_task(P, T, D, smem, tid, sched, s, task_id);
  if (T.kind == MPK_TK_ARGMAX) return argmax_task<NB>(P, D, smem, tid, s, task_id);
  return gemv_task<NB>(P, T, D, s, task_id, smem, tid, sched, next);
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
  lds_vi* ctl = lvi(smem, LDS_CTL);
  if (tid == 0) ctl[0] = 0;
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
  lds_vi* ctl = lvi(smem, LDS_CTL);
  if (tid == 0) ctl[0] = 0;
  // every earlier launch (every earlier iteration) has ended
  if (tid == 0) *lvi(smem, LDS_SYNCED) = 1;
  if (sched) set_positions(P, smem, s, lane);
  __syncthreads();
  run_task<NB>(P, T, task_id, s, smem, tid, sched, -1);
  vm_wait<0>();
}

__global__ void mpk_zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
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
  float* d_rope = nullptr;
  mpk_dev_status* d_status = nullptr;
  mpk_trace_record* d_trace = nullptr;
  int64_t trace_cap = 0;  // records
  int last_iters = 0;
  hipStream_t side = nullptr;
  const void* kernel_persistent = nullptr;
  const void* kernel_op = nullptr;
  int lds_bytes = 0;
  mpk_kparams kp{};
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
    default:
      return mpk_fail(MPK_ERR_SHAPE, "this build runs num_requests in {1, 2}");
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

static int64_t tensor_bytes(const mpk_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.dims[i];
  return n * (t.dtype == MPK_BF16 ? 2 : 4);
}

extern "C" int mpk_compile(mpk_graph_t g, int32_t device, mpk_exec_t* out) {
  mpk_clear_error();
  if (!g || !out) return mpk_fail(MPK_ERR_INVALID_ARG, "mpk_compile: NULL argument");
  *out = nullptr;
  if (g->launch.sched_mode != MPK_SCHED_CORESIDENT)
    return mpk_fail(MPK_ERR_SPLIT, "only the co-resident scheduler mode is implemented");
  HIPCHK(hipSetDevice(device));
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, device));
  if (prop.multiProcessorCount != g->num_workers)
    return mpk_fail(MPK_ERR_SPLIT, "graph built for " + std::to_string(g->num_workers) +
                                       " workers, device has " +
                                       std::to_string(prop.multiProcessorCount) + " CUs");
  int coop = 0;
  HIPCHK(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device));
  if (!coop) return mpk_fail(MPK_ERR_NOT_CORESIDENT, "device has no cooperative launch");

  std::unique_ptr<mpk_exec_s, void (*)(mpk_exec_s*)> x(new mpk_exec_s(), [](mpk_exec_s* e) {
    mpk_destroy_exec(e);
  });
  x->device = device;
  x->g = g;
  x->B = g->meta.num_requests;
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
      if ((rc = dalloc(x.get(), &x->ll_ptr[i], (size_t)n * 8))) return rc;
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
  const mpk_model_cfg& M = g->model;
  const int B = x->B;

  std::vector<mpk_dev_op> dops = g->dops;
  if ((rc = dalloc(x.get(), &x->d_ticket_ctr, 4))) return rc;
  if ((rc = dalloc(x.get(), &x->d_tok_ll, (size_t)B * 8))) return rc;

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
      const int G = D.nq / D.nkv;
      if (G > ATT_MAXG) return mpk_fail(MPK_ERR_SHAPE, "more than 4 query heads per kv head");
      if (D.d > 128) return mpk_fail(MPK_ERR_SHAPE, "head_dim above 128");
      if ((rc = dalloc(x.get(), &D.pll, (size_t)B * D.nkv * D.nsplit * G * (D.d + 2) * 8))) return rc;
      continue;
    }
    const int e_in = o.in[0];
    D.xll = D.x_embed ? nullptr : PL(e_in);
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
    } else if (o.kind == MPK_OP_RMSNORM_GATEUP) {
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.W1 = (const uint16_t*)P(o.in[3]);
      D.y = (float*)PA(o.out[0]);
      D.yll = PL(o.out[0]);
    } else {  // LM head
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.logits = o.out[0] >= 0 ? (float*)P(o.out[0]) : nullptr;
      if ((rc = dalloc(x.get(), &D.pll, (size_t)D.ntiles * B * 2 * 8))) return rc;
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
  if ((rc = dalloc(x.get(), &x->d_status, sizeof(mpk_dev_status)))) return rc;

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
  K.trace = nullptr;
  K.ticket_ctr = x->d_ticket_ctr;
  uint64_t ns = g->launch.spin_timeout_ns ? g->launch.spin_timeout_ns : 2000000000ull;
  K.timeout_ticks = ns / 10;  // s_memrealtime runs at 100 MHz
  K.qstride = g->max_queue;
  K.n_tasks = (int)g->tasks.size();
  K.B = B;
  K.tokens_width = (int)g->tensors[g->meta.tokens].dims[1];
  K.rope_half = half;
  K.rms_eps = M.rms_eps;
  K.vocab = M.vocab;
  // The zero fills above (hipMemset) are ordered on the null stream only;
  // a run on another stream must never see a buffer before it is zeroed (a
  // reused allocation could still hold words stamped by an earlier
  // executable).
  HIPCHK(hipDeviceSynchronize());
  *out = x.release();
  return MPK_OK;
}

// Iteration stamps handed out so far in this process (see prepare_run).
static std::atomic<uint64_t> g_stamps{0};

static int prepare_run(mpk_exec_t x, int32_t n_iter, hipStream_t st) {
  if (!x) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL exec");
  if (n_iter <= 0) return mpk_fail(MPK_ERR_INVALID_ARG, "num_iterations must be positive");
  HIPCHK(hipSetDevice(x->device));
  // bounds of tokens / KV cache for every request
  std::vector<int32_t> step(x->B);
  HIPCHK(hipMemcpyAsync(step.data(), x->kp.step, x->B * 4, hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  std::vector<int32_t> toks((size_t)x->B * x->kp.tokens_width);
  HIPCHK(hipMemcpyAsync(toks.data(), x->kp.tokens, toks.size() * 4, hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  for (int r = 0; r < x->B; ++r) {
    int64_t last = (int64_t)step[r] + n_iter;
    if (step[r] >= 0 && step[r] < x->kp.tokens_width) {
      const int32_t t = toks[(size_t)r * x->kp.tokens_width + step[r]];
      if (t < 0 || t >= x->g->model.vocab)
        return mpk_fail(MPK_ERR_SHAPE, "request " + std::to_string(r) + ": token id " + std::to_string(t) +
                                           " at position " + std::to_string(step[r]) + " is outside the vocabulary");
    }
    if (step[r] < 0 || last >= x->kp.tokens_width || last > x->g->model.max_seq)
      return mpk_fail(MPK_ERR_SHAPE, "request " + std::to_string(r) + ": step " + std::to_string(step[r]) +
                                         " + " + std::to_string(n_iter) +
                                         " iterations leaves the tokens tensor or the KV cache");
  }
  for (size_t i = 0; i < x->g->dops.size(); ++i) {
    const mpk_dev_op& D = x->g->dops[i];
    if (D.kind == MPK_TK_LMHEAD && x->g->ops[i].out[0] >= 0 && D.logits_iters < n_iter)
      return mpk_fail(MPK_ERR_SHAPE, "logits tensor holds fewer iterations than requested");
  }
  // trace buffer
  x->kp.trace = nullptr;
  if (x->g->launch.trace) {
    int64_t need = (int64_t)n_iter * x->kp.n_tasks;
    if (need > x->trace_cap) {
      void* p = nullptr;
      HIPCHK(hipMalloc(&p, (size_t)need * sizeof(mpk_trace_record)));
      x->owned.push_back(p);
      x->d_trace = (mpk_trace_record*)p;
      x->trace_cap = need;
    }
    HIPCHK(hipMemsetAsync(x->d_trace, 0xff, (size_t)need * sizeof(mpk_trace_record), st));
    x->kp.trace = x->d_trace;
    x->kp.trace_tickets = x->g->launch.trace == 1;
  }
  // positions at launch: request r is at step[r] + s in iteration s (the
  // LM-head argmax advances step by one per iteration, on the device)
  for (int r = 0; r < x->B; ++r) x->kp.pos0[r] = step[r];
  // positions at launch: request r is at step[r] + s in iteration s (the
  // LM-head argmax advances step by one per iteration, on the device)
  for (int r = 0; r < x->B; ++r) x->kp.pos0[r] = step[r];
  x->kp.n_iter = n_iter;
  x->last_iters = n_iter;
  // stamps of this run: base + 1 .. base + n_iter, taken from a counter
  // shared by every executable of the process, so no two runs (of this or
  // any other executable) ever use the same stamp
  const uint64_t base = g_stamps.fetch_add((uint64_t)n_iter);
  if (base + (uint64_t)n_iter >= 0xffffffffull)
    return mpk_fail(MPK_ERR_STATE, "iteration stamps exhausted (2^32 iterations per process)");
  x->kp.iter_base = (uint32_t)base;
  hipLaunchKernelGGL(mpk_zero_u32, dim3(1), dim3(64), 0, st, x->d_ticket_ctr, (int64_t)1);
  // clear code / iteration / task; a stop request (abort_req) stays until cleared
  hipLaunchKernelGGL(mpk_zero_u32, dim3(1), dim3(64), 0, st, (uint32_t*)x->d_status, (int64_t)3);
  HIPCHK(hipGetLastError());
  return MPK_OK;
}

extern "C" int mpk_run_steps(mpk_exec_t x, int32_t n_iter, void* stream) {
  mpk_clear_error();
  hipStream_t st = (hipStream_t)stream;
  int rc = prepare_run(x, n_iter, st);
  if (rc) return rc;
  void* args[] = {&x->kp};
  HIPCHK(hipLaunchCooperativeKernel(x->kernel_persistent, dim3(x->g->num_workers), dim3(MPK_THREADS), args,
                                    x->lds_bytes, st));
  return MPK_OK;
}

extern "C" int mpk_run_steps_per_op(mpk_exec_t x, int32_t n_iter, void* stream) {
  mpk_clear_error();
  hipStream_t st = (hipStream_t)stream;
  int rc = prepare_run(x, n_iter, st);
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
  HIPCHK(hipMemcpy(&s, x->d_status, sizeof(s), hipMemcpyDeviceToHost));
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
