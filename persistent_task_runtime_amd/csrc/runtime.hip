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
// worker wavefronts plus one scheduler wavefront.  The scheduler wavefront
// walks the CU's static task queue: for each task it spins (agent-scope
// relaxed loads, then one acquire fence) until every producer event has
// reached count * (iteration + 1), releases the workers through a workgroup
// barrier, and after the task signals the task's event with an agent-scope
// release add.
//
// Weights stream through a per-wavefront ring in LDS, filled by direct
// global->LDS 16-byte loads (global_load_lds_dwordx4).  The ring's producer
// side walks the CU's queue ahead of the consumer and crosses task
// boundaries: while a task's dependencies are still pending, the first
// weight units of that task (and of the next ones) are already in flight.
// This is the "load the next layer while computing this one" pipelining of
// P3 "Why MPK?", done per CU with the queue known at compile time.
//
// The iteration's last operator picks the argmax token, writes it into
// tokens, advances step (P1 "How MPK Works") and releases the next iteration.
#include <hip/hip_runtime.h>

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

// Wait until at most N vector-memory operations of this wavefront are in
// flight.  The compiler does not model the LDS writes of global_load_lds, so
// the ring's consumer waits explicitly; the memory clobber keeps the LDS read
// of the slot after the wait.
template <int N>
DEV void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// LDS layout (bytes)
//   [0, 2048)                 control words, reductions, 1/rms, tile argmax
//   [LDS_X, +XS)              staged activations x (or attention scratch)
//   [LDS_RES, +2048)          staged residual rows of the tile
//   [LDS_RING, +NW*R*1024)    weight rings, R units of 1 KB per wavefront
// x is staged permuted so each 16-byte LDS read is lane-contiguous:
//   column k -> unit u = k / 512, lane l = (k % 512) / 8, half h = (k % 8) / 4
//   offset (floats) = u * 512 + h * 256 + l * 4 + (k % 4)
// ---------------------------------------------------------------------------
#define LDS_CTL 0
#define LDS_RED 256                      // [16][8] floats: per-wave partials
#define LDS_INV (LDS_RED + 16 * 8 * 4)   // [8] floats
#define LDS_BEST (LDS_INV + 64)          // [8 waves][8] (float) + [8][8] (int)
#define LDS_X 2048
#define LDS_RES_BYTES 2048

template <int NB>
struct Lay {
  static constexpr int XS = 49152 * NB;                    // staged x bytes
  static constexpr int RES = LDS_X + XS;                   // residual rows
  static constexpr int RING = RES + LDS_RES_BYTES;         // weight rings
  static constexpr int R = NB == 1 ? 12 : 6;               // ring units per wavefront
  static constexpr int TOTAL = RING + MPK_NW * R * 1024;
};
static_assert(Lay<1>::TOTAL <= 160 * 1024, "LDS budget");
static_assert(Lay<2>::TOTAL <= 160 * 1024, "LDS budget");

DEV int xperm(int k) { return (k & ~511) + ((k & 4) << 6) + (((k & 511) >> 3) << 2) + (k & 3); }

// Token id consumed by request b in this iteration.
DEV int cur_token(const mpk_kparams& P, int b) {
  const int p = gldi(P.step + b);
  const int t = gldi(P.tokens + (int64_t)b * P.tokens_width + p);
  return t < 0 ? 0 : (t >= P.vocab ? P.vocab - 1 : t);  // ids are checked on the host; stay in bounds
}

// ---------------------------------------------------------------------------
// weight units (GEMV and LM-head tiles)
//   A tile covers virtual rows [row0, row0 + nrows).  Rows go to the worker
//   wavefronts in assignment units of `a` rows (a = 2 for gate/up pairs):
//   wave w takes units w, w + 8, w + 16, ...  A row is read as ceil(K/512)
//   units of 512 bf16 (1 KB, 16 bytes per lane); a wavefront's sequence is
//   its rows in order, each row's units in order.
// ---------------------------------------------------------------------------
DEV const uint16_t* row_ptr(cop& D, int vrow) {
  if (D.pairs) return ((vrow & 1) ? D.W1 : D.W0) + (int64_t)(vrow >> 1) * D.K;
  if (vrow < D.N0) return D.W0 + (int64_t)vrow * D.K;
  vrow -= D.N0;
  if (vrow < D.N1) return D.W1 + (int64_t)vrow * D.K;
  return D.W2 + (int64_t)(vrow - D.N1) * D.K;
}

DEV int units_per_row(cop& D) { return (D.K + 511) >> 9; }

DEV int wave_units(cop& D, ctask& T, int wave) {
  const int a = D.pairs ? 2 : 1;
  const int au = T.nrows / a;
  const int mine = au > wave ? (au - wave + MPK_NW - 1) / MPK_NW : 0;
  return mine * a * units_per_row(D);
}

// Producer side of a wavefront's ring: the next unit to load, walking stream
// tasks in queue order across iterations.  Everything the producer needs is
// copied out of the descriptors into wave-uniform scalars when it moves to a
// task, so issuing a unit performs no memory read.
struct Issuer {
  const uint16_t* W0;
  const uint16_t* W1;
  const uint16_t* W2;
  const uint16_t* row;  // current row (lane offset not included)
  int N0, N1, K, pairs, row0;
  int s, k;             // iteration and queue position of the task
  int j, n;             // unit index within the wave's sequence, count
  int kk, rr, u;        // assignment unit, row within unit, unit within row
  int upr, a;
  int live;
};

DEV void issuer_row(Issuer& I, int wave) {
  int vrow = I.row0 + (wave + MPK_NW * I.kk) * I.a + I.rr;
  const uint16_t* r;
  if (I.pairs) {
    r = ((vrow & 1) ? I.W1 : I.W0) + (int64_t)(vrow >> 1) * I.K;
  } else if (vrow < I.N0) {
    r = I.W0 + (int64_t)vrow * I.K;
  } else if (vrow - I.N0 < I.N1) {
    r = I.W1 + (int64_t)(vrow - I.N0) * I.K;
  } else {
    r = I.W2 + (int64_t)(vrow - I.N0 - I.N1) * I.K;
  }
  I.row = unip(r);
}

// Point the issuer at the first stream task at or after queue position k of
// iteration s that gives this wave at least one unit.
DEV void issuer_seek(Issuer& I, const mpk_kparams& P, cqent* Q, int qlen, int s, int k, int wave) {
  int found = 0;
  for (int guard = 0; guard < 2 * qlen + 2 && !found; ++guard) {
    if (k >= qlen) {
      k = uni(k - qlen);
      s = uni(s + 1);
    }
    if (s >= P.n_iter || k < 0) break;
    const int tix = uni(Q[k].task);
    ctask& T = tasks_of(P)[tix];
    const int kind = uni(T.kind);
    if (kind == MPK_TK_GEMV || kind == MPK_TK_LMHEAD) {
      cop& D = ops_of(P)[uni(T.op)];
      const int n = uni(wave_units(D, T, wave));
      if (n > 0) {
        I.W0 = unip(D.W0), I.W1 = unip(D.W1), I.W2 = unip(D.W2);
        I.N0 = uni(D.N0), I.N1 = uni(D.N1), I.K = uni(D.K), I.pairs = uni(D.pairs);
        I.row0 = uni(T.row0);
        I.s = s, I.k = k, I.j = 0, I.n = n;
        I.kk = 0, I.rr = 0, I.u = 0, I.upr = uni(units_per_row(D)), I.a = I.pairs ? 2 : 1;
        found = 1;
        break;
      }
    }
    const int nx = uni(Q[k].next_stream);  // > k; >= qlen means the next iteration
    if (nx < 0) break;
    k = nx;
  }
  I.live = found;
  if (found) issuer_row(I, wave);
}

// Issue the issuer's next unit into LDS slot `slot` and advance.
DEV void issue_unit(Issuer& I, char* ring_wave, int slot, const mpk_kparams& P, cqent* Q, int qlen,
                    int wave, int lane) {
  const int kleft = I.K - I.u * 512;
  const int col = lane * 8 < kleft ? I.u * 512 + lane * 8 : 0;  // lanes past the row re-read its start
  __builtin_amdgcn_global_load_lds((gptr_t)(const void*)(I.row + col),
                                   (lptr_t)(void*)(ring_wave + slot * 1024), 16, 0, 0);
  I.j = uni(I.j + 1);
  I.u = uni(I.u + 1);
  if (I.u == I.upr) {
    I.u = 0;
    I.rr = uni(I.rr + 1);
    if (I.rr == I.a) {
      I.rr = 0;
      I.kk = uni(I.kk + 1);
    }
    if (I.j < I.n) issuer_row(I, wave);
  }
  if (I.j == I.n) issuer_seek(I, P, Q, qlen, I.s, I.k + 1, wave);
}

// Per-wavefront ring state (uniform).
struct RingState {
  int head;      // slot of the oldest unit in flight
  int inflight;  // units issued, not yet consumed
};

template <int R>
DEV void wait_head(int inflight) {
  // the head unit has (inflight - 1) loads issued after it
  if (inflight >= R) {
    vm_wait<R - 1>();
  } else {
    switch (inflight) {
      case 12: vm_wait<11>(); break;
      case 11: vm_wait<10>(); break;
      case 10: vm_wait<9>(); break;
      case 9: vm_wait<8>(); break;
      case 8: vm_wait<7>(); break;
      case 7: vm_wait<6>(); break;
      case 6: vm_wait<5>(); break;
      case 5: vm_wait<4>(); break;
      case 4: vm_wait<3>(); break;
      case 3: vm_wait<2>(); break;
      case 2: vm_wait<1>(); break;
      default: vm_wait<0>(); break;
    }
  }
}

// Issue one unit into the free slot after the ring's last unit, if the
// producer has one; called once per consumed unit (steady state) and in a
// loop at start-up.
template <int R>
DEV void ring_top_up(Issuer& I, RingState& S, char* ring_wave, const mpk_kparams& P, cqent* Q, int qlen,
                     int wave, int lane) {
  if (I.live && S.inflight < R) {
    int slot = S.head + S.inflight;
    if (slot >= R) slot -= R;
    issue_unit(I, ring_wave, uni(slot), P, Q, qlen, wave, lane);
    S.inflight = uni(S.inflight + 1);
  }
}

template <int R>
DEV void ring_fill(Issuer& I, RingState& S, char* ring_wave, const mpk_kparams& P, cqent* Q, int qlen,
                   int wave, int lane) {
  for (int i = 0; i < R; ++i) ring_top_up<R>(I, S, ring_wave, P, Q, qlen, wave, lane);
}

// Stage x (times the RMSNorm gain when the operator normalises) into LDS,
// compute 1 / rms per request, and stage the tile's residual rows.  All
// waves take part in the barriers.
template <int NB>
DEV void stage_x(const mpk_kparams& P, cop& D, ctask& T, char* smem, int tid,
                 bool sched) {
  float* xs = reinterpret_cast<float*>(smem + LDS_X);
  float* res = reinterpret_cast<float*>(smem + Lay<NB>::RES);
  float* red = reinterpret_cast<float*>(smem + LDS_RED);
  float* inv = reinterpret_cast<float*>(smem + LDS_INV);
  const int K = D.K;
  const int Kpad = ((K + 511) / 512) * 512;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float ss[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) ss[b] = 0.f;
  if (!sched) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint16_t* erow = nullptr;
      if (D.x_embed) erow = D.E + (int64_t)cur_token(P, b) * K;
      for (int k = tid * 4; k < Kpad; k += MPK_NW * 64 * 4) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (k < K) {
          if (D.x_embed) {
            const u32x2 e = gldv<u32x2>(erow + k);
            v[0] = bf16lo(e.x), v[1] = bf16hi(e.x), v[2] = bf16lo(e.y), v[3] = bf16hi(e.y);
          } else {
            const f32x4 f = gldv<f32x4>(D.x + (int64_t)b * K + k);
            v[0] = f.x, v[1] = f.y, v[2] = f.z, v[3] = f.w;
          }
          if (D.has_norm) {
            const u32x2 gg = gldv<u32x2>(D.gain + k);
            const float g[4] = {bf16lo(gg.x), bf16hi(gg.x), bf16lo(gg.y), bf16hi(gg.y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ss[b] = fmaf(v[e], v[e], ss[b]);
              v[e] = v[e] * g[e];
            }
          }
        }
        *reinterpret_cast<float4*>(xs + b * Kpad + xperm(k)) = float4{v[0], v[1], v[2], v[3]};
      }
      if (D.epi == MPK_EPI_RESID) {
        for (int i = tid; i < T.nrows; i += MPK_NW * 64) {
          const int row = T.row0 + i;
          float r;
          if (D.res_embed) r = bf16f(gld16(D.E + (int64_t)cur_token(P, b) * D.n_out + row));
          else r = gld(D.resid + (int64_t)b * D.n_out + row);
          res[b * T.nrows + i] = r;
        }
      }
    }
    if (D.has_norm) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float t = wave_sum(ss[b]);
        if ((tid & 63) == 0) red[wave * 8 + b] = t;
      }
    }
  }
  __syncthreads();
  if (tid < NB) {
    if (D.has_norm) {
      float t = 0.f;
      for (int w = 0; w < MPK_NW; ++w) t += red[w * 8 + tid];
      inv[tid] = 1.0f / sqrtf(t / (float)K + P.rms_eps);
    } else {
      inv[tid] = 1.0f;
    }
  }
  __syncthreads();
}

DEV float silu(float g) { return g / (1.0f + expf(-g)); }

// ---------------------------------------------------------------------------
// GEMV-type task: rmsnorm_linear (EPI_STORE), linear + residual (EPI_RESID),
// rmsnorm + gate/up + SiLU-mul (EPI_SILU), final norm + LM head + tile argmax
// (EPI_ARGMAX).  Returns true when the task's completion must be signalled.
// ---------------------------------------------------------------------------
template <int NB>
DEV bool gemv_task(const mpk_kparams& P, ctask& T, cop& D, Issuer& I,
                   RingState& RS, cqent* Q, int qlen, int s, char* smem, int tid,
                   bool sched) {
  constexpr int R = Lay<NB>::R;
  stage_x<NB>(P, D, T, smem, tid, sched);
  const int EPI = D.epi;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const float* xs = reinterpret_cast<const float*>(smem + LDS_X);
  const float* res = reinterpret_cast<const float*>(smem + Lay<NB>::RES);
  const float* inv = reinterpret_cast<const float*>(smem + LDS_INV);
  char* ring_wave = smem + Lay<NB>::RING + wave * R * 1024;
  const int Kpad = ((D.K + 511) / 512) * 512;
  float best_v[NB];
  int best_i[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) best_v[b] = -INFINITY, best_i[b] = 0x7fffffff;
  if (!sched) {
    const int n = wave_units(D, T, wave);
    const int a = D.pairs ? 2 : 1;
    const int upr = units_per_row(D);
    int kk = 0, rr = 0, u = 0;
    float acc[NB], gate[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f, gate[b] = 0.f;
    for (int i = 0; i < n; ++i) {
      wait_head<R>(RS.inflight);
      const u32x4 w = *reinterpret_cast<const u32x4*>(ring_wave + RS.head * 1024 + lane * 16);
      const float wf[8] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                           bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
      const int base = u * 512 + lane * 4;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 x0 = *reinterpret_cast<const float4*>(xs + b * Kpad + base);
        const float4 x1 = *reinterpret_cast<const float4*>(xs + b * Kpad + base + 256);
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
      // the slot just read is refilled with the next unit of the stream
      RS.head = uni(RS.head + 1 == R ? 0 : RS.head + 1);
      RS.inflight = uni(RS.inflight - 1);
      ring_top_up<R>(I, RS, ring_wave, P, Q, qlen, wave, lane);
      if (++u == upr) {
        u = 0;
        const int vrow = T.row0 + (wave + MPK_NW * kk) * a + rr;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float sum = wave_sum(acc[b]);
          acc[b] = 0.f;
          if (EPI == MPK_EPI_STORE) {
            if (lane == 0) gst(D.y + (int64_t)b * D.n_out + vrow, sum * inv[b]);
          } else if (EPI == MPK_EPI_RESID) {
            if (lane == 0) gst(D.y + (int64_t)b * D.n_out + vrow, res[b * T.nrows + (vrow - T.row0)] + sum);
          } else if (EPI == MPK_EPI_SILU) {
            if (rr == 0) {
              gate[b] = sum * inv[b];
            } else if (lane == 0) {
              gst(D.y + (int64_t)b * D.n_out + (vrow >> 1), silu(gate[b]) * (sum * inv[b]));
            }
          } else {  // ARGMAX
            const float logit = sum * inv[b];
            if (D.logits && s < D.logits_iters && lane == 0)
              gst(D.logits + ((int64_t)s * P.B + b) * D.N0 + vrow, logit);
            if (logit > best_v[b]) best_v[b] = logit, best_i[b] = vrow;
          }
        }
        if (++rr == a) {
          rr = 0;
          ++kk;
        }
      }
    }
  }
  if (EPI != MPK_EPI_ARGMAX) return true;

  // ---- LM head: tile argmax, then the last tile picks the token ----
  float* bv = reinterpret_cast<float*>(smem + LDS_BEST);
  int* bi = reinterpret_cast<int*>(smem + LDS_BEST + MPK_NW * 8 * 4);
  volatile int* ctl = reinterpret_cast<volatile int*>(smem + LDS_CTL);
  if (!sched && lane == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) bv[wave * 8 + b] = best_v[b], bi[wave * 8 + b] = best_i[b];
  }
  __syncthreads();
  float* part = D.part;  // [ntiles][NB] (value, index)
  if (tid < NB) {
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int w = 0; w < MPK_NW; ++w) {
      const float vv = bv[w * 8 + tid];
      const int ii = bi[w * 8 + tid];
      if (vv > v || (vv == v && ii < ix)) v = vv, ix = ii;
    }
    gst(part + ((int64_t)T.tile * NB + tid) * 2, v);
    gst(part + ((int64_t)T.tile * NB + tid) * 2 + 1, __int_as_float(ix));
  }
  __syncthreads();
  if (sched && lane == 0) {
    const uint32_t old = __hip_atomic_fetch_add(D.tickets, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    ctl[1] = (old % (uint32_t)D.ntiles) == (uint32_t)D.ntiles - 1;
  }
  __syncthreads();
  const bool last = ctl[1] != 0;
  if (last && tid < NB) {
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int t = 0; t < D.ntiles; ++t) {
      const float vv = gld(part + ((int64_t)t * NB + tid) * 2);
      const int ii = __float_as_int(gld(part + ((int64_t)t * NB + tid) * 2 + 1));
      if (vv > v || (vv == v && ii < ix)) v = vv, ix = ii;
    }
    const int p = gldi(P.step + tid);
    if (p + 1 >= gldi(P.prompt_len + tid)) *(gi32*)(void*)(P.tokens + (int64_t)tid * P.tokens_width + p + 1) = ix;
    *(gi32*)(void*)(P.step + tid) = p + 1;
  }
  return last;
}

// ---------------------------------------------------------------------------
// Attention task (request r, kv head j, split c of nsplit): per-head RMSNorm
// of q and k, RoPE at the request's position p, K/V of p into the caches
// (written by the split that owns p), scores over this split's positions,
// softmax partials (max, sum, weighted V) and, in the last arriving split of
// (r, j), the merge into the attention output of the group's query heads.
// ---------------------------------------------------------------------------
#define ATT_MAXG 4

DEV bool attn_task(const mpk_kparams& P, ctask& T, cop& D, char* smem,
                   int tid, bool sched) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = T.row0, j = T.nrows, c = T.split, NS = D.nsplit;
  const int d = D.d, G = D.nq / D.nkv, half = d >> 1, LP = d >> 3, PPR = 64 / LP;
  const int p = gldi(P.step + r);
  const int n = p + 1;
  const int lo = (int)(((int64_t)c * n) / NS), hi = (int)(((int64_t)(c + 1) * n) / NS);
  float* qs = reinterpret_cast<float*>(smem + LDS_X);  // [G][d]
  float* kv = qs + ATT_MAXG * 128;                      // k [d], v [d] (bf16-rounded)
  float* sc = kv + 256;                                 // [G][SUB]
  float* redm = sc + ATT_MAXG * MPK_ATTN_SUB;           // [NW][G]
  float* reds = redm + MPK_NW * ATT_MAXG;               // [NW][G]
  float* accr = reds + MPK_NW * ATT_MAXG;               // [NW][G][d]
  volatile int* ctl = reinterpret_cast<volatile int*>(smem + LDS_CTL);
  const int qkv_w = (D.nq + 2 * D.nkv) * d;
  const float* qkv = D.x + (int64_t)r * qkv_w;
  uint16_t* kc = D.kc + ((int64_t)(r * D.nkv + j) * D.S) * d;
  uint16_t* vc = D.vc + ((int64_t)(r * D.nkv + j) * D.S) * d;
  const bool owner = (c == NS - 1);

  // ---- q / k / v of the group ----
  if (!sched) {
    for (int hh = wave; hh < G + 2; hh += MPK_NW) {
      const float* src = hh < G ? qkv + (int64_t)(j * G + hh) * d
                                : (hh == G ? qkv + (int64_t)D.nq * d + j * d
                                           : qkv + (int64_t)(D.nq + D.nkv) * d + j * d);
      const float a = lane < half ? gld(src + lane) : 0.f;
      const float b = lane < half ? gld(src + lane + half) : 0.f;
      if (hh <= G) {
        const float ss = wave_sum(a * a + b * b);
        const float inv = 1.0f / sqrtf(ss / (float)d + P.rms_eps);
        if (lane < half) {
          const uint16_t* g = hh < G ? D.qn : D.kn;
          const float na = bf16f(g[lane]) * (a * inv);
          const float nb = bf16f(g[lane + half]) * (b * inv);
          const float cs = gld(P.rope_cos + (int64_t)p * half + lane);
          const float sn = gld(P.rope_sin + (int64_t)p * half + lane);
          const float ra = na * cs - nb * sn;
          const float rb = nb * cs + na * sn;
          if (hh < G) {
            qs[hh * d + lane] = ra;
            qs[hh * d + lane + half] = rb;
          } else {
            const uint16_t ka = f2bf(ra), kb = f2bf(rb);
            kv[lane] = bf16f(ka);
            kv[lane + half] = bf16f(kb);
            if (owner) {
              gst16(kc + (int64_t)p * d + lane, ka);
              gst16(kc + (int64_t)p * d + lane + half, kb);
            }
          }
        }
      } else if (lane < half) {
        const uint16_t va = f2bf(a), vb = f2bf(b);
        kv[d + lane] = bf16f(va);
        kv[d + lane + half] = bf16f(vb);
        if (owner) {
          gst16(vc + (int64_t)p * d + lane, va);
          gst16(vc + (int64_t)p * d + lane + half, vb);
        }
      }
    }
  }
  __syncthreads();

  const float scale = 1.0f / sqrtf((float)d);
  float m_run[ATT_MAXG], l_run[ATT_MAXG];
  float acc[ATT_MAXG][8];
#pragma unroll
  for (int h = 0; h < ATT_MAXG; ++h) {
    m_run[h] = -INFINITY, l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const int dim0 = (lane % LP) * 8;
  const int pg = lane / LP;
  for (int base = lo; base < hi; base += MPK_ATTN_SUB) {
    const int cnt = min(MPK_ATTN_SUB, hi - base);
    // scores
    if (!sched) {
      for (int i0 = wave * PPR; i0 < cnt; i0 += MPK_NW * PPR) {
        const int t = i0 + pg;
        const bool valid = t < cnt;
        const int tau = base + t;
        float kf[8];
        if (valid && tau != p) {
          const u32x4 w = gldv<u32x4>(kc + (int64_t)tau * d + dim0);
          kf[0] = bf16lo(w.x), kf[1] = bf16hi(w.x), kf[2] = bf16lo(w.y), kf[3] = bf16hi(w.y);
          kf[4] = bf16lo(w.z), kf[5] = bf16hi(w.z), kf[6] = bf16lo(w.w), kf[7] = bf16hi(w.w);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kf[e] = valid ? kv[dim0 + e] : 0.f;
        }
#pragma unroll
        for (int h = 0; h < ATT_MAXG; ++h) {
          if (h < G) {
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(qs[h * d + dim0 + e], kf[e], part);
            for (int off = 1; off < LP; off <<= 1) part += __shfl_xor(part, off);
            if (valid && (lane % LP) == 0) sc[h * MPK_ATTN_SUB + t] = part * scale;
          }
        }
      }
    }
    __syncthreads();
    // max per head
    if (!sched) {
#pragma unroll
      for (int h = 0; h < ATT_MAXG; ++h) {
        if (h < G) {
          float mx = -INFINITY;
          for (int t = tid; t < cnt; t += MPK_NW * 64) mx = fmaxf(mx, sc[h * MPK_ATTN_SUB + t]);
          mx = wave_max(mx);
          if (lane == 0) redm[wave * ATT_MAXG + h] = mx;
        }
      }
    }
    __syncthreads();
    float m_new[ATT_MAXG], alpha[ATT_MAXG];
#pragma unroll
    for (int h = 0; h < ATT_MAXG; ++h) {
      float mx = m_run[h];
      if (h < G)
        for (int w = 0; w < MPK_NW; ++w) mx = fmaxf(mx, redm[w * ATT_MAXG + h]);
      m_new[h] = mx;
      alpha[h] = expf(m_run[h] - mx);  // m_run = -inf -> 0
    }
    if (!sched) {
#pragma unroll
      for (int h = 0; h < ATT_MAXG; ++h) {
        if (h < G) {
          float sm = 0.f;
          for (int t = tid; t < cnt; t += MPK_NW * 64) {
            const float e = expf(sc[h * MPK_ATTN_SUB + t] - m_new[h]);
            sc[h * MPK_ATTN_SUB + t] = e;
            sm += e;
          }
          sm = wave_sum(sm);
          if (lane == 0) reds[wave * ATT_MAXG + h] = sm;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < ATT_MAXG; ++h) {
      float sm = 0.f;
      if (h < G)
        for (int w = 0; w < MPK_NW; ++w) sm += reds[w * ATT_MAXG + h];
      l_run[h] = l_run[h] * alpha[h] + sm;
      m_run[h] = m_new[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
    }
    // weighted V
    if (!sched) {
      for (int i0 = wave * PPR; i0 < cnt; i0 += MPK_NW * PPR) {
        const int t = i0 + pg;
        if (t < cnt) {
          const int tau = base + t;
          float vf[8];
          if (tau != p) {
            const u32x4 w = gldv<u32x4>(vc + (int64_t)tau * d + dim0);
            vf[0] = bf16lo(w.x), vf[1] = bf16hi(w.x), vf[2] = bf16lo(w.y), vf[3] = bf16hi(w.y);
            vf[4] = bf16lo(w.z), vf[5] = bf16hi(w.z), vf[6] = bf16lo(w.w), vf[7] = bf16hi(w.w);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = kv[d + dim0 + e];
          }
#pragma unroll
          for (int h = 0; h < ATT_MAXG; ++h) {
            if (h < G) {
              const float wgt = sc[h * MPK_ATTN_SUB + t];
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(wgt, vf[e], acc[h][e]);
            }
          }
        }
      }
    }
    __syncthreads();  // sc is rewritten by the next pass
  }
  // ---- reduce acc over position groups and waves; write the split partial ----
  if (!sched) {
#pragma unroll
    for (int h = 0; h < ATT_MAXG; ++h) {
      if (h < G) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = acc[h][e];
          for (int off = LP; off < 64; off <<= 1) v += __shfl_xor(v, off);
          if (lane < LP) accr[(wave * ATT_MAXG + h) * 128 + dim0 + e] = v;
        }
      }
    }
  }
  __syncthreads();
  const int stride = d + 2;
  float* part = D.part + ((int64_t)((r * D.nkv + j) * NS + c) * G) * stride;
  for (int idx = tid; idx < G * d; idx += MPK_THREADS) {
    const int h = idx / d, i = idx - h * d;
    float v = 0.f;
    for (int w = 0; w < MPK_NW; ++w) v += accr[(w * ATT_MAXG + h) * 128 + i];
    gst(part + h * stride + 2 + i, v);
    if (i == 0) {
      gst(part + h * stride, m_run[h]);
      gst(part + h * stride + 1, l_run[h]);
    }
  }
  __syncthreads();
  if (sched && lane == 0) {
    uint32_t old = __hip_atomic_fetch_add(D.tickets + (r * D.nkv + j), 1u, __ATOMIC_ACQ_REL,
                                          __HIP_MEMORY_SCOPE_AGENT);
    ctl[1] = (old % (uint32_t)NS) == (uint32_t)NS - 1;
  }
  __syncthreads();
  const bool last = ctl[1] != 0;
  if (last) {
    const float* pbase = D.part + ((int64_t)((r * D.nkv + j) * NS) * G) * stride;
    for (int idx = tid; idx < G * d; idx += MPK_THREADS) {
      const int h = idx / d, i = idx - h * d;
      float M = -INFINITY;
      for (int cc = 0; cc < NS; ++cc) M = fmaxf(M, gld(pbase + ((int64_t)cc * G + h) * stride));
      float L = 0.f, O = 0.f;
      for (int cc = 0; cc < NS; ++cc) {
        const float* pp = pbase + ((int64_t)cc * G + h) * stride;
        const float lc = gld(pp + 1);
        if (lc > 0.f) {
          const float wgt = expf(gld(pp) - M);
          L = fmaf(lc, wgt, L);
          O = fmaf(gld(pp + 2 + i), wgt, O);
        }
      }
      gst(D.y + (int64_t)r * D.nq * d + (int64_t)(j * G + h) * d + i, O / L);
    }
  }
  return last;
}

// ---------------------------------------------------------------------------
// dispatch of one task body
// ---------------------------------------------------------------------------
template <int NB>
DEV bool run_task(const mpk_kparams& P, ctask& T, Issuer& I, RingState& RS,
                  cqent* Q, int qlen, int s, char* smem, int tid, bool sched) {
  cop& D = ops_of(P)[T.op];
  if (T.kind == MPK_TK_ATTN) return attn_task(P, T, D, smem, tid, sched);
  return gemv_task<NB>(P, T, D, I, RS, Q, qlen, s, smem, tid, sched);
}

// Spin until every dependency of T for iteration s is satisfied.  Returns
// false (after recording a status) on watchdog timeout or a stop request.
DEV bool wait_deps(const mpk_kparams& P, ctask& T, int s, int task_id) {
  const uint64_t t0 = clock_now();
  for (int k = 0; k < T.n_deps; ++k) {
    const uint32_t target = (uint32_t)T.dep_cnt[k] * (uint32_t)(s + 1 - T.dep_prev[k]);
    uint32_t* ev = P.events + T.dep_ev[k];
    int spins = 0;
    while (__hip_atomic_load(ev, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if ((++spins & 31) == 0) {
        const int code = __hip_atomic_load(&P.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int abort_req =
            __hip_atomic_load(&P.status->abort_req, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        int mine = 0;
        if (abort_req) mine = MPK_ERR_ABORTED;
        else if (clock_now() - t0 > P.timeout_ticks) mine = MPK_ERR_DEVICE_TIMEOUT;
        if (mine) {
          int expected = 0;
          if (__hip_atomic_compare_exchange_strong(&P.status->code, &expected, mine, __ATOMIC_RELAXED,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            __hip_atomic_store(&P.status->iteration, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&P.status->task, task_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          return false;
        }
        if (code) return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
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
  volatile int* ctl = reinterpret_cast<volatile int*>(smem + LDS_CTL);
  Issuer I;
  RingState RS{0, 0};
  I.live = 0;
  if (!sched && qlen > 0) {
    issuer_seek(I, P, Q, qlen, 0, 0, wave);
    ring_fill<Lay<NB>::R>(I, RS, smem + Lay<NB>::RING + wave * Lay<NB>::R * 1024, P, Q, qlen, wave, lane);
  }
  for (int s = 0; s < P.n_iter; ++s) {
    for (int k = 0; k < qlen; ++k) {
      const int task_id = Q[k].task;
      ctask& T = tasks_of(P)[task_id];
      if (sched && lane == 0) {
        const bool ok = wait_deps(P, T, s, task_id);
        ctl[0] = ok ? 0 : 1;
        if (ok && P.trace) {
          mpk_trace_record& Rr = P.trace[(int64_t)s * P.n_tasks + task_id];
          Rr.task = task_id;
          Rr.iteration = s;
          Rr.start_ticket = __hip_atomic_fetch_add(P.ticket_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          Rr.t_start = clock_now();
          Rr.hw_id = hwreg_hw_id();
          Rr.xcc_id = hwreg_xcc_id();
        }
      }
      __syncthreads();
      if (ctl[0]) {
        vm_wait<0>();  // leave no LDS-bound load in flight
        return;
      }
      // An opaque copy of the thread id per task keeps the compiler from
      // hoisting per-lane address arithmetic of every body out of the task
      // loop (it would stay live, and spill, across all bodies).
      int tid_o = tid;
      asm volatile("" : "+v"(tid_o));
      const bool sig = run_task<NB>(P, T, I, RS, Q, qlen, s, smem, tid_o, sched);
      __syncthreads();
      if (sched && lane == 0) {
        if (P.trace) {
          mpk_trace_record& Rr = P.trace[(int64_t)s * P.n_tasks + task_id];
          Rr.end_ticket = __hip_atomic_fetch_add(P.ticket_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          Rr.t_end = clock_now();
        }
        if (sig) __hip_atomic_fetch_add(P.events + T.out_ev, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
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
  // a one-entry queue holding this task, for the ring's producer side
  cqent* q1 = (cqent*)(const void*)P.single_q + task_id;
  Issuer I;
  RingState RS{0, 0};
  I.live = 0;
  mpk_kparams P1 = P;
  P1.n_iter = 1;
  if (!sched) {
    issuer_seek(I, P1, q1, 1, 0, 0, wave);
    ring_fill<Lay<NB>::R>(I, RS, smem + Lay<NB>::RING + wave * Lay<NB>::R * 1024, P1, q1, 1, wave, lane);
  }
  run_task<NB>(P, T, I, RS, q1, 1, s, smem, tid, sched);
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
  mpk_dev_qentry* d_single = nullptr;
  int32_t* d_qlen = nullptr;
  uint32_t* d_counters = nullptr;  // events | attention tickets | LM tickets | trace ticket
  int64_t n_counters = 0;
  uint32_t* d_events = nullptr;
  uint32_t* d_ticket_ctr = nullptr;
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
  for (int i = 0; i < NTEN; ++i) {
    const mpk_tensor& t = g->tensors[i];
    if (t.dev_ptr) {
      x->tensor_ptr[i] = t.dev_ptr;
    } else if (g->embed_src[i] < 0) {
      if ((rc = dalloc(x.get(), &x->tensor_ptr[i], (size_t)tensor_bytes(t)))) return rc;
    }
  }
  auto P = [&](int id) -> void* { return id >= 0 ? x->tensor_ptr[id] : nullptr; };
  const mpk_model_cfg& M = g->model;
  const int B = x->B;

  // counters: events, then per-op tickets
  std::vector<mpk_dev_op> dops = g->dops;
  int64_t ncnt = (int64_t)g->ev_count.size();
  std::vector<int64_t> tick_off(dops.size(), -1);
  for (size_t i = 0; i < dops.size(); ++i) {
    if (dops[i].kind == MPK_TK_ATTN) tick_off[i] = ncnt, ncnt += (int64_t)B * dops[i].nkv;
    if (dops[i].kind == MPK_TK_LMHEAD) tick_off[i] = ncnt, ncnt += 1;
  }
  const int64_t ticket_ctr_off = ncnt++;
  x->n_counters = ncnt;
  if ((rc = dalloc(x.get(), &x->d_counters, (size_t)ncnt * 4))) return rc;
  x->d_events = x->d_counters;
  x->d_ticket_ctr = x->d_counters + ticket_ctr_off;

  for (size_t i = 0; i < dops.size(); ++i) {
    mpk_dev_op& D = dops[i];
    const mpk_op& o = g->ops[i];
    if (!D.kind) continue;
    if (D.kind == MPK_TK_ATTN) {
      D.x = (const float*)P(o.in[0]);
      D.qn = (const uint16_t*)P(o.in[1]);
      D.kn = (const uint16_t*)P(o.in[2]);
      D.kc = (uint16_t*)P(o.in[3]);
      D.vc = (uint16_t*)P(o.in[4]);
      D.y = (float*)P(o.out[0]);
      const int G = D.nq / D.nkv;
      if (G > ATT_MAXG) return mpk_fail(MPK_ERR_SHAPE, "more than 4 query heads per kv head");
      if ((rc = dalloc(x.get(), &D.part, (size_t)B * D.nkv * D.nsplit * G * (D.d + 2) * 4))) return rc;
      D.tickets = x->d_counters + tick_off[i];
      continue;
    }
    const int e_in = o.in[0];
    D.x = D.x_embed ? nullptr : (const float*)P(e_in);
    if (D.x_embed) D.E = (const uint16_t*)P(g->embed_src[e_in]);
    D.gain = D.has_norm ? (const uint16_t*)P(o.in[1]) : nullptr;
    if (o.kind == MPK_OP_RMSNORM_LINEAR) {
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.W1 = (const uint16_t*)P(o.in[3]);
      D.W2 = (const uint16_t*)P(o.in[4]);
      D.y = (float*)P(o.out[0]);
    } else if (o.kind == MPK_OP_LINEAR_RESIDUAL) {
      D.W0 = (const uint16_t*)P(o.in[1]);
      if (D.res_embed) D.E = (const uint16_t*)P(g->embed_src[o.in[2]]);
      else D.resid = (const float*)P(o.in[2]);
      D.y = (float*)P(o.out[0]);
    } else if (o.kind == MPK_OP_RMSNORM_GATEUP) {
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.W1 = (const uint16_t*)P(o.in[3]);
      D.y = (float*)P(o.out[0]);
    } else {  // LM head
      D.W0 = (const uint16_t*)P(o.in[2]);
      D.logits = o.out[0] >= 0 ? (float*)P(o.out[0]) : nullptr;
      if ((rc = dalloc(x.get(), &D.part, (size_t)D.ntiles * B * 2 * 4))) return rc;
      D.tickets = x->d_counters + tick_off[i];
    }
  }
  if ((rc = dalloc(x.get(), &x->d_ops, dops.size() * sizeof(mpk_dev_op)))) return rc;
  HIPCHK(hipMemcpy(x->d_ops, dops.data(), dops.size() * sizeof(mpk_dev_op), hipMemcpyHostToDevice));
  if ((rc = dalloc(x.get(), &x->d_tasks, g->tasks.size() * sizeof(mpk_dev_task)))) return rc;
  HIPCHK(hipMemcpy(x->d_tasks, g->tasks.data(), g->tasks.size() * sizeof(mpk_dev_task), hipMemcpyHostToDevice));
  if ((rc = dalloc(x.get(), &x->d_queues, g->queues.size() * sizeof(mpk_dev_qentry)))) return rc;
  HIPCHK(hipMemcpy(x->d_queues, g->queues.data(), g->queues.size() * sizeof(mpk_dev_qentry), hipMemcpyHostToDevice));
  {
    std::vector<mpk_dev_qentry> single(g->tasks.size());
    for (size_t i = 0; i < single.size(); ++i) single[i] = mpk_dev_qentry{(int32_t)i, -1};
    if ((rc = dalloc(x.get(), &x->d_single, single.size() * sizeof(mpk_dev_qentry)))) return rc;
    HIPCHK(hipMemcpy(x->d_single, single.data(), single.size() * sizeof(mpk_dev_qentry), hipMemcpyHostToDevice));
  }
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
  K.single_q = x->d_single;
  K.qlen = x->d_qlen;
  K.events = x->d_events;
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
  *out = x.release();
  return MPK_OK;
}

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
  }
  x->kp.n_iter = n_iter;
  x->last_iters = n_iter;
  int64_t nz = x->n_counters;
  hipLaunchKernelGGL(mpk_zero_u32, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, x->d_counters, nz);
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
    for (size_t i = 0; i < g->ops.size(); ++i) {
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
  hipSetDevice(x->device);
  for (void* p : x->owned) hipFree(p);
  if (x->side) hipStreamDestroy(x->side);
  delete x;
}
