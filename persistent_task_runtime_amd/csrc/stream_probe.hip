// stream_probe.hip -- measured HBM read-stream ceiling of the device.
//
// The decode step is bound by streaming its weights once per iteration (P3
// "Why MPK?", Figure 1: the bound is the weight bytes over the memory
// bandwidth).  The published 8 TB/s of MI355X is a peak; what a kernel can
// actually read is lower.  This kernel reads a buffer once with the same load
// form the weight streams use (16-byte nontemporal global loads, every lane
// of a 64-wide wavefront on consecutive 16 bytes), so a roofline fraction can
// be stated against both the published peak and this measured ceiling.
//
// It stores nothing unless the XOR of everything it read equals a fixed
// constant, which keeps the loads live without adding traffic.
#include <hip/hip_runtime.h>

#include <string>

#include "graph.hpp"
#include "mpk.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef const v4u __attribute__((address_space(1))) gv4u;

constexpr int kThreads = 512;                  // 8 wavefronts per workgroup
constexpr int kDepth = 16;                     // 16-byte loads in flight per lane
constexpr uint64_t kUnit = kThreads * kDepth;  // 16-byte vectors per workgroup step (128 KiB)

// Workgroup g reads units g, g + G, g + 2G, ... (G = gridDim.x); consecutive
// workgroups land on consecutive XCDs, so every XCD streams a slice of every
// region of the buffer.  A unit's 16 loads per lane are all issued before the
// first is consumed; with several workgroups per CU the units of one overlap
// the tail of another's.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const v4u* __restrict__ src, uint64_t n_units,
                                                               uint32_t* __restrict__ sink) {
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  for (uint64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
    gv4u* p = (gv4u*)(src + u * kUnit + tid);
    v4u v[kDepth];
#pragma unroll
    for (int j = 0; j < kDepth; ++j) v[j] = __builtin_nontemporal_load(p + j * kThreads);
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
#pragma unroll
    for (int j = 0; j < kDepth; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x6a09e667u) sink[0] = acc;
}

}  // namespace

extern "C" int mpk_stream_read(const void* src, uint64_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  mpk_clear_error();
  if (!src || !sink) return mpk_fail(MPK_ERR_INVALID_ARG, "NULL buffer");
  if (workgroups < 1) return mpk_fail(MPK_ERR_INVALID_ARG, "workgroups must be at least 1");
  const uint64_t unit_bytes = kUnit * 16;
  if (bytes == 0 || bytes % unit_bytes)
    return mpk_fail(MPK_ERR_SHAPE, "bytes must be a positive multiple of " + std::to_string(unit_bytes));
  if ((uintptr_t)src % 16 || (uintptr_t)sink % 4) return mpk_fail(MPK_ERR_ALIGN, "src must be 16-byte aligned");
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                     (const v4u*)src, bytes / unit_bytes, sink);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return mpk_fail(MPK_ERR_HIP, std::string("stream_read_kernel: ") + hipGetErrorString(e));
  return MPK_OK;
}
