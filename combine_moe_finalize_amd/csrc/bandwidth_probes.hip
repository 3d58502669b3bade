// gfx950 streaming read and copy kernels: the HBM rates a plain stream
// reaches, measured beside the finalize kernels in the same session; and an
// empty kernel, the per-launch floor that small calls are compared with.
//
// Work layout: one 256-lane workgroup covers 16 KiB, 1024 vectors of 16
// bytes; lane t of the workgroup takes vectors t, t + 256, t + 512 and
// t + 768, so each wave instruction moves 1 KiB of consecutive bytes and a
// lane has four loads in flight before it uses any of them. The byte count is
// a multiple of 16 KiB, so the grid covers it exactly and every access is in
// bounds.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bandwidth_probes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPerLane = 4;
constexpr int kVecsPerBlock = kThreads * kPerLane;          // 16 KiB
static_assert(kVecsPerBlock * 16 == MOEF_PROBE_GRAIN, "one workgroup covers one grain");
constexpr uint32_t kSentinel = 0x9E3779B9u;

__global__ void __launch_bounds__(kThreads)
read_probe_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kVecsPerBlock + threadIdx.x;
  u32x4 v[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) v[u] = __builtin_nontemporal_load(src + base + u * kThreads);
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (x == kSentinel) sink[0] = x;
}

__global__ void __launch_bounds__(kThreads)
copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  const int64_t base = (int64_t)blockIdx.x * kVecsPerBlock + threadIdx.x;
  u32x4 v[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) v[u] = __builtin_nontemporal_load(src + base + u * kThreads);
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) __builtin_nontemporal_store(v[u], dst + base + u * kThreads);
}

// One wave that does nothing: what a launch costs before any memory access.
__global__ void __launch_bounds__(64) empty_probe_kernel() {}

// A dispatch packet counts a grid's work-items in 32 bits: at most
// (2^32 - 1) / 256 workgroups of 256 lanes, one grain each.
bool grain_count_ok(int64_t bytes) {
  return bytes > 0 && bytes % MOEF_PROBE_GRAIN == 0 &&
         bytes / MOEF_PROBE_GRAIN <= MOEF_PROBE_MAX_GRAINS;
}

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace

extern "C" {

int moef_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr) return 1;
  if (!grain_count_ok(bytes)) return 2;
  if (!aligned(src, 16) || !aligned(sink, 4)) return 4;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned int)(bytes / MOEF_PROBE_GRAIN)),
                     dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), sink);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int moef_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr) return 1;
  if (!grain_count_ok(bytes)) return 2;
  if (!aligned(src, 16) || !aligned(dst, 16)) return 4;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes) return 6;
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned int)(bytes / MOEF_PROBE_GRAIN)),
                     dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst));
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int moef_probe_empty(void* stream) {
  hipLaunchKernelGGL(empty_probe_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int moef_probe_mark(void* stream) {
  hipLaunchKernelGGL(empty_probe_kernel, dim3(2), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
