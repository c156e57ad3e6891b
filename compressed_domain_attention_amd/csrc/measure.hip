// Measurement helper: a plain streaming read of device memory, the ceiling
// against which the decode's bandwidth is reported (a read of the same
// bytes, in the same launch pattern, with no arithmetic on them).
//
// Every thread reads 16-byte words in a grid-stride pattern, sixteen of them
// requested at a time, and folds them into one XOR; each workgroup writes one
// word to `sink` so the loads cannot be dropped.

#include "cdattn_measure.h"
#include "internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 16;   // 16-byte loads requested together per thread

// Word i of the read is 16-byte word (g + i * total_threads) of the buffer
// for global thread g: a grid-stride pattern whose every round requests
// kInFlight words per thread at once; words past the end are out of the
// buffer's range and read as zeros without touching memory.
__global__ __launch_bounds__(kThreads) void read_kernel(const void *src, uint32_t bytes, uint32_t per_thread,
                                                        uint32_t *__restrict__ sink) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(src), (short)0, (int)bytes,
                                                                    0x00020000);
  const uint32_t total = gridDim.x * kThreads;
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  uint32_t x = 0;
  for (uint32_t i0 = 0; i0 < per_thread; i0 += kInFlight) {
    uint4 w[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      w[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, 16u * (g + (i0 + u) * total), 0, 0));
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) x ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int k = 0; k < kThreads; ++k) t ^= red[k];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

extern "C" int codec_measure_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups,
                                  hipStream_t stream) {
  if (!src || !sink) return 1;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || bytes % 16 || bytes == 0 || bytes > (1u << 31)) return 2;
  if (workgroups < 1 || workgroups > 65536) return 2;
  const uint64_t words = bytes / 16, threads = (uint64_t)workgroups * kThreads;
  const uint32_t per_thread = (uint32_t)((words + threads - 1) / threads);
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, stream, src, (uint32_t)bytes,
                     per_thread, sink);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}
