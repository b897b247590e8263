// Plain streaming read of a device buffer: the read rate that this chip
// reaches for a given byte count with the simplest well-shaped kernel. The
// decode kernels move the same kind of traffic (large non-temporal 16-byte
// reads from HBM), so this rate is the practical ceiling that their
// measured rates are set against, next to the published HBM peak.
//
// Measurement only: it is not part of the attention API and is built into
// a library of its own (libkvprobe.so).
//
// Each workgroup (256 threads) reads one contiguous range of the buffer,
// every lane keeping 8 independent 16-byte loads in flight, and XORs what
// it reads into one 32-bit word per thread (the sink), so that the loads
// cannot be dropped and a test can check that every byte was read once.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
thread_local hipError_t g_last = hipSuccess;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(
    const u32x4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t base = (size_t)blockIdx.x * per;
  const size_t end = base + per < n16 ? base + per : n16;
  uint32_t acc = 0;
  size_t i = base + threadIdx.x;
  // every load of the unrolled body lies below `end`
  for (; i + (size_t)(kUnroll - 1) * kThreads < end; i += (size_t)kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + i + (size_t)u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// The HIP error of this thread's last failed launch ("no error" if none).
const char* kvprobe_last_error(void) { return hipGetErrorString(g_last); }

// Threads per workgroup of kvprobe_stream_read: the sink holds one 32-bit
// word per thread, workgroups * kvprobe_threads() words in all.
int kvprobe_threads(void) { return kThreads; }

// Reads `bytes` bytes at `src` (device memory, 16-byte aligned, bytes a
// multiple of 16) with `workgroups` workgroups on `stream` (a hipStream_t;
// null = the default stream). `sink` (device memory, at least
// workgroups * 256 * 4 bytes) receives each thread's XOR of the 32-bit
// words it read; the XOR of all sink words is the XOR of the whole
// buffer. Returns 0 once launched, -1 for invalid arguments (nothing is
// launched), -4 if the launch fails (kvprobe_last_error names the error).
int kvprobe_stream_read(const void* src, size_t bytes, void* sink,
                        size_t sink_bytes, int workgroups, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0 || workgroups < 1 ||
      workgroups > (1 << 20) ||
      sink_bytes < (size_t)workgroups * kThreads * sizeof(uint32_t))
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0,
                     (hipStream_t)stream, (const u32x4*)src, bytes / 16,
                     (uint32_t*)sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) g_last = e;
  return e == hipSuccess ? 0 : -4;
}

}  // extern "C"
