// Measurement probes for the benchmark's floors (libmxfp4_probes.so; used by
// bench.py --floors only, never by the GEMM library):
//   - an empty kernel: the cost of one launch on its own;
//   - a streaming read: the least time to bring a buffer of a workload's B
//     size in from memory with one launch of plain coalesced loads;
//   - scaled FP4 matrix instructions back to back: the issue rate the
//     matrix units reach, with the shader clock measured alongside.
// Every access stays inside the buffer sizes the host passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void empty_kernel() {}

// Grid-stride read of n16 16-byte chunks; a lane's chunks are xor-folded and
// written only if the fold equals a value the data never gives (keeps the
// loads alive without writing anything).
__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                     uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t x = 0;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = p[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (x == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = x;
}

// Each wave issues `iters` rounds of eight independent scaled e2m1 x e2m1
// 16x16x128 instructions on register operands.  Lane 0 of each
// workgroup's first wave records the shader-clock counter (s_memtime) and
// the 100 MHz real-time counter (s_memrealtime) before and after.
__global__ __launch_bounds__(256) void mfma_kernel(float *__restrict__ out, uint64_t *__restrict__ stamps, int iters) {
  const int lane = threadIdx.x & 63;
  v8i a = {lane, lane * 3, lane * 5, lane * 7, 0, 0, 0, 0};
  v8i b = {lane * 11, lane * 13, lane * 17, lane * 19, 0, 0, 0, 0};
  v4f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 4, 4, 0, 120, 0, 120);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    stamps[blockIdx.x * 4 + 0] = t0;
    stamps[blockIdx.x * 4 + 1] = t1;
    stamps[blockIdx.x * 4 + 2] = r0;
    stamps[blockIdx.x * 4 + 3] = r1;
  }
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int mxfp4_probe_empty(void *stream) {
  empty_kernel<<<1, 64, 0, (hipStream_t)stream>>>();
  return (int)hipGetLastError();
}

// p: bytes (a multiple of 16) readable; sink: wgs * 256 uint32 writable.
__attribute__((visibility("default"))) int mxfp4_probe_stream(const void *p, size_t bytes, void *sink, int wgs,
                                                              void *stream) {
  if (!p || !sink || wgs < 1 || bytes % 16 != 0) return 1;
  stream_kernel<<<wgs, 256, 0, (hipStream_t)stream>>>((const u32x4 *)p, bytes / 16, (uint32_t *)sink);
  return (int)hipGetLastError();
}

// out: wgs * 256 floats; stamps: wgs * 4 uint64.
__attribute__((visibility("default"))) int mxfp4_probe_mfma(void *out, void *stamps, int wgs, int iters,
                                                            void *stream) {
  if (!out || !stamps || wgs < 1 || iters < 1) return 1;
  mfma_kernel<<<wgs, 256, 0, (hipStream_t)stream>>>((float *)out, (uint64_t *)stamps, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
