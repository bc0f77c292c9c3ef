// Phase-timing probe of the large-M kernel (libmxfp4_probes.so; used by
// bench.py --floors only).  It runs the library's A quantization and the
// 64 x 112-tile, four-wave K loop (the schedule of 256 x 7168 x 7168) with
// the loop's STAMPS flag on, built with the library's flags for that
// source, so the code between the stamps is the library's.  Each wave
// writes five 100 MHz real-time stamps (entry, K loop done, partial tiles
// in LDS, C stores issued, C stores complete) and its XCD number at
// stamps[(workgroup * 4 + wave) * 8 + i]; C is written as by the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_wide.hpp"

extern "C" {

// Bytes of the quad-packed A operand for M x K.
__attribute__((visibility("default"))) size_t mxfp4_probe_wide_operand_bytes(int M, int K) {
  const size_t mq = (size_t)((M + 63) / 64), ks = (size_t)((K + 127) / 128);
  return mq * ks * (4 * 1024 + 256);
}

// A (bf16, M x K) -> quad-packed operand at aop (operand_bytes(M, K) bytes).
__attribute__((visibility("default"))) int mxfp4_probe_wide_quant(const void *A, void *aop, int M, int K,
                                                                  void *stream) {
  if (!A || !aop) return 1;
  if (M < 1 || K < 128 || K % 64 != 0) return 2;
  const int units = ((M + 63) / 64) * ((K + 127) / 128);
  mxfp4::quant_quad_kernel<<<units, 128, 0, (hipStream_t)stream>>>((const uint16_t *)A, (uint8_t *)aop, M, K, 0);
  return (int)hipGetLastError();
}

// The stamped K loop; returns 0, 1 (null pointer), 2 (N not a multiple of
// 112, or bad sizes), 3 (stamp_words below workgroups * 4 * 8), or the HIP
// error.
__attribute__((visibility("default"))) int mxfp4_probe_wide_phases(const void *aop, const void *Bw, const void *Bs,
                                                                   void *C, void *stamps, size_t stamp_words, int M,
                                                                   int N, int K, void *stream) {
  if (!aop || !Bw || !Bs || !C || !stamps) return 1;
  if (M < 1 || N < 112 || N % 112 != 0 || K < 128 || K % 64 != 0) return 2;
  const int n_tiles = N / 112, m_tiles = (M + 63) / 64;
  const size_t grid = (size_t)n_tiles * m_tiles;
  if (stamp_words < grid * 4 * 8) return 3;
  mxfp4::gemm_wide_kernel<4, 7, 4, 2, false, true><<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(
      (const uint8_t *)aop, (const uint8_t *)Bw, (const uint8_t *)Bs, (uint16_t *)C, (float *)stamps, nullptr, M, N,
      K, 1, n_tiles, m_tiles);
  return (int)hipGetLastError();
}

}  // extern "C"
