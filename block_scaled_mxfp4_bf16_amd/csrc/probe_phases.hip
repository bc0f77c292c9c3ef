// Phase-timing probe of the fused small-M kernel (libmxfp4_probes.so; used by
// bench.py --floors only).  It instantiates the fused kernel with its STAMPS
// flag on for four split-1 schedules, built with the same flags as the
// library's own instantiations, so the code between the stamps is the
// library's:
//   which 0: 1 m tile x 2 subtiles x 1 column wave x 4 K waves x 1 step
//            (the schedule of 32 x 4096 x 512);
//   which 1: the same with 1 subtile, 14 K waves of 4 steps, 8-row A blocks
//            (the schedule of 8 x 2112 x 7168);
//   which 2: 2 subtiles, 4 K waves of 3 steps (16 x 3072 x 1536);
//   which 3: 2 subtiles x 4 column waves, 4 K waves of 4 steps
//            (64 x 7168 x 2048).
// Each wave writes six 100 MHz real-time stamps (entry, loads issued, A
// staged, products done, C stores issued, C stores complete) at
// stamps[(workgroup * waves + wave) * 8 + i]; C is written as by the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_fused.hpp"

namespace {

template <int MT, int NT, int WN, int WK, int KPW, int RB>
int launch_stamped(const void *A, const void *Bw, const void *Bs, void *C, void *stamps, size_t stamp_words, int M,
                   int N, int K, int sw, hipStream_t stream) {
  if (N % (16 * NT * WN) != 0 || K % 64 != 0) return 2;
  const int ks = (K + 127) / 128;
  if (ks > WK * KPW) return 2;  // one workgroup must cover the whole K range
  if (RB == 8 ? M > 8 : M < 1) return 2;
  const int n_tiles = N / (16 * NT * WN);
  const int m_tiles = (M + 16 * MT - 1) / (16 * MT);
  const size_t grid = (size_t)n_tiles * m_tiles;
  if (stamp_words < grid * WN * WK * 8) return 3;
  mxfp4::gemm_kernel<MT, NT, WN, WK, KPW, false, RB, 0, true><<<(unsigned)grid, 64 * WN * WK, 0, stream>>>(
      (const uint16_t *)A, nullptr, nullptr, (const uint8_t *)Bw, (const uint8_t *)Bs, (uint16_t *)C, (float *)stamps,
      nullptr, M, N, K, 1, n_tiles, sw ? 1 : 0);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// Returns 0 on success, 1 for a null pointer, 2 for a shape the schedule does
// not serve in one workgroup per tile, 3 if `stamp_words` (uint64 words at
// `stamps`) is below workgroups * waves * 8, else the HIP error.
__attribute__((visibility("default"))) int mxfp4_probe_phases(int which, const void *A, const void *Bw,
                                                              const void *Bs, void *C, void *stamps,
                                                              size_t stamp_words, int M, int N, int K, int sw,
                                                              void *stream) {
  if (!A || !Bw || !Bs || !C || !stamps) return 1;
  if (M < 1 || N < 1 || K < 1) return 2;
  switch (which) {
    case 0: return launch_stamped<1, 2, 1, 4, 1, 16>(A, Bw, Bs, C, stamps, stamp_words, M, N, K, sw,
                                                    (hipStream_t)stream);
    case 1: return launch_stamped<1, 1, 1, 14, 4, 8>(A, Bw, Bs, C, stamps, stamp_words, M, N, K, sw,
                                                    (hipStream_t)stream);
    case 2: return launch_stamped<1, 2, 1, 4, 3, 16>(A, Bw, Bs, C, stamps, stamp_words, M, N, K, sw,
                                                    (hipStream_t)stream);
    case 3: return launch_stamped<1, 2, 4, 4, 4, 16>(A, Bw, Bs, C, stamps, stamp_words, M, N, K, sw,
                                                    (hipStream_t)stream);
    default: return 2;
  }
}

// Waves per workgroup of schedule `which` (0 if unknown).
__attribute__((visibility("default"))) int mxfp4_probe_phases_waves(int which) {
  return which == 0 ? 4 : which == 1 ? 14 : which == 2 ? 4 : which == 3 ? 16 : 0;
}

}  // extern "C"
