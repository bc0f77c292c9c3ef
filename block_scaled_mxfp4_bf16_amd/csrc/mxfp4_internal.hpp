// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxfp4 {

// A GEMM schedule: compile-time tile shape plus the runtime split count.
//   mt    16-row M tiles per workgroup (the workgroup covers 16*mt rows)
//   nt    16-column N subtiles per wave
//   wn    waves side by side along N; they share the A the workgroup stages
//   wk    waves that split the workgroup's K run and add through LDS
//   kpw   128-wide K steps per wave (a workgroup covers wk*kpw steps)
//   split workgroups that split K for one output tile; the last to finish
//         adds the partial sums from the workspace and stores C
//   pq    1: the GEMM reads A already quantized, in the caller's layout
//         (codes [M, K/2] and shuffled scales): mxfp4_gemm_q's A as it is, or
//         bf16 A quantized into the workspace by a launch of its own; 0: the
//         GEMM quantizes A
//   rb    rows per staged A block: 16, or 8 (for M <= 8: no loads or
//         converts are spent on rows that do not exist)
//   wide  1: the large-M kernel -- A quantized once, wk waves per
//         workgroup that split K, each holding the whole 16*mt x 16*nt
//         tile; kpw is then the number of K steps loaded ahead; 3: the
//         same kernel with B staged through LDS
//   epi   how split K partials meet: 0 ticketed slots added in split
//         order; 1 float atomics into one f32 tile (zero-filled by a launch
//         of its own); 2 stream-K -- `split` is then the number of
//         workgroups of the whole grid, each taking an equal run of the
//         tiles x K steps iterations
struct Schedule {
  int mt, nt, wn, wk, kpw, split, pq, rb, wide;
  int epi;
  int variant;  // index into the kernel table
};

// Split-K workspace layout: a fixed prefix of ticket words (one per output
// tile, zero between calls), then the f32 partial tiles.  The prefix has the
// same size for every shape, so a workspace can serve shapes one after
// another without the partials of one landing on the tickets of the next.
constexpr size_t kTicketBytes = 65536;
constexpr int kMaxSplitTiles = (int)(kTicketBytes / 4);
// Largest stream-K grid (its partials take two tiles per workgroup).
constexpr int kMaxStreamKGroups = 8192;

struct GemmArgs {
  const void *A;
  const void *Bw;
  const void *Bs;
  void *C;
  void *workspace;
  int M, N, K;
  // A already quantized (mxfp4_gemm_q): codes [M, K/2] and shuffled scales;
  // then A is unused and only pre-quantized schedules run.
  const void *Aq = nullptr;
  const void *As = nullptr;
};

// Kernel table queries (gemm_kernels.hip).
int num_gemm_variants();
void gemm_variant_shape(int v, Schedule *s);  // fills everything but split
int find_gemm_variant(int mt, int nt, int wn, int wk, int kpw, int pq, int rb, int wide, int epi = 0);

// Bytes of quantized A in the workspace: the larger of the two layouts
// (the caller's -- codes, 256-byte aligned, then shuffled scales with rows
// padded to 256 -- and the large-M kernel's quad-packed one), so one
// workspace size serves either.
inline size_t caller_codes_bytes(int M, int K) { return ((size_t)M * (K / 2) + 255) & ~(size_t)255; }
inline size_t caller_a_bytes(int M, int K) {
  return caller_codes_bytes(M, K) + (size_t)((M + 255) & ~255) * (size_t)(((K / 32) + 7) & ~7);
}
size_t quad_operand_bytes(int M, int K);
inline size_t pq_operand_bytes(int M, int K) {
  const size_t a = caller_a_bytes(M, K), b = quad_operand_bytes(M, K);
  return a > b ? a : b;
}

// Large-M kernels compiled (gemm_wide.hip): (row tiles, column subtiles,
// waves, K steps loaded ahead).
#define MXFP4_WIDE_VARIANTS(X)                                                                          \
  X(4, 7, 8, 2) X(4, 7, 4, 2) X(4, 8, 8, 2) X(4, 6, 8, 2) X(4, 4, 8, 2) X(4, 4, 8, 3) X(4, 3, 8, 2) \
  X(4, 3, 8, 3) X(4, 2, 8, 2) X(4, 2, 8, 4) X(4, 1, 8, 4) X(8, 2, 8, 2) X(8, 3, 8, 2)
#define MXFP4_DECLARE_WIDE(MW, NW, W, D) \
  hipError_t launch_wide_##MW##_##NW##_##W##_##D(const GemmArgs &a, int split, bool sw, hipStream_t stream);
MXFP4_WIDE_VARIANTS(MXFP4_DECLARE_WIDE)
#undef MXFP4_DECLARE_WIDE
// ... with B's codes staged through a per-wave LDS ring of D steps.
#define MXFP4_WIDEL_VARIANTS(X) X(4, 7, 4, 4) X(4, 7, 4, 3) X(4, 4, 8, 2) X(4, 2, 8, 4) X(4, 8, 4, 3)
#define MXFP4_DECLARE_WIDEL(MW, NW, W, D) \
  hipError_t launch_widel_##MW##_##NW##_##W##_##D(const GemmArgs &a, int split, bool sw, hipStream_t stream);
MXFP4_WIDEL_VARIANTS(MXFP4_DECLARE_WIDEL)
#undef MXFP4_DECLARE_WIDEL

size_t gemm_workspace_bytes(const Schedule &s, int M, int N, int K);
hipError_t launch_gemm(const Schedule &s, const GemmArgs &a, bool sw_quant, hipStream_t stream);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);  // bytes: a multiple of 16

hipError_t launch_quantize(const void *x, int64_t rows, int64_t K, void *q, void *scales, bool shuffled, bool sw,
                           hipStream_t stream);
hipError_t launch_preshuffle_b(const void *bq, const void *bs_raw, int64_t N, int64_t K, void *bq_sh, void *bs_sh,
                               hipStream_t stream);
hipError_t launch_prepare_b(const void *b, int64_t N, int64_t K, void *bq_sh, void *bs_sh, bool sw, hipStream_t stream);

}  // namespace mxfp4
