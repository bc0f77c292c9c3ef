// Large-M MXFP4 GEMM for gfx950: A quantized once by its own launch, then a
// K loop in which the waves of a workgroup split K instead of the tile.
//
// Submission 711914 quantizes A with a standalone kernel when M is large
// and hands the FP4 operands to a GEMM; this is that split, with our own
// kernels.  The design follows from what bounds the shape on MI355X:
//   - Each CU's vector cache keeps only about 64 lines (128 bytes each)
//     outstanding to L2, and under this load a line takes ~450 cycles to
//     arrive, so a CU's time is about (lines it requests) x 450 / 64 cycles
//     however many loads its waves have in flight.  A workgroup that owns a
//     BM x BN output tile requests (BM + BN) * K / 2 bytes of codes, so the
//     tile should be as close to square as the grid allows: at 256 x 7168 x
//     7168, 64 x 112 tiles make exactly 256 workgroups, one per CU.
//   - Every wave holds the accumulators of the whole tile and takes every
//     fourth 128-wide K step, loading that step's operands straight into
//     registers three steps ahead.  No byte is loaded twice by one
//     workgroup and nothing passes through LDS in the loop; the four
//     partial tiles are added through LDS once, at the end.
//   - Workgroups that share B columns run on one XCD (workgroups are
//     dealt to the eight XCDs in turn), so B comes from HBM about once and
//     from that XCD's L2 for the other row tiles.
//
// Quad-packed operand layout of quantized A (the workspace holds it):
//   codes   for 16-row tile t < 4*MQ and K step ks < KS (MQ = ceil(M/64),
//           KS = ceil(K/128)): 1 KiB at (t*KS + ks)*1024, operand lane L's
//           16 bytes at 16*L -- rows 16t + L%16, K chunk L/16 of the step,
//           32 codes with element 2i in the low nibble of byte i;
//   scales  after the codes, for tile quad q and step ks: 256 bytes at
//           (q*KS + ks)*256; dword L holds operand lane L's scale bytes of
//           tiles 4q..4q+3 (byte j for tile 4q+j).
// One dword per lane then serves the scale operand of four matrix
// instructions, selected by the instruction's operand byte select.
#include "gemm_wide.hpp"

namespace mxfp4 {

size_t quad_operand_bytes(int M, int K) {
  const size_t mq = (size_t)((M + 63) / 64), ks = (size_t)((K + 127) / 128);
  return mq * ks * (4 * 1024 + 256);
}

// Pre-quantized A (codes [M, K/2] as mxfp4_quantize writes them, scales in
// the shuffled layout) -> quad-packed operand.  One single-wave workgroup
// per (tile quad q, step ks): for each of the quad's four tiles, operand
// lane L takes the 16 code bytes of row 16(4q+j) + L%16, K chunk
// 4ks + L/16; the four tiles' scale bytes of lane L make one dword.  Rows
// past M and chunks past K become zero codes with scale byte 0.
__global__ __launch_bounds__(64) void repack_quad_kernel(const uint8_t *__restrict__ Aq, const uint8_t *__restrict__ As,
                                                         uint8_t *__restrict__ Aop, int M, int K) {
  const int lane = threadIdx.x;
  const int KS = (K + 127) >> 7;
  const int q = blockIdx.x / KS, ks = blockIdx.x - (blockIdx.x / KS) * KS;
  const int G = K >> 5, gp = (G + 7) & ~7;
  const int mq = (M + 63) >> 6;
  const int grp = 4 * ks + (lane >> 4);
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Aq, 0, M * (K >> 1), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)As, 0, ((M + 255) & ~255) * gp, kRsrcWord3);
  u32x4 v[4];
  uint32_t sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (4 * q + j) * 16 + (lane & 15);
    const bool ok = row < M && grp < G;
    v[j] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off_or_oob(ok, row * (K >> 1) + grp * 16), 0, 0);
    sc[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, off_or_oob(ok, (int)shuffled_scale_offset(row, grp, gp)), 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) *(u32x4 *)(Aop + (size_t)((4 * q + j) * KS + ks) * 1024 + lane * 16) = v[j];
  uint32_t *scales = (uint32_t *)(Aop + (size_t)mq * 4 * KS * 1024);
  scales[(size_t)(q * KS + ks) * 64 + lane] = sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24);
}

template <int MW, int NW, int W, int D, bool BL>
static hipError_t launch_wide(const GemmArgs &a, int split, bool sw, hipStream_t stream) {
  char *ws = (char *)a.workspace;
  uint8_t *aop = (uint8_t *)(ws + kTicketBytes);
  const int units = ((a.M + 63) / 64) * ((a.K + 127) / 128);  // (tile quad, K step)
  if (a.Aq)
    repack_quad_kernel<<<units, 64, 0, stream>>>((const uint8_t *)a.Aq, (const uint8_t *)a.As, aop, a.M, a.K);
  else
    quant_quad_kernel<<<units, 128, 0, stream>>>((const uint16_t *)a.A, aop, a.M, a.K, sw ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_tiles = a.N / (16 * NW);
  const int m_tiles = (a.M + 16 * MW - 1) / (16 * MW);
  uint32_t *tickets = (uint32_t *)ws;
  float *partials =
      split > 1 ? (float *)(ws + kTicketBytes + ((pq_operand_bytes(a.M, a.K) + 255) & ~(size_t)255)) : nullptr;
  dim3 grid((unsigned)(n_tiles * m_tiles * split));
  gemm_wide_kernel<MW, NW, W, D, BL><<<grid, 64 * W, 0, stream>>>(aop, (const uint8_t *)a.Bw, (const uint8_t *)a.Bs,
                                                               (uint16_t *)a.C, partials, tickets, a.M, a.N, a.K,
                                                               split, n_tiles, m_tiles);
  return hipGetLastError();
}

#define MXFP4_DEFINE_WIDE(MW, NW, W, D)                                                                          \
  hipError_t launch_wide_##MW##_##NW##_##W##_##D(const GemmArgs &a, int split, bool sw, hipStream_t stream) { \
    return launch_wide<MW, NW, W, D, false>(a, split, sw, stream);                                              \
  }
MXFP4_WIDE_VARIANTS(MXFP4_DEFINE_WIDE)
#undef MXFP4_DEFINE_WIDE
#define MXFP4_DEFINE_WIDEL(MW, NW, W, D)                                                                          \
  hipError_t launch_widel_##MW##_##NW##_##W##_##D(const GemmArgs &a, int split, bool sw, hipStream_t stream) { \
    return launch_wide<MW, NW, W, D, true>(a, split, sw, stream);                                                \
  }
MXFP4_WIDEL_VARIANTS(MXFP4_DEFINE_WIDEL)
#undef MXFP4_DEFINE_WIDEL

}  // namespace mxfp4
