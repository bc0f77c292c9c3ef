// Standalone quantization and B-layout kernels for gfx950.
//
//   quantize_raw      bf16 [rows, K] -> packed e2m1 [rows, K/2] + raw e8m0 [rows, K/32]
//   quantize_shuffled same codes; scales written in the shuffled, padded layout
//   preshuffle_b_data packed e2m1 [N, K/2] -> 16x16-byte tile layout
//   shuffle_scales    raw e8m0 [N, K/32] -> shuffled, padded layout
//   prepare_b         bf16 [N, K] -> both GEMM layouts of B in one pass
//
// One lane owns one 32-element group: a 64-byte load, the group scale, 16
// converts and a 16-byte store; nothing crosses lanes.  These kernels prepare
// B offline and give a standalone A quantization; the GEMM hot path fuses
// the same group quantizer into its K loop.
#include "mxfp4_device.hpp"
#include "mxfp4_internal.hpp"

namespace mxfp4 {

__device__ __forceinline__ void load_group(const uint4 *__restrict__ src, uint32_t (&w)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 v = src[i];
    w[4 * i + 0] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// Group index idx = row * G + g addresses 64 bytes of input at idx * 64 and
// 16 bytes of output at idx * 16 (rows are contiguous).
template <bool SW>
__global__ __launch_bounds__(256) void quantize_raw_kernel(const uint4 *__restrict__ x, uint4 *__restrict__ q,
                                                           uint8_t *__restrict__ scales, uint32_t groups) {
  uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= groups) return;
  uint32_t w[16];
  load_group(x + (size_t)idx * 4, w);
  uint32_t c[4];
  uint32_t s = quant_group32<SW>(w, c);
  q[idx] = make_uint4(c[0], c[1], c[2], c[3]);
  scales[idx] = (uint8_t)s;
}

// One lane per (row, group) slot of the padded scale buffer
// [pad256(rows), gp]; slots outside the matrix get the fill byte 127.
template <bool SW>
__global__ __launch_bounds__(256) void quantize_shuffled_kernel(const uint4 *__restrict__ x, uint4 *__restrict__ q,
                                                                uint8_t *__restrict__ scales, uint32_t rows,
                                                                uint32_t G, uint32_t gp, uint32_t slots) {
  uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= slots) return;
  uint32_t row = idx / gp, g = idx - row * gp;
  uint32_t off = shuffled_scale_offset(row, g, gp);
  if (row >= rows || g >= G) {
    scales[off] = 127;
    return;
  }
  uint32_t gi = row * G + g;
  uint32_t w[16];
  load_group(x + (size_t)gi * 4, w);
  uint32_t c[4];
  uint32_t s = quant_group32<SW>(w, c);
  q[gi] = make_uint4(c[0], c[1], c[2], c[3]);
  scales[off] = (uint8_t)s;
}

// One lane per 16-byte output chunk c = (g * T + t) * 16 + n, T = K/32 tiles
// per 16-row group: chunk holds bytes 16t..16t+15 of row 16g+n.
__global__ __launch_bounds__(256) void preshuffle_b_data_kernel(const uint4 *__restrict__ bq,
                                                                uint4 *__restrict__ out, uint32_t T,
                                                                uint32_t chunks) {
  uint32_t c = blockIdx.x * 256u + threadIdx.x;
  if (c >= chunks) return;
  uint32_t n = c & 15u;
  uint32_t gt = c >> 4;
  uint32_t g = gt / T, t = gt - g * T;
  // input row 16g+n has T chunks of 16 bytes
  out[c] = bq[(size_t)(16u * g + n) * T + t];
}

// One lane per byte of the shuffled buffer: invert the byte address into
// (row, group) and copy, or fill with 127 outside the matrix.
__global__ __launch_bounds__(256) void shuffle_scales_kernel(const uint8_t *__restrict__ raw,
                                                             uint8_t *__restrict__ out, uint32_t rows, uint32_t G,
                                                             uint32_t gp, uint32_t total) {
  uint32_t a = blockIdx.x * 256u + threadIdx.x;
  if (a >= total) return;
  uint32_t blk = 32u * gp;  // bytes per 32-row block
  uint32_t r0 = a / blk, rem = a - r0 * blk;
  uint32_t k0 = rem >> 8, b = rem & 255u;
  uint32_t row = 32u * r0 + 16u * (b & 1u) + ((b >> 2) & 15u);
  uint32_t g = 8u * k0 + 4u * ((b >> 1) & 1u) + (b >> 6);
  out[a] = (row < rows && g < G) ? raw[row * G + g] : (uint8_t)127;
}

// Quantize B and write it straight into the GEMM's layouts (the pages
// prepare B offline with a quantize, then a shuffle of codes and scales).
// One wave per unit (16-row group g, 128-wide step s) of the padded scale
// layout, g < pad256(N)/16, s < pad8(K/32)/4, four waves per workgroup
// (fewer, larger workgroups measured 11% faster at 7168x7168 than one wave
// each).  Each of a wave's four loads covers the 16 rows x one 32-element
// group (four lanes per group, coalesced); lane t = 4r + q then holds
// bytes 4q..4q+3 of row r in tile t' = 4s + ch of the preshuffled layout,
// so the 64 lanes' dwords are one contiguous 256-byte tile.  Rows past N
// and groups past K/32 load as zeros, write no codes and get the scale fill
// byte 127; units past the last touch nothing.
template <bool SW>
__global__ __launch_bounds__(256) void prepare_b_kernel(const uint16_t *__restrict__ B, uint8_t *__restrict__ bq_sh,
                                                        uint8_t *__restrict__ bs_sh, int N, int K, int gp, int units) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool live = unit < units;
  const int steps = gp >> 2;
  const int g = unit / steps, s = unit - (unit / steps) * steps;
  const int G = K >> 5;
  const int rows_p = (N + 255) & ~255;
  const int b_bytes = N * K * 2;
  const int q_bytes = N * (K >> 1);
  const int s_bytes = rows_p * gp;
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)B, 0, b_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)bq_sh, 0, q_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)bs_sh, 0, s_bytes, kRsrcWord3);
  const int row = 16 * g + (lane >> 2);
  u32x4 w[4];
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    const int grp = 4 * s + ch;
    const bool ok = live && row < N && grp < G;
    w[ch] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, off_or_oob(ok, (row * K + grp * 32 + (lane & 3) * 8) * 2), 0,
                                                  0);
  }
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    const int grp = 4 * s + ch;
    uint32_t sc;
    const uint32_t d = quant_quarter_t<SW>(w[ch], &sc);
    const bool codes = live && 16 * g < N && grp < G;
    __builtin_amdgcn_raw_buffer_store_b32(d, q_rsrc, off_or_oob(codes, g * (K >> 1) * 16 + grp * 256 + lane * 4), 0,
                                          0);
    const uint32_t byte = (row < N && grp < G) ? sc : 127u;
    __builtin_amdgcn_raw_buffer_store_b8(
        (uint8_t)byte, s_rsrc, off_or_oob(live && (lane & 3) == 0, (int)shuffled_scale_offset(row, grp, gp)), 0, 0);
  }
}

static inline uint32_t blocks_for(uint64_t n) { return (uint32_t)((n + 255) / 256); }

hipError_t launch_quantize(const void *x, int64_t rows, int64_t K, void *q, void *scales, bool shuffled, bool sw,
                           hipStream_t stream) {
  uint32_t G = (uint32_t)(K / 32);
  if (!shuffled) {
    uint32_t groups = (uint32_t)rows * G;
    if (sw)
      quantize_raw_kernel<true><<<blocks_for(groups), 256, 0, stream>>>((const uint4 *)x, (uint4 *)q,
                                                                          (uint8_t *)scales, groups);
    else
      quantize_raw_kernel<false><<<blocks_for(groups), 256, 0, stream>>>((const uint4 *)x, (uint4 *)q,
                                                                           (uint8_t *)scales, groups);
  } else {
    uint32_t gp = (G + 7) / 8 * 8;
    uint32_t rp = (uint32_t)((rows + 255) / 256 * 256);
    uint32_t slots = rp * gp;
    if (sw)
      quantize_shuffled_kernel<true><<<blocks_for(slots), 256, 0, stream>>>(
          (const uint4 *)x, (uint4 *)q, (uint8_t *)scales, (uint32_t)rows, G, gp, slots);
    else
      quantize_shuffled_kernel<false><<<blocks_for(slots), 256, 0, stream>>>(
          (const uint4 *)x, (uint4 *)q, (uint8_t *)scales, (uint32_t)rows, G, gp, slots);
  }
  return hipGetLastError();
}

hipError_t launch_preshuffle_b(const void *bq, const void *bs_raw, int64_t N, int64_t K, void *bq_sh, void *bs_sh,
                               hipStream_t stream) {
  uint32_t T = (uint32_t)(K / 32);
  uint32_t chunks = (uint32_t)(N / 16) * T * 16u;
  preshuffle_b_data_kernel<<<blocks_for(chunks), 256, 0, stream>>>((const uint4 *)bq, (uint4 *)bq_sh, T, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t G = T;
  uint32_t gp = (G + 7) / 8 * 8;
  uint32_t total = (uint32_t)((N + 255) / 256 * 256) * gp;
  shuffle_scales_kernel<<<blocks_for(total), 256, 0, stream>>>((const uint8_t *)bs_raw, (uint8_t *)bs_sh,
                                                               (uint32_t)N, G, gp, total);
  return hipGetLastError();
}

hipError_t launch_prepare_b(const void *b, int64_t N, int64_t K, void *bq_sh, void *bs_sh, bool sw, hipStream_t stream) {
  const int G = (int)(K / 32);
  const int gp = (G + 7) / 8 * 8;
  const uint32_t units = (uint32_t)((N + 255) / 256 * 16) * (uint32_t)(gp / 4);
  const uint32_t blocks = (units + 3) / 4;
  if (sw)
    prepare_b_kernel<true><<<blocks, 256, 0, stream>>>((const uint16_t *)b, (uint8_t *)bq_sh, (uint8_t *)bs_sh, (int)N,
                                                       (int)K, gp, (int)units);
  else
    prepare_b_kernel<false><<<blocks, 256, 0, stream>>>((const uint16_t *)b, (uint8_t *)bq_sh, (uint8_t *)bs_sh, (int)N,
                                                        (int)K, gp, (int)units);
  return hipGetLastError();
}

}  // namespace mxfp4
