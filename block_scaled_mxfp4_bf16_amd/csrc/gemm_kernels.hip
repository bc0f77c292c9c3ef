// Fused MXFP4 GEMM: the operand-preparation and fill kernels, the joined
// variant table and its queries.  The kernel template itself, with its full
// description, is in gemm_fused.hpp; its instantiations are spread over
// gemm_table_*.hip.
#include <vector>

#include "gemm_fused.hpp"

namespace mxfp4 {

// Zero-fills the f32 tiles the atomic split-K epilogue adds into.
__global__ __launch_bounds__(256) void zero_f32_kernel(float *__restrict__ p, int n4) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n4) ((v4f *)p)[i] = v4f{0.f, 0.f, 0.f, 0.f};
}

// Zero `bytes` (a multiple of 16) at a 16-byte aligned address with a fill
// kernel rather than a memset node, which a graph capturing the call would
// record.
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream) {
  const size_t n4 = bytes / 16;
  if (n4 == 0) return hipSuccess;
  if (n4 > (size_t)INT32_MAX - 255) return hipErrorInvalidValue;
  zero_f32_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, stream>>>((float *)p, (int)n4);
  return hipGetLastError();
}

// A quantized once into operand blocks for the pre-quantized mode: block
// (m tile, step) holds 1 KiB of codes (operand lane L's 16 bytes at 16*L)
// and 64 scale bytes.  One wave per 16 rows x 32 elements, four consecutive
// lanes per group, as in the staging of the fused mode.
__global__ __launch_bounds__(64) void quant_operand_kernel(const uint16_t *__restrict__ A, uint8_t *__restrict__ Aop,
                                                           int M, int K, int units, int sw_quant) {
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;  // (m tile, step, chunk), chunk fastest; one wave per workgroup
  if (unit >= units) return;
  const int KS = (K + 127) >> 7;
  const int ch = unit & 3;
  const int ks = (unit >> 2) % KS;
  const int mtile = (unit >> 2) / KS;
  const int row = mtile * 16 + (lane >> 2);
  const int kel = ks * 128 + ch * 32 + (lane & 3) * 8;
  const int a_bytes = M * K * 2;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, a_bytes, kRsrcWord3);
  const bool ok = (row < M) && (ks * 128 + ch * 32 < K);
  const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, ok ? (row * K + kel) * 2 : a_bytes, 0, 0);
  uint32_t s;
  const uint32_t d = quant_quarter(w, sw_quant, &s);
  uint8_t *blk = Aop + (size_t)(mtile * KS + ks) * 1088;
  ((uint32_t *)blk)[ch * 64 + lane] = d;
  if ((lane & 3) == 0) blk[1024 + ch * 16 + (lane >> 2)] = (uint8_t)s;
}

// Pre-quantized A (codes [M, K/2] as mxfp4_quantize writes them, scales
// in the shuffled layout) -> operand blocks.  One single-wave workgroup per
// (16-row tile t, step ks): operand lane L takes the 16 code bytes of row
// 16t + L%16, K chunk 4ks + L/16, and that group's scale byte.  Rows past M
// and chunks past K become zero codes with scale byte 0, as quantizing
// zeros would give.
__global__ __launch_bounds__(64) void repack_operand_kernel(const uint8_t *__restrict__ Aq,
                                                            const uint8_t *__restrict__ As,
                                                            uint8_t *__restrict__ Aop, int M, int K) {
  const int lane = threadIdx.x;
  const int KS = (K + 127) >> 7;
  const int t = blockIdx.x / KS, ks = blockIdx.x - (blockIdx.x / KS) * KS;
  const int G = K >> 5, gp = (G + 7) & ~7;
  const int row = 16 * t + (lane & 15), grp = 4 * ks + (lane >> 4);
  const bool ok = row < M && grp < G;
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Aq, 0, M * (K >> 1), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)As, 0, ((M + 255) & ~255) * gp, kRsrcWord3);
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off_or_oob(ok, row * (K >> 1) + grp * 16), 0, 0);
  const uint32_t sc =
      __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, off_or_oob(ok, (int)shuffled_scale_offset(row, grp, gp)), 0, 0);
  uint8_t *blk = Aop + (size_t)(t * KS + ks) * 1088;
  *(u32x4 *)(blk + lane * 16) = v;
  blk[1024 + lane] = (uint8_t)sc;
}

size_t operand_a_bytes(int M, int K) { return (size_t)((M + 15) / 16) * (size_t)((K + 127) / 128) * 1088; }

hipError_t launch_operand_prep(const GemmArgs &a, uint8_t *aop, bool sw, hipStream_t stream) {
  if (a.Aq) {
    const int blocks = ((a.M + 15) / 16) * ((a.K + 127) / 128);
    repack_operand_kernel<<<blocks, 64, 0, stream>>>((const uint8_t *)a.Aq, (const uint8_t *)a.As, aop, a.M, a.K);
  } else {
    const int units = ((a.M + 15) / 16) * ((a.K + 127) / 128) * 4;
    quant_operand_kernel<<<units, 64, 0, stream>>>((const uint16_t *)a.A, aop, a.M, a.K, units, sw ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t launch_zero_f32(float *p, int n4, hipStream_t stream) {
  zero_f32_kernel<<<(n4 + 255) / 256, 256, 0, stream>>>(p, n4);
  return hipGetLastError();
}

// ---------------------------------------------------------------- table

const Variant *variants_part0(int *count);
const Variant *variants_part1(int *count);
const Variant *variants_part2(int *count);
const Variant *variants_part3(int *count);
const Variant *variants_part4(int *count);
const Variant *variants_part5(int *count);
const Variant *variants_part6(int *count);
const Variant *variants_part7(int *count);

// The parts joined in order (the order breaks ties in the schedule search).
static const std::vector<Variant> &variants() {
  static const std::vector<Variant> table = [] {
    std::vector<Variant> t;
    const Variant *(*parts[])(int *) = {variants_part0, variants_part1, variants_part2, variants_part3,
                                        variants_part4, variants_part5, variants_part6, variants_part7};
    for (auto part : parts) {
      int n = 0;
      const Variant *v = part(&n);
      t.insert(t.end(), v, v + n);
    }
    return t;
  }();
  return table;
}

int num_gemm_variants() { return (int)variants().size(); }

void gemm_variant_shape(int v, Schedule *s) {
  s->mt = variants()[v].mt;
  s->nt = variants()[v].nt;
  s->wn = variants()[v].wn;
  s->wk = variants()[v].wk;
  s->kpw = variants()[v].kpw;
  s->pq = variants()[v].pq;
  s->rb = variants()[v].rb;
  s->wide = variants()[v].wide;
  s->epi = variants()[v].epi;
  s->variant = v;
}

int find_gemm_variant(int mt, int nt, int wn, int wk, int kpw, int pq, int rb, int wide, int epi) {
  for (int v = 0; v < num_gemm_variants(); ++v)
    if (variants()[v].mt == mt && variants()[v].nt == nt && variants()[v].wn == wn && variants()[v].wk == wk &&
        variants()[v].kpw == kpw && variants()[v].pq == pq && variants()[v].rb == rb && variants()[v].wide == wide &&
        variants()[v].epi == epi)
      return v;
  return -1;
}

size_t gemm_workspace_bytes(const Schedule &s, int M, int N, int K) {
  if (s.split <= 1 && !s.pq && s.epi != 2) return 0;
  size_t bytes = kTicketBytes;
  if (s.pq) bytes += (pq_operand_bytes(M, K) + 255) & ~(size_t)255;
  const size_t tiles = (size_t)(N / (16 * s.nt * s.wn)) * (size_t)((M + 16 * s.mt - 1) / (16 * s.mt));
  const size_t e = (size_t)s.mt * s.nt * s.wn * 256;
  if (s.epi == 2)
    bytes += (size_t)s.split * 2 * e * sizeof(float);  // two slots per workgroup of the grid
  else if (s.epi == 1 && s.split > 1)
    bytes += tiles * e * sizeof(float);  // one f32 tile per output tile
  else if (s.split > 1)
    bytes += tiles * (size_t)s.split * e * sizeof(float);
  return bytes;
}

hipError_t launch_gemm(const Schedule &s, const GemmArgs &a, bool sw_quant, hipStream_t stream) {
  return variants()[s.variant].fn(a, s.split, sw_quant, stream);
}

}  // namespace mxfp4
