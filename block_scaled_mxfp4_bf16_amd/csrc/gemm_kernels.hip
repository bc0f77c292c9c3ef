// Fused MXFP4 GEMM: the fill kernel, the joined variant table and its
// queries.  The kernel template itself, with its full
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
