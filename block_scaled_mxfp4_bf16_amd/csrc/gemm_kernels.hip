// Fused MXFP4 GEMM for gfx950: C[M,N] (bf16) = Q(A[M,K] bf16) * B[N,K]^T.
//
// One matrix instruction, v_mfma_scale_f32_16x16x128_f8f6f4 with both
// operands e2m1 (format code 4), multiplies a 16x128 block of A by a 128x16
// block of B^T, each 32-wide K chunk carrying its own e8m0 scale, into a
// 16x16 f32 accumulator.  Lane l supplies row/column l%16 and K chunk l/16:
// 32 e2m1 codes (16 bytes) and that chunk's scale byte.  A 32-wide K chunk is
// exactly one scale group, so the quantization of A is lane-local: each lane
// loads its 32 bf16 values (64 bytes), takes their amax, derives the scale
// byte and converts with v_cvt_scalef32_pk_fp4_f32 (submission 608632,
// kernel v7 and _hw_mxfp4_quant_op, which do the same per BLOCK_K tile).
//
// B comes preshuffled (16-row x 16-byte tiles, 256 contiguous bytes each),
// so the B operand of one instruction is 1 KiB contiguous and lane l loads
// its 16 bytes at offset 16*l.  The shuffled scale layout puts, in the dword
// at 4*l of a 256-byte block, the scales of rows {l%16, l%16+16} x groups
// {l/16, l/16+4}: one dword per lane serves two 16-column subtiles and two
// K steps (submission 711914, the vectorized scale loads of its kernels).
//
// Work split: a workgroup owns an output tile of 16*MT rows x 16*NT
// columns; its WAVES waves take disjoint runs of 128-wide K steps (at most
// KPW each) and add their accumulators through LDS in wave order.  When one
// tile's K range is split over `split` workgroups (submission 610679, split-K
// kernel), each writes its f32 partial tile to the workspace, then takes a
// ticket; the workgroup that takes the last ticket adds the partials in
// split order, stores bf16 C and resets the ticket.  The sum order is fixed,
// so results are deterministic, and there is no second launch.
#include "mxfp4_device.hpp"
#include "mxfp4_internal.hpp"

namespace mxfp4 {

template <int MT, int NT, int KPW, int WAVES, bool SW>
__global__ __launch_bounds__(64 * WAVES) void gemm_fused_kernel(const uint16_t *__restrict__ A,
                                                                const uint8_t *__restrict__ Bw,
                                                                const uint8_t *__restrict__ Bs,
                                                                uint16_t *__restrict__ C,
                                                                float *__restrict__ partials,
                                                                uint32_t *__restrict__ tickets, int M, int N,
                                                                int K, int split, int n_tiles) {
  constexpr int E = MT * NT * 256;  // outputs of one tile
  constexpr int NTH = 64 * WAVES;
  __shared__ float red[WAVES][MT * NT * 4][64];
  __shared__ uint32_t s_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int bid = blockIdx.x;
  const int n_tile = bid % n_tiles;
  const int rest = bid / n_tiles;
  const int sk = rest % split;
  const int m_tile = rest / split;
  const int m0 = m_tile * 16 * MT;
  const int g0 = n_tile * NT;  // first 16-row group of B (16-column subtile of C)

  const int KS = (K + 127) >> 7;  // 128-wide K steps
  const int W = split * WAVES;
  const int wk = sk * WAVES + wave;
  const int ks_begin = (int)(((int64_t)wk * KS) / W);
  const int ks_end = (int)(((int64_t)(wk + 1) * KS) / W);

  const int r16 = lane & 15;
  const int kc = lane >> 4;
  const size_t b_group_stride = (size_t)K * 8;  // (K/2) * 16 bytes per 16-row group
  const int gp = ((K >> 5) + 7) & ~7;
  const size_t s_block_stride = (size_t)gp * 32;  // bytes per 32-row block of scales

  const uint16_t *arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = m0 + 16 * mt + r16;
    r = r < M ? r : M - 1;
    arow[mt] = A + (size_t)r * K;
  }

  // Phase 1: issue every load of this wave's K run.  Steps past the run are
  // clamped to a valid step (their loads hit cache; their products are
  // skipped); lanes past K in a half step (K % 128 == 64) load nothing.
  uint32_t aw[KPW][MT][16];
  uint4 bv[KPW][NT];
  uint32_t sw[KPW][NT];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    int ks = ks_begin + i;
    ks = ks < KS ? ks : KS - 1;
    const int kel = ks * 128 + kc * 32;
    const bool valid = kel < K;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4 *src = (const uint4 *)(arow[mt] + kel);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 v = valid ? src[j] : make_uint4(0, 0, 0, 0);
        aw[i][mt][4 * j + 0] = v.x;
        aw[i][mt][4 * j + 1] = v.y;
        aw[i][mt][4 * j + 2] = v.z;
        aw[i][mt][4 * j + 3] = v.w;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int g = g0 + nt;
      const uint4 *bp = (const uint4 *)(Bw + (size_t)g * b_group_stride + (size_t)ks * 1024) + lane;
      bv[i][nt] = valid ? *bp : make_uint4(0, 0, 0, 0);
      const uint32_t *sp =
          (const uint32_t *)(Bs + (size_t)(g >> 1) * s_block_stride + (size_t)(ks >> 1) * 256) + lane;
      uint32_t word = *sp;
      uint32_t sel = (uint32_t)((g & 1) | ((ks & 1) << 1));
      sw[i][nt] = valid ? ((word >> (8 * sel)) & 0xFFu) : 127u;
    }
  }

  // Phase 2: quantize A in registers and accumulate.
  v4f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    if (ks_begin + i >= ks_end) break;
    const int kel = (ks_begin + i) * 128 + kc * 32;
    const bool valid = kel < K;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t q[4];
      uint32_t sa = quant_group32<SW>(aw[i][mt], q);
      sa = valid ? sa : 127u;
      v8i a_op = {(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint4 b = bv[i][nt];
        v8i b_op = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_op, b_op, acc[mt][nt], 4, 4, 0, (int)sa,
                                                                       0, (int)sw[i][nt]);
      }
    }
  }

  // Reduce the waves' accumulators through LDS.  Accumulator element r of
  // lane l in subtile (mt, nt) is C row 16*mt + 4*(l/16) + r, column
  // 16*nt + l%16.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(mt * NT + nt) * 4 + r][lane] = acc[mt][nt][r];
  __syncthreads();

  const int tile = m_tile * n_tiles + n_tile;
  if (split == 1) {
    for (int e = threadIdx.x; e < E; e += NTH) {
      const int i = e >> 6, ln = e & 63;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) s += red[w][i][ln];
      const int mt = i / (4 * NT), nt = (i >> 2) % NT, r = i & 3;
      const int row = m0 + 16 * mt + 4 * (ln >> 4) + r;
      const int col = 16 * (g0 + nt) + (ln & 15);
      if (row < M) C[(size_t)row * N + col] = (uint16_t)f32_to_bf16_rne(s);
    }
    return;
  }

  float *mine = partials + ((size_t)tile * split + sk) * E;
  for (int e = threadIdx.x; e < E; e += NTH) {
    const int i = e >> 6, ln = e & 63;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[w][i][ln];
    mine[e] = s;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&tickets[tile], 1u) == (uint32_t)(split - 1)) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float *all = partials + (size_t)tile * split * E;
  for (int e = threadIdx.x; e < E; e += NTH) {
    float s = 0.f;
    for (int j = 0; j < split; ++j) s += __builtin_nontemporal_load(all + (size_t)j * E + e);
    const int i = e >> 6, ln = e & 63;
    const int mt = i / (4 * NT), nt = (i >> 2) % NT, r = i & 3;
    const int row = m0 + 16 * mt + 4 * (ln >> 4) + r;
    const int col = 16 * (g0 + nt) + (ln & 15);
    if (row < M) C[(size_t)row * N + col] = (uint16_t)f32_to_bf16_rne(s);
  }
  if (threadIdx.x == 0) tickets[tile] = 0u;
}

// ---------------------------------------------------------------- table

typedef hipError_t (*launch_fn)(const GemmArgs &, int split, hipStream_t);

template <int MT, int NT, int KPW, int WAVES, bool SW>
static hipError_t launch_variant(const GemmArgs &a, int split, hipStream_t stream) {
  const int n_tiles = a.N / (16 * NT);
  const int m_tiles = (a.M + 16 * MT - 1) / (16 * MT);
  const int tiles = n_tiles * m_tiles;
  uint32_t *tickets = (uint32_t *)a.workspace;
  float *partials = (float *)((char *)a.workspace + kTicketBytes);
  dim3 grid((unsigned)(tiles * split));
  gemm_fused_kernel<MT, NT, KPW, WAVES, SW><<<grid, 64 * WAVES, 0, stream>>>(
      (const uint16_t *)a.A, (const uint8_t *)a.Bw, (const uint8_t *)a.Bs, (uint16_t *)a.C, partials, tickets, a.M,
      a.N, a.K, split, n_tiles);
  return hipGetLastError();
}

struct Variant {
  int mt, nt, kpw, waves;
  launch_fn hw, sw;
};

#define MXFP4_VARIANT(MT, NT, KPW, WAVES) \
  {MT, NT, KPW, WAVES, launch_variant<MT, NT, KPW, WAVES, false>, launch_variant<MT, NT, KPW, WAVES, true>}

static const Variant kVariants[] = {
    MXFP4_VARIANT(1, 2, 1, 4), MXFP4_VARIANT(1, 2, 2, 4), MXFP4_VARIANT(1, 2, 4, 4), MXFP4_VARIANT(1, 2, 8, 4),
    MXFP4_VARIANT(2, 2, 1, 4), MXFP4_VARIANT(2, 2, 2, 4), MXFP4_VARIANT(2, 2, 4, 4), MXFP4_VARIANT(2, 2, 8, 4),
    MXFP4_VARIANT(4, 2, 1, 4), MXFP4_VARIANT(4, 2, 2, 4), MXFP4_VARIANT(4, 2, 4, 4), MXFP4_VARIANT(4, 2, 8, 4),
};

int num_gemm_variants() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }

void gemm_variant_shape(int v, int *mt, int *nt, int *kpw, int *waves) {
  *mt = kVariants[v].mt;
  *nt = kVariants[v].nt;
  *kpw = kVariants[v].kpw;
  *waves = kVariants[v].waves;
}

int find_gemm_variant(int mt, int nt, int kpw, int waves) {
  for (int v = 0; v < num_gemm_variants(); ++v)
    if (kVariants[v].mt == mt && kVariants[v].nt == nt && kVariants[v].kpw == kpw && kVariants[v].waves == waves)
      return v;
  return -1;
}

size_t gemm_workspace_bytes(const Schedule &s, int M, int N, int K) {
  (void)K;
  if (s.split <= 1) return 0;
  const size_t tiles = (size_t)(N / (16 * s.nt)) * (size_t)((M + 16 * s.mt - 1) / (16 * s.mt));
  const size_t e = (size_t)s.mt * s.nt * 256;
  return kTicketBytes + tiles * (size_t)s.split * e * sizeof(float);
}

hipError_t launch_gemm(const Schedule &s, const GemmArgs &a, bool sw_quant, hipStream_t stream) {
  const Variant &v = kVariants[s.variant];
  return (sw_quant ? v.sw : v.hw)(a, s.split, stream);
}

}  // namespace mxfp4
