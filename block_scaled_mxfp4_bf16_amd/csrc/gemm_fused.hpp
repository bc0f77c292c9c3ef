// Fused MXFP4 GEMM for gfx950 (kernel template and its launcher): C[M,N] (bf16) = Q(A[M,K] bf16) * B[N,K]^T.
//
// One matrix instruction, v_mfma_scale_f32_16x16x128_f8f6f4 with both
// operands e2m1 (format code 4), multiplies a 16x128 block of A by a 128x16
// block of B^T, each 32-wide K chunk carrying its own e8m0 scale, into a
// 16x16 f32 accumulator.  Lane l supplies row/column l%16 and K chunk l/16:
// 32 e2m1 codes (16 bytes) and that chunk's scale byte.
//
// B comes preshuffled (16-row x 16-byte tiles, 256 contiguous bytes each),
// so the B operand of one instruction is 1 KiB contiguous and lane l loads
// its 16 bytes at offset 16*l.  The shuffled scale layout puts, in the dword
// at 4*l of a 256-byte block, the scales of rows {l%16, l%16+16} x groups
// {l/16, l/16+4}: one dword per lane serves two 16-column subtiles and two
// K steps (submission 711914, the vectorized scale loads of its kernels).
//
// A is quantized inside the kernel (submission 608632, kernel v7, does the
// same per BLOCK_K tile with the hardware convert) and staged through LDS,
// once per workgroup, in the operand layout:
//   - one load instruction covers 8 rows x two 32-element groups: eight
//     consecutive lanes read one row's 128 contiguous bytes, a whole cache
//     line, so no line is requested twice (the vector cache does not merge
//     two requests for one line in flight).  Schedules of one row tile and
//     one column wave load 16 rows x one group instead (four lanes per
//     64-byte run), whose LDS writes are conflict-free;
//   - the four lanes of a group combine their amax with two DPP steps, then
//     each converts its 8 elements with v_cvt_scalef32_pk_fp4_bf16 into one
//     dword of codes;
//   - the lane of row r, group c, quarter q writes its dword at dword
//     64c + 4r + q of a 1 KiB block and the scale at byte 16c + r; a block
//     is exactly one matrix operand (operand lane L reads 16 bytes at 16*L).
//
// Work split: a workgroup owns an output tile of 16*MT rows x 16*NT*WN
// columns and a run of K steps.  Its waves form a WN x WK grid: WN waves
// share the staged A and take NT subtiles each; WK waves split the run
// (KPW steps each) and add their accumulators through LDS in wave order.
// When one tile's K range is split over several workgroups (submission
// 610679, split-K kernel), the partial tiles meet in the workspace; how is
// the epilogue mode EPI:
//   0  each workgroup writes its f32 partial tile to a slot of its own and
//      takes a ticket; the one that draws the last ticket adds the slots in
//      split order, stores bf16 C and resets the ticket.  The sum order is
//      fixed, so results are deterministic, and there is no second launch
//      (the pages reduce split-K partials with a second kernel).
//   1  each workgroup adds its partial tile into one f32 tile with float
//      atomics (submission 711914, the fused large-K kernel, adds into a
//      zeroed f32 C and casts it afterwards); the last ticket casts the sum
//      to bf16 and stores C.  The order of the additions, and so the
//      rounding, varies from run to run.  The f32 tiles are zero-filled by
//      a small launch before the GEMM.
//   2  stream-K: a grid of G workgroups splits the tiles x K steps
//      iteration space into G equal contiguous runs, so every workgroup has
//      the same work whatever the tile count.  A run may cross tile
//      boundaries; a tile that one run covers whole is stored directly, the
//      others go through ticketed slots as in mode 0, added in workgroup
//      order, so results are deterministic.
#pragma once

#include <type_traits>

#include "mxfp4_device.hpp"
#include "mxfp4_internal.hpp"

namespace mxfp4 {

// `split`: workgroups per tile (EPI 0, 1) or of the whole grid (EPI 2).
// STAMPS (measurement probes only; every schedule of the library has it
// off): each wave records the 100 MHz real-time counter at the kernel's
// phase boundaries -- entry, loads issued, A staged, products reduced, C
// stores issued, C stores completed -- in scalar registers, and lane 0
// writes the six stamps at the end to `partials`, read as uint64
// [workgroups * waves][8].  Split-1 schedules only.
template <int MT, int NT, int WN, int WK, int KPW, bool PREQ, int RB, int EPI, bool STAMPS = false>
__global__ __launch_bounds__(64 * WN * WK) void gemm_kernel(const uint16_t *__restrict__ A,
                                                           const uint8_t *__restrict__ Aq,
                                                           const uint8_t *__restrict__ As,
                                                           const uint8_t *__restrict__ Bw,
                                                           const uint8_t *__restrict__ Bs, uint16_t *__restrict__ C,
                                                           float *__restrict__ partials,
                                                           uint32_t *__restrict__ tickets, int M, int N, int K,
                                                           int split, int n_tiles, int sw_quant) {
  constexpr int WAVES = WN * WK;
  constexpr int NTH = 64 * WAVES;
  constexpr int KW = WK * KPW;                      // K steps one workgroup covers at most
  // staged A blocks: 16 rows x 32 elements each, or (RB == 8, for M <= 8)
  // 8 rows x 64 elements, so that no load is spent on rows that do not exist
  constexpr int UPS = RB == 8 ? 2 : 4;              // blocks per (step, m tile)
  // Whole-line A loads (below).  Their LDS writes conflict two ways, which
  // shows where a single wave stages one tile and uses it at once (one row
  // tile, one column wave); there the half-line order is kept.
  constexpr bool LINES = RB == 8 || MT > 1 || WN > 1;
  constexpr int UNITS = KW * MT * UPS;
  constexpr int UPW = (UNITS + WAVES - 1) / WAVES;  // per wave
  constexpr int TN = NT * WN;                       // 16-column subtiles per workgroup
  constexpr int E = MT * TN * 256;                  // outputs per tile
  constexpr int NP = (NT + 1) / 2;                  // scale dwords per step and wave
  constexpr int A_BYTES = PREQ ? 0 : KW * MT * 1024;  // codes
  constexpr int S_BYTES = PREQ ? 0 : KW * MT * 64;    // scales
  constexpr int RED_BYTES = WK > 1 ? WAVES * MT * NT * 1024 : 0;
  constexpr int LDS_BYTES0 = (A_BYTES + S_BYTES) > RED_BYTES ? (A_BYTES + S_BYTES) : RED_BYTES;
  constexpr int LDS_BYTES = LDS_BYTES0 > 16 ? LDS_BYTES0 : 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ uint32_t s_last;
  uint32_t *a_lds = (uint32_t *)lds;
  uint8_t *s_lds = lds + A_BYTES;
  float *red = (float *)lds;

  constexpr int EPT = (E + NTH - 1) / NTH;         // tile elements per thread in the split epilogue
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % WN;
  const int wk = wave / WN;
  const int KS = (K + 127) >> 7;
  const int gp = ((K >> 5) + 7) & ~7;

  // Buffer descriptors carry the operands' byte sizes: a load whose offset
  // is out of range returns zeros.  That is how rows past M, K chunks past K
  // and steps past the run are handled, without branches: zero codes with a
  // zero scale contribute nothing.
  const int a_bytes = M * K * 2;
  const int b_bytes = (N >> 4) * K * 8;
  const int s_bytes = ((N + 255) >> 8) * 8 * gp * 32;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, a_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Bw, 0, b_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Bs, 0, s_bytes, kRsrcWord3);

  // One segment: steps [S0, S1) of tile (m_tile, n_tile), whose K range is
  // shared by `nparts` workgroups; slot(j) is the partial tile of the j-th
  // of them and this workgroup is number `mine_j`.
  uint64_t stamp[6];
  auto take = [&](int i) {
    if constexpr (STAMPS) stamp[i] = __builtin_amdgcn_s_memrealtime();
  };
  auto write_stamps = [&]() {
    if constexpr (STAMPS) {
      static_assert(EPI == 0, "stamps serve split-1 schedules");
      __builtin_amdgcn_s_waitcnt(0);
      take(5);
      if (lane == 0) {
        uint64_t *out = (uint64_t *)partials + ((size_t)blockIdx.x * WAVES + wave) * 8;
#pragma unroll
        for (int i = 0; i < 6; ++i) out[i] = stamp[i];
      }
    }
  };
  take(0);
  auto segment = [&](const int m_tile, const int n_tile, const int S0, const int S1, const int nparts,
                     const int mine_j, auto slot) {
  const int m0 = m_tile * 16 * MT;
  const int gw = n_tile * TN + wn * NT;  // this wave's first 16-row group of B

  // Phase 1: issue the loads.  A first: it is small and mostly L2-resident,
  // and since the load counter retires in issue order, quantizing it can
  // then start while B (from HBM, the long pole) is still in flight.
  const int kc = lane >> 4;
  u32x4 aw[PREQ ? 1 : UPW];
  u32x4 ap[PREQ ? KPW : 1][PREQ ? MT : 1];
  uint32_t asb[PREQ ? KPW : 1][PREQ ? MT : 1];
  if constexpr (!PREQ) {
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      // (step, m tile, row half, chunk pair) with the chunk pair fastest
      // (LINES): lane t loads 16 bytes of row 8*half + t/8, chunk
      // 2*pair + (t/4)%2, so eight lanes read one row's 128-byte line whole;
      // else (step, m tile, chunk): lane t loads row t/4, chunk unit%4.
      // With one wave per column group each wave stages exactly the blocks
      // of its own steps.
      const int unit = WN == 1 ? wk * (KPW * MT * UPS) + u : wave + u * WAVES;
      const int st = unit / (MT * UPS);
      const int mt = (unit / UPS) % MT;
      const int ch = LINES ? 2 * (unit & 1) + ((lane >> 2) & 1) : (unit & 3);
      const int ks = S0 + st;
      const int row = m0 + 16 * mt + (LINES ? (RB == 8 ? 0 : 8 * ((unit >> 1) & 1)) + (lane >> 3) : (lane >> 2));
      const int kel = ks * 128 + ch * 32 + (lane & 3) * 8;
      const bool ok = (unit < UNITS) && (ks < S1) && (row < M) && (ks * 128 + ch * 32 < K);
      aw[u] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, off_or_oob(ok, (row * K + kel) * 2), 0, 0);
    }
  } else {
    // pre-quantized A as the caller holds it: codes [M, K/2] row-major and
    // scales in the shuffled layout (B's).  Operand lane l takes the 16 code
    // bytes of row 16*mtile + l%16, K chunk l/16 of the step (the two steps
    // of a 128-byte row segment come from two loads), and the scale dword at
    // lane l of the step pair's 256-byte block, as for B.
    const int q_bytes = M * (K >> 1);
    const int as_bytes = ((M + 255) >> 8) * 8 * gp * 32;
    const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Aq, 0, q_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)As, 0, as_bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int ks = S0 + wk * KPW + i;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int mtile = m_tile * MT + mt;
        const int row = mtile * 16 + (lane & 15);
        const bool ok = (ks < S1) && (row < M) && (ks * 128 + kc * 32 < K);
        ap[i][mt] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off_or_oob(ok, row * (K >> 1) + ks * 64 + kc * 16), 0, 0);
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(
            as_rsrc, off_or_oob(ks < S1, (mtile >> 1) * gp * 32 + (ks >> 1) * 256 + lane * 4), 0, 0);
        asb[i][mt] = (w >> (8 * ((mtile & 1) | ((ks & 1) << 1)))) & 0xFFu;
      }
    }
  }
  u32x4 bv[KPW][NT];
  uint32_t sword[KPW][NP];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int ks = S0 + wk * KPW + i;
    const bool step_ok = ks < S1;
    const bool ok = step_ok && (ks * 128 + kc * 32 < K);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int off = off_or_oob(ok, (gw + nt) * K * 8 + ks * 1024 + lane * 16);
      bv[i][nt] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, off, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int g = gw + 2 * p;
      const int off = off_or_oob(step_ok, (g >> 1) * gp * 32 + (ks >> 1) * 256 + lane * 4);
      sword[i][p] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, off, 0, 0);
    }
  }

  take(1);

  // Phase 2: quantize the staged A blocks into LDS (the encoder is chosen
  // once for all blocks, so the hardware path is straight-line code).
  if constexpr (!PREQ) {
    auto stage_all = [&](auto sw_tag) {
      constexpr bool SW = decltype(sw_tag)::value;
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int unit = WN == 1 ? wk * (KPW * MT * UPS) + u : wave + u * WAVES;
        if (UPW * WAVES == UNITS || unit < UNITS) {
          uint32_t s;
          const uint32_t d = quant_quarter_t<SW>(aw[u], &s);
          // the lane's row, group and quarter of the block's 16 x 128 operand
          // (as loaded above)
          const int blk = RB == 8 ? unit >> 1 : unit >> 2;
          const int ch = LINES ? 2 * (unit & 1) + ((lane >> 2) & 1) : (unit & 3);
          const int r = LINES ? (RB == 8 ? 0 : 8 * ((unit >> 1) & 1)) + (lane >> 3) : (lane >> 2);
          a_lds[blk * 256 + ch * 64 + r * 4 + (lane & 3)] = d;
          if ((lane & 3) == 0) s_lds[blk * 64 + ch * 16 + r] = (uint8_t)s;
        }
      }
    };
    if (sw_quant)
      stage_all(std::true_type{});
    else
      stage_all(std::false_type{});
    if constexpr (WN == 1) {
      // the blocks this wave reads are the ones it wrote: LDS keeps one
      // wave's accesses in order, so only the compiler must not reorder
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      __syncthreads();
    }
  }

  take(2);

  // Phase 3: accumulate.
  v4f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int st = wk * KPW + i;
    const int ks = S0 + st;
    uint32_t sb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // subtile nt's 32-row scale block is (gw + nt) / 2: dword nt / 2 of
      // those loaded, or (nt + 1) / 2 when gw is odd (only with NT odd: for
      // NT even every wave's gw is even); a select of two registers, not an
      // indexed one
      const int g = gw + nt;
      const uint32_t sel = (uint32_t)((g & 1) | ((ks & 1) << 1));
      const uint32_t dw = (NT % 2 == 0) ? sword[i][nt >> 1] : ((gw & 1) ? sword[i][(nt + 1) >> 1] : sword[i][nt >> 1]);
      sb[nt] = (dw >> (8 * sel)) & 0xFFu;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int blk = st * MT + mt;
      u32x4 a;
      uint32_t sa;
      if constexpr (PREQ) {
        a = ap[i][mt];
        sa = asb[i][mt];
      } else {
        a = *(const u32x4 *)(a_lds + blk * 256 + lane * 4);
        sa = s_lds[blk * 64 + lane];
        if constexpr (RB == 8) {
          // rows 8..15 of the block were not staged: feed zeros
          if (lane & 8) {
            a = u32x4{0u, 0u, 0u, 0u};
            sa = 0u;
          }
        }
      }
      const v8i a_op = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const u32x4 b = bv[i][nt];
        const v8i b_op = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
        acc[mt][nt] =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_op, b_op, acc[mt][nt], 4, 4, 0, (int)sa, 0, (int)sb[nt]);
      }
    }
  }

  // Epilogue.  Accumulator element r of lane l in subtile (mt, nt) is C row
  // 16*mt + 4*(l/16) + r, column 16*nt + l%16.  Tile element index
  // e = (((mt*WN + wn)*NT + nt)*4 + r)*64 + l.
  const int tile = m_tile * n_tiles + n_tile;
  auto store_c = [&](int e, float v) {
    const int ln = e & 63, i = e >> 6;
    const int r = i & 3, t = i >> 2;  // t = mt*TN + (wn*NT + nt)
    const int mt = t / TN, sub = t % TN;
    const int row = m0 + 16 * mt + 4 * (ln >> 4) + r;
    const int col = 16 * (n_tile * TN + sub) + (ln & 15);
    if (row < M) C[(size_t)row * N + col] = (uint16_t)bf16x2_rne(v, 0.f);
  };
  auto elem = [&](int mt, int nt, int r) { return (((mt * WN + wn) * NT + nt) * 4 + r) * 64 + lane; };

  if constexpr (WK == 1) {
    if (nparts == 1) {
      if constexpr (STAMPS) {
        // the stamp follows the last product: an empty statement that reads
        // every accumulator keeps the compiler from moving it earlier
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) asm volatile("" ::"v"(acc[mt][nt]));
      }
      take(3);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) store_c(elem(mt, nt, r), acc[mt][nt][r]);
      take(4);
      write_stamps();
      return;
    }
  } else {
    // add the WK waves of each column group in wave order
    __syncthreads();  // LDS is reused
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wk * E + elem(mt, nt, r)] = acc[mt][nt][r];
    __syncthreads();
    take(3);
    if (nparts == 1) {
      // eight consecutive elements are eight consecutive columns of one row:
      // add them over the WK waves and store them as one 16-byte write
      for (int j = threadIdx.x; j < E / 8; j += NTH) {
        const int e0 = 8 * j;
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = 0.f;
#pragma unroll
        for (int w = 0; w < WK; ++w) {
          const v4f lo = *(const v4f *)(red + w * E + e0);
          const v4f hi = *(const v4f *)(red + w * E + e0 + 4);
          v[0] += lo[0]; v[1] += lo[1]; v[2] += lo[2]; v[3] += lo[3];
          v[4] += hi[0]; v[5] += hi[1]; v[6] += hi[2]; v[7] += hi[3];
        }
        const int ln = e0 & 63, i = e0 >> 6;
        const int r = i & 3, t = i >> 2;
        const int mt = t / TN, sub = t % TN;
        const int row = m0 + 16 * mt + 4 * (ln >> 4) + r;
        const int col = 16 * (n_tile * TN + sub) + (ln & 15);
        if (row < M) {
          u32x4 pk;
          pk.x = bf16x2_rne(v[0], v[1]);
          pk.y = bf16x2_rne(v[2], v[3]);
          pk.z = bf16x2_rne(v[4], v[5]);
          pk.w = bf16x2_rne(v[6], v[7]);
          *(u32x4 *)(C + (size_t)row * N + col) = pk;
        }
      }
      take(4);
      write_stamps();
      return;
    }
  }

  // Split K across workgroups.  Each writes its partial tile with
  // device-coherent stores (EPI 1: float atomics), waits until they have
  // completed, and takes a ticket; the workgroup that draws the last ticket
  // reads the partials with device-coherent loads, adds them in slot order
  // and stores C.  Only these accesses touch the workspace, so no
  // cache-wide write-back is needed.
  float *const mine = EPI == 1 ? partials + (size_t)tile * E : slot(mine_j);
  auto put = [&](int e, float v) {
    if constexpr (EPI == 1)
      __hip_atomic_fetch_add(mine + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_store(mine + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if constexpr (WK == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) put(elem(mt, nt, r), acc[mt][nt][r]);
  } else {
    for (int e = threadIdx.x; e < E; e += NTH) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < WK; ++w) v += red[w * E + e];
      put(e, v);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's workspace writes have completed
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&tickets[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)(nparts - 1)
                 ? 1u
                 : 0u;
  __syncthreads();
  if (!s_last) return;
  float sum[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) sum[i] = 0.f;
  for (int j = 0; j < (EPI == 1 ? 1 : nparts); ++j) {
    const float *part = EPI == 1 ? mine : slot(j);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (EPT * NTH == E || e < E) sum[i] += __hip_atomic_load(part + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = threadIdx.x + i * NTH;
    if (EPT * NTH == E || e < E) store_c(e, sum[i]);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&tickets[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };  // segment

  if constexpr (EPI == 2) {
    // Workgroup g owns iterations [start(g), start(g+1)) of the tiles x K
    // steps space, tile-major; each run is at most one workgroup's K
    // capacity long (the host checks), so a tile it covers in part is its
    // first or its last, and it keeps those partials in its slots 2g and
    // 2g + 1.
    const int m_tiles = (M + 16 * MT - 1) / (16 * MT);
    const long long T = (long long)n_tiles * m_tiles * KS;
    const int G = split;
    auto start = [&](int g) { return (long long)g * T / G; };
    // the workgroup whose run holds iteration x: the largest g with
    // start(g) <= x; x*G/T is at most one below it
    auto owner = [&](long long x) {
      int g = (int)(x * G / T);
      if (g + 1 < G && start(g + 1) <= x) ++g;
      return g;
    };
    const int g = blockIdx.x;
    const long long end = start(g + 1);
    for (long long it = start(g); it < end;) {
      const int t = (int)(it / KS);
      const int s0 = (int)(it - (long long)t * KS);
      const int s1 = (int)((long long)KS < s0 + (end - it) ? (long long)KS : s0 + (end - it));
      const int glo = owner((long long)t * KS), ghi = owner((long long)t * KS + KS - 1);
      auto slot = [&](int j) {
        const int gg = glo + j;
        const int which = (int)(start(gg) / KS) == t ? 0 : 1;
        return partials + ((size_t)gg * 2 + which) * E;
      };
      segment(t / n_tiles, t - (t / n_tiles) * n_tiles, s0, s1, ghi - glo + 1, g - glo, slot);
      it += s1 - s0;
      __syncthreads();  // LDS and s_last are reused by the next segment
    }
  } else {
    const int bid = blockIdx.x;
    const int n_tile = bid % n_tiles;
    const int rest = bid / n_tiles;
    const int sk = rest % split;
    const int m_tile = rest / split;
    const int tile = m_tile * n_tiles + n_tile;
    auto slot = [&](int j) { return partials + ((size_t)tile * split + j) * E; };
    segment(m_tile, n_tile, (int)((uint32_t)(sk * KS) / (uint32_t)split),
            (int)((uint32_t)((sk + 1) * KS) / (uint32_t)split), split, sk, slot);
  }
}

// The zero fill of the float-atomic epilogue's tiles (gemm_kernels.hip).
hipError_t launch_zero_f32(float *p, int n4, hipStream_t stream);

typedef hipError_t (*launch_fn)(const GemmArgs &, int split, bool sw, hipStream_t);

template <int MT, int NT, int WN, int WK, int KPW, bool PREQ, int RB, int EPI = 0>
hipError_t launch_variant(const GemmArgs &a, int split, bool sw, hipStream_t stream) {
  const int n_tiles = a.N / (16 * NT * WN);
  const int m_tiles = (a.M + 16 * MT - 1) / (16 * MT);
  char *ws = (char *)a.workspace;
  const uint8_t *aq = nullptr, *as = nullptr;
  if (!PREQ && a.Aq) return hipErrorInvalidValue;  // pre-quantized A needs a pre-quantized schedule
  if (PREQ) {
    if (a.Aq) {
      // the caller's codes and shuffled scales, read as they are: one launch
      aq = (const uint8_t *)a.Aq;
      as = (const uint8_t *)a.As;
    } else {
      // bf16 A under a pre-quantized schedule: quantize it into the
      // workspace first, in the caller's layout
      uint8_t *q = (uint8_t *)(ws + kTicketBytes);
      uint8_t *sc = q + caller_codes_bytes(a.M, a.K);
      hipError_t e = launch_quantize(a.A, a.M, a.K, q, sc, true, sw, stream);
      if (e != hipSuccess) return e;
      aq = q;
      as = sc;
    }
  }
  uint32_t *tickets = (uint32_t *)ws;
  float *partials = nullptr;
  if (split > 1 || EPI == 2)
    partials = (float *)(ws + kTicketBytes + (PREQ ? ((pq_operand_bytes(a.M, a.K) + 255) & ~(size_t)255) : 0));
  if (EPI == 1 && split > 1) {
    const int n4 = n_tiles * m_tiles * MT * NT * WN * 64;  // tiles x elements / 4
    hipError_t e = launch_zero_f32(partials, n4, stream);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)(EPI == 2 ? split : n_tiles * m_tiles * split));
  gemm_kernel<MT, NT, WN, WK, KPW, PREQ, RB, EPI><<<grid, 64 * WN * WK, 0, stream>>>(
      (const uint16_t *)a.A, aq, as, (const uint8_t *)a.Bw, (const uint8_t *)a.Bs, (uint16_t *)a.C, partials, tickets,
      a.M, a.N, a.K, split, n_tiles, sw ? 1 : 0);
  return hipGetLastError();
}

struct Variant {
  int mt, nt, wn, wk, kpw, pq;
  launch_fn fn;
  int rb;    // rows per staged A block (8: only for M <= 8)
  int wide;  // the large-M kernel of gemm_wide.hip
  int epi;   // split epilogue: 0 ticketed slots, 1 float atomics, 2 stream-K
};

#define V(MT, NT, WN, WK, KPW) {MT, NT, WN, WK, KPW, 0, launch_variant<MT, NT, WN, WK, KPW, false, 16>, 16, 0, 0}
#define V8(MT, NT, WN, WK, KPW) {MT, NT, WN, WK, KPW, 0, launch_variant<MT, NT, WN, WK, KPW, false, 8>, 8, 0, 0}
#define VQ(MT, NT, WN, WK, KPW) {MT, NT, WN, WK, KPW, 1, launch_variant<MT, NT, WN, WK, KPW, true, 16>, 16, 0, 0}
// the same kernels with the float-atomic (EPI 1) and stream-K (EPI 2)
// epilogues, for the long-K small-M shapes that split K
#define VE(MT, NT, WN, WK, KPW, RB)                                                              \
  {MT, NT, WN, WK, KPW, 0, launch_variant<MT, NT, WN, WK, KPW, false, RB, 1>, RB, 0, 1},        \
      {MT, NT, WN, WK, KPW, 0, launch_variant<MT, NT, WN, WK, KPW, false, RB, 2>, RB, 0, 2},
// large-M kernels: W waves split K; listed with wn = 1, wk = W, kpw = the
// number of steps loaded ahead
#define VW(MW, NW, W, D) {MW, NW, 1, W, D, 1, launch_wide_##MW##_##NW##_##W##_##D, 16, 1, 0},
#define VWL(MW, NW, W, D) {MW, NW, 1, W, D, 1, launch_widel_##MW##_##NW##_##W##_##D, 16, 3, 0},

}  // namespace mxfp4
