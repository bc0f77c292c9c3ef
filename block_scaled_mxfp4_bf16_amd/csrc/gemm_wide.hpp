// Large-M MXFP4 GEMM kernel for gfx950 (template; instantiated by
// gemm_wide.hip): the K loop over A quantized beforehand into quad-packed
// operand blocks, in which the waves of a workgroup split K instead of the
// tile.  The design notes and the operand layout are at the top of
// gemm_wide.hip.
#pragma once

#include <type_traits>

#include "mxfp4_device.hpp"
#include "mxfp4_internal.hpp"

namespace mxfp4 {

// A -> quad-packed operand (internal linkage: each library that launches
// it has its own copy).  One two-wave workgroup per (tile quad q, K step ks): wave h quantizes
// tiles 4q + 2h and 4q + 2h + 1, each 16 rows x 128 elements of bf16 A in
// four coalesced 16-byte loads per lane (one per 32-element group, four
// lanes per group, as in the fused kernels' staging).  All eight loads of a
// lane are issued before any is used, so a workgroup pays one memory round
// trip, and the grid (one workgroup per quad and step) spreads A over the
// CUs.  Codes go to the tiles' 1 KiB blocks; the two tiles' scale bytes of
// an operand lane go to half h of that lane's scale dword as one 16-bit
// store.  Rows past M and chunks past K load as zeros and are written as
// zero codes with scale byte 0; so are the tiles of the last quad past M.
static __global__ __launch_bounds__(128) void quant_quad_kernel(const uint16_t *__restrict__ A, uint8_t *__restrict__ Aop,
                                                         int M, int K, int sw_quant) {
  const int lane = threadIdx.x & 63;
  const int h = threadIdx.x >> 6;
  const int KS = (K + 127) >> 7;
  const int q = blockIdx.x / KS;
  const int ks = blockIdx.x - q * KS;
  const int mq = (M + 63) >> 6;
  const int a_bytes = M * K * 2;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, a_bytes, kRsrcWord3);
  u32x4 w[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (4 * q + 2 * h + j) * 16 + (lane >> 2);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int kel = ks * 128 + ch * 32 + (lane & 3) * 8;
      const bool ok = (row < M) && (ks * 128 + ch * 32 < K);
      w[j][ch] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, off_or_oob(ok, (row * K + kel) * 2), 0, 0);
    }
  }
  uint32_t *codes = (uint32_t *)Aop;
  uint16_t *scales = (uint16_t *)(Aop + (size_t)mq * 4 * KS * 1024);
  auto run = [&](auto sw_tag) {
    constexpr bool SW = decltype(sw_tag)::value;
    uint32_t s[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = 4 * q + 2 * h + j;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        // lane = 4*row + quarter: dword (16*ch + row)*4 + quarter of the block
        codes[(size_t)(t * KS + ks) * 256 + ch * 64 + lane] = quant_quarter_t<SW>(w[j][ch], &s[j][ch]);
      }
    }
    // operand lane 16*ch + row: bytes 2h, 2h + 1 of its dword
    if ((lane & 3) == 0) {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        scales[((size_t)(q * KS + ks) * 64 + ch * 16 + (lane >> 2)) * 2 + h] = (uint16_t)(s[0][ch] | (s[1][ch] << 8));
    }
  };
  if (sw_quant)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// Scaled FP4 x FP4 matrix instruction whose A scale is byte `sel` of the
// scale dword (the instruction's byte select must be a constant; `sel` is
// one after unrolling).
__device__ __forceinline__ v4f mfma_fp4_sel(const v8i &a, const v8i &b, const v4f &c, int sel, uint32_t sa,
                                            uint32_t sb) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 1, (int)sa, 0, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 2, (int)sa, 0, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 3, (int)sa, 0, (int)sb);
  }
}

// Uniform part of a buffer offset, moved out of range (bit 31) unless
// `in_range`; the lane's part is added to it afterwards (all offsets stay
// below 2^31, so the sum is out of range exactly when the flag is set).
__device__ __forceinline__ int uniform_off(bool in_range, int off) {
  return off | (in_range ? 0 : (int)0x80000000u);
}

// Workgroup: W waves (two per SIMD when W = 8), output tile of 16*MW rows x
// 16*NW columns, K steps [S0, S1) of its split; wave w takes steps S0 + w,
// S0 + w + W, ...  Each wave keeps the whole tile's accumulators in
// registers and D steps of operands in flight.
// BL: B's codes go straight from memory into a per-wave LDS ring of D
// slots (one step's NW operand blocks each) instead of registers, so the
// registers that would have held them hold deeper A stages; each lane reads
// back exactly the 16 bytes it loaded, right before the step's MFMAs.
// s_waitcnt for vmcnt <= N, expcnt and lgkmcnt left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// STAMPS (measurement probes only; every schedule of the library has it
// off, and split must be 1): each wave records the 100 MHz real-time counter
// at entry, at the end of its K loop, once the partial tiles are in LDS,
// once its C stores are issued and once they are complete, and lane 0
// writes them, with the XCD number, to `partials` read as uint64
// [workgroups * W][8].
template <int MW, int NW, int W, int D, bool BL, bool STAMPS = false>
__global__ __launch_bounds__(64 * W) void gemm_wide_kernel(const uint8_t *__restrict__ Aop,
                                                          const uint8_t *__restrict__ Bw,
                                                          const uint8_t *__restrict__ Bs, uint16_t *__restrict__ C,
                                                          float *__restrict__ partials,
                                                          uint32_t *__restrict__ tickets, int M, int N, int K,
                                                          int split, int n_tiles, int m_tiles) {
  static_assert(MW % 4 == 0, "A scales come as one dword per four row tiles");
  static_assert(W == 4 || W == 8, "four or eight waves");
  constexpr int NTH = 64 * W;
  constexpr int MQ = MW / 4;
  constexpr int NSD = (NW + 1) / 2;  // B scale dwords per step: 32-row blocks the NW subtiles touch
  constexpr int E = MW * NW * 256;   // outputs per tile
  constexpr int RS = 4;              // partial tiles LDS holds at once
  // the B ring and the partial tiles share one LDS array
  constexpr int kRedBytes = RS * E * 4;
  // per wave: a 1 KiB block the first DMA load lands in, then D slots of NW
  // operand blocks
  constexpr int kWaveRing = (D * NW + 1) * 1024;
  constexpr int kRingBytes = BL ? W * kWaveRing : 0;
  constexpr int kLdsBytes = kRedBytes > kRingBytes ? kRedBytes : kRingBytes;
  static_assert(kLdsBytes <= 160 * 1024 - 64, "partial tiles and B ring must fit in LDS");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  float *const red = (float *)lds;
  uint8_t *const ring = lds;
  __shared__ uint32_t s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint64_t stamp[5];
  auto take = [&](int i) {
    if constexpr (STAMPS) stamp[i] = __builtin_amdgcn_s_memrealtime();
  };
  take(0);

  // Workgroup b runs on XCD b % 8.  Give each XCD a contiguous range of
  // (n tile, m tile, split) indices, split and m tile fastest, so that the
  // workgroups reading the same B columns share one L2.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int g8 = G >> 3, r8 = G & 7;
  const int lin = xcd < r8 ? xcd * (g8 + 1) + slot : r8 * (g8 + 1) + (xcd - r8) * g8 + slot;
  const int sk = lin % split;
  const int mn = lin / split;
  const int m_tile = mn % m_tiles;
  const int n_tile = mn / m_tiles;
  const int gw = n_tile * NW;  // first 16-row group of B
  const int t0 = m_tile * MW;  // first 16-row tile of A

  const int KS = (K + 127) >> 7;
  const int S0 = (int)((uint32_t)(sk * KS) / (uint32_t)split);
  const int S1 = (int)((uint32_t)((sk + 1) * KS) / (uint32_t)split);
  const int gp = ((K >> 5) + 7) & ~7;
  const int kc = lane >> 4;

  // Out-of-range offsets read zeros: tiles past the quantized rows, steps
  // past the run, and the missing half of a final 64-wide step.
  const int mq_all = (M + 63) >> 6;
  const int codes_bytes = mq_all * 4 * KS * 1024;
  const int ascale_bytes = mq_all * KS * 256;
  const int b_bytes = (N >> 4) * K * 8;
  const int s_bytes = ((N + 255) >> 8) * 8 * gp * 32;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Aop, 0, codes_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t as_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(Aop + codes_bytes), 0, ascale_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Bw, 0, b_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)Bs, 0, s_bytes, kRsrcWord3);
  // the lane's byte in a 1 KiB operand block and in a 256-byte scale block;
  // a final half step leaves K chunks 2 and 3 of B out of range (bit 31 is
  // set with an OR, so an offset already out of range stays so)
  const int l16 = lane * 16, l4 = lane * 4;
  const int half_k = (K & 127) != 0;
  const int half_oob = (half_k && kc >= 2) ? (int)0x80000000u : 0;

  struct Stage {
    u32x4 a[MW];
    uint32_t as[MQ];
    u32x4 b[BL ? 1 : NW];
    uint32_t bs[NSD];
  };
  // Byte offset of a ring slot: this wave's slot d, operand block nt.
  auto ring_at = [&](int d, int nt) { return wave * kWaveRing + (1 + d * NW + nt) * 1024; };
  auto load = [&](int ks, Stage &st, int d) {
    const bool ok = ks < S1;
    const int lb = ks == KS - 1 ? half_oob : 0;
    if constexpr (BL) {
      // B first: the step's A (in registers) arrives after it, so waiting
      // for A also covers the ring slot
#pragma unroll
      for (int nt = 0; nt < NW; ++nt)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (__attribute__((address_space(3))) void *)(ring + ring_at(d, nt)),
                                                 16, uniform_off(ok, (gw + nt) * K * 8 + ks * 1024 + l16) | lb, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < NSD; ++q)
        st.bs[q] = __builtin_amdgcn_raw_buffer_load_b32(
            s_rsrc, uniform_off(ok, ((gw >> 1) + q) * gp * 32 + (ks >> 1) * 256) + l4, 0, 0);
    }
#pragma unroll
    for (int mw = 0; mw < MW; ++mw)
      st.a[mw] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, uniform_off(ok, ((t0 + mw) * KS + ks) * 1024) + l16, 0, 0);
#pragma unroll
    for (int q = 0; q < MQ; ++q)
      st.as[q] = __builtin_amdgcn_raw_buffer_load_b32(
          as_rsrc, uniform_off(ok, ((m_tile * MQ + q) * KS + ks) * 256) + l4, 0, 0);
    if constexpr (!BL) {
#pragma unroll
      for (int nt = 0; nt < NW; ++nt)
        st.b[nt] =
            __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, uniform_off(ok, (gw + nt) * K * 8 + ks * 1024 + l16) | lb, 0, 0);
#pragma unroll
      for (int q = 0; q < NSD; ++q)
        st.bs[q] = __builtin_amdgcn_raw_buffer_load_b32(
            s_rsrc, uniform_off(ok, ((gw >> 1) + q) * gp * 32 + (ks >> 1) * 256) + l4, 0, 0);
    }
  };
  // Loads per stage, and how many are issued after a stage's B by the time
  // its slot is read in the steady loop: its own scales and A, and the
  // D - 1 other stages.
  constexpr int kLoadsPerStage = NW + NSD + MW + MQ;
  constexpr int kOwnAfterB = NSD + MW + MQ;
  constexpr int kAfterB = (D - 1) * kLoadsPerStage + kOwnAfterB;
  static_assert(!BL || kAfterB <= 63, "the load counter holds at most 63");

  // The scale byte of B subtile nt: the dword of its 32-row block, byte
  // (row block half) | 2 * (step parity); a wave's steps all share a parity
  // when W is even.
  const int ks0 = S0 + wave;
  const int odd = gw & 1;
  uint32_t bshift[NW];
#pragma unroll
  for (int nt = 0; nt < NW; ++nt) bshift[nt] = 8u * (uint32_t)(((gw + nt) & 1) | ((ks0 & 1) << 1));

  v4f acc[MW][NW];
#pragma unroll
  for (int mw = 0; mw < MW; ++mw)
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) acc[mw][nt] = v4f{0.f, 0.f, 0.f, 0.f};

  // B operand blocks of ring slot d, read back once the slot's loads have
  // landed.  The slot is written by the memory system, not by an
  // instruction the compiler tracks, so the wait is explicit: `after` loads
  // issued after the slot's B may still be outstanding.
  // `later` stages (0 .. D-1) issued their loads after slot d's.
  auto ring_read = [&](int d, int later, u32x4 (&bl)[NW]) {
    if constexpr (BL) {
      switch (later) {
        case 0: wait_vmcnt<kOwnAfterB>(); break;
        case 1: wait_vmcnt<kOwnAfterB + (D > 1 ? kLoadsPerStage : 0)>(); break;
        case 2: wait_vmcnt<kOwnAfterB + (D > 2 ? 2 * kLoadsPerStage : 0)>(); break;
        default: wait_vmcnt<kAfterB>(); break;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) bl[nt] = *(const u32x4 *)(ring + ring_at(d, nt) + l16);
    }
  };
  auto compute = [&](const Stage &st, const u32x4 (&bl)[NW]) {
    const u32x4 *bv = BL ? bl : st.b;
    uint32_t sb[NW];
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      const uint32_t dw = (NW % 2 == 0) ? st.bs[nt >> 1] : (odd ? st.bs[(nt + 1) >> 1] : st.bs[nt >> 1]);
      sb[nt] = (dw >> bshift[nt]) & 0xFFu;
    }
#pragma unroll
    for (int mw = 0; mw < MW; ++mw) {
      const v8i a_op = {(int)st.a[mw].x, (int)st.a[mw].y, (int)st.a[mw].z, (int)st.a[mw].w, 0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) {
        const v8i b_op = {(int)bv[nt].x, (int)bv[nt].y, (int)bv[nt].z, (int)bv[nt].w, 0, 0, 0, 0};
        acc[mw][nt] = mfma_fp4_sel(a_op, b_op, acc[mw][nt], mw & 3, st.as[mw >> 2], sb[nt]);
      }
    }
  };

  // The load counter retires in issue order, so a stage's data has arrived
  // once no more than D - 1 stages' loads are outstanding, provided the
  // loads go out stage by stage: scheduling barriers keep the compiler from
  // interleaving them.  The loop has no branch inside (a branch that skips
  // a load or a use makes the compiler wait for every load in flight where
  // the paths meet); steps past the run load zeros and add nothing, and the
  // last round issues no loads.
  // With BL the loop is rotated so that each stage reads the next slot
  // after issuing its own reload: a ring read at the top of the loop would
  // follow the previous iteration's last ring load across the back edge,
  // where the compiler can no longer tell the slots apart and waits for it.
  if constexpr (BL) {
    // The compiler checks an LDS read against the first LDS-DMA load of the
    // array it meets and, unless their addresses differ by a constant that
    // keeps them apart, waits for every DMA load in flight.  Make that first
    // load one out of range (it fetches nothing and writes zeros) into this
    // wave's block below its ring, which no read touches; the ring reads
    // carry their own exact waits.
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        b_rsrc, (__attribute__((address_space(3))) void *)(ring + wave * kWaveRing), 16, (int)0x80000000u, 0, 0, 0);
  }
  Stage st[D];
  u32x4 bl[NW];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load(ks0 + W * d, st[d], d);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nsteps = ks0 < S1 ? (S1 - ks0 + W - 1) / W : 0;
  const int rounds = (nsteps + D - 1) / D;
  if (rounds > 0) ring_read(0, D - 1, bl);
  for (int it = 0; it + 1 < rounds; ++it) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(st[d], bl);
      __builtin_amdgcn_sched_barrier(0);
      load(ks0 + W * ((it + 1) * D + d), st[d], d);
      __builtin_amdgcn_sched_barrier(0);
      ring_read((d + 1) % D, D - 1, bl);
    }
  }
  if (rounds > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(st[d], bl);
      // last round: no reloads, so fewer loads follow each slot's B
      if (d + 1 < D) ring_read(d + 1, D - 2 - d, bl);
    }
  }
  if constexpr (BL) {
    // the partial tiles reuse the ring: every wave's loads must have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if constexpr (STAMPS) {
    // the stamp follows the last product
#pragma unroll
    for (int mw = 0; mw < MW; ++mw)
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) asm volatile("" ::"v"(acc[mw][nt]));
  }
  take(1);

  // Add the waves' tiles through LDS, four at a time.  Element index e =
  // ((mw*NW + nt)*4 + r)*64 + l is accumulator element r of lane l in
  // subtile (mw, nt): C row 16*mw + 4*(l/16) + r, column 16*nt + l%16, so
  // eight consecutive e are eight consecutive columns of one row.  With
  // eight waves, waves 4..7 hand their tiles to waves 0..3 first.
  auto put = [&](int slot) {
#pragma unroll
    for (int mw = 0; mw < MW; ++mw)
#pragma unroll
      for (int nt = 0; nt < NW; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[slot * E + ((mw * NW + nt) * 4 + r) * 64 + lane] = acc[mw][nt][r];
  };
  if constexpr (W == 8) {
    if (wave >= 4) put(wave - 4);
    __syncthreads();
    if (wave < 4) {
#pragma unroll
      for (int mw = 0; mw < MW; ++mw)
#pragma unroll
        for (int nt = 0; nt < NW; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mw][nt][r] += red[wave * E + ((mw * NW + nt) * 4 + r) * 64 + lane];
    }
    __syncthreads();
    if (wave < 4) put(wave);
  } else {
    put(wave);
  }
  __syncthreads();
  take(2);

  const int m0 = t0 * 16;
  auto sum8 = [&](int e0, float (&v)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
#pragma unroll
    for (int w = 0; w < RS; ++w) {
      const v4f lo = *(const v4f *)(red + w * E + e0);
      const v4f hi = *(const v4f *)(red + w * E + e0 + 4);
      v[0] += lo[0]; v[1] += lo[1]; v[2] += lo[2]; v[3] += lo[3];
      v[4] += hi[0]; v[5] += hi[1]; v[6] += hi[2]; v[7] += hi[3];
    }
  };
  auto store8 = [&](int e0, const float (&v)[8]) {
    const int ln = e0 & 63, i = e0 >> 6;
    const int r = i & 3, t = i >> 2;
    const int mw = t / NW, nt = t % NW;
    const int row = m0 + 16 * mw + 4 * (ln >> 4) + r;
    const int col = 16 * (gw + nt) + (ln & 15);
    if (row < M) {
      u32x4 pk;
      pk.x = bf16x2_rne(v[0], v[1]);
      pk.y = bf16x2_rne(v[2], v[3]);
      pk.z = bf16x2_rne(v[4], v[5]);
      pk.w = bf16x2_rne(v[6], v[7]);
      *(u32x4 *)(C + (size_t)row * N + col) = pk;
    }
  };

  if (split == 1) {
    for (int j = threadIdx.x; j < E / 8; j += NTH) {
      float v[8];
      sum8(8 * j, v);
      store8(8 * j, v);
    }
    if constexpr (STAMPS) {
      take(3);
      __builtin_amdgcn_s_waitcnt(0);
      take(4);
      uint32_t xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      if (lane == 0) {
        uint64_t *out = (uint64_t *)partials + ((size_t)blockIdx.x * W + wave) * 8;
#pragma unroll
        for (int i = 0; i < 5; ++i) out[i] = stamp[i];
        out[5] = xcc & 0xFu;
      }
    }
    return;
  }

  // Split K across workgroups: the same slot-and-ticket protocol as the
  // fused kernels (device-coherent slot stores, wait, ticket; the last
  // workgroup adds the slots in split order and resets the ticket).  Slots
  // move 16-byte chunks: buffer stores and loads with the device-coherence
  // bit, which is what relaxed agent-scope atomic accesses compile to.
  constexpr int kSc1 = 16;
  const int tile = m_tile * n_tiles + n_tile;
  auto slot_rsrc = [&](int s) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)(partials + ((size_t)tile * split + s) * E), 0, E * 4,
                                             kRsrcWord3);
  };
  auto as_u = [](float a, float b, float c, float d) {
    return u32x4{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
  };
  {
    const __amdgpu_buffer_rsrc_t w_rsrc = slot_rsrc(sk);
    for (int j = threadIdx.x; j < E / 8; j += NTH) {
      float v[8];
      sum8(8 * j, v);
      __builtin_amdgcn_raw_buffer_store_b128(as_u(v[0], v[1], v[2], v[3]), w_rsrc, 32 * j, 0, kSc1);
      __builtin_amdgcn_raw_buffer_store_b128(as_u(v[4], v[5], v[6], v[7]), w_rsrc, 32 * j + 16, 0, kSc1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&tickets[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)(split - 1)
                 ? 1u
                 : 0u;
  __syncthreads();
  if (!s_last) return;
  for (int j = threadIdx.x; j < E / 8; j += NTH) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
    for (int s = 0; s < split; ++s) {
      const __amdgpu_buffer_rsrc_t r_rsrc = slot_rsrc(s);
      const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r_rsrc, 32 * j, 0, kSc1);
      const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r_rsrc, 32 * j + 16, 0, kSc1);
      v[0] += __uint_as_float(lo.x); v[1] += __uint_as_float(lo.y);
      v[2] += __uint_as_float(lo.z); v[3] += __uint_as_float(lo.w);
      v[4] += __uint_as_float(hi.x); v[5] += __uint_as_float(hi.y);
      v[6] += __uint_as_float(hi.z); v[7] += __uint_as_float(hi.w);
    }
    store8(8 * j, v);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&tickets[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mxfp4
