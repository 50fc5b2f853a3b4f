// W4A16 tile kernel: C[M][N] = s_tW * X[M][K] (BF16) x deq(W)[N][K] (NVFP4),
// one workgroup per MT x NT output tile, over all of K.
//
// Source: "Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic"
// (bitsandbytes PR #2030), sections "The SIMT / MMA layer" (matrix cores take
// over from the vector ALU as M grows) and the tile-selection follow-up (the
// tile width along N is chosen per shape).
//
// Layout.  KS = 2: 8 waves, two per SIMD: wave (ng = w % 4, kh = w / 4) owns W rows
// [NTW ng, NTW ng + NTW) of the tile and all MT rows of X, and the kh-th half
// of every K stage; the two halves are summed through LDS at the end (KS = 1:
// 4 waves, each over whole stages).  Every W element of the tile is
// dequantised exactly once.
//   - W is the MFMA's A operand and X its B operand, so each output lane holds
//     4 consecutive columns n of one row m of C: 8-byte stores.
//   - K stages of SK elements flow through an NS-stage ring in LDS, filled by
//     direct loads: per stage the tile's X [MT][2 SK bytes], W codes
//     [NT][SK / 2 bytes] and E4M3 scales [NT][SK / 16 bytes].  NS - 1 stages
//     are in flight while one is computed: enough bytes to cover the HBM
//     latency for the thin tiles of small M (measured: with 64-element
//     stages the 16 x 64 tile took 20 us at 14336 x 4096, with 512-element
//     stages 12 us).
//   - W codes are expanded exactly to BF16 in registers (dequant2_bf16: the
//     product e2m1 * e4m3 has at most 6 significant bits) and the BF16 MFMA
//     accumulates in FP32; the epilogue multiplies by s_tW.
// MFMA shapes: NTW = 32 takes v_mfma_f32_32x32x16_bf16, NTW = 16
// v_mfma_f32_16x16x32_bf16.  K assignment (identical for W and X, so products
// pair up), within a wave's SKW = SK / KS elements of a stage:
//   32x32x16: sub-step t, lane half g:    K [g SKW / 2 + 8 t, + 8);
//   16x16x32: sub-step t, lane quarter q: K [q SKW / 4 + 8 t, + 8);
// so each lane's W codes and scale bytes for a stage are contiguous.
#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

// 16-byte chunk c of a row of nc chunks, swizzled so that 16 lanes reading
// the same chunk of consecutive rows hit 16 different bank groups.
template <int NC>
__device__ __forceinline__ int tswz(int r, int c) {
  if constexpr (NC >= 16) return c ^ (r & 15);
  else return c ^ ((r / (16 / NC)) & (NC - 1));
}

template <int MT, int NT, int SK, int NS>
struct TileSmem {
  uint4 x[NS][MT * SK / 8];       // X rows: 2 SK bytes
  uint4 w[NS][NT * SK / 32];      // W code rows: SK / 2 bytes
  uint32_t s[NS][NT * SK / 64];   // W scale rows: SK / 16 bytes
  uint4 dummy[64];                // target of the padding loads that keep every wave's load count equal
};

template <int MT, int NTW, int WN, int KS, int SK, int NS>
__global__ __launch_bounds__(64 * WN * KS, 1) void w4_tile_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wc, const uint8_t* __restrict__ Ws,
    const float* __restrict__ Wts, uint16_t* __restrict__ C, int M, int N, int K, int tiles_m) {
  constexpr int NT = WN * NTW;
  constexpr int TW = WN * KS;                         // waves
  constexpr int SKW = SK / KS;                        // K elements per wave per stage
  constexpr bool BIG = NTW % 32 == 0;                 // 32x32x16 MFMAs, else 16x16x32
  constexpr int TS = BIG ? 32 : 16;                   // MFMA tile edge
  constexpr int WT = NTW / TS;                        // W tiles per wave
  constexpr int MJ = MT / TS;                         // m tiles per wave
  constexpr int SUB = BIG ? SKW / 16 : SKW / 32;      // sub-steps per wave per stage
  constexpr int XNC = SK / 8, WNC = SK / 32;          // 16-byte chunks per X / W row
  constexpr int SBR = SK / 16;                        // scale bytes per W row per stage
  // direct loads per stage: 16-byte lanes (1 KB each) for X and W, 4-byte
  // lanes (256 B each) for the scales, padded to a multiple of the wave
  // count; every wave loads a share of everything.  (Splitting the streams
  // between the two K halves' waves, W 5 stages ahead and X 2, so that each
  // stream has its own in-order load counter, measured 2-12% slower.)
  constexpr int XCNT = MT * 2 * SK / 1024, WCNT = NT * SK / 2 / 1024, SCNT = NT * SBR / 256;
  constexpr int XL = (XCNT + TW - 1) / TW, WL = (WCNT + TW - 1) / TW, SL = (SCNT + TW - 1) / TW;
  constexpr int LOADS = XL + WL + SL;
  static_assert(XCNT >= 1 && WCNT >= 1 && SCNT >= 1 && NTW * SKW / 2 >= 64, "tile too small");
  static_assert(LOADS * (NS - 1) < 64, "vmcnt range");
  static_assert(XNC <= 64 && WNC <= 64, "row geometry");
  __shared__ TileSmem<MT, NT, SK, NS> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar load selection
  const int ng = wave % WN, kh = wave / WN;
  // the m tiles of one W slab run on one XCD, one after another
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int n0 = (lin / tiles_m) * NT, m0 = (lin % tiles_m) * MT;
  const int KT = K / SK;                              // > 0 (K % SK == 0)
  const int KH = K / 2, KB = K / 16;
  const int rows_w = min(N - n0, NT), rows_x = min(M - m0, MT);
  const rsrc4_t rw = make_rsrc4(Wc + (int64_t)n0 * KH, rows_w * KH);
  const rsrc4_t rs = make_rsrc4(Ws + (int64_t)n0 * KB, rows_w * KB);
  const rsrc4_t rx = make_rsrc4(X + (int64_t)m0 * K, rows_x * K * 2);

  // --- direct loads of stage st into a ring slot SLOT.  The per-lane part of
  // every offset is computed once; a stage adds its K position.  Padding
  // loads read zeros out of range into the dummy area.  Stages past KT need
  // no masking: they land in slots that are never computed on, and past the
  // end of a buffer the resource returns zeros.
  int xo[XL], wo[WL], so[SL];
#pragma unroll
  for (int u = 0; u < XL; ++u) {                      // X: 1 KB = 1024 / (2 SK) rows per load
    const int j = wave * XL + u;
    const int row = j * (1024 / (2 * SK)) + lane / XNC, sl = lane % XNC;
    xo[u] = j < XCNT ? row * K * 2 + 16 * tswz<XNC>(row, sl) : -1;
  }
#pragma unroll
  for (int u = 0; u < WL; ++u) {                      // W codes: 1 KB = 2048 / SK rows per load
    const int j = wave * WL + u;
    const int row = j * (2048 / SK) + lane / WNC, sl = lane % WNC;
    wo[u] = j < WCNT ? row * KH + 16 * tswz<WNC>(row, sl) : -1;
  }
#pragma unroll
  for (int u = 0; u < SL; ++u) {                      // scales: 256 B = 256 / SBR rows per load
    const int j = wave * SL + u;
    const int b = 256 * j + 4 * lane;                 // byte in the stage's scale block
    so[u] = j < SCNT ? (b / SBR) * KB + b % SBR : -1;
  }
  auto issue_x = [&](int st, auto SLOTC) {
    constexpr int slot = decltype(SLOTC)::value;
#pragma unroll
    for (int u = 0; u < XL; ++u) {
      const bool real = wave * XL + u < XCNT;           // wave-uniform
      dma_x4(rx, lds_addr(real ? &sm.x[slot][(wave * XL + u) * 64] : &sm.dummy[0]), real ? xo[u] + st * SK * 2 : OOB);
    }
  };
  auto issue_w = [&](int st, auto SLOTC) {
    constexpr int slot = decltype(SLOTC)::value;
#pragma unroll
    for (int u = 0; u < WL; ++u) {
      const bool real = wave * WL + u < WCNT;
      dma_x4(rw, lds_addr(real ? &sm.w[slot][(wave * WL + u) * 64] : &sm.dummy[0]), real ? wo[u] + st * (SK / 2) : OOB);
    }
#pragma unroll
    for (int u = 0; u < SL; ++u) {
      const bool real = wave * SL + u < SCNT;
      dma_x1(rs, lds_addr(real ? &sm.s[slot][(wave * SL + u) * 64] : reinterpret_cast<uint32_t*>(&sm.dummy[0])),
             real ? so[u] + st * SBR : OOB);
    }
  };

  // --- fragments of one stage for this lane
  const int r = BIG ? (lane & 31) : (lane & 15);
  const int g = BIG ? (lane >> 5) : (lane >> 4);      // lane half (32x32) or quarter (16x16)
  // this lane's W row of W tile wt: NTW ng + TS wt + r
  constexpr int WB = BIG ? SKW / 4 : SKW / 8;         // W code bytes per lane per stage
  constexpr int WQ = WB / 16;                         // ... in 16-byte chunks
  constexpr int NSB = BIG ? SKW / 32 : SKW / 64;      // scale bytes per lane per stage
  static_assert(WB % 16 == 0 && (NSB == 1 || NSB == 2 || NSB == 4), "fragment geometry");
  constexpr int NACC = BIG ? 16 : 4;
  typedef float vacc __attribute__((ext_vector_type(NACC)));
  vacc acc[WT][MJ];
#pragma unroll
  for (int wt = 0; wt < WT; ++wt)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[wt][j] = vacc{};

  // One stage (X in ring slot SX, W and scales in slot SW): the lane's W
  // codes and scale bytes are read and the scales decoded exactly (byte t / 2
  // serves sub-step t); then, sub-step by sub-step, the X fragments of
  // sub-step t + 1 are read while sub-step t's W codes are expanded to BF16
  // and its MFMAs run.  Reading a whole stage's fragments up front instead
  // left the LDS busy and the matrix cores idle at the start of every step
  // and the reverse at its end (timing-only builds at 14336 x 4096, m = 256:
  // 35.7 us with no global loads at all, 33.7 us with no MFMAs).
  const int xc = (kh * SKW + g * (BIG ? SKW / 2 : SKW / 4)) / 8;   // the lane's first X chunk of a stage
  const int wbyte = kh * SKW / 2 + g * WB;                          // ... and first W code byte
  auto stage = [&](auto SXC, auto SWC) {
    constexpr int sx = decltype(SXC)::value, sw = decltype(SWC)::value;
    uint4 wc[WT][WQ];
    uint32_t sc[WT];
#pragma unroll
    for (int wt = 0; wt < WT; ++wt) {
      const int wr = NTW * ng + TS * wt + r;
#pragma unroll
      for (int c = 0; c < WQ; ++c) wc[wt][c] = sm.w[sw][wr * WNC + tswz<WNC>(wr, wbyte / 16 + c)];
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(&sm.s[sw][0]) + wr * SBR + kh * SKW / 16 + g * NSB;
      if constexpr (NSB == 4) sc[wt] = *reinterpret_cast<const uint32_t*>(sb);
      else if constexpr (NSB == 2) sc[wt] = *reinterpret_cast<const uint16_t*>(sb);
      else sc[wt] = *sb;
    }
    auto read_x = [&](int t, uint4* xf) {
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        const int row = TS * j + r;
        xf[j] = sm.x[sx][row * XNC + tswz<XNC>(row, xc + t)];
      }
    };
    uint4 xf[2][MJ];
    read_x(0, xf[0]);
    float s[WT][NSB];
#pragma unroll
    for (int wt = 0; wt < WT; ++wt) {
      static_for<0, (NSB + 1) / 2>([&](auto BC) {
        constexpr int b = 2 * decltype(BC)::value;
        const v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc[wt], 1.0f, b >= 2);   // exact E4M3 decode
        s[wt][b] = v[0];
        if constexpr (b + 1 < NSB) s[wt][b + 1] = v[1];
      });
    }
    static_for<0, SUB>([&](auto TC) {
      constexpr int t = decltype(TC)::value;
      if constexpr (t + 1 < SUB) read_x(t + 1, xf[(t + 1) & 1]);
      v8bf wv[WT];
#pragma unroll
      for (int wt = 0; wt < WT; ++wt) {
        const uint4& q = wc[wt][t / 4];
        const uint32_t d = (t & 3) == 0 ? q.x : (t & 3) == 1 ? q.y : (t & 3) == 2 ? q.z : q.w;
        wv[wt] = dequant8_bf16(d, s[wt][t >> 1]);
      }
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        v8bf xv;
        __builtin_memcpy(&xv, &xf[t & 1][j], 16);
#pragma unroll
        for (int wt = 0; wt < WT; ++wt) {
          if constexpr (BIG)
            acc[wt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[wt], xv, acc[wt][j], 0, 0, 0);
          else
            acc[wt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[wt], xv, acc[wt][j], 0, 0, 0);
        }
      }
      // keep sub-step t + 2's reads out of sub-step t's region
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // --- pipeline.  Step kt: wait for stage kt and cross the barrier (after
  // which stage kt has landed and no wave still reads stage kt-1's slot),
  // issue stage kt+NS-1 into that slot and compute stage kt; NS - 1 stages
  // stay in flight.  A stage's X and W loads go out together, stage by stage,
  // so the wait count covers whole stages.  The loop body is NS steps, so
  // every ring slot is a compile-time constant (static LDS offsets); steps
  // past KT are skipped.
  static_for<0, NS - 1>([&](auto SC) {
    issue_x(decltype(SC)::value, SC);
    issue_w(decltype(SC)::value, SC);
  });
  auto step = [&](int kt, auto IC) {
    constexpr int i = decltype(IC)::value;
    using SL_ = std::integral_constant<int, (i + NS - 1) % NS>;
    wait_vm_barrier<LOADS * (NS - 2)>();     // stage kt landed; stage kt-1's slot is free
    issue_x(kt + NS - 1, SL_{});
    issue_w(kt + NS - 1, SL_{});
    stage(std::integral_constant<int, i>{}, std::integral_constant<int, i>{});
  };
  for (int kt = 0; kt < KT; kt += NS) {
    static_for<0, NS>([&](auto IC) {
      if (kt + decltype(IC)::value < KT) step(kt + decltype(IC)::value, IC);
    });
  }

  // --- with two K halves, sum them through LDS (the ring is free once
  // every wave's loads, padding included, have landed and every wave is past
  // its last read)
  if constexpr (KS == 2) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    vacc* red = reinterpret_cast<vacc*>(&sm.x[0][0]);
    static_assert(WN * WT * MJ * 64 * sizeof(vacc) <= sizeof(sm.x), "reduction space");
    if (kh == 1) {
#pragma unroll
      for (int wt = 0; wt < WT; ++wt)
#pragma unroll
        for (int j = 0; j < MJ; ++j) red[((ng * WT + wt) * MJ + j) * 64 + lane] = acc[wt][j];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kh == 1) return;
#pragma unroll
    for (int wt = 0; wt < WT; ++wt)
#pragma unroll
      for (int j = 0; j < MJ; ++j) acc[wt][j] += red[((ng * WT + wt) * MJ + j) * 64 + lane];
  }

  // --- epilogue: x s_tW, BF16 RNE; lane holds 4 consecutive n of one m
  const float ts = *Wts;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int wt = 0; wt < WT; ++wt)
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int m = m0 + TS * j + r;
    if (m >= M) continue;
#pragma unroll
    for (int grp = 0; grp < NACC / 4; ++grp) {
      const int n = n0 + NTW * ng + TS * wt + (BIG ? 8 * grp + 4 * g : 4 * g);
      const uint32_t lo = pack_bf16x2(acc[wt][j][4 * grp] * ts, acc[wt][j][4 * grp + 1] * ts);
      const uint32_t hi = pack_bf16x2(acc[wt][j][4 * grp + 2] * ts, acc[wt][j][4 * grp + 3] * ts);
      uint16_t* p = C + (int64_t)m * N + n;
      if (vec && n + 4 <= N) {
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
      } else {
        const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < N) p[i] = e[i];
      }
    }
  }
}

template <int MT, int NTW, int WN, int KS, int SK, int NS>
hipError_t launch_tile(int64_t m, int64_t n, int64_t k, const uint16_t* x, const uint8_t* w, const uint8_t* ws,
                       const float* wts, uint16_t* c, hipStream_t stream) {
  const int tiles_m = (int)ceil_div(m, MT), tiles_n = (int)ceil_div(n, WN * NTW);
  hipLaunchKernelGGL((w4_tile_kernel<MT, NTW, WN, KS, SK, NS>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(64 * WN * KS), 0, stream,
                     x, w, ws, wts, c, (int)m, (int)n, (int)k, tiles_m);
  return hipGetLastError();
}

}  // namespace

int w4_tile_k_multiple(int shape) { return shape == 0 ? 512 : shape == 1 ? 256 : 128; }

// Tile shapes (m x n, K per stage, ring stages), all with 8 waves (4 W row
// groups x two K halves per stage):
//   0: 16 x 64,   K 512, 4 stages (136 KB of LDS);
//   1: 64 x 64,   K 256, 3 stages (123 KB);
//   2: 128 x 128, K 128, 3 stages (123 KB).
// Measured on 14336 x 4096, m = 256 (graph replay, cold weights), against
// the 8-wave shape 2: 4 waves with K 64 x 4 stages and 4 waves with K 128 x 3
// stages within 3%; 4 waves of 2 x 2 (each two W tiles, half the LDS reads of
// X per MFMA) within 3% (box-to-box spread ~10%).  The 128 x 128 tile takes
// ~40 us per 128 x 128 x 4096 tile whichever of these it is, ~3x its MFMA
// time per stage: the two stages in flight do not cover the load latency.
hipError_t launch_w4_tile(int shape, int64_t m, int64_t n, int64_t k, const uint16_t* x, const uint8_t* w,
                          const uint8_t* ws, const float* wts, uint16_t* c, hipStream_t stream) {
  if (shape == 0) return launch_tile<16, 16, 4, 2, 512, 4>(m, n, k, x, w, ws, wts, c, stream);
  if (shape == 1) return launch_tile<64, 16, 4, 2, 256, 3>(m, n, k, x, w, ws, wts, c, stream);
  return launch_tile<128, 32, 4, 2, 128, 3>(m, n, k, x, w, ws, wts, c, stream);
}

}  // namespace bsg
