// NVFP4 x NVFP4 GEMM: exact dequantisation to FP16 in registers + FP16 MFMA.
//
// Prior art: "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera
// Rubin NVL72", section "Building the GEMM".  There, block-scaled NVFP4 MMAs
// consume the E4M3 scales in hardware.
//
// gfx950's scaled MFMA instead takes one E8M0 (power-of-two) scale per
// 32-element K block.  NVFP4 has an E4M3 scale per 16 elements, whose
// mantissa (1 + f, f in eighths) cannot be folded exactly into 4-, 6- or
// 8-bit MFMA operands.  The exact mapping used here:
//   - e2m1(code) * e4m3(scale) has at most 6 significant bits and lies in
//     [2^-10, 2688], so it is exact in FP16;
//   - the FP4->FP16 conversion gives the code value and one packed FP16
//     multiply the whole scale (both E4M3 scales of a lane's two blocks
//     decoded to an FP16 pair by one conversion);
//   - the FP16 MFMA (v_mfma_f32_32x32x16_f16) accumulates in FP32;
//   - the epilogue multiplies by s_tA * s_tB.
// The roofline of this path is therefore the FP16/BF16 dense MFMA peak.
//
// Layout of one workgroup (256 threads, 4 waves):
//   - Output tile 256 x 256; each wave owns 128 x 128 (4 x 4 tiles of 32 x 32).
//   - K step 128 elements, double-buffered in LDS:
//       codes [256][64] bytes per operand, 16-byte chunks swizzled by
//       ((row >> 2) & 3);
//       scales [256] x 8 bytes (the step's eight 16-element blocks).
//   - K assignment (identical for A and B, so products pair up): in half h of
//     a step, lane (r = l % 32, g = l / 32) reads chunk 2h+g of its row, i.e.
//     K elements [64h + 32g, 64h + 32g + 32).  Dword s' of that chunk feeds
//     MFMA sub-step s' (8 elements at MFMA positions 8g..8g+7) and belongs to
//     scale block 4h + 2g + s'/2.
#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

constexpr int BM = 256, BN = 256, BK = 128, NT = 256;
constexpr int ROWB = BK / 2;   // code bytes per row per step
constexpr int GROUP_M = 8;

// Tiles are uint4 arrays: the compiler then knows every access is 16-byte
// aligned and emits single ds_read_b128 / ds_write_b128 instructions.
constexpr int RC = ROWB / 16;   // 16-byte chunks per row
struct Smem {
  uint4 a[2][BM * RC];
  uint4 b[2][BN * RC];
  uint2 as[2][BM];
  uint2 bs[2][BN];
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * RC + (chunk ^ ((row >> 2) & 3)); }

__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in = t - group * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

template <bool SCALE_QW>
__global__ __launch_bounds__(NT, 1) void nvfp4_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ Ats,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const float* __restrict__ Bts,
    uint16_t* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = (K + BK - 1) / BK;
  const int KH = K / 2;          // code bytes per row
  const int KB = K / 16;         // scale bytes per row

  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const auto ca_rsrc = make_rsrc(A + (int64_t)m0 * KH, rows_a * KH);
  const auto cb_rsrc = make_rsrc(B + (int64_t)n0 * KH, rows_b * KH);
  const auto sa_rsrc = make_rsrc(As + (int64_t)m0 * KB, rows_a * KB);
  const auto sb_rsrc = make_rsrc(Bs + (int64_t)n0 * KB, rows_b * KB);

  // staging: thread owns chunk (tid & 3) of rows (tid >> 2) + 64 i, and the
  // scale bytes of row tid
  const int lc = tid & 3, lr = tid >> 2;
  uint4 ra[4], rb[4];
  uint32_t sa_raw[4], sb_raw[4];
  const int off0 = lr * KH + lc * 16;
  // Loads only issue here (no branches, no uses); scale words are assembled
  // in sstore, after the MFMAs of the current step.
  auto gload = [&](int kt) {
    const int kofs = kt * ROWB + lc * 16 < KH ? kt * ROWB : OOB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = kofs == OOB ? OOB : off0 + 64 * i * KH + kofs;
      ra[i] = buffer_load_x4(ca_rsrc, off);
      rb[i] = buffer_load_x4(cb_rsrc, off);
    }
    if (SCALE_QW) {            // K % 128 == 0: the step's 8 scale bytes are one qword
      const uint2 va = buffer_load_x2(sa_rsrc, tid * KB + kt * 8);
      const uint2 vb = buffer_load_x2(sb_rsrc, tid * KB + kt * 8);
      sa_raw[0] = va.x; sa_raw[1] = va.y; sb_raw[0] = vb.x; sb_raw[1] = vb.y;
    } else {                   // pairs of blocks; pairs past K read as 0
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = kt * 8 + 2 * j;
        sa_raw[j] = buffer_load_u16(sa_rsrc, kb < KB ? tid * KB + kb : OOB);
        sb_raw[j] = buffer_load_u16(sb_rsrc, kb < KB ? tid * KB + kb : OOB);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lr + 64 * i;
      sm.a[buf][swz(row, lc)] = ra[i];
      sm.b[buf][swz(row, lc)] = rb[i];
    }
    if (SCALE_QW) {
      sm.as[buf][tid] = make_uint2(sa_raw[0], sa_raw[1]);
      sm.bs[buf][tid] = make_uint2(sb_raw[0], sb_raw[1]);
    } else {
      sm.as[buf][tid] = make_uint2(sa_raw[0] | (sa_raw[1] << 16), sa_raw[2] | (sa_raw[3] << 16));
      sm.bs[buf][tid] = make_uint2(sb_raw[0] | (sb_raw[1] << 16), sb_raw[2] | (sb_raw[3] << 16));
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  if (KT > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 ca[4], cb[4];
      uint32_t da[4], db[4];   // the lane's two block scales per row, FP16 pair
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r;
        ca[i] = sm.a[buf][swz(row, 2 * h + g)];
        const uint2 sc = sm.as[buf][row];
        const uint32_t w = h ? sc.y : sc.x;           // blocks 4h .. 4h+3
        da[i] = e4m3_pair_f16(w >> (16 * g));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + r;
        cb[j] = sm.b[buf][swz(row, 2 * h + g)];
        const uint2 sc = sm.bs[buf][row];
        const uint32_t w = h ? sc.y : sc.x;
        db[j] = e4m3_pair_f16(w >> (16 * g));
      }
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        v8h av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t d = sp == 0 ? ca[i].x : sp == 1 ? ca[i].y : sp == 2 ? ca[i].z : ca[i].w;
          av[i] = dequant8_f16(d, da[i], sp >> 1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t d = sp == 0 ? cb[j].x : sp == 1 ? cb[j].y : sp == 2 ? cb[j].z : cb[j].w;
          bv[j] = dequant8_f16(d, db[j], sp >> 1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  const float alpha = __fmul_rn(*Ats, *Bts);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        if (row < M && col < N)
          C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v] * alpha);
      }
    }
}


// Decoded scales of one lane for one half step: the E4M3 scales of its two
// 16-element blocks as an FP16 pair (block 0 low, block 1 high).
struct Scales2 {
  uint32_t mp;
};

__device__ __forceinline__ Scales2 decode_scale_pair(uint32_t word16) {
  return Scales2{e4m3_pair_f16(word16)};
}

// The two halves of the exact expansion are issued apart: the code values
// (e2m1x8_f16) under one half of a sub-step's MFMAs and the multiply by the
// block's whole scale (scale8_f16) under the other.  (An earlier form had the
// conversion take 2^E from an FP32 scale and the multiply only (1 + f), which
// cost two more instructions per scale pair to build; same bits, 1.2-2.4%
// slower.)

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int sp) {
  return sp == 0 ? q.x : sp == 1 ? q.y : sp == 2 ? q.z : q.w;
}

// ---------------------------------------------------------------------------
// Ring kernel (K % 256 == 0).  The operands stream HBM -> LDS by direct loads
// into two pair slots; a pair is two 128-element K steps, so each row of a
// slot holds the 128 code bytes of two steps and every direct load fetches
// whole 128-byte lines (against 64-byte half lines with one step per slot:
// half the L2 requests for the same bytes; same-process A/B against a 4-stage
// ring of single steps, bit-identical: 16384^3 2.5% faster, 4096^3 and
// ragged shapes 2-3.5%).  A step is ~4096 MFMA cycles, so the 1.5-2 steps a
// pair has to land cover the load latency.
//
// Per pair slot and operand, codes are [256][128] bytes, 16-byte chunk c of
// row r at c ^ ((r >> 1) & 7) (conflict-free ds_read_b128); step 2p of pair p
// is chunks 0-3, step 2p + 1 chunks 4-7.  Scales are the pair's 16 bytes per
// row (eight 16-element blocks per step), one lane per row.  Each wave issues
// 8 code loads per operand per pair (1 KiB = 8 rows each) and one scale load.
// Pair p, steps 2p and 2p + 1:
//   - step 2p: the B loads of pair p + 1 go out two per sub-step over its
//     first four sub-steps (into the slot of pair p - 1, free since the last
//     barrier); no barrier, the next step is in the same slot;
//   - step 2p + 1: between sub-steps 3 and 4 the wave waits for every load
//     (pair p + 1) and crosses the barrier, after which nobody reads slot p;
//     the A loads of pair p + 2 go out two per sub-step over sub-steps 4-7.
//
// A step is 8 sub-steps of 16 MFMAs (K16 each); sub-step t uses half t/4 of
// the step's K range and dword t%4 of the lane's code chunk.  Software
// pipeline inside a step:
//   - the operands of sub-step t+1 are prepared during sub-step t: the
//     code conversions under its first 8 MFMAs, the scale multiplies
//     under its last 8, so no multiply waits on a conversion just issued
//     (measured: +3% over issuing them in pairs);
//   - half 1's codes and scale words are read from LDS during sub-step 0 and
//     decoded in four quarters over sub-steps 1 and 2;
//   - the next step's half-0 data is read during sub-step 4 (after the
//     barrier in odd steps), decoded over sub-steps 5 and 6, and prepared for
//     its sub-step 0 during sub-step 7.
struct NRingSmem {
  uint4 a[2][BM * 8];             // pair slots: the 128 code bytes of two steps per row
  uint4 b[2][BN * 8];
  uint4 as[2][BM];                // 16 scale bytes per row: step 2p then 2p + 1
  uint4 bs[2][BN];
};

// Codes and scale words of one half step for one lane: chunk 2h+g of its 4 A
// and 4 B rows, and the 16-bit pair of E4M3 bytes of its two blocks (in the
// low half of each word).
struct NHalf {
  uint4 ca[4], cb[4];
  uint32_t wa[4], wb[4];
};
struct NDec {
  Scales2 a[4], b[4];
};

__global__ __launch_bounds__(NT, 1) void nvfp4_gemm_ring_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ Ats,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const float* __restrict__ Bts,
    uint16_t* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ NRingSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases in SGPRs
  int tm, tn;
  if (tiles_m % 16 == 0 && tiles_n % 16 == 0)
    supertile_order(blockIdx.x, tiles_n, tm, tn);
  else
    raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = K / BK;          // even and > 0 (K % 256 == 0)
  const int KH = K / 2, KB = K / 16;
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const rsrc4_t ra = make_rsrc4(A + (int64_t)m0 * KH, rows_a * KH);
  const rsrc4_t rb = make_rsrc4(B + (int64_t)n0 * KH, rows_b * KH);
  const rsrc4_t rsa = make_rsrc4(As + (int64_t)m0 * KB, rows_a * KB);
  const rsrc4_t rsb = make_rsrc4(Bs + (int64_t)n0 * KB, rows_b * KB);
  // Past-the-end stages load through empty resources: every offset is then
  // out of range and reads zero.
  const rsrc4_t ra0 = make_rsrc4(A, 0), rb0 = make_rsrc4(B, 0);
  const rsrc4_t rsa0 = make_rsrc4(As, 0), rsb0 = make_rsrc4(Bs, 0);

  // load u (0..7) of an operand covers rows 8 (8 wave + u) .. + 7, the 128
  // bytes of one pair per row; lane i fills chunk position i & 7
  int code_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 8 * (8 * wave + u) + (lane >> 3);
    code_off[u] = row * KH + (((lane & 7) ^ ((row >> 1) & 7)) * 16);
  }
  const int scale_off = (64 * wave + lane) * KB;
  const int KPR = KT / 2;         // pairs

  // Stage st: code load u (A rows for u < 4, B rows for u >= 4) and the
  // scale loads.  The lane's offset within the tile's panel is a loop
  // constant, the stage's K offset is the load's scalar offset, and
  // past-the-end stages load zeros through the empty resources, so issuing a
  // load costs no vector instructions (measured against per-lane offsets with
  // a select: 2.3% faster at 16384^3, 1.3-1.6% at 4096^3 and 4096^2 x 16384,
  // bit-identical).
  auto issue_a = [&](int p, int u) {
    dma_x4_so(p < KPR ? ra : ra0, (uint32_t)(uintptr_t)&sm.a[p & 1][64 * (8 * wave + u)], code_off[u], p * 128);
  };
  auto issue_b = [&](int p, int u) {
    dma_x4_so(p < KPR ? rb : rb0, (uint32_t)(uintptr_t)&sm.b[p & 1][64 * (8 * wave + u)], code_off[u], p * 128);
  };
  auto issue_sa = [&](int p) {
    dma_x4_so(p < KPR ? rsa : rsa0, (uint32_t)(uintptr_t)&sm.as[p & 1][64 * wave], scale_off, p * 16);
  };
  auto issue_sb = [&](int p) {
    dma_x4_so(p < KPR ? rsb : rsb0, (uint32_t)(uintptr_t)&sm.bs[p & 1][64 * wave], scale_off, p * 16);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  // Half h of stage st; `par` = st & 1 selects the stage's 8 bytes of the
  // 16-byte super-stage entry (static).
  auto read_half = [&](int st, auto PARC, auto HC, NHalf& x) {
    constexpr int par = decltype(PARC)::value, h = decltype(HC)::value;
    const int slot = (st >> 1) & 1;
    constexpr int chunk = 4 * par + 2 * h;   // + g: the lane's chunk of the pair row
    // lane g's two scale bytes: the 16-bit half g of the half step's dword
    const uint16_t* sa16 = reinterpret_cast<const uint16_t*>(&sm.as[slot][0]);
    const uint16_t* sb16 = reinterpret_cast<const uint16_t*>(&sm.bs[slot][0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + r;
      x.ca[i] = sm.a[slot][row * 8 + ((chunk + g) ^ ((row >> 1) & 7))];
      x.wa[i] = sa16[(row * 4 + par * 2 + h) * 2 + g];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + r;
      x.cb[j] = sm.b[slot][row * 8 + ((chunk + g) ^ ((row >> 1) & 7))];
      x.wb[j] = sb16[(row * 4 + par * 2 + h) * 2 + g];
    }
  };
  auto decode = [&](const NHalf& x, NDec& d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) d.a[i] = decode_scale_pair(x.wa[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) d.b[j] = decode_scale_pair(x.wb[j]);
  };
  // quarter q of decode: A fragments 2q, 2q + 1 (q < 2) or B fragments
  // 2q - 4, 2q - 3
  auto decode_part = [&](const NHalf& x, NDec& d, auto QC) {
    constexpr int q = decltype(QC)::value;
#pragma unroll
    for (int i = 2 * (q & 1); i < 2 * (q & 1) + 2; ++i) {
      if (q < 2) d.a[i] = decode_scale_pair(x.wa[i]);
      else d.b[i] = decode_scale_pair(x.wb[i]);
    }
  };
  auto dequant = [&](const NHalf& x, const NDec& d, int sp, v8h* av, v8h* bv) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      av[i] = scale8_f16(e2m1x8_f16(dword_of(x.ca[i], sp)), d.a[i].mp, sp >> 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bv[j] = scale8_f16(e2m1x8_f16(dword_of(x.cb[j], sp)), d.b[j].mp, sp >> 1);
  };
  auto convert = [&](const NHalf& x, const NDec& d, int sp, v8h* av, v8h* bv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = e2m1x8_f16(dword_of(x.ca[i], sp));
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = e2m1x8_f16(dword_of(x.cb[j], sp));
  };
  auto rescale = [&](const NDec& d, int sp, v8h* av, v8h* bv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = scale8_f16(av[i], d.a[i].mp, sp >> 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = scale8_f16(bv[j], d.b[j].mp, sp >> 1);
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  // MFMAs of tile rows i0, i0 + 1 (8 of the sub-step's 16)
  auto mfma_half = [&](const v8h* av, const v8h* bv, int i0) {
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[j], av[i], acc[i][j], 0, 0, 0);   // B first
  };
  // 8 groups of 1 MFMA, NV VALU and NL LDS reads
  auto interleave = [](auto NV, auto NL) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(NV)::value, 0);
      if (decltype(NL)::value) __builtin_amdgcn_sched_group_barrier(0x100, decltype(NL)::value, 0);
    }
  };
  using N0 = std::integral_constant<int, 0>;
  using N2 = std::integral_constant<int, 2>;
  using N4 = std::integral_constant<int, 4>;
  using N6 = std::integral_constant<int, 6>;

  NHalf x0, x1;     // current stage half 0 / half 1 (x0 is reused for the next stage)
  NDec d0, d1;
  v8h av[2][4], bv[2][4];

  // Sub-step: MFMAs on operands (ca, cb); prepares (na, nb) from (x, d, sp):
  // conversions under the first 8 MFMAs (with `first`), multiplies under the
  // last 8 (with `second`).  Scheduling regions end at the sched_barriers.
  auto sub = [&](const v8h* ca, const v8h* cb, const NHalf& x, const NDec& d, int sp, v8h* na, v8h* nb,
                 auto first, auto second, auto NV1, auto NV2, auto NL2, auto pre) {
    pre();   // direct loads placed ahead of the sub-step's scheduling region
    __builtin_amdgcn_sched_barrier(0);
    mfma_half(ca, cb, 0);
    convert(x, d, sp, na, nb);
    first();
    interleave(NV1, N0{});
    __builtin_amdgcn_sched_barrier(0);
    mfma_half(ca, cb, 2);
    rescale(d, sp, na, nb);
    second();
    interleave(NV2, NL2);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto none = [] {};

  // Step kt with parity PAR = kt & 1 (static).  On entry x0/d0 hold stage
  // kt's half 0 and av[0]/bv[0] its sub-step 0.
  auto step = [&](int kt, auto PARC) {
    constexpr int PAR = decltype(PARC)::value;
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    // pair p = kt / 2.  Even step: the B loads (and B scales) of pair p + 1,
    // two per sub-step over the first four.  Odd step: after the mid-step
    // barrier, the A loads (and A scales) of pair p + 2 over sub-steps 4-7.
    // (Loads spread over sub-steps: a burst of ten direct loads held up the
    // wave's MFMA issue while the memory queue drained, measured -2.7% at
    // 16384^3 with single-step stages.)
    const int p = kt >> 1;
    auto loads = [&](auto Q) {
      constexpr int q = decltype(Q)::value;
      return [&] {
        if constexpr (PAR == 0) {
          if (q == 0) issue_sb(p + 1);
          if (q < 4) {
            issue_b(p + 1, 2 * q);
            issue_b(p + 1, 2 * q + 1);
          }
        } else {
          if (q == 4) issue_sa(p + 2);
          if (q >= 4) {
            issue_a(p + 2, 2 * (q - 4));
            issue_a(p + 2, 2 * (q - 4) + 1);
          }
        }
      };
    };
    sub(av[0], bv[0], x0, d0, 1, av[1], bv[1], none, [&] { read_half(kt, PARC, H1{}, x1); }, N4{}, N4{}, N2{},
        loads(std::integral_constant<int, 0>{}));
    sub(av[1], bv[1], x0, d0, 2, av[0], bv[0], [&] { decode_part(x1, d1, std::integral_constant<int, 0>{}); },
        [&] { decode_part(x1, d1, std::integral_constant<int, 1>{}); }, N6{}, N6{}, N0{},
        loads(std::integral_constant<int, 1>{}));
    sub(av[0], bv[0], x0, d0, 3, av[1], bv[1], [&] { decode_part(x1, d1, std::integral_constant<int, 2>{}); },
        [&] { decode_part(x1, d1, std::integral_constant<int, 3>{}); }, N6{}, N6{}, N0{},
        loads(std::integral_constant<int, 2>{}));
    sub(av[1], bv[1], x1, d1, 0, av[0], bv[0], none, none, N4{}, N4{}, N0{}, loads(std::integral_constant<int, 3>{}));
    // odd step: pair p + 1 (every load issued so far) landed, and nobody reads
    // slot p any more; even step: the next stage is in the same pair slot
    if constexpr (PAR == 1) wait_vm_barrier<0>();
    else __builtin_amdgcn_sched_barrier(0);
    sub(av[0], bv[0], x1, d1, 1, av[1], bv[1], none,
        [&] { read_half(kt + 1, std::integral_constant<int, PAR ^ 1>{}, H0{}, x0); }, N4{}, N4{}, N2{},
        loads(std::integral_constant<int, 4>{}));
    sub(av[1], bv[1], x1, d1, 2, av[0], bv[0], [&] { decode_part(x0, d0, std::integral_constant<int, 0>{}); },
        [&] { decode_part(x0, d0, std::integral_constant<int, 1>{}); }, N6{}, N6{}, N0{},
        loads(std::integral_constant<int, 5>{}));
    sub(av[0], bv[0], x1, d1, 3, av[1], bv[1], [&] { decode_part(x0, d0, std::integral_constant<int, 2>{}); },
        [&] { decode_part(x0, d0, std::integral_constant<int, 3>{}); }, N6{}, N6{}, N0{},
        loads(std::integral_constant<int, 6>{}));
    sub(av[1], bv[1], x0, d0, 0, av[0], bv[0], none, none, N4{}, N4{}, N0{}, loads(std::integral_constant<int, 7>{}));
  };

  // prologue: pair 0 and the A half of pair 1; wait for pair 0
  issue_sa(0);
  issue_sb(0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    issue_a(0, u);
    issue_b(0, u);
  }
  issue_sa(1);
#pragma unroll
  for (int u = 0; u < 8; ++u) issue_a(1, u);
  wait_vm_barrier<9>();
  read_half(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, x0);
  decode(x0, d0);
  dequant(x0, d0, 0, av[0], bv[0]);
  // Uniform body to the end: the last step issues zero loads past KT and
  // prepares "stage KT" (zeros), which is never used.
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }

  // Epilogue: x s_tA s_tB, BF16, through the (now idle) A and B rings as
  // whole row segments (the MFMAs took the B operand first, so each lane holds
  // 4 consecutive columns per accumulator quad).
  const float alpha = __fmul_rn(*Ats, *Bts);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the out-of-range tail loads
  __syncthreads();                                   // every wave is done with the rings
  static_assert(sizeof(sm.a) + sizeof(sm.b) >= 4 * 128 * 256, "epilogue staging needs 32 KB per wave");
  store_block128_bf16<true>(acc, &sm.a[0][0] + wave * (128 * 16), C, M, N, m0 + wm * 128, n0 + wn * 128, alpha);
}


// ---------------------------------------------------------------------------
// Small-problem kernel: 64 x 64 output tiles, one 32 x 32 FP16 MFMA tile per
// wave, operands straight from global memory (L2) into registers.  It serves
// grids that would leave most CUs idle with 256 x 256 tiles: the
// 256 x 256 x 128 GEMM is one such tile, and one workgroup would then run
// every load, MFMA and store of the problem in series (14 us).
//
// K runs in chunks of 128 elements.  In a chunk, lane (r = l % 32,
// g = l / 32) supplies A row r (and B row r) at K [64 g, 64 g + 64): 32
// contiguous code bytes and the 4 scale bytes of their blocks.  MFMA t
// (0..7) takes K positions 64 g + 8 t .. + 7 from each lane half, so A and B
// pair the same K positions in every product and each position is used once.
// Codes are dequantised exactly to FP16 as in the other kernels.
constexpr int SMALL_T = 64;
// Grids of fewer 256 x 256 tiles than this run the small kernel (measured:
// 2.4-2.9x faster up to 25 tiles, equal at 32, 8% slower at 36).
constexpr int NV_SMALL_TILES = 32;

__global__ __launch_bounds__(256) void nvfp4_small_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ Ats,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const float* __restrict__ Bts,
    uint16_t* __restrict__ C, int M, int N, int K, int tiles_n) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * SMALL_T + 32 * (wave & 1), n0 = tn * SMALL_T + 32 * (wave >> 1);
  const int KH = K / 2, KB = K / 16;
  // wave-uniform (readfirstlane), so the buffer resources stay scalar
  const int rows_a = __builtin_amdgcn_readfirstlane(max(0, min(32, M - m0)));
  const int rows_b = __builtin_amdgcn_readfirstlane(max(0, min(32, N - n0)));
  const auto ca = make_rsrc(A + (int64_t)max(0, min(m0, M)) * KH, rows_a * KH);
  const auto cb = make_rsrc(B + (int64_t)max(0, min(n0, N)) * KH, rows_b * KH);
  const auto sa = make_rsrc(As + (int64_t)max(0, min(m0, M)) * KB, rows_a * KB);
  const auto sb = make_rsrc(Bs + (int64_t)max(0, min(n0, N)) * KB, rows_b * KB);
  const int r = lane & 31, g = lane >> 5;
  v16f acc = v16f{};
  for (int kc = 0; kc < K; kc += 128) {
    // K % 32 == 0: each 32-element half of the lane's range is wholly in or out of K
    const int k0 = kc + 64 * g;
    const bool in0 = k0 < K, in1 = k0 + 32 < K;
    const uint4 a0 = buffer_load_x4(ca, in0 ? r * KH + k0 / 2 : OOB);
    const uint4 a1 = buffer_load_x4(ca, in1 ? r * KH + k0 / 2 + 16 : OOB);
    const uint4 b0 = buffer_load_x4(cb, in0 ? r * KH + k0 / 2 : OOB);
    const uint4 b1 = buffer_load_x4(cb, in1 ? r * KH + k0 / 2 + 16 : OOB);
    // the scale row pitch K / 16 is only 2-byte aligned: 16-bit loads
    const uint32_t sa0 = buffer_load_u16(sa, in0 ? r * KB + k0 / 16 : OOB);
    const uint32_t sa1 = buffer_load_u16(sa, in1 ? r * KB + k0 / 16 + 2 : OOB);
    const uint32_t sb0 = buffer_load_u16(sb, in0 ? r * KB + k0 / 16 : OOB);
    const uint32_t sb1 = buffer_load_u16(sb, in1 ? r * KB + k0 / 16 + 2 : OOB);
    // blocks 0-1 and 2-3 of the lane's range as FP16 scale pairs
    const uint32_t xp[2] = {e4m3_pair_f16(sa0), e4m3_pair_f16(sa1)};
    const uint32_t yp[2] = {e4m3_pair_f16(sb0), e4m3_pair_f16(sb1)};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t da = t < 4 ? dword_of(a0, t) : dword_of(a1, t - 4);
      const uint32_t db = t < 4 ? dword_of(b0, t) : dword_of(b1, t - 4);
      const v8h av = dequant8_f16(da, xp[t / 4], (t / 2) & 1);
      const v8h bv = dequant8_f16(db, yp[t / 4], (t / 2) & 1);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
  }
  const float alpha = __fmul_rn(*Ats, *Bts);
  const int col = n0 + r;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = m0 + (v >> 2) * 8 + g * 4 + (v & 3);
    if (row < M && col < N) C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[v] * alpha);
  }
}
}  // namespace

hipError_t launch_gemm_nvfp4(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const float* ats, const uint8_t* b,
                             const uint8_t* bs, const float* bts, uint16_t* c,
                             hipStream_t stream) {
  const int tiles_m = (int)ceil_div(m, BM), tiles_n = (int)ceil_div(n, BN);
  if (tiles_m * tiles_n < NV_SMALL_TILES) {
    const int sm = (int)ceil_div(m, SMALL_T), sn = (int)ceil_div(n, SMALL_T);
    hipLaunchKernelGGL(nvfp4_small_kernel, dim3(sm * sn), dim3(256), 0, stream, a, as, ats, b, bs, bts, c, (int)m,
                       (int)n, (int)k, sn);
  } else if (k % 256 == 0 && k > 0)
    hipLaunchKernelGGL(nvfp4_gemm_ring_kernel, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, ats, b, bs, bts, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else if (k % 128 == 0)
    hipLaunchKernelGGL(nvfp4_gemm_kernel<true>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, ats, b, bs, bts, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(nvfp4_gemm_kernel<false>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, ats, b, bs, bts, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bsg
