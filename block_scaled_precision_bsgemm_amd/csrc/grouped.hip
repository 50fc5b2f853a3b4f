// Ragged grouped GEMM: NVFP4 activations x dense BF16 or FP16 weights, BF16
// output, with the optional epilogue and routing variants.
//
// Source: "Triton #11171 -- Why Two New NVFP4 Test Cases Produced Twelve
// Tensor-Memory Failures", sections "Ragged mode added routing rather than a
// plain matrix" and "NVFP4 x dense matmul".  Routed activation rows are
// grouped per slice (expert), and each slice meets its own dense operand.
// That page stages an expanded (dequantised) copy of the NVFP4 operand for
// the dense MMA.  Here each wave expands its own fragments in registers
// instead, exactly: to BF16 for BF16 weights (BF16 MFMA), to FP16 for FP16
// weights (FP16 MFMA; e2m1 * e4m3 is exact in FP16 too).
//
// Variants (same page: "Scatter changes where output rows are written",
// "Gamma adds a per-row scaling input", "The ordinary variants also exercise
// the shared bias route", "Filter 3: gather variants are excluded"), for
// logical row r of group g:
//   A row read   src(r) = gather[r] (else r);
//   y[r][n]      = (s_t * acc + bias[g][n]) * gamma[r];
//   stored at    C[scatter[r]][n] (else C[r][n]).
// Gather changes only the A load offsets (computed once per tile); the
// epilogue reads the tile's gamma and destination rows from LDS.  Indices
// outside [0, a_rows) (gather) or [0, m_total) (scatter) read zeros or skip
// the store, so malformed indices stay inside the buffers.
//
// Scheduling.  The host knows only G, m_total and n; the row counts stay on
// the device.  The grid therefore covers an upper bound on the number of
// tiles (256-row tiles: sum_g ceil(c_g / BM) <= m_total / BM + G; the
// ping-pong kernel's two tile heights: see grouped_grid_blocks).  Each
// workgroup finds its (group, m-tile) with a wave-wide prefix scan over the
// offsets.  Workgroups past the real tile count exit at once.  Tiles are
// ordered n-tile-major, so the m-tiles of one group (same W panel) run close
// together; xcd_remap keeps neighbours on one XCD's L2.
//
// Tile: 256 rows x 256 columns, 4 waves of 128 x 128, K step 64 elements:
//   - A codes [256][32] bytes (chunks swizzled by (row >> 3) & 1), A scales
//     [256] dwords (4 E4M3 bytes);
//   - W [256][64] BF16, 16-byte chunks swizzled by ((row >> 1) & 7).
// K assignment (A and W agree): lane (r = l % 32, g = l / 32) takes K
// elements [32g, 32g + 32) of the step.  Dword sp of that range feeds MFMA
// sub-step sp at positions 8g..8g+7; its scale block is 2g + sp/2, and its W
// chunk is 4g + sp.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int AROWB = BK / 2;        // A code bytes per row per step
constexpr int WROWB = BK * 2;        // W bytes per row per step

// Tiles are uint4 arrays: the compiler then knows every access is 16-byte
// aligned and emits single ds_read_b128 / ds_write_b128 instructions.
constexpr int ARC = AROWB / 16, WRC = WROWB / 16;   // 16-byte chunks per row
struct Smem {
  uint4 a[2][BM * ARC];
  uint4 w[2][BN * WRC];
  uint32_t as[2][BM];
  int tile_info[4];
};

// 16-byte chunk c of A row r sits at c ^ ((r >> 3) & 1) (conflict-free for
// 32 consecutive rows reading one chunk).
__device__ __forceinline__ int aswz(int row, int chunk) { return row * ARC + (chunk ^ ((row >> 3) & 1)); }

// 16-byte chunk c of W row r sits at c ^ ((r >> 1) & 7): 16 consecutive rows
// reading one chunk cover all 16 bank groups.
__device__ __forceinline__ int wswz(int row, int chunk) { return row * WRC + (chunk ^ ((row >> 1) & 7)); }

// Everything a grouped launch needs.  bias, gamma, gather and scatter may be
// null.  W holds BF16 or FP16 bit patterns (the kernel's F16 parameter).
struct GArgs {
  const uint8_t* A;
  const uint8_t* As;
  const float* Ats;
  const int32_t* off;
  const uint16_t* W;
  uint16_t* C;
  const float* bias;      // [G][N]
  const float* gamma;     // [M]
  const int32_t* gather;  // [M], rows of A
  const int32_t* scatter; // [M], rows of C
  const int32_t* koff;    // K-ragged mode: [G + 1] K offsets (multiples of 256); C is [G][M][N]
  int G, M, a_rows, N, K, tiles_n, tiles_m;
  int mbig;               // ping-pong kernel: 256-row tile slots per n-tile
};

// Operand type, exact dequantisation and MFMA of the two weight types.
template <bool F16> struct GMath;
template <> struct GMath<false> {
  typedef v8bf vec;
  typedef v2f scales;   // a lane's two block scales (bytes 0, 1 of a word), FP32
  static __device__ __forceinline__ scales decode(uint32_t word) { return e4m3_pair_f32(word); }
  static __device__ __forceinline__ vec dq8(uint32_t codes, const scales& s, int b) {
    return dequant8_bf16(codes, b ? s[1] : s[0]);
  }
  static __device__ __forceinline__ v16f mfma(const vec& a, const vec& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct GMath<true> {
  typedef v8h vec;
  typedef uint32_t scales;   // the two block scales as an FP16 pair
  static __device__ __forceinline__ scales decode(uint32_t word) { return e4m3_pair_f16(word); }
  static __device__ __forceinline__ vec dq8(uint32_t codes, const scales& s, int b) { return dequant8_f16(codes, s, b); }
  static __device__ __forceinline__ v16f mfma(const vec& a, const vec& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Per-tile epilogue data in LDS: the destination row of each of the tile's
// 256 logical rows (-1: no store) and its gamma.
struct GEpi {
  int dst[BM];
  float gamma[BM];
};

// Thread t < BM fills row t of the tile starting at logical row r0 with
// rows_a valid rows.
__device__ __forceinline__ void fill_epi(const GArgs& p, int r0, int rows_a, int t, GEpi& e) {
  if (t >= BM) return;
  int dst = -1;
  float gm = 1.0f;
  if (t < rows_a) {
    dst = p.scatter ? p.scatter[r0 + t] : r0 + t;
    if ((unsigned)dst >= (unsigned)p.M) dst = -1;
    if (p.gamma) gm = p.gamma[r0 + t];
  }
  e.dst[t] = dst;
  e.gamma[t] = gm;
}

// Source row of logical tile row `row` (gather), or -1 when it reads zeros.
__device__ __forceinline__ int gather_row(const GArgs& p, int r0, int rows_a, int row) {
  if (row >= rows_a) return -1;
  const int src = p.gather[r0 + row];
  return (unsigned)src < (unsigned)p.a_rows ? src : -1;
}

// Find the group holding global m-tile `mt` (tiles of BM rows counted group by
// group).  Run by wave 0.  Writes {group, first row, end row} to `info`, or
// group = -1 when mt is past the last tile.
__device__ void find_tile(const int32_t* __restrict__ off, int G, int mt, int lane, int* info) {
  int base = 0;   // m-tiles before the current chunk of 64 groups
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int tiles = 0, lo = 0;
    if (g < G) {
      lo = off[g];
      tiles = (off[g + 1] - lo + BM - 1) / BM;
    }
    int incl = tiles;   // inclusive prefix sum over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int excl = incl - tiles;
    if (g < G && mt >= base + excl && mt < base + incl) {
      const int local = mt - base - excl;
      info[0] = g;
      info[1] = lo + local * BM;
      info[2] = min(lo + (local + 1) * BM, (int)off[g + 1]);
    }
    base += __shfl(incl, 63);
    if (mt < base) return;
  }
  if (lane == 0) info[0] = -1;
}

template <bool F16>
__global__ __launch_bounds__(NT, 1) void grouped_kernel(const GArgs p) {
  using GM = GMath<F16>;
  using VT = typename GM::vec;
  __shared__ Smem sm;
  __shared__ GEpi epi;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = t / p.tiles_n, nt = t - mt * p.tiles_n;
  if (wave == 0) find_tile(p.off, p.G, mt, lane, sm.tile_info);
  __syncthreads();
  const int grp = sm.tile_info[0];
  if (grp < 0) return;                      // uniform over the workgroup
  const int M = p.M, N = p.N, K = p.K;
  // Offsets are a documented precondition; clamping keeps even malformed
  // ones inside the A and C buffers.
  const int r0 = min(max(sm.tile_info[1], 0), M), r1 = min(max(sm.tile_info[2], r0), M);
  const int n0 = nt * BN;
  const int KT = (K + BK - 1) / BK;
  const int KH = K / 2, KB = K / 16;

  const int rows_a = r1 - r0, rows_w = min(N - n0, BN);
  const bool gat = p.gather != nullptr;
  // With gather the resources span all of A and rows are addressed by their
  // source index; otherwise they span the tile's rows.
  const auto ca_rsrc = make_rsrc(gat ? p.A : p.A + (int64_t)r0 * KH, (gat ? p.a_rows : rows_a) * KH);
  const auto sa_rsrc = make_rsrc(gat ? p.As : p.As + (int64_t)r0 * KB, (gat ? p.a_rows : rows_a) * KB);
  const auto w_rsrc = make_rsrc(p.W + ((int64_t)grp * N + n0) * K, rows_w * K * 2);
  fill_epi(p, r0, rows_a, tid, epi);

  // staging: A chunk (tid & 1) of rows (tid >> 1) + 128 i; A scale bytes of
  // row tid; W chunk (tid & 7) of rows (tid >> 3) + 32 i.
  const int alc = tid & 1, alr = tid >> 1;
  const int wlc = tid & 7, wlr = tid >> 3;
  int a_base[2], s_base;
  bool a_ok[2], s_ok;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int src = gat ? gather_row(p, r0, rows_a, alr + 128 * i) : alr + 128 * i;
    a_ok[i] = src >= 0;
    a_base[i] = src * KH;
  }
  {
    const int src = gat ? gather_row(p, r0, rows_a, tid) : tid;
    s_ok = src >= 0;
    s_base = src * KB;
  }
  uint4 ra[2], rw[8];
  uint32_t sa_raw[2];
  // Loads only issue here (no branches, no uses); see sstore.
  auto gload = [&](int kt) {
    const int aofs = kt * AROWB + alc * 16 < KH ? kt * AROWB + alc * 16 : OOB;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra[i] = buffer_load_x4(ca_rsrc, (aofs == OOB || !a_ok[i]) ? OOB : a_base[i] + aofs);
    // two pairs of blocks; a pair past K reads as 0
    sa_raw[0] = buffer_load_u16(sa_rsrc, s_ok ? s_base + kt * 4 : OOB);
    sa_raw[1] = buffer_load_u16(sa_rsrc, (s_ok && kt * 4 + 2 < KB) ? s_base + kt * 4 + 2 : OOB);
    const int wofs = kt * BK + wlc * 8 < K ? (kt * BK + wlc * 8) * 2 : OOB;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rw[i] = buffer_load_x4(w_rsrc, wofs == OOB ? OOB : (wlr + 32 * i) * K * 2 + wofs);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      sm.a[buf][aswz(alr + 128 * i, alc)] = ra[i];
    sm.as[buf][tid] = sa_raw[0] | (sa_raw[1] << 16);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sm.w[buf][wswz(wlr + 32 * i, wlc)] = rw[i];
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
    uint4 ca[4];
    typename GM::scales sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + r;
      ca[i] = sm.a[buf][aswz(row, g)];
      const uint32_t sw = sm.as[buf][row];
      sc[i] = GM::decode(sw >> (16 * g));
    }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      VT av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t d = sp == 0 ? ca[i].x : sp == 1 ? ca[i].y : sp == 2 ? ca[i].z : ca[i].w;
        av[i] = GM::dq8(d, sc[i], sp >> 1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + r;
        const uint4 q = sm.w[buf][wswz(row, 4 * g + sp)];
        __builtin_memcpy(&bv[j], &q, 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = GM::mfma(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  const float alpha = *p.Ats;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 128 + j * 32 + r;
    const float b = (p.bias && col < N) ? p.bias[(int64_t)grp * N + col] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = wm * 128 + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        const int dst = epi.dst[lr];
        float y = acc[i][j][v] * alpha;
        if (p.bias) y += b;
        if (p.gamma) y *= epi.gamma[lr];
        if (dst >= 0 && col < N) store_nt2(&p.C[(int64_t)dst * N + col], (uint16_t)f32_to_bf16_rne(y));
      }
  }
}

// ---------------------------------------------------------------------------
// Ring kernel (K % 64 == 0).  The same tiles and K assignment as above (tile
// order n-major, see below), but
// the operands stream HBM -> LDS by direct loads through a 3-stage ring of
// 64-element K steps (two steps in flight while one is computed), and the
// BF16 dequantisation of A runs one MFMA sub-step ahead, under the previous
// sub-step's MFMAs.  One barrier per step.
//
// Per stage: A codes [256][32] bytes (chunk swizzle (r >> 3) & 1, 2 loads per
// wave), W [256][128] bytes (chunk swizzle (r >> 1) & 7, 8 loads per wave).
// A scales come SB bytes per row at a time (SB = 16, four steps, when
// K % 256 == 0; else 4): one load per wave per SB/4 steps, into a ring of 3
// buffers, so a buffer is rewritten only after a barrier has passed since
// its last read.
constexpr int GR_NS = 3, GR_SBUF = 3;
constexpr int GR_LOADS = 2 + 8;   // code loads per wave per stage

template <int SB>
struct GRingSmem {
  uint4 a[GR_NS][BM * ARC];
  uint4 w[GR_NS][BN * WRC];
  uint32_t as[GR_SBUF][BM * SB / 4];
  int tile_info[4];
  GEpi epi;
};

// KRAG: the inner-expert (K-ragged) mode.  The groups split K instead of the
// rows: workgroup (g, m tile, n tile) runs the K slice [koff[g], koff[g+1])
// of the shared A and W and writes C[g].  Slices are multiples of 256, so
// the 16-byte-scale ring serves every group; an empty slice writes zeros.
template <int SB, bool F16, bool KRAG = false, bool IL = true>
__global__ __launch_bounds__(NT, 1) void grouped_ring_kernel(const GArgs p) {
  using GM = GMath<F16>;
  using VT = typename GM::vec;
  constexpr int U = SB / 4;                  // steps per scale load
  __shared__ GRingSmem<SB> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases in SGPRs
  const int M = p.M, N = p.N, K = p.K;
  const int KH = K / 2, KB = K / 16;
  int grp, r0, r1, nt, k0 = 0, k1 = K;
  if constexpr (KRAG) {
    // Unit u = (group, n tile): its tiles_m m-tiles run back to back on one
    // XCD and share the unit's W slice through L2.  Units go round-robin over
    // the 8 XCDs (workgroup b runs on XCD b % 8), so each XCD gets every
    // group's n-tiles in turn: with contiguous blocks of units, the XCD that
    // drew the longest K slices set the kernel time (up to 2.7x its share
    // for Dirichlet-sized experts).  XCD x starts x/8 of the way along its
    // sequence, so the XCDs do not all reach their epilogues together (equal
    // K slices: 669 -> 643 us).  The grid is padded to whole rounds of 8
    // units; padding workgroups exit here.
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int upx = (gridDim.x >> 3) / p.tiles_m;   // units per XCD
    const int u = (((i / p.tiles_m) + x * upx / 8) % upx) * 8 + x;
    if (u >= p.G * p.tiles_n) return;        // uniform over the workgroup
    grp = u / p.tiles_n;
    nt = u - grp * p.tiles_n;
    r0 = (i % p.tiles_m) * BM;
    r1 = min(r0 + BM, M);
    // offsets are a documented precondition; clamped and rounded down to
    // multiples of 256, a malformed one still stays inside A and W
    k0 = min(max(p.koff[grp], 0), K) & ~255;
    k1 = min(max(p.koff[grp + 1], k0), K) & ~255;
  } else {
    // n-tile-major order: consecutive tiles (kept on one XCD by xcd_remap)
    // are the m-tiles of one W column panel, so each group's W panel is
    // fetched from HBM about once and re-read from L2; A (small) is shared
    // through the infinity cache across panels.
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int mtiles = gridDim.x / p.tiles_n;
    nt = t / mtiles;
    const int mt = t - nt * mtiles;
    if (wave == 0) find_tile(p.off, p.G, mt, lane, sm.tile_info);
    __syncthreads();
    grp = sm.tile_info[0];
    if (grp < 0) return;                      // uniform over the workgroup
    // Offsets are a documented precondition; clamping keeps even malformed
    // ones inside the A and C buffers.
    r0 = min(max(sm.tile_info[1], 0), M);
    r1 = min(max(sm.tile_info[2], r0), M);
  }
  const int n0 = nt * BN;
  const int KT = (k1 - k0) / BK;            // a multiple of U
  const int rows_a = r1 - r0, rows_w = min(N - n0, BN);
  const bool gat = p.gather != nullptr;
  // With gather the A resources span all of A and rows are addressed by
  // their source index; otherwise they span the tile's rows.  The K slice
  // start is folded into the bases (k0 = 0 outside the K-ragged mode).
  const rsrc4_t ra = make_rsrc4(gat ? p.A : p.A + (int64_t)r0 * KH + k0 / 2, (gat ? p.a_rows : rows_a) * KH - k0 / 2);
  const rsrc4_t rsa = make_rsrc4(gat ? p.As : p.As + (int64_t)r0 * KB + k0 / 16,
                                 (gat ? p.a_rows : rows_a) * KB - k0 / 16);
  const rsrc4_t rw = make_rsrc4(p.W + (KRAG ? (int64_t)n0 * K : ((int64_t)grp * N + n0) * K) + k0,
                                rows_w * K * 2 - k0 * 2);
  // Past-the-end stages load through empty resources: every offset is then
  // out of range and reads zero.
  const rsrc4_t ra0 = make_rsrc4(p.A, 0), rsa0 = make_rsrc4(p.As, 0), rw0 = make_rsrc4(p.W, 0);
  uint16_t* const Cb = KRAG ? p.C + (int64_t)grp * M * N : p.C;
  fill_epi(p, r0, rows_a, tid, sm.epi);   // visible after the prologue's barrier

  // Load geometry.  A instruction u covers rows 32 (2 wave + u) .. +31 (two
  // lanes per row); W instruction u covers rows 8 (8 wave + u) .. +7 (eight
  // lanes per row).  Each lane fetches the global chunk that the swizzle puts
  // in its LDS slot.
  int a_off[2];
  bool a_ok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 32 * (2 * wave + u) + (lane >> 1);
    const int src = gat ? gather_row(p, r0, rows_a, row) : row;
    a_ok[u] = src >= 0;
    a_off[u] = a_ok[u] ? src * KH + (((lane & 1) ^ ((row >> 3) & 1)) * 16) : OOB;
  }
  int w_off[2];   // even and odd u differ in the swizzle; rows step by 16 per pair
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 8 * (8 * wave + u) + (lane >> 3);
    w_off[u] = row * K * 2 + (((lane & 7) ^ ((row >> 1) & 7)) * 16);
  }
  const int s_src = gat ? gather_row(p, r0, rows_a, 64 * wave + lane) : 64 * wave + lane;
  const bool s_ok = s_src >= 0;
  const int s_off = s_ok ? s_src * KB : OOB;

  // Part `part` of stage st's loads (IL spreads them over three sub-steps):
  // 0: the scales (when the stage starts a super-stage), A and W loads 0-1;
  // 1: W loads 2-4; 2: W loads 5-7.  part < 0: all of them.  Each lane's
  // offset is a loop constant (rows with no source carry the out-of-range
  // offset), the stage's K offset and the row block are the load's scalar
  // offset, and past-the-end stages use the empty resources, so issuing a
  // load costs no vector instructions.
  auto issue_part = [&](int st, int part, bool with_scales) {
    const int slot = st % GR_NS;
    const bool live = st < KT;
    if (part <= 0) {
      if (with_scales) {
        const int sbuf = (st / U) % GR_SBUF;
        const int so = (st / U) * SB;
        if (SB == 16) dma_x4_so(live ? rsa : rsa0, (uint32_t)(uintptr_t)&sm.as[sbuf][64 * wave * 4], s_off, so);
        else dma_x1_so(live ? rsa : rsa0, (uint32_t)(uintptr_t)&sm.as[sbuf][64 * wave], s_off, so);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        dma_x4_so(live ? ra : ra0, (uint32_t)(uintptr_t)&sm.a[slot][64 * (2 * wave + u)], a_off[u], st * AROWB);
    }
    const int u0 = part < 0 ? 0 : part == 0 ? 0 : part == 1 ? 2 : 5;
    const int u1 = part < 0 ? 8 : part == 0 ? 2 : part == 1 ? 5 : 8;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u >= u0 && u < u1)
        dma_x4_so(live ? rw : rw0, (uint32_t)(uintptr_t)&sm.w[slot][64 * (8 * wave + u)], w_off[u & 1],
                  (u >> 1) * 16 * K * 2 + st * WROWB);
  };
  auto issue = [&](int st, auto WITH_SCALES) { issue_part(st, -1, decltype(WITH_SCALES)::value); };

  // Wave w computes rows [64 w, 64 w + 64) x all 256 columns: 2 x 8 MFMA
  // tiles.  Each A row is then dequantised by exactly one wave (the BF16
  // expansion is the kernel's VALU cost); the W fragments, which need no
  // arithmetic, are read from LDS by all four waves.
  const int r = lane & 31, g = lane >> 5;

  struct AFrag {
    uint4 c[2];
    typename GM::scales s[2];   // the lane's two block scales per row fragment
  };
  // A codes and decoded scales of stage st for this lane's 2 row fragments.
  // The step's 4 scale bytes are dword `in` of the row's SB-byte entry; lane
  // g takes bytes 2g and 2g + 1 (its two 16-element blocks).
  auto read_a = [&](int st, auto INC, AFrag& f) {
    constexpr int in = decltype(INC)::value;
    const int slot = st % GR_NS, sbuf = (st / U) % GR_SBUF;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wave * 64 + i * 32 + r;
      f.c[i] = sm.a[slot][aswz(row, g)];
      const uint32_t word = sm.as[sbuf][row * (SB / 4) + in] >> (16 * g);
      f.s[i] = GM::decode(word);
    }
  };
  auto read_w = [&](int st, int sp, VT* bv) {
    const int slot = st % GR_NS;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 q = sm.w[slot][wswz(j * 32 + r, 4 * g + sp)];
      __builtin_memcpy(&bv[j], &q, 16);
    }
  };
  auto dequant = [&](const AFrag& f, int sp, VT* av) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t d = sp == 0 ? f.c[i].x : sp == 1 ? f.c[i].y : sp == 2 ? f.c[i].z : f.c[i].w;
      av[i] = GM::dq8(d, f.s[i], sp >> 1);
    }
  };

  v16f acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v16f{};
  auto mfmas = [&](const VT* av, const VT* bv) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = GM::mfma(bv[j], av[i], acc[i][j]);   // W first: see the epilogue
  };
  // The next sub-step's 8 W reads go out two at a time ahead of the first
  // four MFMA pairs (1-2% faster than one read per pair, the reads then
  // having the whole second half of the sub-step to land); the dequant VALU
  // is spread evenly.
  auto interleave = [] {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
    }
  };
  auto loads_of = [](int s_mod) { return GR_LOADS + (s_mod == 0 ? 1 : 0); };

  AFrag fa[2];
  VT av[2][2], bv[2][8];
  // Step kt, kt % U == IN (static); fa[CUR] holds stage kt's A data, and
  // av[0] / bv[0] its sub-step 0 operands.
  auto step = [&](int kt, auto INC) {
    constexpr int IN = decltype(INC)::value;
    constexpr int CUR = IN & 1;
    constexpr int AFTER = loads_of((IN + 2) % U);   // stage kt+2 stays in flight
    constexpr bool WS = ((IN + 2) % U) == 0;
    // IL: stage kt+2's loads over the first three sub-steps (one burst at
    // the head of the step holds up the wave's MFMA issue)
    issue_part(kt + 2, IL ? 0 : -1, WS);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(av[0], bv[0]);
    read_w(kt, 1, bv[1]);
    dequant(fa[CUR], 1, av[1]);
    interleave();
    if constexpr (IL) {
      issue_part(kt + 2, 1, WS);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfmas(av[1], bv[1]);
    read_w(kt, 2, bv[0]);
    dequant(fa[CUR], 2, av[0]);
    interleave();
    if constexpr (IL) {
      issue_part(kt + 2, 2, WS);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfmas(av[0], bv[0]);
    read_w(kt, 3, bv[1]);
    dequant(fa[CUR], 3, av[1]);
    interleave();
    wait_vm_barrier<AFTER>();         // stage kt+1 landed
    read_a(kt + 1, std::integral_constant<int, (IN + 1) % U>{}, fa[CUR ^ 1]);
    mfmas(av[1], bv[1]);
    read_w(kt + 1, 0, bv[0]);
    dequant(fa[CUR ^ 1], 0, av[0]);
    interleave();
  };

  issue(0, std::true_type{});
  issue(1, std::integral_constant<bool, (1 % U) == 0>{});
  wait_vm_barrier<loads_of(1 % U)>();
  read_a(0, std::integral_constant<int, 0>{}, fa[0]);
  read_w(0, 0, bv[0]);
  dequant(fa[0], 0, av[0]);
  // U is 1 or 4; the body below covers 2 steps when U == 1 so that the fa
  // double buffer index stays static.
  if constexpr (U == 1) {
    for (int kt = 0; kt < KT; kt += 2) {
      step(kt, std::integral_constant<int, 0>{});
      // second step of the pair: same code with the buffers swapped
      constexpr int IN = 1;
      issue_part(kt + 3, IL ? 0 : -1, true);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(av[0], bv[0]);
      read_w(kt + 1, 1, bv[1]);
      dequant(fa[1], 1, av[1]);
      interleave();
      if constexpr (IL) {
        issue_part(kt + 3, 1, true);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfmas(av[1], bv[1]);
      read_w(kt + 1, 2, bv[0]);
      dequant(fa[1], 2, av[0]);
      interleave();
      if constexpr (IL) {
        issue_part(kt + 3, 2, true);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfmas(av[0], bv[0]);
      read_w(kt + 1, 3, bv[1]);
      dequant(fa[1], 3, av[1]);
      interleave();
      wait_vm_barrier<loads_of(0)>();
      read_a(kt + 2, std::integral_constant<int, 0>{}, fa[0]);
      mfmas(av[1], bv[1]);
      read_w(kt + 2, 0, bv[0]);
      dequant(fa[0], 0, av[0]);
      interleave();
      (void)IN;
    }
  } else {
    for (int kt = 0; kt < KT; kt += U) {
      static_for<0, U>([&](auto IC) { step(kt + decltype(IC)::value, IC); });
    }
  }

  // Epilogue: C rows r0..r1 of this group (row table in LDS: ragged edge,
  // scatter), y = (s_t * acc + bias) * gamma rounded once to BF16.  With W
  // as the MFMA's first operand, lane (r, g) holds tile row 64 wave + 32 i + r
  // and, for q = v / 4, the four consecutive columns 32 j + 8 q + 4 g + 0..3.
  // Each wave passes its 64 x 256 block through a private 16 KB of the ring's
  // LDS in two halves of 128 columns: the lanes write their 4-column pieces
  // as BF16, then read back 16-byte row chunks and store whole 256-byte row
  // segments.  Storing from the MFMA layout directly takes one 2-byte store
  // per element: 784 us against 744 us for the 32-expert K-ragged problem.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the out-of-range tail loads
  __syncthreads();                                   // every wave is done with the ring
  const float alpha = *p.Ats;
  uint4* const eb = &sm.w[0][0] + wave * (64 * 16);  // 64 rows x 16 chunks of 16 bytes
  const bool vec_ok = (N & 7) == 0;                  // 16-byte aligned row chunks
  // Phase 1 of half h: the wave's values as BF16 into its LDS rows; the
  // variants are decided once per launch, outside the element loops.
  auto to_lds = [&](int h, auto BIAS, auto GAMMA) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 32 * i + r;                    // wave-local row
      const float gm = decltype(GAMMA)::value ? sm.epi.gamma[64 * wave + row] : 1.0f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * h + jj;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[e] = acc[i][j][4 * q + e] * alpha;
            if constexpr (decltype(BIAS)::value) {
              const int col = n0 + 32 * j + 8 * q + 4 * g + e;
              y[e] += col < N ? p.bias[(int64_t)grp * N + col] : 0.0f;
            }
            if constexpr (decltype(GAMMA)::value) y[e] *= gm;
          }
          const int chunk = 4 * jj + q;
          uint2* dstp = reinterpret_cast<uint2*>(eb + row * 16 + (chunk ^ (row & 15))) + g;
          *dstp = make_uint2(cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3]));
        }
      }
    }
  };
  const bool has_bias = !KRAG && p.bias, has_gamma = !KRAG && p.gamma;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (has_bias && has_gamma) to_lds(h, std::true_type{}, std::true_type{});
    else if (has_bias) to_lds(h, std::true_type{}, std::false_type{});
    else if (has_gamma) to_lds(h, std::false_type{}, std::true_type{});
    else to_lds(h, std::false_type{}, std::false_type{});
    // All 16 row chunks and destination rows of the half are read before the
    // first store, so the LDS latency is paid once, not once per store.
    const int cbase = n0 + 128 * h + 8 * (lane & 15);
    uint4 vals[16];
    int dsts[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int row = 4 * t + (lane >> 4);
      const int c = lane & 15;
      vals[t] = eb[row * 16 + (c ^ (row & 15))];
      dsts[t] = sm.epi.dst[64 * wave + row];
    }
    if (cbase < N) {
      if (vec_ok) {
#pragma unroll
        for (int t = 0; t < 16; ++t)
          if (dsts[t] >= 0) store_nt16(Cb + (int64_t)dsts[t] * N + cbase, vals[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          if (dsts[t] < 0) continue;
          uint16_t* cp = Cb + (int64_t)dsts[t] * N + cbase;
          const uint32_t wd[4] = {vals[t].x, vals[t].y, vals[t].z, vals[t].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (cbase + e < N) cp[e] = (uint16_t)(wd[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// Ping-pong form of the ring kernel for K % 256 == 0: eight waves, two per
// SIMD (waves w and w + 4 share SIMD w % 4 under the round-robin placement),
// in two groups that take turns.  While group 0 runs the MFMAs of step k,
// group 1 reads stage k's A codes, scales and W fragments from LDS and
// expands A; then the roles swap.  The matrix core of each SIMD is fed from
// one wave while the other wave's LDS and VALU work overlaps it.
//
// Wave (pg, wq) computes rows [64 wq, 64 wq + 64) x columns
// [128 pg, 128 pg + 128): 2 x 4 MFMA tiles, 128 accumulator registers.  The
// MFMAs run in the same K order as in the ring kernel, so the two give
// identical results.
//
// Ring: 3 stages, loads two stages ahead.  B_a(k) is the barrier at which
// group 0 enters the MFMA phase of step k, B_b(k) the one at which group 1
// does.  Each group issues the loads of stage k + 2 at the start of its
// MFMA phase of step k (after B_a(k), resp. B_b(k)); every read of stage
// k - 1, whose slot they overwrite, ends by B_a(k).  That leaves the MFMA
// phase free to read W fragments of the current stage too.
struct GPPSmem {
  uint4 a[GR_NS][BM * ARC];
  uint4 w[GR_NS][BN * WRC];
  uint32_t as[GR_SBUF][BM * 4];
  int tile_info[4];
  GEpi epi;
};

// Tiles of the ping-pong kernel.  Group g's c rows take c / 256 full
// 256-row tiles; a remainder of more than 128 rows takes one more 256-row
// tile, a remainder of 1..128 rows one 128-row tile.  Padding stays under 128
// rows per group, and the 128-row tiles, dispatched after the 256-row ones,
// shorten the last round.
// A 512 x 128 tile (eight waves of 64 distinct rows, so each A row expanded
// once; 32 KB staged a step instead of 40; a 4-stage ring) was measured no
// faster per tile: 8 groups of 2048 rows, K = 7168, N = 2048, exactly two
// rounds of tiles: 428 us against 419 us for the 256 x 256 tile.
__device__ __forceinline__ int pp_big_tiles(int c) { return (c >> 8) + ((c & 255) > 128 ? 1 : 0); }
__device__ __forceinline__ int pp_small_tiles(int c) { return ((c & 255) != 0 && (c & 255) <= 128) ? 1 : 0; }

// find_tile for the ping-pong kernel's two tile sizes: tile `mt` among the
// 256-row tiles (SMALL false) or among the 128-row tiles (SMALL true), counted
// group by group.  Run by wave 0; writes {group, first row, end row} to
// `info`, or group = -1 when mt is past the last tile of that size.
template <bool SMALL>
__device__ void find_tile_pp(const int32_t* __restrict__ off, int G, int mt, int lane, int* info) {
  int base = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int tiles = 0, lo = 0, hi = 0, c = 0;
    if (g < G) {
      lo = off[g];
      hi = off[g + 1];
      c = max(hi - lo, 0);
      tiles = SMALL ? pp_small_tiles(c) : pp_big_tiles(c);
    }
    int incl = tiles;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int excl = incl - tiles;
    if (g < G && mt >= base + excl && mt < base + incl) {
      const int local = mt - base - excl;
      info[0] = g;
      if (SMALL) {
        info[1] = lo + (c & ~255);
        info[2] = hi;
      } else {
        info[1] = lo + local * 256;
        info[2] = lo + min((local + 1) * 256, c);
      }
    }
    base += __shfl(incl, 63);
    if (mt < base) return;
  }
  if (lane == 0) info[0] = -1;
}

// One tile of the ping-pong kernel.  MI = 2: 256 rows, wave (pg, wq) owns
// rows [64 wq, 64 wq + 64); MI = 1: 128 rows, wave (pg, wq) owns rows
// [32 wq, 32 wq + 32).  Either way its columns are [128 pg, 128 pg + 128).
// The loads are those of the 256-row tile in both cases: for a 128-row tile
// rows 128..255 lie past rows_a and land in LDS as zeros without touching
// memory.
__shared__ GPPSmem pp_sm;

template <bool F16, int MI>
__device__ __forceinline__ void pp_tile(const GArgs& p, int grp, int r0, int r1, int nt) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  using GM = GMath<F16>;
  using VT = typename GM::vec;
  constexpr int U = 4;                       // steps per 16-byte scale load
  constexpr int TM = 128 * MI;               // tile rows
  const int pg = wave >> 2, wq = wave & 3;
  const int N = p.N, K = p.K;
  const int KH = K / 2, KB = K / 16;
  const int n0 = nt * BN;
  const int KT = K / BK;                      // a multiple of U
  const int rows_a = r1 - r0, rows_w = min(N - n0, BN);
  const bool gat = p.gather != nullptr;
  const rsrc4_t ra = make_rsrc4(gat ? p.A : p.A + (int64_t)r0 * KH, (gat ? p.a_rows : rows_a) * KH);
  const rsrc4_t rsa = make_rsrc4(gat ? p.As : p.As + (int64_t)r0 * KB, (gat ? p.a_rows : rows_a) * KB);
  const rsrc4_t rw = make_rsrc4(p.W + ((int64_t)grp * N + n0) * K, rows_w * K * 2);
  // Past-the-end stages load through empty resources: every offset is then
  // out of range and reads zero.
  const rsrc4_t ra0 = make_rsrc4(p.A, 0), rsa0 = make_rsrc4(p.As, 0), rw0 = make_rsrc4(p.W, 0);
  fill_epi(p, r0, rows_a, tid, pp_sm.epi);   // visible after the prologue's barrier

  // Load geometry.  Wave w's A load covers rows 32 w .. +31 (two lanes per
  // row); its W load u (0..3) covers rows 8 (4 w + u) .. +7 (eight lanes per
  // row); group 0's waves also load the scales of rows 64 wq .. +63.
  const int arow = 32 * wave + (lane >> 1);
  const int asrc = gat ? gather_row(p, r0, rows_a, arow) : arow;
  // Lane offsets are loop constants (rows with no source carry the
  // out-of-range offset); the stage's K offset and the row block are the
  // load's scalar offset; past-the-end stages use the empty resources.
  const int a_off = asrc >= 0 ? asrc * KH + (((lane & 1) ^ ((arow >> 3) & 1)) * 16) : OOB;
  int w_off[2];   // loads u and u + 2 differ by 16 rows and share the swizzle
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 8 * (4 * wave + u) + (lane >> 3);
    w_off[u] = row * K * 2 + (((lane & 7) ^ ((row >> 1) & 7)) * 16);
  }
  const int s_src = gat ? gather_row(p, r0, rows_a, 64 * wq + lane) : 64 * wq + lane;
  const int s_off = s_src >= 0 ? s_src * KB : OOB;

  auto issue = [&](int st, auto PG, auto WITH_SCALES) {
    const int slot = st % GR_NS;
    const bool live = st < KT;
    if constexpr (decltype(PG)::value == 0 && decltype(WITH_SCALES)::value) {
      const int sbuf = (st / U) % GR_SBUF;
      dma_x4_so(live ? rsa : rsa0, (uint32_t)(uintptr_t)&pp_sm.as[sbuf][64 * wq * 4], s_off, (st / U) * 16);
    }
    dma_x4_so(live ? ra : ra0, (uint32_t)(uintptr_t)&pp_sm.a[slot][64 * wave], a_off, st * AROWB);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      dma_x4_so(live ? rw : rw0, (uint32_t)(uintptr_t)&pp_sm.w[slot][64 * (4 * wave + u)], w_off[u & 1],
                (u >> 1) * 16 * K * 2 + st * WROWB);
  };
  // loads per wave for stage st (st % U == s_mod): the scale load joins
  // group 0's A and W loads at the start of each 4-step scale batch
  auto loads_of = [](int pg_, int s_mod) { return 5 + ((pg_ == 0 && s_mod == 0) ? 1 : 0); };

  const int r = lane & 31, g = lane >> 5;
  VT av[4][MI];
  // This wave's MI A row fragments of stage st (st % U == IN), expanded for
  // all four K16 sub-steps.  Sub-step sp pairs lane half g with K
  // 32 g + 8 sp .. + 7, whose scale is byte 2 g + sp / 2 of the row's 4 scale
  // bytes for the step.
  auto read_a = [&](int st, auto INC) {
    constexpr int IN = decltype(INC)::value;
    const int slot = st % GR_NS, sbuf = (st / U) % GR_SBUF;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = wq * 32 * MI + i * 32 + r;
      const uint4 c = pp_sm.a[slot][aswz(row, g)];
      const uint32_t word = pp_sm.as[sbuf][row * 4 + IN] >> (16 * g);
      const typename GM::scales sv = GM::decode(word);
      av[0][i] = GM::dq8(c.x, sv, 0);
      av[1][i] = GM::dq8(c.y, sv, 0);
      av[2][i] = GM::dq8(c.z, sv, 1);
      av[3][i] = GM::dq8(c.w, sv, 1);
    }
  };
  // This wave's 4 W fragments of sub-step sp of stage st.
  auto read_w = [&](int st, int sp, VT* bv) {
    const int slot = st % GR_NS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 q = pp_sm.w[slot][wswz(pg * 128 + j * 32 + r, 4 * g + sp)];
      __builtin_memcpy(&bv[j], &q, 16);
    }
  };

  v16f acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  auto mfmas = [&](const VT* a, const VT* b) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = GM::mfma(a[i], b[j], acc[i][j]);
  };

  VT bv0[4], bv1[4], bv2[4], bv3[4];
  // Memory phase of step k: A expanded for the whole step, W of sub-steps 0-1.
  auto mem_phase = [&](int k, auto INC) {
    read_a(k, INC);
    read_w(k, 0, bv0);
    read_w(k, 1, bv1);
  };
  // MFMA phase of step k: the loads of stage k + 2, then the MFMAs, with the
  // W fragments of sub-steps 2-3 read under those of sub-steps 0-1.
  auto mfma_phase = [&](int k, auto PG, auto WS) {
    issue(k + 2, PG, WS);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(av[0], bv0);
    read_w(k, 2, bv2);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(av[1], bv1);
    read_w(k, 3, bv3);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(av[2], bv2);
    mfmas(av[3], bv3);
  };

  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  // Prologue: stages 0 and 1; stage 0 complete everywhere before the first read.
  if (pg == 0) {
    issue(0, Z{}, std::true_type{});
    issue(1, Z{}, std::false_type{});
    wait_vm_barrier<loads_of(0, 1)>();
  } else {
    issue(0, O{}, std::true_type{});
    issue(1, O{}, std::false_type{});
    wait_vm_barrier<loads_of(1, 1)>();
  }
  // Group 0: [mem k] B_a(k) [MFMA k] B_b(k).
  // Group 1: B_a(0), then [mem k] B_b(k) [MFMA k] B_a(k+1).
  // At B_b(k) every wave's stage k + 1 loads have landed (group 0 may still
  // have stage k + 2 in flight; group 1 issues it after B_b(k)), so group 0's
  // reads of stage k + 1 after B_b(k), and group 1's after B_a(k + 1), see
  // the whole stage.
  if (pg == 0) {
    for (int kt = 0; kt < KT; kt += U) {
      static_for<0, U>([&](auto IC) {
        constexpr int IN = decltype(IC)::value;
        const int k = kt + IN;
        mem_phase(k, IC);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        mfma_phase(k, Z{}, std::integral_constant<bool, ((IN + 2) % U) == 0>{});
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_barrier<loads_of(0, (IN + 2) % U)>();
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    asm volatile("s_barrier" ::: "memory");
  } else {
    asm volatile("s_barrier" ::: "memory");
    for (int kt = 0; kt < KT; kt += U) {
      static_for<0, U>([&](auto IC) {
        constexpr int IN = decltype(IC)::value;
        const int k = kt + IN;
        mem_phase(k, IC);
        wait_vm_barrier<0>();
        __builtin_amdgcn_sched_barrier(0);
        mfma_phase(k, O{}, std::integral_constant<bool, ((IN + 2) % U) == 0>{});
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the out-of-range tail loads

  // Epilogue as in the ring kernel, for this wave's (32 MI) x 128 block.
  const float alpha = *p.Ats;
  const bool plain = !p.bias && !p.gamma && !p.scatter;
  const int cn0 = n0 + pg * 128;
  const int wr0 = wq * 32 * MI;               // the wave's first tile row
  if (plain && r0 + TM <= r1 && n0 + BN <= N) {
    uint16_t* cw = p.C + (int64_t)(r0 + wr0 + g * 4) * N + cn0 + r;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          store_nt2(&cw[(int64_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * N + j * 32],
                    (uint16_t)f32_to_bf16_rne(acc[i][j][v] * alpha));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = cn0 + j * 32 + r;
      const float b = (p.bias && col < N) ? p.bias[(int64_t)grp * N + col] : 0.0f;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = wr0 + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
          const int dst = pp_sm.epi.dst[lr];
          float y = acc[i][j][v] * alpha;
          if (p.bias) y += b;
          if (p.gamma) y *= pp_sm.epi.gamma[lr];
          if (dst >= 0 && col < N) store_nt2(&p.C[(int64_t)dst * N + col], (uint16_t)f32_to_bf16_rne(y));
        }
    }
  }
}

// Grid: tiles_n n-tiles x (mbig 256-row slots, then min(G, M) 128-row slots),
// n-major after xcd_remap, so each XCD takes a contiguous run of slots: the
// 256-row tiles of an n-tile column first, then its 128-row tiles.  Slots
// past the real tile count exit at once.
template <bool F16>
__global__ __launch_bounds__(512, 1) void grouped_pp_kernel(const GArgs p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int mslots = gridDim.x / p.tiles_n;
  const int nt = t / mslots;
  const int slot = t - nt * mslots;
  const bool small = slot >= p.mbig;
  if (wave == 0) {
    if (small) find_tile_pp<true>(p.off, p.G, slot - p.mbig, lane, pp_sm.tile_info);
    else find_tile_pp<false>(p.off, p.G, slot, lane, pp_sm.tile_info);
  }
  __syncthreads();
  const int grp = pp_sm.tile_info[0];
  if (grp < 0) return;                        // uniform over the workgroup
  // Offsets are a documented precondition; clamping keeps even malformed
  // ones inside the A and C buffers, and a tile within its row count.
  const int r0 = min(max(pp_sm.tile_info[1], 0), p.M);
  const int r1 = min(max(pp_sm.tile_info[2], r0), min(p.M, r0 + (small ? 128 : 256)));
  if (small) pp_tile<F16, 1>(p, grp, r0, r1, nt);
  else pp_tile<F16, 2>(p, grp, r0, r1, nt);
}

}  // namespace

hipError_t launch_grouped_kragged(const KRaggedCall& c, hipStream_t stream) {
  GArgs p{};
  p.A = c.a; p.As = c.as; p.Ats = c.ats; p.W = c.w; p.C = c.c; p.koff = c.k_offsets;
  p.G = c.num_groups; p.M = (int)c.m; p.a_rows = (int)c.m; p.N = (int)c.n; p.K = (int)c.k;
  p.tiles_n = (int)ceil_div(c.n, BN);
  p.tiles_m = (int)ceil_div(c.m, BM);
  const int64_t units = (int64_t)c.num_groups * p.tiles_n;   // padded to whole rounds of 8 (one per XCD)
  const dim3 grid((unsigned)(ceil_div(units, 8) * 8 * p.tiles_m));
  if (c.w_f16)
    hipLaunchKernelGGL((grouped_ring_kernel<16, true, true>), grid, dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((grouped_ring_kernel<16, false, true>), grid, dim3(NT), 0, stream, p);
  return hipGetLastError();
}

// 256-row tile slots of the ping-pong kernel: sum_g big_tiles(c_g) <=
// sum_g (c_g + 127) / 256 <= (m_total + 127 G) / 256.
static int64_t pp_big_slots(int64_t m_total, int num_groups) { return (m_total + 127 * (int64_t)num_groups) / 256; }

// 128-row tile slots: at most one per non-empty group.
static int64_t pp_small_slots(int64_t m_total, int num_groups) { return std::min<int64_t>(num_groups, m_total); }

int64_t grouped_grid_blocks(int num_groups, int64_t m_total, int64_t n, int64_t k) {
  const int64_t tiles_n = ceil_div(n, BN);
  if (k % 256 == 0 && k > 0) return (pp_big_slots(m_total, num_groups) + pp_small_slots(m_total, num_groups)) * tiles_n;
  return (m_total / BM + num_groups) * tiles_n;   // >= sum_g ceil(c_g / BM)
}

hipError_t launch_grouped(const GroupedCall& c, hipStream_t stream) {
  GArgs p{};
  p.A = c.a; p.As = c.as; p.Ats = c.ats; p.off = c.offsets; p.W = c.w; p.C = c.c;
  p.bias = c.bias; p.gamma = c.gamma; p.gather = c.gather; p.scatter = c.scatter;
  p.G = c.num_groups; p.M = (int)c.m_total; p.a_rows = (int)c.a_rows; p.N = (int)c.n; p.K = (int)c.k;
  p.tiles_n = (int)ceil_div(c.n, BN);
  p.mbig = (int)pp_big_slots(c.m_total, c.num_groups);
  const dim3 grid((unsigned)grouped_grid_blocks(c.num_groups, c.m_total, c.n, c.k));
  const int64_t k = c.k;
  if (c.w_f16) {
    if (k % 256 == 0 && k > 0)
      hipLaunchKernelGGL((grouped_pp_kernel<true>), grid, dim3(512), 0, stream, p);
    else if (k % 64 == 0 && k > 0)
      hipLaunchKernelGGL((grouped_ring_kernel<4, true>), grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL(grouped_kernel<true>, grid, dim3(NT), 0, stream, p);
  } else {
    if (k % 256 == 0 && k > 0)
      hipLaunchKernelGGL((grouped_pp_kernel<false>), grid, dim3(512), 0, stream, p);
    else if (k % 64 == 0 && k > 0)
      hipLaunchKernelGGL((grouped_ring_kernel<4, false>), grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL(grouped_kernel<false>, grid, dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace bsg
