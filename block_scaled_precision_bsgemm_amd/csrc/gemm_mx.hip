// MX-format GEMMs (MXFP8 x MXFP8 and MXFP4 x MXFP4) on the gfx950 scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Both block formats (E4M3 or E2M1 values, one E8M0 scale per 32 K-elements)
// are ones this MFMA consumes natively.  Each lane supplies one E8M0 byte for
// its row and its 32-element K block, so no dequantisation happens anywhere.
// Prior art: "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera
// Rubin NVL72", section "Building the GEMM".  That page stages FP8 E4M3
// operands through a multi-stage shared-memory ring and sweeps its depth.
//
// Both kernels are templated on the element format.  Everything is counted in
// bytes of a code row: one byte holds one E4M3 element or two E2M1 elements,
// so a 16-byte chunk is 16 (FP8) or 32 (FP4) K-elements.
//
// Layout of one workgroup (256 threads, 4 waves):
//   - Output tile 256 x 256; each wave owns 128 x 128 (4 x 4 MFMA tiles of
//     32 x 32).
//   - Operand register layout of the 32x32x64 MFMA, checked on the device
//     against the oracle: lane (r = l % 32, g = l / 32) holds row r, and its
//     scale byte applies to the MFMA's 32-element K block g.
//       FP8: dwords 0-3 = K [16g, 16g+16) of block 0, dwords 4-7 = K
//            [32+16g, 32+16g+16) of block 1 (two 16-byte chunks);
//       FP4: dwords 0-3 = K [32g, 32g+32), element 2j in the low nibble of
//            byte j (one 16-byte chunk, block g whole).
//     So an FP8 MFMA over code bytes [64s, 64s+64) takes chunks 4s+g and
//     4s+2+g, and an FP4 MFMA over bytes [32s, 32s+32) takes chunk 2s+g.
//     Either way the lane's scale is that of block 2s+g.
//   - Output lane layout: lane l holds column l % 32, rows
//     8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

constexpr int BM = 256, BN = 256, BK = 128, NT = 256;   // BK: code bytes per row per step
constexpr int GROUP_M = 8;   // tile rows per rasterisation group

// K-elements per code byte.
template <bool FP4>
constexpr int per_byte() { return FP4 ? 2 : 1; }

// Tiles are uint4 arrays: the compiler then knows every access is 16-byte
// aligned and emits single ds_read_b128 / ds_write_b128 instructions.
constexpr int RC = BK / 16;   // 16-byte chunks per row
template <bool FP4>
struct Smem {
  static constexpr int SW = per_byte<FP4>();   // scale dwords per row per step
  uint4 a[2][BM * RC];
  uint4 b[2][BN * RC];
  uint32_t as[2][BM * SW];
  uint32_t bs[2][BN * SW];
};

// 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7): any 16
// consecutive rows reading one chunk then cover all 16 bank groups of
// 16 bytes (two 128-byte rows per 256 bytes of banks).
__device__ __forceinline__ int swz(int row, int chunk) { return row * RC + (chunk ^ ((row >> 1) & 7)); }

// Map a linear tile index to (tile_m, tile_n): groups of GROUP_M tile rows
// are walked column by column, so consecutive tiles share B columns and the
// group's A rows.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in = t - group * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// Operand of one MFMA from a lane's fragment registers (lo = the first
// 16-byte chunk, hi = the second): FP8 takes both, FP4 one.  The compiler
// narrows an FP4 operand to its 4 used registers.
__device__ __forceinline__ v8i frag8(const uint4& lo, const uint4& hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
__device__ __forceinline__ v8i frag4(const uint4& c) {
  return v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
}

// FP4 is the E2M1 source format (4) of the MFMA's cbsz/blgp fields, FP8 the
// E4M3 one (0).
template <bool FP4>
constexpr int mfma_fmt() { return FP4 ? 4 : 0; }

// General kernel (any K % 32 == 0): operands go HBM -> registers -> LDS,
// double-buffered, 128 code bytes per row per step; scales come byte by byte
// so blocks past K read as 0.
template <bool FP4>
__global__ __launch_bounds__(NT, 1) void mx_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  constexpr int SPS = 4 * per_byte<FP4>();   // scale bytes per row per step
  constexpr int SW = SPS / 4;                // ... in dwords
  __shared__ Smem<FP4> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KP = K / per_byte<FP4>();   // code bytes per row
  const int KT = (KP + BK - 1) / BK;
  const int KB = K / 32;

  // ---- global -> register staging: thread owns chunk (tid & 7) of rows
  //      (tid >> 3) + 32 i, i = 0..7, and the SPS scale bytes of row tid.
  const int lc = tid & 7, lr = tid >> 3;
  uint4 ra[8], rb[8];
  // Per-tile buffer resources: loads past the tile's last valid row return 0.
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const auto ra_rsrc = make_rsrc(A + (int64_t)m0 * KP, rows_a * KP);
  const auto rb_rsrc = make_rsrc(B + (int64_t)n0 * KP, rows_b * KP);
  const auto sa_rsrc = make_rsrc(As + (int64_t)m0 * KB, rows_a * KB);
  const auto sb_rsrc = make_rsrc(Bs + (int64_t)n0 * KB, rows_b * KB);
  const int off0 = lr * KP + lc * 16;

  // Loads only issue here; the scale bytes are assembled in sstore, after the
  // MFMAs of the current step, so nothing waits on them early.
  uint32_t sa_raw[SPS], sb_raw[SPS];
  auto gload = [&](int kt) {
    const int kc = kt * BK + lc * 16;
    const int kofs = kc < KP ? kt * BK : OOB;   // KP % 16 == 0: chunks are wholly in or out
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = kofs == OOB ? OOB : off0 + 32 * i * KP + kofs;
      ra[i] = buffer_load_x4(ra_rsrc, off);
      rb[i] = buffer_load_x4(rb_rsrc, off);
    }
    // one offset register; bytes of blocks past K are zeroed in sstore
    const int sbase = tid * KB + kt * SPS;
#pragma unroll
    for (int j = 0; j < SPS; ++j) {
      sa_raw[j] = buffer_load_u8(sa_rsrc, sbase + j);
      sb_raw[j] = buffer_load_u8(sb_rsrc, sbase + j);
    }
  };
  // Scale bytes of blocks past K (read from the next row, or as 0 past the
  // tile) become 0, like their codes: 2^-127 * 0 contributes nothing.
  auto sstore = [&](int buf, int kt) {
#pragma unroll
    for (int j = 0; j < SPS; ++j) {
      if (kt * SPS + j >= KB) { sa_raw[j] = 0u; sb_raw[j] = 0u; }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = lr + 32 * i;
      sm.a[buf][swz(row, lc)] = ra[i];
      sm.b[buf][swz(row, lc)] = rb[i];
    }
#pragma unroll
    for (int w = 0; w < SW; ++w) {
      const uint32_t* x = sa_raw + 4 * w;
      const uint32_t* y = sb_raw + 4 * w;
      sm.as[buf][tid * SW + w] = x[0] | (x[1] << 8) | (x[2] << 16) | (x[3] << 24);
      sm.bs[buf][tid * SW + w] = y[0] | (y[1] << 8) | (y[2] << 16) | (y[3] << 24);
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
    sstore(0, 0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    // sub-step s: one MFMA per tile over 64 K-elements, scale byte 2s + g
#pragma unroll
    for (int s = 0; s < SPS / 2; ++s) {
      v8i af[4], bf[4];
      int sa[4], sb[4];
      const int sbyte = 2 * s + g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r;
        af[i] = FP4 ? frag4(sm.a[buf][swz(row, 2 * s + g)])
                    : frag8(sm.a[buf][swz(row, 4 * s + g)], sm.a[buf][swz(row, 4 * s + 2 + g)]);
        sa[i] = (int)((sm.as[buf][row * SW + sbyte / 4] >> (8 * (sbyte % 4))) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + r;
        bf[j] = FP4 ? frag4(sm.b[buf][swz(row, 2 * s + g)])
                    : frag8(sm.b[buf][swz(row, 4 * s + g)], sm.b[buf][swz(row, 4 * s + 2 + g)]);
        sb[j] = (int)((sm.bs[buf][row * SW + sbyte / 4] >> (8 * (sbyte % 4))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], bf[j], acc[i][j], mfma_fmt<FP4>(), mfma_fmt<FP4>(), 0, sa[i], 0, sb[j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1, kt + 1);
    __syncthreads();
  }

  // ---- epilogue: FP32 -> BF16 (RNE), masked stores
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        if (row < M && col < N) C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
      }
    }
}


// ---------------------------------------------------------------------------
// Ring kernel (K % 128 == 0; launched for K % 512 != 0, where the pair ring
// below does not apply): the operands stream HBM -> LDS by direct loads
// through a 4-stage ring of 64-code-byte K steps (64 K-elements of FP8, 128
// of FP4), so three steps are in flight while one is computed.  The pages'
// FP8 GEMM got its gains from the same lever: ring depth.
//
// Codes, per stage and operand: [256][64] bytes, 16-byte chunk c of row r at
// c ^ ((r >> 2) & 3) (conflict-free reads).  Each wave issues 8 code loads
// per stage (4 A, 4 B; 1 KiB = 16 rows each).
//
// Scales are loaded in batches.  With one lane per row, a scale load touches
// 64 cache lines for a few bytes each, and the address path costs about one
// clock per line.  Per-stage 4-byte scale loads cost as much as all the code
// loads.  So one load brings SB bytes per row: the scales of U K steps (SB =
// 16 when K % 512 == 0, else 4; a stage takes 2 scale bytes per row for FP8,
// 4 for FP4).  That is one load per operand per wave every U stages, into a
// ring of per-super-stage buffers.
//
// Per stage each wave runs 16 MFMA issues' worth of work: its 4 x 4 tiles,
// one K64 FP8 MFMA or two K64 FP4 MFMAs each (an FP4 MFMA takes half the
// cycles of an FP8 one, so a stage costs the same matrix-core time in both
// formats).  The stage's fragments were read into registers during the second
// half of the previous stage.  Halfway through the MFMAs the wave waits for
// the next stage's loads, crosses the barrier and reads the next fragments,
// overlapping the remaining MFMAs.  The K loop is unrolled by one
// super-stage, so every step's load count and wait count are static.
constexpr int RB_K = 64, RB_NS = 4, RB_ROW = RB_K / 16;   // code bytes per stage row; 4 chunks per row
constexpr int RB_CODE_LOADS = 8;                           // code loads per wave per stage

// Scale buffers per super-stage of U stages.  Stage st + 3 is issued at the
// head of step st; the buffer it overwrites must have had its last read
// (made in the step before the stage it serves, after that step's barrier)
// before a barrier that precedes step st.
template <int U>
constexpr int ring_scale_bufs() { return U >= 4 ? 2 : (U >= 2 ? 3 : 4); }

template <int SB, bool FP4>
struct RingSmem {
  static constexpr int U = SB / (2 * per_byte<FP4>());
  uint4 a[RB_NS][BM * RB_ROW];
  uint4 b[RB_NS][BN * RB_ROW];
  uint32_t as[ring_scale_bufs<U>()][BM * SB / 4];   // [super-stage buffer][row][SB bytes]
  uint32_t bs[ring_scale_bufs<U>()][BN * SB / 4];
};

__device__ __forceinline__ int rswz(int row, int chunk) { return row * RB_ROW + (chunk ^ ((row >> 2) & 3)); }

// One stage's fragments, from chunks g and 2 + g of the lane's rows: one
// 8-dword MFMA operand per tile (FP8), or two 4-dword ones (FP4, lo and hi).
template <bool FP4> struct Frags;
template <> struct Frags<false> {
  v8i a[4], b[4];
  int sa[4], sb[4];
};
template <> struct Frags<true> {
  uint4 alo[4], ahi[4], blo[4], bhi[4];
  int sa[4], sb[4];
};

template <int SB, bool FP4, int IL = 2>
__global__ __launch_bounds__(NT, 1) void mx_gemm_ring_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  using Sm = RingSmem<SB, FP4>;
  constexpr int U = Sm::U;                        // stages per scale super-stage
  constexpr int NSB = ring_scale_bufs<U>();
  __shared__ Sm sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases in SGPRs
  int tm, tn;
  if (tiles_m % 16 == 0 && tiles_n % 16 == 0)
    supertile_order(blockIdx.x, tiles_n, tm, tn);
  else
    raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KP = K / per_byte<FP4>();   // code bytes per row
  const int KT = KP / RB_K;             // a positive multiple of U
  const int KB = K / 32;
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const rsrc4_t ra = make_rsrc4(A + (int64_t)m0 * KP, rows_a * KP);
  const rsrc4_t rb = make_rsrc4(B + (int64_t)n0 * KP, rows_b * KP);
  const rsrc4_t rsa = make_rsrc4(As + (int64_t)m0 * KB, rows_a * KB);
  const rsrc4_t rsb = make_rsrc4(Bs + (int64_t)n0 * KB, rows_b * KB);
  // Past-the-end stages load through empty resources: every offset is then
  // out of range and reads zero.
  const rsrc4_t ra0 = make_rsrc4(A, 0), rb0 = make_rsrc4(B, 0);
  const rsrc4_t rsa0 = make_rsrc4(As, 0), rsb0 = make_rsrc4(Bs, 0);

  // Code-load geometry: instruction u of this wave covers rows 16 (4 wave + u)
  // .. +15; lane i fills LDS slot i & 3 of row 16 (4 wave + u) + (i >> 2) with
  // the chunk that the swizzle puts there.
  int code_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 16 * (4 * wave + u) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    code_off[u] = row * KP + chunk * 16;
  }
  const int scale_off = (64 * wave + lane) * KB;

  // Stage st: its codes, plus (when st starts a super-stage) the scales of the
  // whole super-stage.  Stages past the last load through the empty
  // resources: zeros land in slots nobody reads, and every step keeps the same
  // static wait count.  The lane's offset is a loop constant and the stage's
  // K offset the load's scalar offset, so a load costs no vector
  // instructions.
  // code load u (0..7) of stage st: A rows for u < 4, B rows for u >= 4
  auto issue_code = [&](int st, int u) {
    const int slot = st % RB_NS;
    const bool live = st < KT;
    if (u < 4)
      dma_x4_so(live ? ra : ra0, (uint32_t)(uintptr_t)&sm.a[slot][64 * (4 * wave + u)], code_off[u & 3], st * RB_K);
    else
      dma_x4_so(live ? rb : rb0, (uint32_t)(uintptr_t)&sm.b[slot][64 * (4 * wave + (u & 3))], code_off[u & 3],
                st * RB_K);
  };
  auto issue_scales = [&](int st) {
    const int sbuf = (st / U) % NSB;
    const bool live = st < KT;
    const int so = (st / U) * SB;
    if (SB == 16) {
      dma_x4_so(live ? rsa : rsa0, (uint32_t)(uintptr_t)&sm.as[sbuf][64 * wave * 4], scale_off, so);
      dma_x4_so(live ? rsb : rsb0, (uint32_t)(uintptr_t)&sm.bs[sbuf][64 * wave * 4], scale_off, so);
    } else {
      dma_x1_so(live ? rsa : rsa0, (uint32_t)(uintptr_t)&sm.as[sbuf][64 * wave], scale_off, so);
      dma_x1_so(live ? rsb : rsb0, (uint32_t)(uintptr_t)&sm.bs[sbuf][64 * wave], scale_off, so);
    }
  };
  auto issue = [&](int st, auto WITH_SCALES) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      issue_code(st, u);
      issue_code(st, 4 + u);
    }
    if (decltype(WITH_SCALES)::value) issue_scales(st);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  // Fragments of stage st; `in` = st % U is static.  FP8: the stage's E8M0
  // bytes are 2 in and 2 in + 1 of the row's SB-byte scale entry and lane g
  // takes byte 2 in + g; both sit in dword in / 2.  FP4: the stage's bytes
  // are dword in, and lane g takes byte 2 s + g for MFMA s = 0, 1.  Shifting
  // the dword right by 8 g puts lane g's byte at the same position for both
  // lane halves (2 (in % 2) for FP8, 2 s for FP4), and the MFMA's scale byte
  // select (op_sel) picks it there: no per-byte extraction.  The scale dwords
  // are read first, so the first MFMA never waits on a drained LDS queue.
  auto read_frags = [&](int st, auto INC, Frags<FP4>& f) {
    constexpr int in = decltype(INC)::value;
    constexpr int word = FP4 ? in : in / 2;
    const int slot = st % RB_NS, sbuf = (st / U) % NSB;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.sa[i] = (int)(sm.as[sbuf][(wm * 128 + i * 32 + r) * (SB / 4) + word] >> (8 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) f.sb[j] = (int)(sm.bs[sbuf][(wn * 128 + j * 32 + r) * (SB / 4) + word] >> (8 * g));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + r;
      const uint4 lo = sm.a[slot][rswz(row, g)], hi = sm.a[slot][rswz(row, 2 + g)];
      if constexpr (FP4) {
        f.alo[i] = lo;
        f.ahi[i] = hi;
      } else {
        f.a[i] = frag8(lo, hi);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + r;
      const uint4 lo = sm.b[slot][rswz(row, g)], hi = sm.b[slot][rswz(row, 2 + g)];
      if constexpr (FP4) {
        f.blo[j] = lo;
        f.bhi[j] = hi;
      } else {
        f.b[j] = frag8(lo, hi);
      }
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  // MFMA of A fragment a and B fragment b (scale byte select sel).  WFIRST:
  // the B operand goes first, giving the row-chunk epilogue its layout.  The
  // FP4 ring with 4-byte scale batches keeps A first: with B first the
  // compiler spilled ~200 VGPRs in its main loop.
  constexpr bool WFIRST = !(FP4 && SB == 4);
  auto mfma_ab = [](const v8i& a, const v8i& b, const v16f& c, auto sel_c, int sa, int sb) {
    constexpr int fmt = mfma_fmt<FP4>();
    constexpr int sel = decltype(sel_c)::value;
    if constexpr (WFIRST) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, fmt, fmt, sel, sb, sel, sa);
    else return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, fmt, fmt, sel, sa, sel, sb);
  };
  // MFMAs of tile rows i0, i0 + 1.  OPSEL: byte of the (shifted) scale dwords
  // that holds this stage's FP8 scale.  FP4 runs its two K64 halves in turn
  // (all 8 tiles of the first, then the second), so the two MFMAs into one
  // accumulator are 7 issues apart.
  auto mfma_rows = [&](const Frags<FP4>& f, int i0, auto OPSEL) {
    if constexpr (FP4) {
      static_for<0, 2>([&](auto SC) {
        constexpr int s = decltype(SC)::value;
#pragma unroll
        for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = mfma_ab(frag4(s ? f.ahi[i] : f.alo[i]), frag4(s ? f.bhi[j] : f.blo[j]), acc[i][j],
                                std::integral_constant<int, 2 * s>{}, f.sa[i], f.sb[j]);
      });
    } else {
      constexpr int sel = decltype(OPSEL)::value;
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma_ab(f.a[i], f.b[j], acc[i][j], std::integral_constant<int, sel>{}, f.sa[i], f.sb[j]);
    }
  };

  // One MFMA of tile (i, j) of a stage: the FP8 one, or the FP4 one of K64
  // half SC.
  auto mfma_one = [&](const Frags<FP4>& f, int i, int j, auto OPSEL, auto SC) {
    if constexpr (FP4) {
      constexpr int s = decltype(SC)::value;
      acc[i][j] = mfma_ab(frag4(s ? f.ahi[i] : f.alo[i]), frag4(s ? f.bhi[j] : f.blo[j]), acc[i][j],
                          std::integral_constant<int, 2 * s>{}, f.sa[i], f.sb[j]);
    } else {
      constexpr int sel = decltype(OPSEL)::value;
      acc[i][j] = mfma_ab(f.a[i], f.b[j], acc[i][j], std::integral_constant<int, sel>{}, f.sa[i], f.sb[j]);
    }
  };

  // Loads issued for stage s: codes, plus 2 scale loads when s starts a
  // super-stage.  Waiting for stage kt+1 leaves stages kt+2 and kt+3 in flight.
  auto loads_of = [](int s_mod) { return RB_CODE_LOADS + (s_mod == 0 ? 2 : 0); };

  // Step kt with kt % U == IN; fragments alternate between f[0] and f[1] with
  // the step's parity, which IN fixes when U is even (U == 1 unrolls by 2).
  Frags<FP4> f[2];
  auto step = [&](int kt, auto INC, auto CURC) {
    constexpr int IN = decltype(INC)::value;
    constexpr int CUR = decltype(CURC)::value;
    constexpr int ISSUE_MOD = (IN + RB_NS - 1) % U;   // stage kt+3 within its super-stage
    // Direct loads of stage kt+3 (a burst of 8 at the head of the step, IL
    // == 0, fills the wave's memory queue and holds up its MFMA issue):
    //   IL == 1: interleaved with the first half's MFMAs (+11% at 16384^3
    //            for MXFP8 and MXFP4 over IL == 0);
    //   IL == 2: the A half interleaved with the first half's MFMAs, the B
    //            half right after the mid-step barrier, so the wait leaves
    //            fewer loads outstanding (+1.3% MXFP8, +3.4% MXFP4 at 16384^3
    //            over IL == 1).  All three give bit-identical output.
    constexpr int LATE = IL == 2 ? 4 : 0;
    constexpr int AFTER = loads_of((IN + 2) % U) + loads_of((IN + 3) % U) - LATE;
    constexpr auto SEL = std::integral_constant<int, 2 * (IN % 2)>{};
    if constexpr (IL == 2) {
      if constexpr (ISSUE_MOD == 0) issue_scales(kt + RB_NS - 1);
      static_for<0, 8 * per_byte<FP4>()>([&](auto IX) {
        constexpr int ix = decltype(IX)::value, t = ix % 8;
        if (ix % (2 * per_byte<FP4>()) == 0) issue_code(kt + RB_NS - 1, ix / (2 * per_byte<FP4>()));
        __builtin_amdgcn_sched_barrier(0);
        mfma_one(f[CUR], t >> 2, t & 3, SEL, std::integral_constant<int, ix / 8>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    } else if constexpr (IL == 1) {
      if constexpr (ISSUE_MOD == 0) issue_scales(kt + RB_NS - 1);
      // FP4: the 8 tiles' first K64 halves, then their second halves (two
      // MFMAs into one accumulator stay 7 issues apart)
      static_for<0, 8 * per_byte<FP4>()>([&](auto IX) {
        constexpr int ix = decltype(IX)::value, t = ix % 8;
        if (ix % per_byte<FP4>() == 0) issue_code(kt + RB_NS - 1, ix / per_byte<FP4>());
        __builtin_amdgcn_sched_barrier(0);
        mfma_one(f[CUR], t >> 2, t & 3, SEL, std::integral_constant<int, ix / 8>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      issue(kt + RB_NS - 1, std::integral_constant<bool, ISSUE_MOD == 0>{});
      // keep the loads at the head of the step: the compiler would otherwise
      // sink them below the first MFMAs and shorten the ring's lead
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows(f[CUR], 0, SEL);
    }
    wait_vm_barrier<AFTER>();        // stage kt+1 landed; kt+2, kt+3 in flight
    if constexpr (IL == 2) {
#pragma unroll
      for (int u = 4; u < 8; ++u) issue_code(kt + RB_NS - 1, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_frags(kt + 1, std::integral_constant<int, (IN + 1) % U>{}, f[CUR ^ 1]);
    mfma_rows(f[CUR], 2, SEL);
    // 8 MFMAs (FP8) or 16 (FP4) interleaved with the 24 LDS reads
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, per_byte<FP4>(), 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                  // 3 LDS reads
    }
  };

  // prologue: stages 0..2 (stage 0 carries the first super-stage's scales)
  issue(0, std::true_type{});
  issue(1, std::integral_constant<bool, (1 % U) == 0>{});
  issue(2, std::integral_constant<bool, (2 % U) == 0>{});
  wait_vm_barrier<loads_of(1 % U) + loads_of(2 % U)>();
  read_frags(0, std::integral_constant<int, 0>{}, f[0]);
  // Every step has the same shape, the last ones included: they issue
  // out-of-range (zero, no traffic) loads for stages past KT and read the
  // zero fragments of "stage KT", which are never used.  One copy of the
  // loop body (U steps, or 2 when U == 1) therefore serves the whole loop;
  // with U == 1 and KT odd the second step of the last pass is skipped.
  constexpr int UNROLL = U == 1 ? 2 : U;
  for (int kt = 0; kt < KT; kt += UNROLL) {
    static_for<0, UNROLL>([&](auto IC) {
      constexpr int i = decltype(IC)::value;
      if (U == 1 && i == 1 && kt + 1 == KT) return;
      step(kt + i, std::integral_constant<int, i % U>{}, std::integral_constant<int, i & 1>{});
    });
  }

  // Epilogue.  The MFMAs take the B (column) operand first, so each lane
  // holds 4 consecutive columns per accumulator quad; the block goes out as
  // BF16 through the (now idle) A and B rings: 16-byte row-chunk stores
  // instead of one 2-byte store per element.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the out-of-range tail loads
  __syncthreads();                                   // every wave is done with the rings
  static_assert(sizeof(sm.a) + sizeof(sm.b) >= 4 * 128 * 256, "epilogue staging needs 32 KB per wave");
  if constexpr (WFIRST) {
    store_block128_bf16<false>(acc, &sm.a[0][0] + wave * (128 * 16), C, M, N, m0 + wm * 128, n0 + wn * 128, 1.0f);
  } else {
    // A first: lane (r, g) holds column 32 j + r, rows 32 i + 8 (v / 4) + 4 g + v % 4
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 128 + j * 32 + r;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
          if (row < M && col < N) C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Pair ring kernel (K % 512 == 0): the ring of the kernel above, but each
// direct load fetches whole 128-byte lines, two K steps of a row at once.
//
// What bounds the single-step ring is the rate at which a CU's L1 completes
// requests to L2: it keeps about 130 of them in flight, so at ~380 cycles of
// L2 latency it completes ~0.35 per clock, and with 64-byte row segments a
// step of 32 KiB needs 512 requests (MXFP8 at the full MFMA rate needs 0.5
// per clock).  A 128-byte segment per row halves the requests for the same
// bytes.
//
// Ring: two pair slots, each [256][128] code bytes per operand (the two K
// steps of a row side by side), 16-byte chunk c of row r at c ^ ((r >> 1) &
// 7); the same 128 KiB as four single-step stages.  Scales in batches per
// row, two batch buffers: WIDE (K % 1024 == 0) 32 bytes per row (2 U steps),
// else 16 bytes (U steps).  Every scale row is a separate L2 request, so the
// wide batches halve the scale requests (MXFP4 16384^3 -3.0%, MXFP8 -0.8%,
// bit-identical).  A 32-byte row holds two 16-byte chunks, swapped on bit 3
// of the row, so the 32 lanes that read one scale dword of 32 consecutive
// rows meet 2-way bank conflicts, as with 16-byte rows (4-way unswapped).
// The K loop then covers a whole 32-byte batch (both halves unrolled, the
// half a compile-time constant): a run-time half split the loop body and
// made the compiler spill.
// Schedule, for pair p = steps 2p and 2p + 1:
//   step 2p:     its first-half MFMAs interleaved with the B loads of pair
//                p + 1; then the fragments of step 2p + 1 (same slot) are
//                read under the second-half MFMAs.  No barrier.
//   step 2p + 1: first-half MFMAs; wait for every load (all of pair p + 1)
//                and cross the barrier (after which no wave still reads
//                slot p); issue the A loads of pair p + 2 (and a scale batch
//                when it starts one) into slot p; read the fragments of step
//                2p + 2 under the second-half MFMAs.
// So one barrier per two steps, and pair p + 1's loads have 1.5-2 steps to
// land.
constexpr int PR_CH = 8;   // 16-byte chunks per row of a pair slot

template <bool FP4, bool WIDE>
struct PairSmem {
  static constexpr int U = 16 / (2 * per_byte<FP4>());   // steps per 16 scale bytes of a row
  static constexpr int SCW = WIDE ? 8 : 4;                // scale dwords per row of a batch
  uint4 a[2][BM * PR_CH];
  uint4 b[2][BN * PR_CH];
  uint32_t as[2][BM * SCW];
  uint32_t bs[2][BN * SCW];
};

__device__ __forceinline__ int prswz(int row, int chunk) { return row * PR_CH + (chunk ^ ((row >> 1) & 7)); }

template <bool FP4, bool WIDE>
__global__ __launch_bounds__(NT, 1) void mx_pair_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  using Sm = PairSmem<FP4, WIDE>;
  constexpr int U = Sm::U;             // FP8 8, FP4 4: an even number of steps
  constexpr int SCW = Sm::SCW;
  constexpr int PB = WIDE ? U : U / 2; // pairs per scale batch
  __shared__ Sm sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  if (tiles_m % 16 == 0 && tiles_n % 16 == 0)
    supertile_order(blockIdx.x, tiles_n, tm, tn);
  else
    raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KP = K / per_byte<FP4>();  // code bytes per row
  const int KT = KP / RB_K;            // steps: a positive multiple of U
  const int KPR = KT / 2;              // pairs
  const int KB = K / 32;
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const rsrc4_t ra = make_rsrc4(A + (int64_t)m0 * KP, rows_a * KP);
  const rsrc4_t rb = make_rsrc4(B + (int64_t)n0 * KP, rows_b * KP);
  const rsrc4_t rsa = make_rsrc4(As + (int64_t)m0 * KB, rows_a * KB);
  const rsrc4_t rsb = make_rsrc4(Bs + (int64_t)n0 * KB, rows_b * KB);
  const rsrc4_t ra0 = make_rsrc4(A, 0), rb0 = make_rsrc4(B, 0);
  const rsrc4_t rsa0 = make_rsrc4(As, 0), rsb0 = make_rsrc4(Bs, 0);

  // Load u (0..7) of an operand covers rows 8 (8 wave + u) .. + 7; lane i
  // fills chunk position i & 7 of row 8 (8 wave + u) + (i >> 3) with the
  // chunk that the swizzle puts there.
  int code_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 8 * (8 * wave + u) + (lane >> 3);
    code_off[u] = row * KP + (((lane & 7) ^ ((row >> 1) & 7)) * 16);
  }
  // 16-byte batches: lane i loads row 64 wave + i.  32-byte batches: scale
  // load v covers rows 64 wave + 32 v .. + 31, two lanes per row, each lane
  // the chunk that the swap puts in its slot (rows r and r + 32 swap alike).
  const int srow = WIDE ? 64 * wave + (lane >> 1) : 64 * wave + lane;
  const int scale_off = WIDE ? srow * KB + 16 * ((lane & 1) ^ ((srow >> 3) & 1)) : srow * KB;
  auto issue_a = [&](int p, int u) {
    dma_x4_so(p < KPR ? ra : ra0, (uint32_t)(uintptr_t)&sm.a[p & 1][64 * (8 * wave + u)], code_off[u],
              p * (2 * RB_K));
  };
  auto issue_b = [&](int p, int u) {
    dma_x4_so(p < KPR ? rb : rb0, (uint32_t)(uintptr_t)&sm.b[p & 1][64 * (8 * wave + u)], code_off[u],
              p * (2 * RB_K));
  };
  auto issue_scales = [&](int p) {   // p starts a batch
    const int bat = p / PB, buf = bat & 1;
    const bool live = p < KPR;
#pragma unroll
    for (int v = 0; v < (WIDE ? 2 : 1); ++v) {
      const int lds = 64 * wave * SCW + 256 * v, so = bat * (4 * SCW) + v * 32 * KB;
      dma_x4_so(live ? rsa : rsa0, (uint32_t)(uintptr_t)&sm.as[buf][lds], scale_off, so);
      dma_x4_so(live ? rsb : rsb0, (uint32_t)(uintptr_t)&sm.bs[buf][lds], scale_off, so);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  const int ssw = WIDE ? ((r >> 3) & 1) << 2 : 0;   // the chunk swap of this lane's rows (32 i + r)
  // Fragments of step st (st % U == in): its half st & 1 of the pair slot,
  // chunks 4 h + g and 4 h + 2 + g; scales as in the single-step ring.
  // (HALF: which 16 bytes of a 32-byte batch row hold step st's scales.)
  auto read_frags = [&](int st, auto INC, auto HALFC, Frags<FP4>& f) {
    constexpr int in = decltype(INC)::value;
    constexpr int word = FP4 ? in : in / 2;
    constexpr int h = in & 1;
    const int slot = (st >> 1) & 1, buf = (st / (WIDE ? 2 * U : U)) & 1;
    const int sdw = (decltype(HALFC)::value ? 4 - ssw : ssw) + word;   // the step's dword of its row
#pragma unroll
    for (int i = 0; i < 4; ++i) f.sa[i] = (int)(sm.as[buf][(wm * 128 + i * 32 + r) * SCW + sdw] >> (8 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) f.sb[j] = (int)(sm.bs[buf][(wn * 128 + j * 32 + r) * SCW + sdw] >> (8 * g));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + r;
      const uint4 lo = sm.a[slot][prswz(row, 4 * h + g)], hi = sm.a[slot][prswz(row, 4 * h + 2 + g)];
      if constexpr (FP4) {
        f.alo[i] = lo;
        f.ahi[i] = hi;
      } else {
        f.a[i] = frag8(lo, hi);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + r;
      const uint4 lo = sm.b[slot][prswz(row, 4 * h + g)], hi = sm.b[slot][prswz(row, 4 * h + 2 + g)];
      if constexpr (FP4) {
        f.blo[j] = lo;
        f.bhi[j] = hi;
      } else {
        f.b[j] = frag8(lo, hi);
      }
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  auto mfma_ab = [](const v8i& a, const v8i& b, const v16f& c, auto sel_c, int sa, int sb) {
    constexpr int fmt = mfma_fmt<FP4>();
    constexpr int sel = decltype(sel_c)::value;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, fmt, fmt, sel, sb, sel, sa);   // B first
  };
  auto mfma_one = [&](const Frags<FP4>& f, int i, int j, auto OPSEL, auto SC) {
    if constexpr (FP4) {
      constexpr int s = decltype(SC)::value;
      acc[i][j] = mfma_ab(frag4(s ? f.ahi[i] : f.alo[i]), frag4(s ? f.bhi[j] : f.blo[j]), acc[i][j],
                          std::integral_constant<int, 2 * s>{}, f.sa[i], f.sb[j]);
    } else {
      constexpr int sel = decltype(OPSEL)::value;
      acc[i][j] = mfma_ab(f.a[i], f.b[j], acc[i][j], std::integral_constant<int, sel>{}, f.sa[i], f.sb[j]);
    }
  };
  // the MFMAs of tile rows 2 hf, 2 hf + 1 (FP4: all 8 tiles' first K64 halves,
  // then their second halves), one load of `ld` (if any) before each of the
  // first 8 issues
  auto mfma_half = [&](const Frags<FP4>& f, int hf, auto OPSEL, auto ld) {
    static_for<0, 8 * per_byte<FP4>()>([&](auto IX) {
      constexpr int ix = decltype(IX)::value, t = ix % 8;
      if constexpr (ix % per_byte<FP4>() == 0) ld(ix / per_byte<FP4>());
      __builtin_amdgcn_sched_barrier(0);
      mfma_one(f, 2 * hf + (t >> 2), t & 3, OPSEL, std::integral_constant<int, ix / 8>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto no_load = [](int) {};

  Frags<FP4> f[2];
  // step kt (kt % U == IN; parity IN & 1; fragments in f[IN & 1])
  auto step = [&](int kt, auto INC, auto HALFC) {
    constexpr int IN = decltype(INC)::value;
    constexpr int HALF = decltype(HALFC)::value;
    constexpr int CUR = IN & 1;
    constexpr auto SEL = std::integral_constant<int, 2 * (IN % 2)>{};
    const int p = kt >> 1;
    if constexpr (CUR == 0) {
      mfma_half(f[CUR], 0, SEL, [&](int u) { issue_b(p + 1, u); });
    } else {
      mfma_half(f[CUR], 0, SEL, no_load);
      wait_vm_barrier<0>();            // pair p + 1 landed; nobody reads slot p any more
      // pair p + 2 starts a scale batch
      constexpr bool NEW_BATCH = WIDE ? HALF == 1 && ((IN + 3) / 2) % (U / 2) == 0 : ((IN + 3) / 2) % PB == 0;
      if constexpr (NEW_BATCH) issue_scales(p + 2);
#pragma unroll
      for (int u = 0; u < 8; ++u) issue_a(p + 2, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_frags(kt + 1, std::integral_constant<int, (IN + 1) % U>{},
               std::integral_constant<int, WIDE && (IN + 1 == U) ? 1 - HALF : HALF>{}, f[CUR ^ 1]);
    if constexpr (FP4) {
      static_for<0, 2>([&](auto SC) {
#pragma unroll
        for (int i = 2; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) mfma_one(f[CUR], i, j, SEL, SC);
      });
    } else {
#pragma unroll
      for (int i = 2; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma_one(f[CUR], i, j, SEL, std::integral_constant<int, 0>{});
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, per_byte<FP4>(), 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                  // 3 LDS reads
    }
  };

  // prologue: pair 0 (with the first scale batch) and the A loads of pair 1;
  // wait for pair 0
  issue_scales(0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    issue_a(0, u);
    issue_b(0, u);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) issue_a(1, u);
  wait_vm_barrier<8>();
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  read_frags(0, std::integral_constant<int, 0>{}, H0{}, f[0]);
  if constexpr (WIDE) {
    for (int kt = 0; kt < KT; kt += 2 * U) {   // one 32-byte scale batch (KT % (2 U) == 0)
      static_for<0, U>([&](auto IC) { step(kt + decltype(IC)::value, IC, H0{}); });
      static_for<0, U>([&](auto IC) { step(kt + U + decltype(IC)::value, IC, H1{}); });
    }
  } else {
    for (int kt = 0; kt < KT; kt += U) {
      static_for<0, U>([&](auto IC) { step(kt + decltype(IC)::value, IC, H0{}); });
    }
  }

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the out-of-range tail loads
  __syncthreads();                                   // every wave is done with the rings
  static_assert(sizeof(sm.a) + sizeof(sm.b) >= 4 * 128 * 256, "epilogue staging needs 32 KB per wave");
  store_block128_bf16<false>(acc, &sm.a[0][0] + wave * (128 * 16), C, M, N, m0 + wm * 128, n0 + wn * 128, 1.0f);
}

// K % 512 == 0: the pair ring (same-process A/B against the single-step ring,
// bit-identical output: MXFP8 16384^3 -7.6%, MXFP4 16384^3 -6.7%, MXFP8
// 4096^3 -5%; loads of the next pair spread one per MFMA beat bursts after the
// barrier by 3-5%), with 32-byte scale batches when K % 1024 == 0.  K % 128
// == 0 otherwise: the single-step ring with 4-byte scale batches.  Any other
// K: the register-staged kernel.
template <bool FP4>
hipError_t launch_mx(int64_t m, int64_t n, int64_t k, const uint8_t* a, const uint8_t* as,
                     const uint8_t* b, const uint8_t* bs, uint16_t* c, hipStream_t stream) {
  const int tiles_m = (int)ceil_div(m, BM), tiles_n = (int)ceil_div(n, BN);
  if (k % 1024 == 0 && k > 0)
    hipLaunchKernelGGL((mx_pair_kernel<FP4, true>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else if (k % 512 == 0 && k > 0)
    hipLaunchKernelGGL((mx_pair_kernel<FP4, false>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else if (k % 128 == 0 && k > 0)
    hipLaunchKernelGGL((mx_gemm_ring_kernel<4, FP4>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<FP4>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a, as, b,
                       bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mxfp8(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* c,
                             hipStream_t stream) {
  return launch_mx<false>(m, n, k, a, as, b, bs, c, stream);
}

hipError_t launch_gemm_mxfp4(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* c,
                             hipStream_t stream) {
  return launch_mx<true>(m, n, k, a, as, b, bs, c, stream);
}

}  // namespace bsg
