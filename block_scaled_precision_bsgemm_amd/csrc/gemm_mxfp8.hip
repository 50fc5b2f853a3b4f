// MXFP8 x MXFP8 GEMM on the gfx950 scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The block format (E4M3 values, one E8M0 scale per 32 K-elements) is the one
// this MFMA consumes natively.  Each lane supplies one E8M0 byte for its row
// and its 32-element K block, so no dequantisation happens anywhere.
// Prior art: "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera
// Rubin NVL72", section "Building the GEMM".  That page stages FP8 E4M3
// operands through a multi-stage shared-memory ring and sweeps its depth.
//
// Layout of one workgroup (256 threads, 4 waves):
//   - Output tile 256 x 256; each wave owns 128 x 128 (4 x 4 MFMA tiles of
//     32 x 32).
//   - K step 128 bytes, double-buffered in LDS:
//       A and B codes [256][128] bytes each, 16-byte chunks XOR-swizzled
//       by ((row >> 1) & 7), conflict-free for the MFMA operand reads;
//       A and B scales [256] dwords (4 E8M0 bytes of the step).
//   - Operand register layout of the 32x32x64 FP8 MFMA, checked on the device
//     against the oracle: lane (r = l % 32, g = l / 32) holds row r;
//       dwords 0-3 = K bytes [16g, 16g+16) of the MFMA's first 32-block;
//       dwords 4-7 = K bytes [32+16g, 32+16g+16) of its second 32-block;
//       the lane's scale byte applies to 32-block g.
//     So lane g loads chunks (4s+g) and (4s+2+g) of sub-step s, and its scale
//     is the one of block 2s+g.
//   - Output lane layout: lane l holds column l % 32, rows
//     8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

constexpr int BM = 256, BN = 256, BK = 128, NT = 256;
constexpr int GROUP_M = 8;   // tile rows per rasterisation group

// Tiles are uint4 arrays: the compiler then knows every access is 16-byte
// aligned and emits single ds_read_b128 / ds_write_b128 instructions.
constexpr int RC = BK / 16;   // 16-byte chunks per row
struct Smem {
  uint4 a[2][BM * RC];
  uint4 b[2][BN * RC];
  uint32_t as[2][BM];
  uint32_t bs[2][BN];
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

template <bool SCALE_DW>
__global__ __launch_bounds__(NT, 1) void mxfp8_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = (K + BK - 1) / BK;
  const int KB = K / 32;

  // ---- global -> register staging: thread owns chunk (tid & 7) of rows
  //      (tid >> 3) + 32 i, i = 0..7, and the scale dword of row tid.
  const int lc = tid & 7, lr = tid >> 3;
  uint4 ra[8], rb[8];
  // Per-tile buffer resources: loads past the tile's last valid row return 0.
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const auto ra_rsrc = make_rsrc(A + (int64_t)m0 * K, rows_a * K);
  const auto rb_rsrc = make_rsrc(B + (int64_t)n0 * K, rows_b * K);
  const auto sa_rsrc = make_rsrc(As + (int64_t)m0 * KB, rows_a * KB);
  const auto sb_rsrc = make_rsrc(Bs + (int64_t)n0 * KB, rows_b * KB);
  const int off0 = lr * K + lc * 16;

  // Loads only issue here; the scale bytes are assembled in sstore, after the
  // MFMAs of the current step, so nothing waits on them early.
  uint32_t sa_raw[4], sb_raw[4];
  auto gload = [&](int kt) {
    const int kc = kt * BK + lc * 16;
    const int kofs = kc < K ? kt * BK : OOB;   // K % 32 == 0: chunks are wholly in or out
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = kofs == OOB ? OOB : off0 + 32 * i * K + kofs;
      ra[i] = buffer_load_x4(ra_rsrc, off);
      rb[i] = buffer_load_x4(rb_rsrc, off);
    }
    if (SCALE_DW) {            // K % 128 == 0: the step's 4 scale bytes are one dword
      sa_raw[0] = buffer_load_u32(sa_rsrc, tid * KB + kt * 4);
      sb_raw[0] = buffer_load_u32(sb_rsrc, tid * KB + kt * 4);
    } else {                   // blocks past K read as 0 (their codes are 0 too)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = kt * 4 + j;
        sa_raw[j] = buffer_load_u8(sa_rsrc, kb < KB ? tid * KB + kb : OOB);
        sb_raw[j] = buffer_load_u8(sb_rsrc, kb < KB ? tid * KB + kb : OOB);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = lr + 32 * i;
      sm.a[buf][swz(row, lc)] = ra[i];
      sm.b[buf][swz(row, lc)] = rb[i];
    }
    if (SCALE_DW) {
      sm.as[buf][tid] = sa_raw[0];
      sm.bs[buf][tid] = sb_raw[0];
    } else {
      sm.as[buf][tid] = sa_raw[0] | (sa_raw[1] << 8) | (sa_raw[2] << 16) | (sa_raw[3] << 24);
      sm.bs[buf][tid] = sb_raw[0] | (sb_raw[1] << 8) | (sb_raw[2] << 16) | (sb_raw[3] << 24);
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
    for (int s = 0; s < 2; ++s) {
      v8i af[4], bf[4];
      int sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r;
        const uint4 lo = sm.a[buf][swz(row, 4 * s + g)];
        const uint4 hi = sm.a[buf][swz(row, 4 * s + 2 + g)];
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sa[i] = (int)((sm.as[buf][row] >> (8 * (2 * s + g))) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + r;
        const uint4 lo = sm.b[buf][swz(row, 4 * s + g)];
        const uint4 hi = sm.b[buf][swz(row, 4 * s + 2 + g)];
        bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sb[j] = (int)((sm.bs[buf][row] >> (8 * (2 * s + g))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], bf[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
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
// Ring kernel (K % 128 == 0): the operands stream HBM -> LDS by direct
// loads through a 4-stage ring of 64-byte K steps, so three steps are in
// flight while one is computed.  The pages' FP8 GEMM got its gains from the
// same lever: ring depth.
//
// Codes, per stage and operand: [256][64] bytes, 16-byte chunk c of row r at
// c ^ ((r >> 2) & 3) (conflict-free reads).  Each wave issues 8 code loads
// per stage (4 A, 4 B; 1 KiB = 16 rows each).
//
// Scales are loaded in batches.  With one lane per row, a scale load touches
// 64 cache lines for a few bytes each, and the address path costs about one
// clock per line.  Per-stage 4-byte scale loads cost as much as all the code
// loads.  So one load brings SB bytes per row: the scales of SB/2 K steps
// (SB = 16 when K % 512 == 0, else 4).  That is one load per operand per wave
// every SB/2 stages, into a ring of per-super-stage buffers.
//
// Per stage each wave runs 16 MFMAs (its 4 x 4 tiles, one K64 MFMA each).
// The stage's fragments were read into registers during the second half of
// the previous stage.  Halfway through the MFMAs the wave waits for the next
// stage's loads, crosses the barrier and reads the next fragments, overlapping
// the remaining MFMAs.  The K loop is unrolled by one super-stage, so every
// step's load count and wait count are static.
constexpr int RB_K = 64, RB_NS = 4, RB_ROW = RB_K / 16;   // 4 chunks per row
constexpr int RB_CODE_LOADS = 8;                           // code loads per wave per stage

// Scale buffers per super-stage: a buffer is rewritten only after at least
// two barriers have passed since its last read (3 buffers when a
// super-stage is only 2 stages long).
template <int SB>
constexpr int ring_scale_bufs() { return SB / 2 >= 4 ? 2 : 3; }

template <int SB>
struct RingSmem {
  uint4 a[RB_NS][BM * RB_ROW];
  uint4 b[RB_NS][BN * RB_ROW];
  uint32_t as[ring_scale_bufs<SB>()][BM * SB / 4];   // [super-stage buffer][row][SB bytes]
  uint32_t bs[ring_scale_bufs<SB>()][BN * SB / 4];
};

__device__ __forceinline__ int rswz(int row, int chunk) { return row * RB_ROW + (chunk ^ ((row >> 2) & 3)); }

struct Frags {
  v8i a[4], b[4];
  int sa[4], sb[4];
};

template <int SB>
__global__ __launch_bounds__(NT, 1) void mxfp8_gemm_ring_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  constexpr int U = SB / 2;                       // stages per scale super-stage
  __shared__ RingSmem<SB> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  if (tiles_m % 16 == 0 && tiles_n % 16 == 0)
    supertile_order(blockIdx.x, tiles_n, tm, tn);
  else
    raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = K / RB_K;   // a positive multiple of U
  const int KB = K / 32;
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const rsrc4_t ra = make_rsrc4(A + (int64_t)m0 * K, rows_a * K);
  const rsrc4_t rb = make_rsrc4(B + (int64_t)n0 * K, rows_b * K);
  const rsrc4_t rsa = make_rsrc4(As + (int64_t)m0 * KB, rows_a * KB);
  const rsrc4_t rsb = make_rsrc4(Bs + (int64_t)n0 * KB, rows_b * KB);

  // Code-load geometry: instruction u of this wave covers rows 16 (4 wave + u)
  // .. +15; lane i fills LDS slot i & 3 of row 16 (4 wave + u) + (i >> 2) with
  // the chunk that the swizzle puts there.
  int code_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 16 * (4 * wave + u) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    code_off[u] = row * K + chunk * 16;
  }
  const int scale_off = (64 * wave + lane) * KB;

  // Stage st: its codes, plus (when st starts a super-stage) the scales of the
  // whole super-stage.  Stages past the last are issued at an out-of-range
  // offset: zeros land in slots nobody reads, and every step keeps the same
  // static wait count.
  auto issue = [&](int st, auto WITH_SCALES) {
    const int slot = st % RB_NS;
    const bool live = st < KT;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int off = live ? code_off[u] + st * RB_K : OOB;
      dma_x4(ra, lds_addr(&sm.a[slot][64 * (4 * wave + u)]), off);
      dma_x4(rb, lds_addr(&sm.b[slot][64 * (4 * wave + u)]), off);
    }
    if (decltype(WITH_SCALES)::value) {
      const int sbuf = (st / U) % ring_scale_bufs<SB>();
      const int soff = live ? scale_off + (st / U) * SB : OOB;
      if (SB == 16) {
        dma_x4(rsa, lds_addr(&sm.as[sbuf][64 * wave * 4]), soff);
        dma_x4(rsb, lds_addr(&sm.bs[sbuf][64 * wave * 4]), soff);
      } else {
        dma_x1(rsa, lds_addr(&sm.as[sbuf][64 * wave]), soff);
        dma_x1(rsb, lds_addr(&sm.bs[sbuf][64 * wave]), soff);
      }
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  // Fragments of stage st; `in` = st % U is static.  The stage's E8M0 bytes
  // are 2 in and 2 in + 1 of the row's SB-byte scale entry; lane g takes byte
  // 2 in + g.  Both sit in dword in / 2; shifting it right by 8 g puts lane
  // g's byte at position 2 (in % 2) for both lane halves, and the MFMA's
  // scale byte select (op_sel) picks it there: no per-byte extraction.  The
  // scale dwords are read first, so the first MFMA never waits on a drained
  // LDS queue.
  auto read_frags = [&](int st, auto INC, Frags& f) {
    constexpr int in = decltype(INC)::value;
    constexpr int word = in / 2;
    const int slot = st % RB_NS, sbuf = (st / U) % ring_scale_bufs<SB>();
#pragma unroll
    for (int i = 0; i < 4; ++i) f.sa[i] = (int)(sm.as[sbuf][(wm * 128 + i * 32 + r) * (SB / 4) + word] >> (8 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) f.sb[j] = (int)(sm.bs[sbuf][(wn * 128 + j * 32 + r) * (SB / 4) + word] >> (8 * g));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + r;
      const uint4 lo = sm.a[slot][rswz(row, g)], hi = sm.a[slot][rswz(row, 2 + g)];
      f.a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + r;
      const uint4 lo = sm.b[slot][rswz(row, g)], hi = sm.b[slot][rswz(row, 2 + g)];
      f.b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  // OPSEL: byte of the (shifted) scale dwords that holds this stage's scale
  auto mfma_rows = [&](const Frags& f, int i0, auto OPSEL) {
    constexpr int sel = decltype(OPSEL)::value;
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, sel,
                                                                    f.sa[i], sel, f.sb[j]);
  };

  // Loads issued for stage s: codes, plus 2 scale loads when s starts a
  // super-stage.  Waiting for stage kt+1 leaves stages kt+2 and kt+3 in flight.
  auto loads_of = [](int s_mod) { return RB_CODE_LOADS + (s_mod == 0 ? 2 : 0); };

  // Step kt with kt % U == IN and CUR = kt & 1 (U is even, so IN fixes CUR).
  Frags f[2];
  auto step = [&](int kt, auto INC, auto LASTC) {
    constexpr int IN = decltype(INC)::value;
    constexpr int CUR = IN & 1;
    constexpr bool LAST = decltype(LASTC)::value;
    constexpr int ISSUE_MOD = (IN + RB_NS - 1) % U;   // stage kt+3 within its super-stage
    constexpr int AFTER = loads_of((IN + 2) % U) + loads_of((IN + 3) % U);
    constexpr auto SEL = std::integral_constant<int, 2 * (IN % 2)>{};
    if (!LAST) issue(kt + RB_NS - 1, std::integral_constant<bool, ISSUE_MOD == 0>{});
    // keep the loads at the head of the step: the compiler would otherwise
    // sink them below the first MFMAs and shorten the ring's lead
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows(f[CUR], 0, SEL);
    if (!LAST) {
      wait_vm_barrier<AFTER>();        // stage kt+1 landed; kt+2, kt+3 in flight
      read_frags(kt + 1, std::integral_constant<int, (IN + 1) % U>{}, f[CUR ^ 1]);
    }
    mfma_rows(f[CUR], 2, SEL);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // 3 LDS reads
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
  // U-step body therefore serves the whole loop.
  for (int kt = 0; kt < KT; kt += U) {
    static_for<0, U>([&](auto IC) {
      constexpr int i = decltype(IC)::value;
      step(kt + i, std::integral_constant<int, i>{}, std::false_type{});
    });
  }

  // Epilogue.  Tiles wholly inside C (all but the ragged edge) store without
  // per-element bounds checks; each store writes two 64-byte row segments.
  uint16_t* cw = C + (int64_t)(m0 + wm * 128 + g * 4) * N + n0 + wn * 128 + r;
  if (m0 + BM <= M && n0 + BN <= N) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          cw[(int64_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * N + j * 32] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
  } else {
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

}  // namespace

hipError_t launch_gemm_mxfp8(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* c,
                             hipStream_t stream) {
  const int tiles_m = (int)ceil_div(m, BM), tiles_n = (int)ceil_div(n, BN);
  if (k % 512 == 0 && k > 0)
    hipLaunchKernelGGL(mxfp8_gemm_ring_kernel<16>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else if (k % 128 == 0 && k > 0)
    hipLaunchKernelGGL(mxfp8_gemm_ring_kernel<4>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(mxfp8_gemm_kernel<false>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bsg
