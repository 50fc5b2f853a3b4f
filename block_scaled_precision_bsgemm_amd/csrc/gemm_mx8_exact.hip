// MXFP8 x MXFP8 GEMM with exact products: every E4M3 code times its E8M0
// block scale is expanded to BF16, and the BF16 MFMA
// (v_mfma_f32_32x32x16_bf16) accumulates in FP32.
//
// Why a second MXFP8 path.  The native scaled FP8 MFMA (gemm_mx.hip) sums
// each aligned group of 8 products to about 14 bits below the group's largest
// product.  Where one 32-element block mixes values ~2^17 apart, that error
// exceeds the FP32-summation-order bound (1e-5 * sum |a b|) on some elements.
// Here no product is ever rounded:
//   - e4m3(code) has 4 significant bits and 2^(scale - 127) is a power of
//     two, so their product is exact in BF16, which has FP32's exponent range
//     (checked on the device for all 256 codes and every scale whose products
//     stay inside BF16's normal range);
//   - one packed scaled conversion (v_cvt_scalef32_pk_bf16_fp8) produces two
//     such products; it takes the scale's power of two from the exponent field
//     of its FP32 operand, which is exactly the E8M0 code shifted into place;
//   - the BF16 MFMA multiplies pairs exactly and accumulates in FP32.
// The results then differ from the exact sum only by FP32 summation order,
// for every operand whose decoded values and products lie in FP32's normal
// range.  The price is the BF16 MFMA rate, half of FP8's.
//
// Sources: "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera Rubin
// NVL72", section "Building the GEMM" (FP8 E4M3 GEMM at 16k square, staged
// through a multi-stage ring); "MXFP" is named in "Triton #11171 ...",
// section "The broader related matrix protected neighboring policy".
//
// Ring kernel layout (one workgroup of 4 waves per 256 x 256 output tile;
// each wave owns 128 x 128 = 4 x 4 tiles of 32 x 32):
//   - stage = 64 K elements = 64 code bytes per row; 4-stage direct-to-LDS
//     ring; 16-byte chunk c of row r at c ^ ((r >> 2) & 3);
//   - scales: SB bytes per row per load (16 when K % 512 == 0, else 4), 2
//     bytes per row per stage (the stage's two 32-element blocks);
//   - lane (r = l % 32, g = l / 32) reads chunks g and 2 + g of its row: K
//     [16g, 16g + 16) of block 0 and [32 + 16g, ...) of block 1;
//   - sub-step u (0..3) of a stage runs one 32x32x16 BF16 MFMA per tile on 8
//     K elements per lane half: bytes 8 (u & 1) .. + 7 of chunk u < 2 ? g :
//     2 + g.  A and B take the same bytes, so products pair the same K;
//   - the operands of sub-step u + 1 are converted under the 16 MFMAs of
//     sub-step u (2 conversions per MFMA).
#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

constexpr int BM = 256, BN = 256, NT = 256;
constexpr int XK = 64;                 // code bytes (= K elements) per row per stage
constexpr int XNS = 4;                 // ring stages
constexpr int XROW = XK / 16;          // 16-byte chunks per stage row
constexpr int XCODE_LOADS = 8;         // direct code loads per wave per stage
constexpr int GROUP_M = 8;

// Scale buffers per batch of U stages.  Stage st + 3's loads are issued at
// the head of step st; the buffer they overwrite had its last read in the step
// before the stage it served, after that step's mid-step barrier, so a
// barrier must separate the two.
template <int U>
constexpr int scale_bufs() { return U >= 4 ? 2 : (U >= 2 ? 3 : 4); }

template <int SB>
struct XSmem {
  static constexpr int U = SB / 2;     // stages per scale batch
  uint4 a[XNS][BM * XROW];
  uint4 b[XNS][BN * XROW];
  uint32_t as[scale_bufs<U>()][BM * SB / 4];
  uint32_t bs[scale_bufs<U>()][BN * SB / 4];
};

__device__ __forceinline__ int xswz(int row, int chunk) { return row * XROW + (chunk ^ ((row >> 2) & 3)); }

__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in = t - group * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// E8M0 code -> the FP32 whose exponent field is that code: the scale operand
// of the scaled conversions, which use only its exponent field.
__device__ __forceinline__ float e8m0_as_scale(uint32_t code) { return __uint_as_float(code << 23); }

// Eight E4M3 codes (two dwords, element j in byte j) times 2^(scale - 127),
// as exact BF16 values in MFMA operand order.
__device__ __forceinline__ v8bf expand8_bf16(uint32_t d0, uint32_t d1, float s) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, s, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, s, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, s, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, s, true);
  v8bf out;
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
  return out;
}

// Raw fragments of one stage for one lane: chunks g (lo) and 2 + g (hi) of
// its 4 A and 4 B rows, and the scale dword that holds the stage's two bytes.
struct XFrag {
  uint4 alo[4], ahi[4], blo[4], bhi[4];
  uint32_t sa[4], sb[4];
};

// Bytes 8 (u & 1) .. + 7 of the sub-step's chunk, as two dwords.
__device__ __forceinline__ void sub_dwords(const uint4& lo, const uint4& hi, int u, uint32_t& d0, uint32_t& d1) {
  const uint4& c = u < 2 ? lo : hi;
  d0 = (u & 1) ? c.z : c.x;
  d1 = (u & 1) ? c.w : c.y;
}

template <int SB>
__global__ __launch_bounds__(NT, 1) void mx8x_ring_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  using Sm = XSmem<SB>;
  constexpr int U = Sm::U;
  constexpr int NSB = scale_bufs<U>();
  __shared__ Sm sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  if (tiles_m % 16 == 0 && tiles_n % 16 == 0)
    supertile_order(blockIdx.x, tiles_n, tm, tn);
  else
    raster(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = K / XK;               // a positive multiple of U
  const int KB = K / 32;
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
  const rsrc4_t ra = make_rsrc4(A + (int64_t)m0 * K, rows_a * K);
  const rsrc4_t rb = make_rsrc4(B + (int64_t)n0 * K, rows_b * K);
  const rsrc4_t rsa = make_rsrc4(As + (int64_t)m0 * KB, rows_a * KB);
  const rsrc4_t rsb = make_rsrc4(Bs + (int64_t)n0 * KB, rows_b * KB);

  // Code load u of this wave covers rows 16 (4 wave + u) .. + 15; lane i
  // fills LDS slot i & 3 of row 16 (4 wave + u) + (i >> 2) with the chunk the
  // swizzle puts there.
  int code_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 16 * (4 * wave + u) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    code_off[u] = row * K + chunk * 16;
  }
  const int scale_off = (64 * wave + lane) * KB;

  // Stages past the last load zeros from an out-of-range offset into slots
  // nobody reads, so every step keeps the same static wait count.
  auto issue_code = [&](int st, int u) {
    const int slot = st % XNS;
    const int off = st < KT ? code_off[u & 3] + st * XK : OOB;
    if (u < 4)
      dma_x4(ra, lds_addr(&sm.a[slot][64 * (4 * wave + u)]), off);
    else
      dma_x4(rb, lds_addr(&sm.b[slot][64 * (4 * wave + (u & 3))]), off);
  };
  auto issue_scales = [&](int st) {
    const int sbuf = (st / U) % NSB;
    const int soff = st < KT ? scale_off + (st / U) * SB : OOB;
    if (SB == 16) {
      dma_x4(rsa, lds_addr(&sm.as[sbuf][64 * wave * 4]), soff);
      dma_x4(rsb, lds_addr(&sm.bs[sbuf][64 * wave * 4]), soff);
    } else {
      dma_x1(rsa, lds_addr(&sm.as[sbuf][64 * wave]), soff);
      dma_x1(rsb, lds_addr(&sm.bs[sbuf][64 * wave]), soff);
    }
  };
  auto loads_of = [](int s_mod) { return XCODE_LOADS + (s_mod == 0 ? 2 : 0); };

  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  // Stage st's fragments; the stage's two scale bytes sit in dword (st % U) / 2
  // of the row's SB-byte entry.
  auto read_frags = [&](int st, auto INC, XFrag& f) {
    constexpr int word = decltype(INC)::value / 2;
    const int slot = st % XNS, sbuf = (st / U) % NSB;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.sa[i] = sm.as[sbuf][(wm * 128 + i * 32 + r) * (SB / 4) + word];
#pragma unroll
    for (int j = 0; j < 4; ++j) f.sb[j] = sm.bs[sbuf][(wn * 128 + j * 32 + r) * (SB / 4) + word];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + r;
      f.alo[i] = sm.a[slot][xswz(row, g)];
      f.ahi[i] = sm.a[slot][xswz(row, 2 + g)];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + r;
      f.blo[j] = sm.b[slot][xswz(row, g)];
      f.bhi[j] = sm.b[slot][xswz(row, 2 + g)];
    }
  };

  // Scale operands of block b of a stage with parity P (which 16-bit half of
  // the dword holds the stage's bytes).
  float ssa[4], ssb[4];
  auto scales_of = [&](const XFrag& f, auto PC, auto BC) {
    constexpr int sh = 16 * decltype(PC)::value + 8 * decltype(BC)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) ssa[i] = e8m0_as_scale((f.sa[i] >> sh) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) ssb[j] = e8m0_as_scale((f.sb[j] >> sh) & 0xFFu);
  };
  auto expand = [&](const XFrag& f, int u, v8bf* av, v8bf* bv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t d0, d1;
      sub_dwords(f.alo[i], f.ahi[i], u, d0, d1);
      av[i] = expand8_bf16(d0, d1, ssa[i]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t d0, d1;
      sub_dwords(f.blo[j], f.bhi[j], u, d0, d1);
      bv[j] = expand8_bf16(d0, d1, ssb[j]);
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  auto mfmas = [&](const v8bf* av, const v8bf* bv) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], av[i], acc[i][j], 0, 0, 0);   // B first
  };
  // 16 groups of 1 MFMA, NV VALU and NL LDS reads
  auto interleave = [](auto NV, auto NL) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(NV)::value, 0);
      if (decltype(NL)::value) __builtin_amdgcn_sched_group_barrier(0x100, decltype(NL)::value, 0);
    }
  };
  using N0 = std::integral_constant<int, 0>;
  using N1 = std::integral_constant<int, 1>;
  using N2 = std::integral_constant<int, 2>;
  using N3 = std::integral_constant<int, 3>;

  XFrag f[2];
  v8bf cva[2][4], cvb[2][4];

  // Step kt (IN = kt % U, CUR = kt & 1, both static).  On entry f[CUR] holds
  // stage kt's fragments, ssa/ssb its block-0 scales and cva/cvb[0] its
  // sub-step 0 operands.
  auto step = [&](int kt, auto INC, auto CURC) {
    constexpr int IN = decltype(INC)::value;
    constexpr int CUR = decltype(CURC)::value;
    constexpr int P = IN % 2, PN = ((IN + 1) % U) % 2;
    constexpr int ISSUE_MOD = (IN + XNS - 1) % U;    // stage kt+3 within its scale batch
    // at the mid-step wait, stage kt+2 and the A half of stage kt+3 stay in flight
    constexpr int AFTER = loads_of((IN + 2) % U) + loads_of((IN + 3) % U) - 4;
    XFrag& fc = f[CUR];
    XFrag& fn = f[CUR ^ 1];
    // sub-step 0: A loads 0, 1 of stage kt+3 (and its scale batch) ahead of
    // the region; sub-step 1's operands converted under the MFMAs
    if constexpr (ISSUE_MOD == 0) issue_scales(kt + XNS - 1);
    issue_code(kt + XNS - 1, 0);
    issue_code(kt + XNS - 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(cva[0], cvb[0]);
    expand(fc, 1, cva[1], cvb[1]);
    interleave(N2{}, N0{});
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1: A loads 2, 3; block-1 scales and sub-step 2's operands
    issue_code(kt + XNS - 1, 2);
    issue_code(kt + XNS - 1, 3);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(cva[1], cvb[1]);
    scales_of(fc, std::integral_constant<int, P>{}, N1{});
    expand(fc, 2, cva[0], cvb[0]);
    interleave(N3{}, N0{});
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 landed; the B half of stage kt+3 goes out, then stage kt+1's
    // fragments are read under sub-step 2's MFMAs
    wait_vm_barrier<AFTER>();
#pragma unroll
    for (int u = 4; u < 8; ++u) issue_code(kt + XNS - 1, u);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(cva[0], cvb[0]);
    expand(fc, 3, cva[1], cvb[1]);
    read_frags(kt + 1, std::integral_constant<int, (IN + 1) % U>{}, fn);
    interleave(N2{}, N2{});
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 3: stage kt+1's block-0 scales and its sub-step 0 operands
    mfmas(cva[1], cvb[1]);
    scales_of(fn, std::integral_constant<int, PN>{}, N0{});
    expand(fn, 0, cva[0], cvb[0]);
    interleave(N3{}, N0{});
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: stages 0..2 (stage 0 carries the first scale batch); wait for stage 0
  static_for<0, XNS - 1>([&](auto SC) {
    constexpr int st = decltype(SC)::value;
    if constexpr (st % U == 0) issue_scales(st);
#pragma unroll
    for (int u = 0; u < 8; ++u) issue_code(st, u);
  });
  wait_vm_barrier<loads_of(1 % U) + loads_of(2 % U)>();
  read_frags(0, N0{}, f[0]);
  scales_of(f[0], N0{}, N0{});
  expand(f[0], 0, cva[0], cvb[0]);
  // Every step has the same shape, the last ones included: they issue
  // zero loads past KT and prepare "stage KT" (zeros), which is never used.
  for (int kt = 0; kt < KT; kt += U) {
    static_for<0, U>([&](auto IC) {
      constexpr int i = decltype(IC)::value;
      step(kt + i, std::integral_constant<int, i>{}, std::integral_constant<int, i & 1>{});
    });
  }

  // Epilogue: BF16 through the (now idle) A and B rings as whole row
  // segments (the MFMAs took the B operand first).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the out-of-range tail loads
  __syncthreads();                                   // every wave is done with the rings
  static_assert(sizeof(sm.a) + sizeof(sm.b) >= 4 * 128 * 256, "epilogue staging needs 32 KB per wave");
  store_block128_bf16<false>(acc, &sm.a[0][0] + wave * (128 * 16), C, M, N, m0 + wm * 128, n0 + wn * 128, 1.0f);
}

// ---------------------------------------------------------------------------
// Small-problem and any-K kernel: 64 x 64 output tiles, one 32 x 32 tile per
// wave, operands loaded from global memory (L2) straight into registers.  It
// serves grids under 32 tiles of 256 x 256 and K % 128 != 0.  Per 32-element
// block kb, lane (r, g) loads the 16 code bytes at K [32 kb + 16 g, + 16) of
// its A row and B row and the block's two scale bytes; MFMA 0 takes bytes
// 0..7, MFMA 1 bytes 8..15, so A and B pair the same K positions.
constexpr int SMALL_T = 64;
constexpr int X_SMALL_TILES = 32;

__global__ __launch_bounds__(256) void mx8x_small_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int tiles_n) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * SMALL_T + 32 * (wave & 1), n0 = tn * SMALL_T + 32 * (wave >> 1);
  const int KB = K / 32;
  // wave-uniform (readfirstlane), so the buffer resources stay scalar
  const int rows_a = __builtin_amdgcn_readfirstlane(max(0, min(32, M - m0)));
  const int rows_b = __builtin_amdgcn_readfirstlane(max(0, min(32, N - n0)));
  const auto ca = make_rsrc(A + (int64_t)max(0, min(m0, M)) * K, rows_a * K);
  const auto cb = make_rsrc(B + (int64_t)max(0, min(n0, N)) * K, rows_b * K);
  const auto sa = make_rsrc(As + (int64_t)max(0, min(m0, M)) * KB, rows_a * KB);
  const auto sb = make_rsrc(Bs + (int64_t)max(0, min(n0, N)) * KB, rows_b * KB);
  const int r = lane & 31, g = lane >> 5;
  v16f acc = v16f{};
  for (int kb0 = 0; kb0 < KB; kb0 += 4) {
    uint4 a[4], b[4];
    uint32_t xa[4], xb[4];
    // blocks past K load zeros (codes and scales): they add nothing
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool in = kb0 + q < KB;
      a[q] = buffer_load_x4(ca, in ? r * K + (kb0 + q) * 32 + 16 * g : OOB);
      b[q] = buffer_load_x4(cb, in ? r * K + (kb0 + q) * 32 + 16 * g : OOB);
      xa[q] = buffer_load_u8(sa, in ? r * KB + kb0 + q : OOB);
      xb[q] = buffer_load_u8(sb, in ? r * KB + kb0 + q : OOB);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float s_a = e8m0_as_scale(xa[q]), s_b = e8m0_as_scale(xb[q]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(expand8_bf16(a[q].x, a[q].y, s_a),
                                                    expand8_bf16(b[q].x, b[q].y, s_b), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(expand8_bf16(a[q].z, a[q].w, s_a),
                                                    expand8_bf16(b[q].z, b[q].w, s_b), acc, 0, 0, 0);
    }
  }
  const int col = n0 + r;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = m0 + (v >> 2) * 8 + g * 4 + (v & 3);
    if (row < M && col < N) C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[v]);
  }
}

}  // namespace

hipError_t launch_gemm_mxfp8_exact(int64_t m, int64_t n, int64_t k, const uint8_t* a, const uint8_t* as,
                                   const uint8_t* b, const uint8_t* bs, uint16_t* c, hipStream_t stream) {
  const int tiles_m = (int)ceil_div(m, BM), tiles_n = (int)ceil_div(n, BN);
  if (k > 0 && tiles_m * tiles_n >= X_SMALL_TILES && k % 512 == 0)
    hipLaunchKernelGGL((mx8x_ring_kernel<16>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a, as, b, bs, c,
                       (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else if (k > 0 && tiles_m * tiles_n >= X_SMALL_TILES && k % 128 == 0)
    hipLaunchKernelGGL((mx8x_ring_kernel<4>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a, as, b, bs, c,
                       (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else {
    const int sm = (int)ceil_div(m, SMALL_T), sn = (int)ceil_div(n, SMALL_T);
    hipLaunchKernelGGL(mx8x_small_kernel, dim3(sm * sn), dim3(256), 0, stream, a, as, b, bs, c, (int)m, (int)n,
                       (int)k, sn);
  }
  return hipGetLastError();
}

}  // namespace bsg
