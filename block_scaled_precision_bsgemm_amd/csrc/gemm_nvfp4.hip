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
//   - the scaled FP4->FP16 conversion supplies the scale's power of two;
//   - one packed FP16 multiply supplies (1 + f);
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

struct Scale2 {
  float s;        // E4M3 scale as FP32 (its exponent drives the conversion)
  uint32_t m2;    // (1 + f) as an FP16 pair
};

__device__ __forceinline__ Scale2 decode_scale(uint32_t byte) {
  Scale2 d;
  d.s = e4m3_scale_value(byte);
  d.m2 = scale_mantissa_f16x2(d.s);
  return d;
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
      Scale2 da[4][2], db[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r;
        ca[i] = sm.a[buf][swz(row, 2 * h + g)];
        const uint2 sc = sm.as[buf][row];
        const uint32_t w = h ? sc.y : sc.x;           // blocks 4h .. 4h+3
        da[i][0] = decode_scale((w >> (16 * g)) & 0xFFu);
        da[i][1] = decode_scale((w >> (16 * g + 8)) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + r;
        cb[j] = sm.b[buf][swz(row, 2 * h + g)];
        const uint2 sc = sm.bs[buf][row];
        const uint32_t w = h ? sc.y : sc.x;
        db[j][0] = decode_scale((w >> (16 * g)) & 0xFFu);
        db[j][1] = decode_scale((w >> (16 * g + 8)) & 0xFFu);
      }
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        v8h av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t d = sp == 0 ? ca[i].x : sp == 1 ? ca[i].y : sp == 2 ? ca[i].z : ca[i].w;
          av[i] = dequant8_f16(d, da[i][sp >> 1].s, da[i][sp >> 1].m2);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t d = sp == 0 ? cb[j].x : sp == 1 ? cb[j].y : sp == 2 ? cb[j].z : cb[j].w;
          bv[j] = dequant8_f16(d, db[j][sp >> 1].s, db[j][sp >> 1].m2);
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

}  // namespace

hipError_t launch_gemm_nvfp4(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const float* ats, const uint8_t* b,
                             const uint8_t* bs, const float* bts, uint16_t* c,
                             hipStream_t stream) {
  const int tiles_m = (int)ceil_div(m, BM), tiles_n = (int)ceil_div(n, BN);
  if (k % 128 == 0)
    hipLaunchKernelGGL(nvfp4_gemm_kernel<true>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, ats, b, bs, bts, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(nvfp4_gemm_kernel<false>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, ats, b, bs, bts, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bsg
