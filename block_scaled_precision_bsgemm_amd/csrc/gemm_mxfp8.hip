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

}  // namespace

hipError_t launch_gemm_mxfp8(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* c,
                             hipStream_t stream) {
  const int tiles_m = (int)ceil_div(m, BM), tiles_n = (int)ceil_div(n, BN);
  if (k % 128 == 0)
    hipLaunchKernelGGL(mxfp8_gemm_kernel<true>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(mxfp8_gemm_kernel<false>, dim3(tiles_m * tiles_n), dim3(NT), 0, stream, a,
                       as, b, bs, c, (int)m, (int)n, (int)k, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bsg
