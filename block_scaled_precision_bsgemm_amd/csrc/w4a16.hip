// Small-M weight-only 4-bit GEMM: BF16 activations X[M][K] x NVFP4 weights
// W[N][K], BF16 output.
//
// Source: "Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic"
// (bitsandbytes PR #2030), sections "Methodology" and "The SIMT / MMA layer".
// That PR measures a fused dequant+GEMM against dequantise-then-linear, and a
// SIMT (vector ALU) kernel against a matrix-core kernel at small M.  Here:
//   - m == 1: gemv_kernel.  Vector ALU only.  Each 16-element block's dot
//     product is taken on the unscaled E2M1 values (exact in BF16, via fdot2);
//     the block's full E4M3 scale is applied once, in FP32.
//   - m >= 2: mfma_kernel.  W fragments go straight from HBM into registers,
//     are dequantised exactly to BF16 and meet X on the 16x16x32 BF16 MFMA.
//     The 4 waves of a workgroup split K; partial tiles are summed through LDS.
// Either way, every weight byte is read from HBM once per M tile; X is small
// and stays in L2.
#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ m == 1

constexpr int GV_THREADS = 256;
constexpr int GV_ROWS_PER_WAVE = 4;
constexpr int GV_ROWS = (GV_THREADS / 64) * GV_ROWS_PER_WAVE;   // rows per workgroup
constexpr int GV_CHUNK = 64 * 64;                               // K elements per wave pass

template <int J>
__device__ __forceinline__ float dot_e2m1_pair(uint32_t codes, uint32_t xpair, float acc) {
  const v2bf_t w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, J);   // exact
  v2bf_t xv;
  __builtin_memcpy(&xv, &xpair, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(w, xv, acc, false);
}

// Sum over one 16-element block: two code dwords, eight X pairs.
__device__ __forceinline__ float block_dot(uint32_t c0, uint32_t c1, const uint4& x0, const uint4& x1) {
  float p = 0.0f;
  p = dot_e2m1_pair<0>(c0, x0.x, p);
  p = dot_e2m1_pair<1>(c0, x0.y, p);
  p = dot_e2m1_pair<2>(c0, x0.z, p);
  p = dot_e2m1_pair<3>(c0, x0.w, p);
  p = dot_e2m1_pair<0>(c1, x1.x, p);
  p = dot_e2m1_pair<1>(c1, x1.y, p);
  p = dot_e2m1_pair<2>(c1, x1.z, p);
  p = dot_e2m1_pair<3>(c1, x1.w, p);
  return p;
}

// Lane l of a wave handles K elements [kc + 64 l, kc + 64 l + 64) of every
// chunk kc, as two halves of 32 (K % 32 == 0, so a half is wholly in or out).
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wc, const uint8_t* __restrict__ Ws,
    const float* __restrict__ Wts, uint16_t* __restrict__ C, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nbase = blockIdx.x * GV_ROWS + wave * GV_ROWS_PER_WAVE;
  const int KH = K / 2, KB = K / 16;
  const int rows = max(0, min(N - nbase, GV_ROWS_PER_WAVE));
  const auto c_rsrc = make_rsrc(Wc + (int64_t)nbase * KH, rows * KH);
  const auto s_rsrc = make_rsrc(Ws + (int64_t)nbase * KB, rows * KB);
  const auto x_rsrc = make_rsrc(X, K * 2);
  float acc[GV_ROWS_PER_WAVE] = {};
  for (int kc = 0; kc < K; kc += GV_CHUNK) {
    const int k0 = kc + 64 * lane;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kh = k0 + 32 * h;
      if (kh >= K) break;
      uint4 x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = buffer_load_x4(x_rsrc, (kh + 8 * q) * 2);
      uint4 cw[GV_ROWS_PER_WAVE];
      uint32_t sw[GV_ROWS_PER_WAVE];
#pragma unroll
      for (int rr = 0; rr < GV_ROWS_PER_WAVE; ++rr) {
        // 16 code bytes (32 elements) and 2 scale bytes per row
        const uint4 v = buffer_load_x4(c_rsrc, rr * KH + kh / 2);
        cw[rr] = v;
        sw[rr] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, rr * KB + kh / 16, 0, 0);
      }
#pragma unroll
      for (int rr = 0; rr < GV_ROWS_PER_WAVE; ++rr) {
        const float s0 = e4m3_scale_value(sw[rr] & 0xFFu);
        const float s1 = e4m3_scale_value((sw[rr] >> 8) & 0xFFu);
        acc[rr] = fmaf(block_dot(cw[rr].x, cw[rr].y, x[0], x[1]), s0, acc[rr]);
        acc[rr] = fmaf(block_dot(cw[rr].z, cw[rr].w, x[2], x[3]), s1, acc[rr]);
      }
    }
  }
  const float ts = *Wts;
#pragma unroll
  for (int rr = 0; rr < GV_ROWS_PER_WAVE; ++rr) {
    float v = acc[rr];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == rr && rr < rows) C[nbase + rr] = (uint16_t)f32_to_bf16_rne(v * ts);
  }
}

// ------------------------------------------------------------------ m >= 2

constexpr int MM_THREADS = 256;
constexpr int MM_NB = 32;   // weight rows (output columns) per workgroup

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

// K assignment (W and X agree): in each 128-element step, lane (r = l % 16,
// q = l / 16) takes elements [32q, 32q + 32).  Dword sp of those 32 feeds MFMA
// sub-step sp at positions 8q..8q+7, with scale block 2q + sp/2.
template <int MT>
__global__ __launch_bounds__(MM_THREADS, 1) void mfma_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wc, const uint8_t* __restrict__ Ws,
    const float* __restrict__ Wts, uint16_t* __restrict__ C, int M, int N, int K) {
  constexpr int NI = MM_NB / 16, NJ = MT / 16;
  __shared__ v4f red[3][NI * NJ][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * MM_NB, m0 = blockIdx.y * MT;
  const int KH = K / 2, KB = K / 16;
  const int rows_w = min(N - n0, MM_NB), rows_x = min(M - m0, MT);
  const auto c_rsrc = make_rsrc(Wc + (int64_t)n0 * KH, rows_w * KH);
  const auto s_rsrc = make_rsrc(Ws + (int64_t)n0 * KB, rows_w * KB);
  const auto x_rsrc = make_rsrc(X + (int64_t)m0 * K, rows_x * K * 2);
  // this wave's K range: a quarter of the 128-element steps
  const int steps = (K + 127) / 128;
  const int per = (steps + 3) / 4;
  const int s_begin = wave * per, s_end = min(steps, s_begin + per);

  v4f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{};

  for (int st = s_begin; st < s_end; ++st) {
    const int kq = st * 128 + 32 * q;          // first K element of this lane
    const bool kin = kq < K;                   // K % 32 == 0: 32 elements wholly in or out
    uint4 wc[NI];
    uint32_t ws[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = 16 * i + r;
      wc[i] = buffer_load_x4(c_rsrc, kin ? row * KH + kq / 2 : OOB);
      ws[i] = buffer_load_u16(s_rsrc, kin ? row * KB + kq / 16 : OOB);
    }
    uint4 xv[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int sp = 0; sp < 4; ++sp)
        xv[j][sp] = buffer_load_x4(x_rsrc, kin ? ((16 * j + r) * K + kq + 8 * sp) * 2 : OOB);
    float s[NI][2], mant[NI][2];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[i][b] = e4m3_scale_value((ws[i] >> (8 * b)) & 0xFFu);
        mant[i][b] = scale_mantissa_f32(s[i][b]);
      }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      v8bf_t wv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t d = sp == 0 ? wc[i].x : sp == 1 ? wc[i].y : sp == 2 ? wc[i].z : wc[i].w;
        const v8bf w8 = dequant8_bf16(d, s[i][sp >> 1], mant[i][sp >> 1]);
        __builtin_memcpy(&wv[i], &w8, 16);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        v8bf_t x8;
        __builtin_memcpy(&x8, &xv[j][sp], 16);
#pragma unroll
        for (int i = 0; i < NI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[i], x8, acc[i][j], 0, 0, 0);
      }
    }
  }

  // sum the four waves' partial tiles
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) red[wave - 1][i * NJ + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave == 0) {
    const float ts = *Wts;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        v4f v = acc[i][j];
#pragma unroll
        for (int w = 0; w < 3; ++w) v += red[w][i * NJ + j][lane];
        // D[n][m] lane layout: column m = 16 j + r, rows n = 16 i + 4 q + e
        const int m = m0 + 16 * j + r;
        if (m < M) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = n0 + 16 * i + 4 * q + e;
            if (n < N) C[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v[e] * ts);
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_w4a16(int64_t m, int64_t n, int64_t k, const uint16_t* x, const uint8_t* w,
                        const uint8_t* ws, const float* wts, uint16_t* c, hipStream_t stream) {
  if (m == 1) {
    hipLaunchKernelGGL(gemv_kernel, dim3((unsigned)ceil_div(n, GV_ROWS)), dim3(GV_THREADS), 0,
                       stream, x, w, ws, wts, c, (int)n, (int)k);
  } else if (m <= 16) {
    hipLaunchKernelGGL(mfma_kernel<16>, dim3((unsigned)ceil_div(n, MM_NB), (unsigned)ceil_div(m, 16)),
                       dim3(MM_THREADS), 0, stream, x, w, ws, wts, c, (int)m, (int)n, (int)k);
  } else {
    hipLaunchKernelGGL(mfma_kernel<64>, dim3((unsigned)ceil_div(n, MM_NB), (unsigned)ceil_div(m, 64)),
                       dim3(MM_THREADS), 0, stream, x, w, ws, wts, c, (int)m, (int)n, (int)k);
  }
  return hipGetLastError();
}

}  // namespace bsg
