// NVFP4, MXFP8 and MXFP4 quantizers (HBM-bound streaming kernels).
//
// Recipes: the problem statement of this library (header bsgemm.h).
// Formats named on "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA
// Vera Rubin NVL72", section "Building the GEMM" (NVFP4, FP8 E4M3), and on
// "Triton #11171 ...", section "The broader related matrix protected
// neighboring policy" (MXFP).
//
// Both inputs are flat: X[rows][k] with k % 32 == 0, so no 16- or 32-element
// block straddles a row.  Element i of the flat array belongs to block
// i / 16 (NVFP4) or i / 32 (MX formats), and that is also the flat index of
// its scale byte.  Each thread owns 8 consecutive elements: two 16-byte loads,
// one 4-byte (FP4) or 8-byte (FP8) code store.  The 2 (NVFP4) or 4 (MX)
// threads of a block combine their maxima with lane shuffles.
//
// Bit-exactness: every FP32 step uses the correctly rounded __fdiv_rn and
// __fmul_rn, and this file is compiled with -ffp-contract=off.
#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

constexpr int QTHREADS = 256;

__device__ __forceinline__ float max8_abs(const float4& a, const float4& b) {
  float m = fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
  return fmaxf(m, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

__device__ __forceinline__ uint32_t signbit_u32(float x) { return __float_as_uint(x) >> 31; }

// ------------------------------------------------------------------ MX formats

// Block exponent e = min{e : top * 2^e >= bamax}, clamped to [-127, 127],
// for the element format's largest value top = 1.t * 2^ET: 448 = 1.75 * 2^8
// (E4M3), 6 = 1.5 * 2^2 (E2M1).  For bamax = 1.f * 2^E, e = E - ET if
// 1.f <= 1.t, else E - ET + 1.  Zero and FP32 subnormals fall below -127 and
// clamp.  Finite inputs give e <= 126, so 2^-e is a normal float.
template <bool FP4>
__device__ __forceinline__ int mx_block_exponent(float bamax) {
  constexpr int ET = FP4 ? 2 : 8;
  constexpr uint32_t TMANT = FP4 ? 0x400000u : 0x600000u;
  const uint32_t u = __float_as_uint(bamax);
  const int E = (int)(u >> 23) - 127;
  int e = E - ET + (((u & 0x7FFFFFu) > TMANT) ? 1 : 0);
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// |x| * 2^-e is exact unless it falls below 2^-126, where it encodes to 0
// either way.  E2M1 never saturates here (|x| * 2^-e <= 6 by the choice of
// e); E4M3 does not either.
__device__ __forceinline__ uint32_t mx8_code(float x, float inv) {
  return (signbit_u32(x) << 7) | e4m3_encode_mag(__fmul_rn(fabsf(x), inv));
}
__device__ __forceinline__ uint32_t mx4_code(float x, float inv) {
  return (signbit_u32(x) << 3) | e2m1_encode_mag(__fmul_rn(fabsf(x), inv));
}

// Codes of 8 consecutive elements: 8 bytes (FP8) or 8 nibbles, element 0 in
// the lowest (FP4).
template <bool FP4> struct MxOut;
template <> struct MxOut<false> {
  typedef uint2 type;
  static __device__ __forceinline__ uint2 pack(const float4& a, const float4& b, float inv) {
    uint2 o;
    o.x = mx8_code(a.x, inv) | (mx8_code(a.y, inv) << 8) | (mx8_code(a.z, inv) << 16) | (mx8_code(a.w, inv) << 24);
    o.y = mx8_code(b.x, inv) | (mx8_code(b.y, inv) << 8) | (mx8_code(b.z, inv) << 16) | (mx8_code(b.w, inv) << 24);
    return o;
  }
};
template <> struct MxOut<true> {
  typedef uint32_t type;
  static __device__ __forceinline__ uint32_t pack(const float4& a, const float4& b, float inv) {
    return mx4_code(a.x, inv) | (mx4_code(a.y, inv) << 4) | (mx4_code(a.z, inv) << 8) |
           (mx4_code(a.w, inv) << 12) | (mx4_code(b.x, inv) << 16) | (mx4_code(b.y, inv) << 20) |
           (mx4_code(b.z, inv) << 24) | (mx4_code(b.w, inv) << 28);
  }
};

template <bool FP4>
__global__ __launch_bounds__(QTHREADS) void quantize_mx_kernel(
    const float4* __restrict__ x, typename MxOut<FP4>::type* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t n_oct) {
  const int64_t stride = (int64_t)gridDim.x * QTHREADS;
  for (int64_t o = (int64_t)blockIdx.x * QTHREADS + threadIdx.x; o - (threadIdx.x & 3) < n_oct;
       o += stride) {
    // Every thread of a 4-thread group runs the loop body together (the
    // shuffles below need all four); n_oct is a multiple of 4.
    const bool live = o < n_oct;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (live) { a = x[2 * o]; b = x[2 * o + 1]; }
    float m = max8_abs(a, b);
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int e = mx_block_exponent<FP4>(m);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, normal
    const auto out = MxOut<FP4>::pack(a, b, inv);
    if (live) {
      codes[o] = out;
      if ((threadIdx.x & 3) == 0) scales[o >> 2] = (uint8_t)(e + 127);
    }
  }
}

// ------------------------------------------------------------------ NVFP4

__global__ void nvfp4_reset_kernel(uint32_t* slot) { *slot = 0u; }

// amax over the tensor: per-workgroup maximum, then one atomic max on the
// FP32 bits in the slot.  For non-negative floats the unsigned order of the
// bit patterns is the numeric order.
__global__ __launch_bounds__(QTHREADS) void nvfp4_amax_kernel(const float4* __restrict__ x,
                                                              int64_t n4, uint32_t* slot) {
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * QTHREADS;
  for (int64_t i = (int64_t)blockIdx.x * QTHREADS + threadIdx.x; i < n4; i += stride) {
    const float4 v = x[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wmax[QTHREADS / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int w = 1; w < QTHREADS / 64; ++w) b = fmaxf(b, wmax[w]);
    atomicMax(slot, __float_as_uint(b));
  }
}

// s_t = fl32(amax / 2688) written over the amax bits.
__global__ void nvfp4_finalize_kernel(uint32_t* slot) {
  const float amax = __uint_as_float(*slot);
  *reinterpret_cast<float*>(slot) = __fdiv_rn(amax, 2688.0f);
}

__device__ __forceinline__ uint32_t nv_code(float x, float S) {
  const uint32_t mag = (S == 0.0f) ? 0u : e2m1_encode_mag(__fdiv_rn(fabsf(x), S));
  return (signbit_u32(x) << 3) | mag;
}

__global__ __launch_bounds__(QTHREADS) void nvfp4_encode_kernel(
    const float4* __restrict__ x, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, int64_t n_oct) {
  const float s_t = *tscale;
  const int64_t stride = (int64_t)gridDim.x * QTHREADS;
  for (int64_t o = (int64_t)blockIdx.x * QTHREADS + threadIdx.x; o - (threadIdx.x & 1) < n_oct;
       o += stride) {
    const bool live = o < n_oct;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (live) { a = x[2 * o]; b = x[2 * o + 1]; }
    float m = max8_abs(a, b);
    m = fmaxf(m, __shfl_xor(m, 1));
    uint32_t sc = 0u;
    if (s_t != 0.0f) sc = e4m3_encode_mag(__fdiv_rn(__fdiv_rn(m, 6.0f), s_t));
    const float S = __fmul_rn(e4m3_decode_mag(sc), s_t);
    const uint32_t w = nv_code(a.x, S) | (nv_code(a.y, S) << 4) | (nv_code(a.z, S) << 8) |
                       (nv_code(a.w, S) << 12) | (nv_code(b.x, S) << 16) |
                       (nv_code(b.y, S) << 20) | (nv_code(b.z, S) << 24) |
                       (nv_code(b.w, S) << 28);
    if (live) {
      codes[o] = w;
      if ((threadIdx.x & 1) == 0) scales[o >> 1] = (uint8_t)sc;
    }
  }
}

int grid_for(int64_t work_items, int num_cus) {
  int64_t g = ceil_div(work_items, QTHREADS);
  const int64_t cap = (int64_t)num_cus * 16;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

template <bool FP4>
hipError_t launch_quantize_mx(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream, int num_cus) {
  const int64_t n_oct = rows * k / 8;
  if (n_oct == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mx_kernel<FP4>, dim3(grid_for(n_oct, num_cus)), dim3(QTHREADS), 0,
                     stream, reinterpret_cast<const float4*>(x),
                     reinterpret_cast<typename MxOut<FP4>::type*>(codes), scales, n_oct);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mxfp8(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream, int num_cus) {
  return launch_quantize_mx<false>(rows, k, x, codes, scales, stream, num_cus);
}

hipError_t launch_quantize_mxfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream, int num_cus) {
  return launch_quantize_mx<true>(rows, k, x, codes, scales, stream, num_cus);
}

hipError_t launch_quantize_nvfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                                 uint8_t* scales, float* tensor_scale, hipStream_t stream,
                                 int num_cus) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(tensor_scale);
  const int64_t n = rows * k;
  hipLaunchKernelGGL(nvfp4_reset_kernel, dim3(1), dim3(1), 0, stream, slot);
  if (n > 0) {
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(grid_for(n / 4, num_cus)), dim3(QTHREADS), 0,
                       stream, reinterpret_cast<const float4*>(x), n / 4, slot);
  }
  hipLaunchKernelGGL(nvfp4_finalize_kernel, dim3(1), dim3(1), 0, stream, slot);
  if (n > 0) {
    hipLaunchKernelGGL(nvfp4_encode_kernel, dim3(grid_for(n / 8, num_cus)), dim3(QTHREADS), 0,
                       stream, reinterpret_cast<const float4*>(x),
                       reinterpret_cast<uint32_t*>(codes), scales, tensor_scale, n / 8);
  }
  return hipGetLastError();
}

}  // namespace bsg
