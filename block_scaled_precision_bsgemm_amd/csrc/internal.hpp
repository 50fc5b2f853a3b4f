// Host-side launchers of the bsgemm kernels.  Arguments are validated by the
// C ABI layer (api.cpp) before any of these is called; the launchers only
// choose a configuration and enqueue kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

hipError_t launch_quantize_mxfp8(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream, int num_cus);
hipError_t launch_quantize_mxfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream, int num_cus);
hipError_t launch_quantize_nvfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                                 uint8_t* scales, float* tensor_scale, hipStream_t stream,
                                 int num_cus);

hipError_t launch_gemm_mxfp8(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* c,
                             hipStream_t stream);
// MXFP8 operands, products expanded exactly to BF16, BF16 MFMA (FP32 accumulation).
hipError_t launch_gemm_mxfp8_exact(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                                   const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* c,
                                   hipStream_t stream);
hipError_t launch_gemm_mxfp4(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* c,
                             hipStream_t stream);
hipError_t launch_gemm_nvfp4(int64_t m, int64_t n, int64_t k, const uint8_t* a,
                             const uint8_t* as, const float* ats, const uint8_t* b,
                             const uint8_t* bs, const float* bts, uint16_t* c,
                             hipStream_t stream);
// One grouped launch: bias, gamma, gather and scatter may be null; w holds
// BF16 (w_f16 false) or FP16 bit patterns.
struct GroupedCall {
  int num_groups;
  int64_t m_total, a_rows, n, k;
  const uint8_t* a;
  const uint8_t* as;
  const float* ats;
  const int32_t* offsets;
  const uint16_t* w;
  bool w_f16;
  const float* bias;
  const float* gamma;
  const int32_t* gather;
  const int32_t* scatter;
  uint16_t* c;
};
hipError_t launch_grouped(const GroupedCall& call, hipStream_t stream);
// Workgroups launch_grouped launches for these sizes (an upper bound on the
// tile count; surplus workgroups exit at once).
int64_t grouped_grid_blocks(int num_groups, int64_t m_total, int64_t n, int64_t k);

// One K-ragged (inner-expert) grouped launch: k % 256 == 0; k_offsets on the
// device; c is [num_groups][m][n].
struct KRaggedCall {
  int num_groups;
  int64_t m, n, k;
  const uint8_t* a;
  const uint8_t* as;
  const float* ats;
  const int32_t* k_offsets;
  const uint16_t* w;
  bool w_f16;
  uint16_t* c;
};
hipError_t launch_grouped_kragged(const KRaggedCall& call, hipStream_t stream);
// W4A16 configurations: count, names, largest m each accepts, the selector,
// and a launch of one configuration (config must be a valid id).
int w4a16_num_configs();
const char* w4a16_config_name(int config);
int w4a16_config_max_m(int config);
// K must be a multiple of this for the configuration (32, or 256 for the tile kernels)
int w4a16_config_k_multiple(int config);
int w4a16_select(int64_t m, int64_t n, int64_t k);
// The W4A16 tile kernel (w4a16_tile.hip): shape 0 = 16 x 64, 1 = 64 x 64, 2 = 128 x 128 (m x n);
// k must be a multiple of w4_tile_k_multiple(shape) (its K per ring stage).
int w4_tile_k_multiple(int shape);
hipError_t launch_w4_tile(int shape, int64_t m, int64_t n, int64_t k, const uint16_t* x, const uint8_t* w,
                          const uint8_t* ws, const float* wts, uint16_t* c, hipStream_t stream);
hipError_t launch_w4a16(int config, int64_t m, int64_t n, int64_t k, const uint16_t* x, const uint8_t* w,
                        const uint8_t* ws, const float* wts, uint16_t* c, hipStream_t stream);

}  // namespace bsg
