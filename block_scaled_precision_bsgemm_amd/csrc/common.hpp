// Shared device helpers for the bsgemm kernels (gfx950 / CDNA4).
//
// The codecs below encode and decode the element and scale formats with integer
// operations on IEEE binary32 bit patterns:
//   - E2M1, E4M3 (FN) and E8M0, as in the OCP Microscaling Formats (MX) v1.0 spec;
//   - BF16.
// Every encoder rounds to nearest with ties to even and saturates at the
// format's largest finite value, so the quantizers are bit-exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bsg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v8us __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ encoders

// |a| -> 7-bit E4M3 magnitude code.  RNE, saturating at 0x7E (448).
// Below 2^-6 the E4M3 grid is uniform with step 2^-9: scale by 512 (exact) and
// round to an integer (ties to even).  At and above 2^-6, keep 3 mantissa bits
// of the binary32 pattern with a round-half-even carry, then rebias the
// exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode_mag(float a) {
  const uint32_t u = __float_as_uint(a);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;   // [exp8 | mant3]
  const uint32_t nrm = r - (120u << 3);
  const uint32_t c = (a < 0.015625f) ? sub : nrm;
  return c > 0x7Eu ? 0x7Eu : c;
}

// |a| -> 3-bit E2M1 magnitude code.  RNE, saturating at 7 (6.0).
// Below 1 the grid is uniform with step 0.5.  At and above 1, keep 1 mantissa
// bit and rebias the exponent from 127 to 1.
__device__ __forceinline__ uint32_t e2m1_encode_mag(float a) {
  const uint32_t u = __float_as_uint(a);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 2.0f);
  const uint32_t r = (u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22;  // [exp8 | mant1]
  const uint32_t nrm = r - (126u << 1);
  const uint32_t c = (a < 1.0f) ? sub : nrm;
  return c > 7u ? 7u : c;
}

// ------------------------------------------------------------------ decoders

// E4M3 magnitude code (0..0x7E) -> its exact FP32 value.
__device__ __forceinline__ float e4m3_decode_mag(uint32_t c) {
  const float nrm = __uint_as_float((c + 960u) << 20);   // rebias exponent 7 -> 127
  const float sub = (float)c * 0.001953125f;             // c * 2^-9, exact
  return c < 8u ? sub : nrm;
}

// Bytes 0 and 1 of `word` as two exact E4M3 (FN) values in FP32, signs
// included; the NaN codes 0x7F and 0xFF give NaN.
__device__ __forceinline__ v2f e4m3_pair_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, false);
}

// Bytes 0 and 1 of `word` as two E4M3 values in an FP16 pair (byte 0 in bits
// 15:0).  Exact: every E4M3 value, subnormals included, is an FP16 normal or
// zero.
__device__ __forceinline__ uint32_t e4m3_pair_f16(uint32_t word) {
  const v2h h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// ---------------------------------------------------------------------- BF16

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two FP32 -> packed BF16 pair (lo in bits 15:0), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Two FP32 values -> packed BF16 pair (lo in bits 15:0) by gfx950's pair
// conversion (v_cvt_pk_bf16_f32): round to nearest even, the same bits as
// pack_bf16x2 for finite inputs, in one instruction.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
  const v2bf16 r = __builtin_convertvector((v2f){lo, hi}, v2bf16);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// ------------------------------------------------------- FP4 -> 16-bit dequant
//
// A block-scaled element is e2m1(code) * e4m3(scale).  Both factors are
// decoded exactly (the FP4 conversions at scale 1.0 give the code values)
// and multiplied once: the product has at most 6 significant bits and its
// magnitude is zero or in [2^-10, 2688], so it is exact in FP16, BF16 and
// FP32.  The scale keeps its sign; a NaN scale code gives NaN products.

// Eight E2M1 codes (one dword; element j in nibble j) as exact FP16 values.
__device__ __forceinline__ v8h e2m1x8_f16(uint32_t codes) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  v8h out;
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
  return out;
}

// v times the scale in half `b` (0 or 1; a constant once inlined) of the FP16
// pair `pair` (e4m3_pair_f16): four packed multiplies with the scale half
// selected by the instruction's operand select.
__device__ __forceinline__ v8h scale8_f16(const v8h& v, uint32_t pair, int b) {
  v2h m;
  __builtin_memcpy(&m, &pair, 4);
  const _Float16 s = b ? m[1] : m[0];
  const v8h mm = {s, s, s, s, s, s, s, s};
  return v * mm;
}

// Eight E2M1 codes times the E4M3 scale in half `b` of `pair`, exact FP16.
__device__ __forceinline__ v8h dequant8_f16(uint32_t codes, uint32_t pair, int b) {
  return scale8_f16(e2m1x8_f16(codes), pair, b);
}

// Two E2M1 codes (pair J of the dword) times the E4M3 scale `s` (FP32),
// packed as BF16 (low element in bits 15:0): the FP32 products are exact and
// their high halves are the BF16 patterns, packed by one byte permute.
template <int J>
__device__ __forceinline__ uint32_t dequant2_bf16(uint32_t codes, float s) {
  const v2f p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, J);
  return __builtin_amdgcn_perm(__float_as_uint(p[1] * s), __float_as_uint(p[0] * s), 0x07060302u);
}

__device__ __forceinline__ v8bf dequant8_bf16(uint32_t codes, float s) {
  const uint32_t w[4] = {dequant2_bf16<0>(codes, s), dequant2_bf16<1>(codes, s),
                         dequant2_bf16<2>(codes, s), dequant2_bf16<3>(codes, s)};
  v8bf out;
  __builtin_memcpy(&out, w, 16);
  return out;
}

// ----------------------------------------------------------- buffer loads

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads at offsets outside it
// return zero.  `bytes` must be < 2^31.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load_x4(rsrc_t r, int off) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// The same with cache policy nt (streaming), for data that one launch reads
// exactly once: it then does not evict data that the launch re-reads.
__device__ __forceinline__ uint4 buffer_load_x4_nt(rsrc_t r, int off) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t buffer_load_u32(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_load_u8(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_load_u16(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

__device__ __forceinline__ uint2 buffer_load_x2(rsrc_t r, int off) {
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
}

// An offset past every resource this library builds (all are < 2^31 bytes):
// a buffer load there returns zero without touching memory.  Selecting it
// instead of branching keeps loads unconditional, so the compiler never has
// to wait for them inside the issuing block.
constexpr int OOB = 0x7FFFFFF0;

// --------------------------------------------------------- direct-to-LDS loads

// Buffer resource as an SGPR quad, for inline assembly.  Same layout as
// make_rsrc: base address, stride 0, `bytes` records, raw (untyped) access.
typedef int rsrc4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc4_t make_rsrc4(const void* base, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  rsrc4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}

// Direct global->LDS loads (buffer_load ... lds): lane l's 16 (or 4) bytes
// from `voff` within the resource land in LDS at lds_base + 16 l (4 l), where
// lds_base is wave-uniform.  Offsets past the resource write zeros.
//
// They are issued from inline assembly on purpose.  The compiler cannot tell
// which LDS bytes such a load writes, so for its own builtin it waits for all
// outstanding loads before every later LDS read, which serialises a
// multi-stage ring.  Hidden in assembly, the loads are invisible to its wait
// insertion.  The kernel waits for them itself (vmcnt) before the barrier that
// publishes a stage.  The compiler never holds a value in m0 in these
// kernels; the assembly sets m0 itself, with the one wait state that an LDS
// DMA load needs after a scalar write of m0 (the compiler puts the same
// s_nop 0 there for its own LDS DMA builtins on gfx950).
__device__ __forceinline__ void dma_x4(rsrc4_t rsrc, uint32_t lds_base, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// The same with a wave-uniform scalar offset added to the address.  Callers
// keep the whole address (vector + scalar offset) of every load that must
// read data inside the resource, and pass an empty resource (0 bytes) for
// loads that must read zero, so the result does not depend on whether the
// range check counts the scalar offset.
__device__ __forceinline__ void dma_x4_so(rsrc4_t rsrc, uint32_t lds_base, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma_x1_so(rsrc4_t rsrc, uint32_t lds_base, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma_x1(rsrc4_t rsrc, uint32_t lds_base, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}

// Wait until at most N of this wave's vector-memory loads are outstanding and
// all of its LDS reads have returned, then cross the workgroup barrier.  After
// it, every wave's loads up to that point have landed in LDS, and no wave
// still reads an LDS slot that the next direct loads may overwrite.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// ------------------------------------------------------------------ epilogue

// Streaming (non-temporal) stores for GEMM outputs, which no tile of the
// launch reads back: the output stream then does not evict the operand
// panels that neighbouring tiles still share through L2 (32-expert K-ragged
// problem, 940 MB of C: 707 -> 633 us; MXFP8 4096^3 -5%, MXFP4 16384^3 -2%;
// bit-identical output).  Only for stores that write whole 64-byte or longer
// row segments per instruction: streaming writes of 8- or 16-byte pieces of
// many lines made the same kernel 4-6x slower, so the element-wise edge
// paths keep plain stores.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void* p, const uint4& v) {
  const u32x4_t x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_nt2(uint16_t* p, uint16_t v) { __builtin_nontemporal_store(v, p); }

// Stores one wave's 128 x 128 block of FP32 accumulators to C as BF16 through
// LDS.  acc[i][j] is the 32 x 32 MFMA tile (i, j) computed with the column
// operand first, so lane (r, g) holds row 32 i + r and, at acc[i][j][4 q + e],
// column 32 j + 8 q + 4 g + e.  The lanes write their 4-column pieces (scaled
// by alpha when SCALE) as BF16 pairs into the wave's private 32 KB at `eb`
// (128 rows of 256 bytes, 16-byte chunks swizzled by the row), then read
// back 16-byte row chunks and store 4 whole 256-byte row segments per
// instruction, instead of one 2-byte store per element.  C block origin
// (row0, col0); rows >= M and columns >= N are not stored.  The caller makes
// sure nothing else reads or writes `eb` meanwhile.
template <bool SCALE>
__device__ __forceinline__ void store_block128_bf16(const v16f (&acc)[4][4], uint4* eb, uint16_t* C, int M, int N,
                                                    int row0, int col0, float alpha) {
  const int lane = threadIdx.x & 63, r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * i + r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = SCALE ? acc[i][j][4 * q + e] * alpha : acc[i][j][4 * q + e];
        const int chunk = 4 * j + q;
        uint2* d = reinterpret_cast<uint2*>(eb + row * 16 + (chunk ^ (row & 15))) + g;
        *d = make_uint2(cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3]));
      }
  }
  const int c = lane & 15;
  const int col = col0 + 8 * c;
  const bool full = (N & 7) == 0 && col + 8 <= N;   // 16-byte aligned and inside C
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    // 16 row chunks read as a batch: the LDS latency is paid once per batch
    uint4 v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int row = 4 * (16 * b + t) + (lane >> 4);
      v[t] = eb[row * 16 + (c ^ (row & 15))];
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int grow = row0 + 4 * (16 * b + t) + (lane >> 4);
      if (grow >= M || col >= N) continue;
      uint16_t* cp = C + (int64_t)grow * N + col;
      if (full) {
        store_nt16(cp, v[t]);
      } else {
        const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < N) cp[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// ------------------------------------------------------------- tile order

// Output-tile order for large GEMM grids (tiles_m and tiles_n multiples of
// 16).  Workgroups are dispatched round-robin over the 8 XCDs, and one wave
// of 256 workgroups (one per CU, 32 per XCD) runs at a time.  Each such wave
// covers one 16 x 16 block of output tiles (a "super-tile"): XCD x takes the
// 4 x 8 sub-block at tile rows 4 (x % 4) and tile columns 8 (x / 4), so its
// L2 serves 4 A panels and 8 B panels per K step.  Super-tiles are walked
// along a row, so their 16 A panels stay in the infinity cache while the B
// panels stream through it.
__device__ __forceinline__ void supertile_order(int bid, int tiles_n, int& tm, int& tn) {
  const int x = bid & 7, i = bid >> 3;
  const int st = i >> 5, w = i & 31;
  const int per_row = tiles_n >> 4;
  tm = (st / per_row) * 16 + 4 * (x & 3) + (w & 3);
  tn = (st % per_row) * 16 + 8 * (x >> 2) + (w >> 2);
}

// -------------------------------------------------------------------- misc

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8), and each XCD has its own L2.  Remap the linear workgroup index so
// that each XCD processes one contiguous range of tile indices; neighbouring
// tiles then share operands in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int XCD = 8;
  const int per = nblocks / XCD;       // full rounds
  const int rem = nblocks % XCD;
  const int x = bid % XCD, i = bid / XCD;
  // XCD x owns per (+1 if x < rem) consecutive indices.
  const int base = x * per + (x < rem ? x : rem);
  return base + i;
}

}  // namespace bsg
