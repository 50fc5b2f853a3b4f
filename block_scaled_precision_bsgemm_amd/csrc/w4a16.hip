// Small-M weight-only 4-bit GEMM: BF16 activations X[M][K] x NVFP4 weights
// W[N][K], BF16 output C[M][N].
//
// Source: "Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic"
// (bitsandbytes PR #2030), sections "Methodology" and "The SIMT / MMA layer".
// That PR measures a fused dequant+GEMM against dequantise-then-linear, and a
// SIMT (vector ALU) kernel against a matrix-core kernel at small M.  Here:
//   - the smallest m: gemv_kernel, vector ALU only;
//   - larger m: skinny_kernel (K-split and four-tile forms), BF16 MFMA, or the
//     tile kernel of w4a16_tile.hip;
// chosen per shape by the selector at the end of this file.  The kernels read
// every weight byte from HBM once per m tile and keep X in L2.  At these sizes
// they are bound by the weight stream and the exact expansion of the weights,
// so they are built to keep as much of the stream in flight as they can.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace bsg {

namespace {

typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ m == 1
// (one X row per blockIdx.y)
//
// Wave = R weight rows.  In each 4096-element chunk of K, lane l owns K
// [32 l, 32 l + 32) and [2048 + 32 l, 2048 + 32 l + 32): one 16-byte code
// load per row and half, so every load instruction reads 1 KB of one row.
// The chunk of X is loaded once per workgroup and shared through LDS.  All
// loads of a chunk are issued before any arithmetic.  Each 16-element
// block's dot product is taken on the unscaled E2M1 values (exact in BF16,
// via fdot2); the block's full E4M3 scale is applied once, in FP32.

constexpr int GV_WAVES = 4;   // waves per workgroup; the rows per wave are a template parameter

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

// Sum R per-lane partial sums over the 64 lanes with a halving butterfly:
// each step sends half of the remaining values to the partner lane, so the
// R rows cost R - 1 + (6 - log2 R) shuffles instead of 6 R.  Afterwards lane
// l holds the total of row rows_lane<R>(l).
template <int R>
__device__ __forceinline__ float reduce_rows(float (&v)[R], int lane) {
  static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "R must be a power of two");
  int cnt = R;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    if (cnt > 1) {
      const bool hi = (lane & s) != 0;
#pragma unroll
      for (int i = 0; i < R / 2; ++i) {
        if (i < cnt / 2) {
          const float send = hi ? v[i] : v[i + cnt / 2];
          const float keep = hi ? v[i + cnt / 2] : v[i];
          v[i] = keep + __shfl_xor(send, s);
        }
      }
      cnt /= 2;
    } else {
      v[0] += __shfl_xor(v[0], s);
    }
  }
  return v[0];
}
template <int R>
__device__ __forceinline__ int rows_lane(int lane) {
  int r = 0, half = R / 2, s = 32;
  for (int i = 0; (1 << i) < R; ++i) {
    if (lane & s) r += half;
    half >>= 1;
    s >>= 1;
  }
  return r;
}

// WNT: W is read once per launch (one row of X), so its loads stream (cache
// policy nt) and leave X in the caches (m = 1: -3%).  With more rows every
// row's workgroups re-read W, and plain loads keep it cached for them.
template <int R, bool WNT>
__global__ __launch_bounds__(64 * GV_WAVES) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wc, const uint8_t* __restrict__ Ws,
    const float* __restrict__ Wts, uint16_t* __restrict__ C, int N, int K) {
  // wave and rows are wave-uniform; readfirstlane tells the compiler so,
  // otherwise it builds the W buffer resources in vector registers and wraps
  // every W load in a waterfall loop
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // row blockIdx.y of X and C (the vector-ALU path forced on m > 1 re-reads
  // W once per row)
  X += (int64_t)blockIdx.y * K;
  C += (int64_t)blockIdx.y * N;
  const int n0 = (blockIdx.x * GV_WAVES + wave) * R;
  const int KH = K / 2, KB = K / 16;
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(N - n0, R)));
  const auto c_rsrc = make_rsrc(Wc + (int64_t)n0 * KH, rows * KH);
  const auto s_rsrc = make_rsrc(Ws + (int64_t)n0 * KB, rows * KB);
  const auto x_rsrc = make_rsrc(X, K * 2);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  __shared__ uint4 xs[512];   // one 4096-element chunk of X
  for (int kc = 0; kc < K; kc += 4096) {
    // K % 32 == 0, so each lane's 32-element group is wholly in or out of K
    const int g0 = kc + 32 * lane, g1 = kc + 2048 + 32 * lane;
    const bool in0 = g0 < K, in1 = g1 < K;
    // The workgroup loads the chunk of X once (16 bytes per thread and half)
    // and shares it through LDS: loaded by every wave, X took as many
    // L2-to-CU bytes as the W stream itself.  It goes out ahead of the W
    // loads, so waiting for it leaves W in flight.
    uint4 xl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = kc + 8 * (threadIdx.x + 256 * h);
      xl[h] = buffer_load_x4(x_rsrc, e < K ? e * 2 : OOB);
    }
    uint4 c0[R], c1[R];
    uint32_t s0[R], s1[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int o = in0 ? r * KH + g0 / 2 : OOB;
      c0[r] = WNT ? buffer_load_x4_nt(c_rsrc, o) : buffer_load_x4(c_rsrc, o);
      s0[r] = buffer_load_u16(s_rsrc, in0 ? r * KB + g0 / 16 : OOB);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int o = in1 ? r * KH + g1 / 2 : OOB;
      c1[r] = WNT ? buffer_load_x4_nt(c_rsrc, o) : buffer_load_x4(c_rsrc, o);
      s1[r] = buffer_load_u16(s_rsrc, in1 ? r * KB + g1 / 16 : OOB);
    }
    if (kc > 0) __syncthreads();   // the previous chunk's reads are done
    xs[threadIdx.x] = xl[0];
    xs[threadIdx.x + 256] = xl[1];
    __syncthreads();
    uint4 x0[4], x1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x0[q] = xs[4 * lane + q];        // K g0 .. g0 + 31
      x1[q] = xs[256 + 4 * lane + q];  // K g1 .. g1 + 31
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = acc[r];
      const v2f e0 = e4m3_pair_f32(s0[r]), e1 = e4m3_pair_f32(s1[r]);
      a = fmaf(block_dot(c0[r].x, c0[r].y, x0[0], x0[1]), e0[0], a);
      a = fmaf(block_dot(c0[r].z, c0[r].w, x0[2], x0[3]), e0[1], a);
      a = fmaf(block_dot(c1[r].x, c1[r].y, x1[0], x1[1]), e1[0], a);
      a = fmaf(block_dot(c1[r].z, c1[r].w, x1[2], x1[3]), e1[1], a);
      acc[r] = a;
    }
  }
  const float tot = reduce_rows<R>(acc, lane);
  const int r = rows_lane<R>(lane);
  if ((lane & (64 / R - 1)) == 0 && r < rows) C[n0 + r] = (uint16_t)f32_to_bf16_rne(tot * *Wts);
}

// ------------------------------------------------------------------ m >= 2
//
// Workgroup = SK_CONS consumer waves + SK_PROD producer waves.  It owns W rows
// [n0, n0 + nb) (nb <= 16 TP NT: TP NT 16-row MFMA tiles; rows past nb are
// masked) and X rows [m0, m0 + MT), over all of K.
//
// K is cut into 128-element blocks; stage s holds SB = KS BPS consecutive
// blocks, KS = SK_CONS / TP.  Consumer c = (tile group g = c % TP, K split
// h = c / TP) owns the NT W tiles of group g and, in stage s, blocks
// SB s + KS b + h for b < BPS.  With one tile (TP = NT = 1, nb = 16) all
// eight consumers split K, so a narrow slab still has eight waves streaming
// W.  More blocks per stage (BPS > 1) mean fewer workgroup barriers, each of
// which holds all ten waves to the slowest one.  A consumer loads its W codes
// straight from HBM into registers, RING stages ahead, dequantises them exactly
// to BF16 (dequant2_bf16) and runs 16x16x32 BF16 MFMAs against X fragments
// from LDS.
// The producers direct-load each stage's X blocks (and, when K % 256 == 0,
// the stage's scales) into an NSLOT-deep LDS ring, NSLOT - 1 stages ahead.
// Producers and consumers are separate waves so that the deep weight stream
// and the shallow X stream each have their own in-order load counter.
// One workgroup barrier per stage publishes a slot and retires the oldest.
// At the end the K splits are summed through LDS.
//
// K inside a block: lane (r, q) of a W tile holds the codes of K
// [32 q, 32 q + 32) (one 16-byte load); its dword sp feeds MFMA sub-step sp at
// K positions 8 q .. 8 q + 7.  X fragments use the same assignment, so each
// MFMA sums a consistent set of 32 K positions.

constexpr int SK_CONS = 8, SK_PROD = 2, SK_THREADS = 64 * (SK_CONS + SK_PROD);

template <int MT, int SB>
struct SkStage {
  uint4 x[SB][MT * 16];    // [block][row m: 16 chunks of 16 B; chunk c at c ^ (m & 15)]
  uint4 s[64 * SB / 2];    // W scales of the stage: row r at bytes [8 SB r, 8 SB r + 8 SB)
};

template <int MT, int SB, int NSLOT, bool SDMA, int P>
__device__ __forceinline__ void sk_produce(SkStage<MT, SB>* st, const uint16_t* X, const uint8_t* Ws, int m0,
                                           int n0, int rows_x, int rows_w, int K, int S, int lane) {
  constexpr int XD = SB * MT / 4;             // X loads per stage (1 KB each)
  constexpr int SD = SDMA ? SB / 2 : 0;       // scale loads per stage (1 KB each)
  constexpr int CNT = (XD + SK_PROD - 1 - P) / SK_PROD + (SD + SK_PROD - 1 - P) / SK_PROD;
  static_assert(CNT * (NSLOT - 2) < 64, "outstanding loads exceed the vmcnt range");
  const int KB = K / 16;
  const auto x_rsrc = make_rsrc4(X + (int64_t)m0 * K, rows_x * K * 2);
  const auto s_rsrc = make_rsrc4(Ws + (int64_t)n0 * KB, rows_w * KB);
  auto issue = [&](int s) {
    SkStage<MT, SB>& t = st[s % NSLOT];
    const int kst = s * 128 * SB;
#pragma unroll
    for (int i = P; i < XD; i += SK_PROD) {
      // 4 rows of block j: lane -> (row m, LDS chunk lane & 15)
      const int j = i / (MT / 4), m = 4 * (i % (MT / 4)) + (lane >> 4);
      const int c = (lane & 15) ^ (m & 15);
      const int k = kst + 128 * j + 8 * c;
      dma_x4(x_rsrc, lds_addr(&t.x[j][4 * (i % (MT / 4)) * 16]), k < K ? (m * K + k) * 2 : OOB);
    }
#pragma unroll
    for (int i = P; i < SD; i += SK_PROD) {
      const int e = 64 * i + lane;                      // 16-byte piece: row e / (SB/2)
      const int r = e / (SB / 2), b = kst / 16 + 16 * (e % (SB / 2));
      dma_x4(s_rsrc, lds_addr(&t.s[64 * i]), b < KB ? r * KB + b : OOB);
    }
  };
#pragma unroll
  for (int p = 0; p < NSLOT - 1; ++p) issue(p);
  for (int s = 0; s < S; ++s) {
    wait_vm_barrier<CNT * (NSLOT - 2)>();   // stage s has landed: publish it
    issue(s + NSLOT - 1);                   // into the slot retired by that barrier
  }
  // the consumers' two final barriers: stage reads done, partial sums written
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier\n\ts_barrier" ::: "memory");
}

template <int MT, int TP, int NT, int NSLOT, int RING, int BPS, bool SDMA>
__global__ __launch_bounds__(SK_THREADS, 1) void skinny_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wc, const uint8_t* __restrict__ Ws,
    const float* __restrict__ Wts, uint16_t* __restrict__ C, int M, int N, int K, int nb, int m_tiles) {
  constexpr int NJ = MT / 16, KS = SK_CONS / TP, NTILE = TP * NT, SB = KS * BPS;
  static_assert(KS % 2 == 0 && NTILE <= 4, "consumer split");
  __shared__ SkStage<MT, SB> st[NSLOT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // consecutive workgroups (the m tiles of one W slab) share an XCD's L2
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int n0 = (lin / m_tiles) * nb, m0 = (lin % m_tiles) * MT;
  const int KH = K / 2, KB = K / 16;
  // wave-uniform (readfirstlane): a min/max evaluated in vector registers
  // would put the W and X buffer resources there and wrap every load in a
  // waterfall loop
  const int rows_w = __builtin_amdgcn_readfirstlane(max(0, min(nb, N - n0)));
  const int rows_x = __builtin_amdgcn_readfirstlane(max(0, min(MT, M - m0)));
  const int S = (K + 128 * SB - 1) / (128 * SB);

  if (wave >= SK_CONS) {
    if (wave == SK_CONS) sk_produce<MT, SB, NSLOT, SDMA, 0>(st, X, Ws, m0, n0, rows_x, rows_w, K, S, lane);
    else sk_produce<MT, SB, NSLOT, SDMA, 1>(st, X, Ws, m0, n0, rows_x, rows_w, K, S, lane);
    return;
  }

  // ------------------------------------------------------------ consumers
  // In stage s consumer h takes the stage's blocks KS b + h, b < BPS (block
  // SB s + KS b + h of K).
  const int g = wave % TP, h = wave / TP;
  const int r = lane & 15, q = lane >> 4;
  const auto c_rsrc = make_rsrc(Wc + (int64_t)n0 * KH, rows_w * KH);
  const auto s_rsrc = make_rsrc(Ws + (int64_t)n0 * KB, rows_w * KB);
  auto wrow = [&](int il) { return 16 * (g * NT + il) + r; };
  auto wload = [&](int s, int b, int il) -> uint4 {
    const int t = SB * s + KS * b + h, k = 128 * t + 32 * q;
    return buffer_load_x4(c_rsrc, (s < S && k < K) ? wrow(il) * KH + 64 * t + 16 * q : OOB);
  };
  auto sload = [&](int s, int b, int il) -> uint32_t {   // scales of blocks 8t + 2q, 8t + 2q + 1
    const int t = SB * s + KS * b + h, k = 128 * t + 32 * q;
    return SDMA ? 0u : buffer_load_u16(s_rsrc, (s < S && k < K) ? wrow(il) * KB + 8 * t + 2 * q : OOB);
  };
  uint4 wr[RING][BPS][NT];
  uint32_t sr[RING][BPS][NT];
  static_for<0, RING>([&](auto B) {
#pragma unroll
    for (int b = 0; b < BPS; ++b)
#pragma unroll
      for (int il = 0; il < NT; ++il) {
        wr[B][b][il] = wload(B, b, il);
        sr[B][b][il] = sload(B, b, il);
      }
  });
  v4f acc[NT][NJ];
#pragma unroll
  for (int il = 0; il < NT; ++il)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[il][j] = v4f{};

  // One stage: ring slot B holds stage s's W codes.
  auto stage = [&](const int s, auto B) __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stage s published
    const SkStage<MT, SB>& t = st[s % NSLOT];
    static_for<0, BPS>([&](auto b) {
      const int jb = KS * b + h;   // the block's index in the stage
      // every LDS read of the block (X fragments, scales) is issued before
      // any arithmetic, so their latency overlaps the dequantisation
      // instead of stalling each MFMA on its own read
      uint4 xf[4][NJ];
      uint32_t w16s[NT];
#pragma unroll
      for (int sp = 0; sp < 4; ++sp)
#pragma unroll
        for (int j = 0; j < NJ; ++j) xf[sp][j] = t.x[jb][(16 * j + r) * 16 + ((4 * q + sp) ^ r)];
#pragma unroll
      for (int il = 0; il < NT; ++il)
        w16s[il] = SDMA ? *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(t.s) +
                                                             wrow(il) * 8 * SB + 8 * jb + 2 * q)
                        : sr[B][b][il];
      __builtin_amdgcn_sched_barrier(0);
      v2f sc[NT];
#pragma unroll
      for (int il = 0; il < NT; ++il) sc[il] = e4m3_pair_f32(w16s[il]);
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        v8bf_t wv[NT];
#pragma unroll
        for (int il = 0; il < NT; ++il) {
          const uint4& wq = wr[B][b][il];
          const uint32_t d = sp == 0 ? wq.x : sp == 1 ? wq.y : sp == 2 ? wq.z : wq.w;
          const float sv = sc[il][sp >> 1];
          const uint32_t w4[4] = {dequant2_bf16<0>(d, sv), dequant2_bf16<1>(d, sv),
                                  dequant2_bf16<2>(d, sv), dequant2_bf16<3>(d, sv)};
          __builtin_memcpy(&wv[il], w4, 16);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          v8bf_t x8;
          __builtin_memcpy(&x8, &xf[sp][j], 16);
#pragma unroll
          for (int il = 0; il < NT; ++il)
            acc[il][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[il], x8, acc[il][j], 0, 0, 0);
        }
      }
      // refill this ring slot with the block RING stages ahead
#pragma unroll
      for (int il = 0; il < NT; ++il) {
        wr[B][b][il] = wload(s + RING, b, il);
        sr[B][b][il] = sload(s + RING, b, il);
      }
    });
  };
  // Whole rounds of RING stages run without a branch around any load, so the
  // compiler's load counting waits only for the slot each stage consumes;
  // the last partial round checks each stage.
  int s0 = 0;
  for (; s0 + RING <= S; s0 += RING) static_for<0, RING>([&](auto B) { stage(s0 + B, B); });
  static_for<0, RING>([&](auto B) {
    if (s0 + B < S) stage(s0 + B, B);
  });

  // ---- sum the K splits through LDS; consumer i (< NTILE) finishes W tile i
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  v4f* red = reinterpret_cast<v4f*>(&st[0]);   // [consumer][il][j][lane]
  static_assert(SK_CONS * NT * NJ * 64 * sizeof(v4f) <= sizeof(st), "reduction space");
#pragma unroll
  for (int il = 0; il < NT; ++il)
#pragma unroll
    for (int j = 0; j < NJ; ++j) red[((wave * NT + il) * NJ + j) * 64 + lane] = acc[il][j];
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (wave >= NTILE) return;
  const float ts = *Wts;
  const int i = wave, gi = i / NT, il = i % NT;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    v4f v = v4f{};
#pragma unroll
    for (int hh = 0; hh < KS; ++hh) v += red[(((hh * TP + gi) * NT + il) * NJ + j) * 64 + lane];
    // D[n][m] fragment: column m = 16 j + r, rows n = 16 i + 4 q + e
    const int m = m0 + 16 * j + r;
    const int nl = 16 * i + 4 * q;
    if (m < M) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nl + e < rows_w) C[(int64_t)m * N + n0 + nl + e] = (uint16_t)f32_to_bf16_rne(v[e] * ts);
    }
  }
}

constexpr int64_t kW4Workgroups = 256;   // one wave of workgroups: the MI355X CU count

// "fit" tile width along N: the narrowest W slab (16..64 rows) for which the
// whole grid still fits in one wave of workgroups.
int64_t w4a16_fit_nb(int64_t m, int64_t n, int mt) {
  const int64_t per_mtile = std::max<int64_t>(1, kW4Workgroups / ceil_div(m, mt));   // n tiles allowed
  return std::min<int64_t>(64, std::max<int64_t>(16, ceil_div(n, per_mtile)));
}

template <int MT, int TP, int NT, int NSLOT, int RING, int BPS = 1>
hipError_t launch_skinny(int64_t m, int64_t n, int64_t k, const uint16_t* x, const uint8_t* w, const uint8_t* ws,
                         const float* wts, uint16_t* c, int nb_forced, hipStream_t stream) {
  // W rows per workgroup (the tile width along N): forced, or the fit width
  const int nb = nb_forced > 0 ? nb_forced : (int)w4a16_fit_nb(m, n, MT);
  if (nb > 16 * TP * NT) return hipErrorInvalidValue;   // the table pairs slab widths with tilings
  const int n_tiles = (int)ceil_div(n, nb), m_tiles = (int)ceil_div(m, MT);
  const dim3 grid((unsigned)(n_tiles * m_tiles));
  if (k % 256 == 0)
    hipLaunchKernelGGL((skinny_kernel<MT, TP, NT, NSLOT, RING, BPS, true>), grid, dim3(SK_THREADS), 0, stream, x, w, ws,
                       wts, c, (int)m, (int)n, (int)k, nb, m_tiles);
  else
    hipLaunchKernelGGL((skinny_kernel<MT, TP, NT, NSLOT, RING, BPS, false>), grid, dim3(SK_THREADS), 0, stream, x, w, ws,
                       wts, c, (int)m, (int)n, (int)k, nb, m_tiles);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------ dispatch
//
// The configurations a W4A16 call can run, the selector, and a forced path
// that runs any configuration on any shape: the calibration method of "Add
// sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic", tile-selection
// follow-up (one build runs every legal tile on every shape through the same
// forced path, and the selector is changed only where rechecked measurements
// support a rule).  Every configuration is legal for every shape the C ABI
// accepts (the vector-ALU one for m <= 65535), and the dispatch below has a
// final else: no configuration id can launch nothing.

namespace {

struct W4Config {
  const char* name;
  int mt;     // 0: vector-ALU gemv (one X row per grid row); else the MFMA kernel's m tile
  int nb;     // MFMA: W rows per workgroup, 0 = the fit width (w4a16_fit_nb);
              // vector ALU: W rows per wave, 0 = 4
  int ring;   // W register ring depth in stages; 0 = the m tile's default (16, 32: 1; 64: 4)
  bool ksplit = false;   // MFMA: one 16-row W tile per workgroup, K split over all 8 consumers
  int bps = 1;           // MFMA: K blocks per consumer per stage (one workgroup barrier each)
  int tp = 0;            // MFMA, 64-row m tile: tile groups (0: 4 groups of one tile; 2: 2 groups of two)
  int tile = -1;         // tile kernel (w4a16_tile.hip) shape: 0 = 16 x 64, 1 = 64 x 64, 2 = 128 x 128 (m x n);
                         // needs k % 512, 256, 128 == 0 respectively
};

constexpr W4Config kW4Configs[] = {
    {"valu_gemv", 0, 0},
    {"mfma_m16_nfit", 16, 0}, {"mfma_m16_n16", 16, 16}, {"mfma_m16_n32", 16, 32}, {"mfma_m16_n64", 16, 64},
    {"mfma_m32_nfit", 32, 0}, {"mfma_m32_n16", 32, 16}, {"mfma_m32_n32", 32, 32}, {"mfma_m32_n64", 32, 64},
    {"mfma_m64_nfit", 64, 0}, {"mfma_m64_n16", 64, 16}, {"mfma_m64_n32", 64, 32}, {"mfma_m64_n64", 64, 64},
    {"mfma_m16_nfit_r2", 16, 0, 2}, {"mfma_m16_nfit_r4", 16, 0, 4},
    {"mfma_m32_nfit_r2", 32, 0, 2}, {"mfma_m32_nfit_r4", 32, 0, 4},
    {"mfma_m64_nfit_r2", 64, 0, 2},
    {"valu_gemv_w2", 0, 2}, {"valu_gemv_w8", 0, 8},
    {"mfma_m16_n16_ks8", 16, 16, 8, true}, {"mfma_m16_n16_ks8_r4", 16, 16, 4, true},
    {"mfma_m32_n16_ks8", 32, 16, 8, true},
    {"mfma_m16_nfit_b2", 16, 0, 1, false, 2}, {"mfma_m16_nfit_b4", 16, 0, 1, false, 4},
    {"mfma_m32_nfit_b2", 32, 0, 1, false, 2}, {"mfma_m64_nfit_b2", 64, 0, 2, false, 2},
    {"mfma_m64_n64_b2", 64, 64, 2, false, 2}, {"mfma_m16_n16_ks8_b2", 16, 16, 2, true, 2},
    {"mfma_m64_nfit_t2", 64, 0, 2, false, 1, 2}, {"mfma_m64_n64_t2", 64, 64, 2, false, 1, 2},
    {"tile_m16_n64", 16, 64, 0, false, 1, 0, 0}, {"tile_m64_n64", 64, 64, 0, false, 1, 0, 1},
    {"tile_m128_n128", 128, 128, 0, false, 1, 0, 2},
};
constexpr int kW4NumConfigs = sizeof(kW4Configs) / sizeof(kW4Configs[0]);

}  // namespace

int w4a16_num_configs() { return kW4NumConfigs; }

const char* w4a16_config_name(int config) {
  return (config >= 0 && config < kW4NumConfigs) ? kW4Configs[config].name : nullptr;
}

int w4a16_config_max_m(int config) { return kW4Configs[config].mt == 0 ? 65535 : (1 << 30); }

int w4a16_config_k_multiple(int config) {
  return kW4Configs[config].tile >= 0 ? w4_tile_k_multiple(kW4Configs[config].tile) : 32;
}

// The selector, fitted to rechecked calibration measurements (N x K in
// {14336 x 4096, 4096 x 14336, 4096 x 4096, 1536 x 8960}) and checked on
// further shapes (2048 x 8192, 3072 x 4096, 5120 x 4096, 8192 x 2048,
// 896 x 4864, 6144 x 4096, 10240 x 2560, 2560 x 10240, 1024 x 1024,
// 768 x 3072, 1280 x 5120, 3584 x 7168, 2048 x 2048, 12288 x 3072,
// 2048 x 6144, 1792 x 7168, 2304 x 9216, 3328 x 5120, 7168 x 7168), M from 1
// to 256.  Rules, each with a physical reason:
//   - vector ALU for m <= 2, or m <= 4 at n <= 2048: no fixed MFMA-pipeline
//     cost, and the second to fourth passes over W come from the caches;
//   - 16-row W slabs with K split over all eight consumer waves while that
//     grid fits one wave of workgroups (m tile 16, else 32), or two waves
//     for k >= 7168 with the 16-row tile: every consumer streams W, and the
//     W slab is read once per 16 or 32 rows of X.  Rechecked 2-2.3x faster
//     than the four-tile kernel at n = 1536-4096 (whose 16-row slabs left six
//     of eight consumers streaming nothing) and 1.1-3x faster than the vector
//     ALU from m = 3 where n > 2048;
//   - vector ALU for m <= 8 with m * n <= 24576;
//   - otherwise the four-tile MFMA kernel, whose workgroups each hold a
//     whole CU.  While the grid fits in one wave of workgroups (one per CU),
//     time follows the work per workgroup: take the smallest m tile whose
//     grid fits with 64-row W slabs, then the narrowest slab that still fits
//     (the fit width), which fills the wave.
//   - If no m tile fits, 64-row slabs and the m tile with the fewest
//     weighted waves: a wave of 16-, 32- and 64-row tiles costs about 0.8,
//     1 and 1.5 (measured: workgroup time is mostly the W stream, not the
//     MFMA work); ties go to the larger tile.
//   - Four-tile variant per m tile, from the screen medians of every
//     variant over all cells relative to the best of them (max loss of the
//     pick in brackets): 16 rows: 2-stage W ring below k = 7168 (3.2%), 2
//     blocks per stage from there (3.2%); 32 rows: 2 blocks per stage from
//     k = 4096 (0%), 1 ring stage below (1.2%); 64 rows: two tile groups of
//     two tiles (2.4%), which halves the LDS reads of X, against 10-16% for
//     the four-group tiling.
// The first rule (m tile by m alone, slab width from n alone) was within
// 3% only for n >= 12288; at n = 4096 its 16-row slabs re-read X for little W
// and ran up to 3.4x slower.
int w4a16_config_id(int mt, int nb) {
  const int base = mt == 16 ? 1 : mt == 32 ? 5 : 9;
  return base + (nb == 0 ? 0 : nb == 16 ? 1 : nb == 32 ? 2 : 3);
}

//   - The vector-ALU kernel takes 2 W rows per wave instead of 4 where 4 rows
//     leave fewer than about 3 waves per CU per X row (n <= 2560, or m = 1
//     at n <= 4096): rechecked +7-12% at 2560 x 10240 and 1536 x 8960; at
//     larger m or n the extra waves re-read X and lose (-9-16% rechecked at
//     m = 2-8, n = 1536-4096).
//   - The K-split kernel keeps a 4-stage W ring: against 8 stages the median
//     ratio over 180 cells was within 2.5% at every K but 8960 (4.6%).
int w4a16_select(int64_t m, int64_t n, int64_t k) {
  const int gemv = (n <= 2560 || (m <= 1 && n <= 4096)) ? 18 : 0;   // valu_gemv_w2 / valu_gemv
  if (m <= 2 || (m <= 4 && n <= 2048)) return gemv;
  // The tile kernel's thin tiles where their grid fills about one wave of
  // workgroups with 64-row W slabs (n >= 14336): 14336 x 4096 at m = 4 .. 16:
  // 11.6-11.8 us against 12.1-12.9; 28672 x 4096, m = 16: 22.2 against 24.3;
  // at m = 64: 18.8 against 20.0.  (Smaller n leaves CUs idle; there the
  // K-split kernels below win, e.g. 4096 x 4096, m = 16: 7.1 against 10.5.)
  if (ceil_div(n, 64) >= 224) {
    if (m <= 16 && k % 512 == 0) return 31;                                   // tile_m16_n64
    if (m > 48 && m <= 64 && k % 256 == 0 && ceil_div(n, 64) <= 256) return 32;   // tile_m64_n64
  }
  const int64_t slabs = ceil_div(n, 16);
  if (slabs * ceil_div(m, 16) <= kW4Workgroups) return 21;                   // mfma_m16_n16_ks8_r4
  if (slabs * ceil_div(m, 32) <= kW4Workgroups) return 22;                   // mfma_m32_n16_ks8
  if (k >= 7168 && slabs * ceil_div(m, 16) <= 2 * kW4Workgroups) return 21;
  if (m <= 8 && m * n <= 24576) return gemv;
  // The tile kernel's 128 x 128 tiles, once they fill a wave of workgroups:
  // 14336 x 4096 at m = 192 and 256: 38 and 40 us against 50 and 64 us;
  // 28672 x 4096 at m = 96 .. 256: 1.4-1.6x; with fewer tiles (14336 at
  // m <= 128, 8192 at m <= 256) it ties or loses.
  if (m > 64 && k % 128 == 0 && ceil_div(m, 128) * ceil_div(n, 128) >= 224) return 33;   // tile_m128_n128
  // Where the four-tile kernel would take 16-row m tiles, the 16 x 64 tile
  // kernel is faster whenever it takes the K (the calibration's 278 cells:
  // 22 cells 3-19% faster, e.g. 2048 x 6144, m = 128: 1.19x; 2 cells 3-4%
  // slower); likewise its 64 x 64 tile in place of the 64-row four-tile
  // kernel from n = 6144.
  for (int mt : {16, 32, 64})
    if (ceil_div(n, 64) * ceil_div(m, mt) <= kW4Workgroups) {
      if (mt == 64) return n >= 6144 && k % 256 == 0 ? 32 : 29;   // tile_m64_n64 / mfma_m64_nfit_t2
      if (mt == 32) return k >= 4096 ? 25 : 5;                    // mfma_m32_nfit_b2 / mfma_m32_nfit
      if (k % 512 == 0) return 31;                                // tile_m16_n64
      return k >= 7168 ? 23 : 13;                                 // mfma_m16_nfit_b2 / mfma_m16_nfit_r2
    }
  int best = 64;
  double best_cost = 0;
  for (int mt : {64, 32, 16}) {
    const double weight = mt == 16 ? 0.8 : mt == 32 ? 1.0 : 1.5;
    const double cost = weight * (double)ceil_div(ceil_div(n, 64) * ceil_div(m, mt), kW4Workgroups);
    if (mt == 64 || cost < best_cost) {
      best = mt;
      best_cost = cost;
    }
  }
  if (best != 64) return w4a16_config_id(best, 64);
  // 64-row slabs over more than one wave: the tile kernel (5-12% faster than
  // the four-tile one on every calibrated cell), with 128 x 128 tiles where
  // their rounds of workgroups cost less: a 128 x 128 tile takes ~2.5x a
  // 64 x 64 one (14336 x 4096, m = 256: one round of 128 x 128 tiles, 43 us;
  // four of 64 x 64 tiles, 66 us).  10240 x 2560, m = 256: 1 round against 3,
  // 1.42x; 8192 x 2048: 1 against 2, and the 64 x 64 tiles win by 8%.
  if (m > 128 && k % 128 == 0) {
    const int64_t r128 = ceil_div(ceil_div(m, 128) * ceil_div(n, 128), kW4Workgroups);
    const int64_t r64 = ceil_div(ceil_div(m, 64) * ceil_div(n, 64), kW4Workgroups);
    if (5 * r128 < 2 * r64) return 33;   // tile_m128_n128
  }
  return k % 256 == 0 ? 32 : 30;   // tile_m64_n64 / mfma_m64_n64_t2
}

hipError_t launch_w4a16(int config, int64_t m, int64_t n, int64_t k, const uint16_t* x, const uint8_t* w,
                        const uint8_t* ws, const float* wts, uint16_t* c, hipStream_t stream) {
  const W4Config& cf = kW4Configs[config];
  if (cf.tile >= 0) return launch_w4_tile(cf.tile, m, n, k, x, w, ws, wts, c, stream);
  if (cf.mt == 0) {
    const int rows = cf.nb > 0 ? cf.nb : 4;   // W rows per wave
    const dim3 grid((unsigned)ceil_div(n, rows * GV_WAVES), (unsigned)m);
    auto go = [&](auto RC, auto WNTC) {
      hipLaunchKernelGGL((gemv_kernel<decltype(RC)::value, decltype(WNTC)::value>), grid, dim3(64 * GV_WAVES), 0,
                         stream, x, w, ws, wts, c, (int)n, (int)k);
    };
    using R2 = std::integral_constant<int, 2>;
    using R4 = std::integral_constant<int, 4>;
    using R8 = std::integral_constant<int, 8>;
    if (m == 1) {
      if (rows == 8) go(R8{}, std::true_type{});
      else if (rows == 2) go(R2{}, std::true_type{});
      else go(R4{}, std::true_type{});
    } else {
      if (rows == 8) go(R8{}, std::false_type{});
      else if (rows == 2) go(R2{}, std::false_type{});
      else go(R4{}, std::false_type{});
    }
  } else if (cf.tp == 2 && cf.mt == 64) {
    return launch_skinny<64, 2, 2, 2, 2, 1>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
  } else if (cf.bps > 1) {
    if (cf.ksplit) return launch_skinny<16, 1, 1, 2, 2, 2>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    if (cf.mt == 16 && cf.bps == 4) return launch_skinny<16, 2, 2, 2, 1, 4>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    if (cf.mt == 16) return launch_skinny<16, 2, 2, 4, 1, 2>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    if (cf.mt == 32) return launch_skinny<32, 2, 2, 2, 1, 2>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    return launch_skinny<64, 4, 1, 2, 2, 2>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
  } else if (cf.ksplit) {
    if (cf.mt == 32) return launch_skinny<32, 1, 1, 2, 8>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    if (cf.ring == 4) return launch_skinny<16, 1, 1, 4, 4>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    return launch_skinny<16, 1, 1, 4, 8>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
  } else if (cf.mt == 16) {
    if (cf.ring == 4) return launch_skinny<16, 2, 2, 8, 4>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    if (cf.ring == 2) return launch_skinny<16, 2, 2, 8, 2>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    return launch_skinny<16, 2, 2, 8, 1>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
  } else if (cf.mt == 32) {
    if (cf.ring == 4) return launch_skinny<32, 2, 2, 4, 4>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    if (cf.ring == 2) return launch_skinny<32, 2, 2, 4, 2>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    return launch_skinny<32, 2, 2, 4, 1>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
  } else {
    if (cf.ring == 2) return launch_skinny<64, 4, 1, 4, 2>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
    return launch_skinny<64, 4, 1, 4, 4>(m, n, k, x, w, ws, wts, c, cf.nb, stream);
  }
  return hipGetLastError();
}

}  // namespace bsg
