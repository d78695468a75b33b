// gemv.hip -- decode GEMV for 1 <= M <= 8 activation rows.
//
// Method (vibevoice.c README, "The kernels that matter" and "Quantization" >
// "Weights", decode GEMV bullet): single-token decode reads every packed
// weight once and is bound by memory bandwidth, so dequantization is fused
// into the multiply-accumulate and the weights stay 4-bit up to the product;
// 128-bit loads; split over K when the rows alone would not cover the GPU.
//
// Kernels on gfx950 (a lane's 16-byte load holds 32 codes of one row; each
// byte, two codes, indexes a replicated LDS table of bf16 code pairs; the
// codes are bf16 values, so every product is exact in fp32, and the fp32
// block scale multiplies each 64-block's sum):
//   gemv_fast_kernel<M, ARGMAX, AFF>  workgroups own runs of whole row
//     groups, their 8 waves split the tiles; x and the partial sums live in
//     LDS; the products run on the matrix cores (below); optional argmax of
//     y (ARGMAX) and the asymmetric int4 format (AFF, no table); loads past
//     a wave's share read ahead into the next launch's matrix when named;
//   gemv_generic_kernel  codebooks needing three bf16 terms, v_dot2_f32_bf16
//     products, one workgroup per row group, lanes combined by shuffles;
//   argmax_kernel  the argmax of y after the generic path.
// Partial sums combine in a fixed order, so results are reproducible bit for
// bit.
#include <atomic>
#include <climits>

#include "nf4_internal.h"

namespace nf4 {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Waves per workgroup and the largest tile batch TT that stay in registers
// (no scratch) at that wave count: 16 waves leave 128 VGPRs per lane, 8
// waves 256; the batch's loads and the M rows' sums grow with M and NTERM.
template <int M>
constexpr int generic_waves() { return M <= 4 ? 16 : 8; }
template <int M, int NTERM>
constexpr int generic_tt_max() {
  return M <= 1 ? 8 : M == 2 ? (NTERM == 1 ? 8 : 4) : M == 3 ? (NTERM == 1 ? 4 : 2)
       : M == 4 ? (NTERM == 1 ? 4 : 1) : 8;
}

template <int M, int NTERM, int TT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_generic_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw,
    const float2 *__restrict__ am, CodeTerms ct, int64_t N, int64_t K, int64_t KT, int T,
    float *__restrict__ y) {
  __shared__ uint32_t table[NTERM * kPairWords];
  __shared__ float red[WAVES][16][M];

  for (int e = threadIdx.x; e < NTERM * kPairWords; e += blockDim.x) {
    const int term = e / kPairWords;
    const int entry = (e % kPairWords) / kPairCopies;
    table[e] = (uint32_t)ct.t[term][entry & 15] | ((uint32_t)ct.t[term][entry >> 4] << 16);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, h = lane >> 4;
  const int64_t g = blockIdx.x;
  const int64_t t_begin = (int64_t)wave * T;
  const int64_t t_end = t_begin + T < KT ? t_begin + T : KT;
  const uint32_t *tab = table + (lane & (kPairCopies - 1));

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  for (int64_t tb = t_begin; tb < t_end; tb += TT) {
    uint4 wv[TT];
    float2 sv[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      if (tb + i < t_end) {
        wv[i] = qw[(g * KT + tb + i) * 64 + lane];
        sv[i] = am[(g * KT + tb + i) * 16 + r];
      }
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      if (tb + i >= t_end) break;
      const int64_t t = tb + i;
      const uint32_t wd[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
      float p[2][M];
#pragma unroll
      for (int m = 0; m < M; ++m) p[0][m] = p[1][m] = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k0 = t * kTileK + 32 * j + 8 * h;
        uint4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
          xv[m] = k0 < K ? *reinterpret_cast<const uint4 *>(x + m * K + k0)
                         : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t e = (wd[j] >> (8 * q)) & 0xFFu;
#pragma unroll
          for (int term = 0; term < NTERM; ++term) {
            const uint32_t pr = tab[term * kPairWords + e * kPairCopies];
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const uint32_t xp = q == 0 ? xv[m].x : q == 1 ? xv[m].y : q == 2 ? xv[m].z : xv[m].w;
              p[j >> 1][m] = dot2(pr, xp, p[j >> 1][m]);
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        acc[m] = fmaf(sv[i].x, p[0][m], acc[m]);
        acc[m] = fmaf(sv[i].y, p[1][m], acc[m]);
      }
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m) {
    acc[m] += __shfl_xor(acc[m], 16);
    acc[m] += __shfl_xor(acc[m], 32);
  }
  if (h == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][r][m] = acc[m];
  }
  __syncthreads();
  const int nwaves = blockDim.x >> 6;
  for (int idx = threadIdx.x; idx < 16 * M; idx += blockDim.x) {
    const int rr = idx & 15, m = idx >> 4;
    float s = 0.0f;
    for (int w = 0; w < nwaves; ++w) s += red[w][rr][m];
    y[(int64_t)m * N + g * 16 + rr] = s;
  }
}


// ---------------------------------------------------------------------------
// Argmax of y over n for every row m (the lm_head step that picks the next
// token; vibevoice.c README, "The kernels that matter": the decode step ends
// in one index per row instead of a copy of the logits).  Each workgroup
// reduces its outputs to one candidate (value, n) per row m and stores it in
// the workspace; the last workgroup to arrive (a device-scope counter, no
// waiting on other workgroups) reduces the candidates and resets the counter
// to zero.  Candidates are ordered by value, then by the lower n: a total
// order, so any reduction tree picks the same winner, the first n that
// holds the maximum.  NaN never wins; an all-NaN row gives index -1.
// Workspace: [0, 4) arrival counter; from byte 256, P x M candidates of 8 B.
// ---------------------------------------------------------------------------
namespace amax {
constexpr size_t kCandOffset = 256;
__device__ inline bool better(float v, int n, float bv, int bn) {
  return v > bv || (v == bv && n < bn);
}
__device__ inline uint64_t pack(float v, int n) {
  return ((uint64_t)(uint32_t)n << 32) | (uint64_t)__float_as_uint(v);
}
__device__ inline void unpack(uint64_t c, float &v, int &n) {
  v = __uint_as_float((uint32_t)c);
  n = (int)(uint32_t)(c >> 32);
}
template <int M>
__device__ inline void wave_reduce(float (&bv)[M], int (&bn)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv[m], off);
      const int on = __shfl_xor(bn[m], off);
      if (better(ov, on, bv[m], bn[m])) {
        bv[m] = ov;
        bn[m] = on;
      }
    }
}
// Reduce the workgroup's candidates across waves into lds[M] (threads < M
// return them in v, n).  lds holds (waves x M) entries.
template <int M>
__device__ inline void block_reduce(float (&bv)[M], int (&bn)[M], uint64_t *lds, float &v,
                                    int &n) {
  wave_reduce<M>(bv, bn);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) lds[wave * M + m] = pack(bv[m], bn[m]);
  }
  __syncthreads();
  v = -INFINITY;
  n = INT_MAX;
  if (threadIdx.x < M) {
    for (int w = 0; w < nw; ++w) {
      float ov;
      int on;
      unpack(lds[w * M + threadIdx.x], ov, on);
      if (better(ov, on, v, n)) {
        v = ov;
        n = on;
      }
    }
  }
}
// Every thread of the workgroup calls this with its own candidates.
template <int M>
__device__ void finish(float (&bv)[M], int (&bn)[M], int b, int P, uint32_t *counter,
                       uint64_t *cand, int32_t *index, uint64_t *lds, int *flag) {
  float v;
  int n;
  block_reduce<M>(bv, bn, lds, v, n);
  if (threadIdx.x < M) {
    __hip_atomic_store(cand + (size_t)b * M + threadIdx.x, pack(v, n), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    // the candidate's store has completed before the arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  // Release/acquire through the arrival counter: the barrier orders the
  // candidates' agent-scope stores before the counting read-modify-write,
  // which is acquire-release at agent scope, and the barrier after it orders
  // that acquire before the last workgroup's loads of the candidates.
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == (uint32_t)(P - 1);
  }
  __syncthreads();
  if (!*flag) return;
  // the last workgroup: every candidate is stored
#pragma unroll
  for (int m = 0; m < M; ++m) {
    bv[m] = -INFINITY;
    bn[m] = INT_MAX;
  }
  for (int c = threadIdx.x; c < P; c += blockDim.x) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float ov;
      int on;
      unpack(__hip_atomic_load(cand + (size_t)c * M + m, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT),
             ov, on);
      if (better(ov, on, bv[m], bn[m])) {
        bv[m] = ov;
        bn[m] = on;
      }
    }
  }
  __syncthreads();  // lds is reused
  block_reduce<M>(bv, bn, lds, v, n);
  if (threadIdx.x < M) index[threadIdx.x] = n == INT_MAX ? -1 : n;
  if (threadIdx.x == 0)
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace amax

// Argmax over an already written y (the generic GEMV path): workgroup b
// scans columns [N b / P, N (b + 1) / P).
template <int M>
__global__ __launch_bounds__(256) void argmax_kernel(const float *__restrict__ y, int N,
                                                     uint32_t *counter, uint64_t *cand,
                                                     int32_t *index) {
  __shared__ uint64_t lds[4 * M];
  __shared__ int flag;
  const int P = gridDim.x, b = blockIdx.x;
  const int n0 = (int)((int64_t)N * b / P), n1 = (int)((int64_t)N * (b + 1) / P);
  float bv[M];
  int bn[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    bv[m] = -INFINITY;
    bn[m] = INT_MAX;
  }
  for (int n = n0 + (int)threadIdx.x; n < n1; n += blockDim.x) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = y[(int64_t)m * N + n];
      if (amax::better(v, n, bv[m], bn[m])) {
        bv[m] = v;
        bn[m] = n;
      }
    }
  }
  amax::finish<M>(bv, bn, b, P, counter, cand, index, lds, &flag);
}


// ---------------------------------------------------------------------------
// Fast path (codebook of bf16 values, x small enough for LDS).
//
// Work split: workgroup b owns the whole row groups [G*b/P, G*(b+1)/P), a
// contiguous run of device tiles in memory order.  Its 8 waves take the run's
// tiles round robin (wave w: local tiles w, w+8, w+16, ...), so each round
// the workgroup reads 8 KB of consecutive codes, and every wave gets the same
// number of tiles to within one.  A wave keeps kFastDepth tiles in flight.
// Each wave accumulates one partial per row group it touches and leaves it in
// LDS; after one barrier the partials of every row group are summed in wave
// order.  No workspace, no atomics, and a fixed summation order.
//
// A tile's products run on the matrix cores: per 32-k step one
// v_mfma_f32_16x16x32_bf16 with the x rows as operand A (lane row = lane % 16,
// clamped to M - 1; rows past M are computed and dropped) and the looked-up
// weights as operand B, whose fragment is exactly the lane's 8 codes of that
// step.  Two steps make one 64-block, which is scaled and folded into the
// lane's accumulators: D row 4 (lane / 16) + i is output row m, D column
// lane % 16 the weight row.  The cost per tile is four matrix instructions
// whatever M (up to 8), and the vector ALU is left with the lookups.
//
// LDS: the pair table (static) in 32 copies at a 256-byte entry stride
// (entry e in bytes 256 e .. 256 e + 127), so the address (code byte << 8) |
// ((lane % 32) << 2) is one v_perm_b32 and each half of a wave hits 32
// different banks; writing half of a 64-copy table shortens the set-up of
// every launch.  Dynamic, sized per launch: x for all M
// rows, each padded with zeros to a whole number of 128-k tiles and stored
// with a 16-byte skew per row (so the M rows of one operand-A read fall in
// different banks); and the partial sums [row group][wave][16 rows][M].
//
// Affine variant (AFF, the asymmetric int4 format in groups of 128 k): a
// tile row is one group with scale s and zero point z (one params dword per
// row: binary16 s | z << 16), and the workgroup first sums x over every
// tile, X[t][m] (in LDS after the partials, 8 floats per tile).  There is
// no table: the code words interleave their nibbles so that a shift and a
// mask put codes 2p, 2p + 1 into the mantissas of the bf16 pair
// (1 + c/16, 1 + c'/16) (0x3F80 is bf16 1.0), the B operand as it stands.
// A tile's four products form two sums of 64 k each (as in the codebook
// variant, so two MFMA chains overlap), P = P0 + P1 = sum x (1 + q/16), then
// g = fmaf(-(16 + z)/16, X, P) = sum x (q - z) / 16 with one rounding, and
// acc = fmaf(16 s, g, acc) (both constants exact).
// ---------------------------------------------------------------------------
constexpr int kFastWaves = 8;
constexpr int kFastThreads = kFastWaves * 64;  // the launch's block size

// Code i (as its bf16 bit pattern) of the first term, i in 0..15 per lane
// or per wave: each code is read from the kernel argument at a fixed index
// (readfirstlane keeps it a scalar value, so the selects cannot be folded
// back into one read at an index that varies by lane).  The 16 codes are
// contiguous halfwords, code 2 j in the low half of dword j.
__device__ __forceinline__ uint32_t pick_code(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                              int i) {
  const uint32_t w[8] = {(uint32_t)c0, (uint32_t)(c0 >> 32), (uint32_t)c1, (uint32_t)(c1 >> 32),
                         (uint32_t)c2, (uint32_t)(c2 >> 32), (uint32_t)c3, (uint32_t)(c3 >> 32)};
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const uint32_t pj = w[j >> 1];
    v = i == j ? (pj & 0xFFFFu) : i == j + 1 ? (pj >> 16) : v;
  }
  return v;
}
constexpr int kFastCopies = 64;                     // copy slots per 256-byte entry line
constexpr int kFastTableWords = 256 * kFastCopies;  // 64 KB of LDS, copies 0 .. 31 written
constexpr int kFastDepth = 4;                        // tiles in flight per wave
constexpr int kFastSkew = 8;                         // x row skew in LDS, elements
constexpr int kLdsBytes = 160 * 1024;                // LDS per workgroup on gfx950
// sched_barrier mask: ALU, VALU, SALU, MFMA, all LDS and transcendental
// instructions may cross; vector memory instructions may not.
constexpr int kSchedAllButGlobalLoads = 0x1 | 0x2 | 0x4 | 0x8 | 0x80 | 0x100 | 0x200 | 0x400;

template <int M, bool ARGMAX, bool AFF>
__global__ __launch_bounds__(kFastWaves * 64) void gemv_fast_kernel(
    const uint4 *__restrict__ qw, const float2 *__restrict__ am, const uint16_t *__restrict__ x,
    int KT, int gbase_, int grem_, int K, int N, uint64_t cw0, uint64_t cw1, uint64_t cw2, uint64_t cw3,
    float *__restrict__ y, uint32_t *counter, uint64_t *cand, int32_t *index,
    const char *__restrict__ nq, const char *__restrict__ nsb, int nG, int nKT, int nP) {
  constexpr int D = kFastDepth;
  // The table is the kernel's only static LDS array, so it sits at address
  // 0 and a lookup address needs no base added; x and the partials follow in
  // dynamic LDS.
  __shared__ __attribute__((aligned(16))) uint32_t table[AFF ? 4 : kFastTableWords];
  extern __shared__ __attribute__((aligned(16))) uint32_t lds_dyn[];
  // The arguments the first weight loads need lead the list, and the build
  // preloads the first eight arguments into scalar registers at dispatch, so
  // those loads wait for no read of the argument memory (left to itself the
  // compiler reads each argument in the block that first uses it, and each
  // such block waits again).  The empty asm statement needs them in
  // registers here; the read-ahead cursor, which needs later arguments, is
  // formed after the prefetch.
  asm volatile("" ::"s"(x), "s"(qw), "s"(am), "s"(N), "s"(K), "s"(KT), "s"(gbase_), "s"(grem_));
  const int KP = KT * kTileK;                 // padded x row length
  const int XS = KP + kFastSkew;              // x row stride in LDS
  uint16_t *xs = reinterpret_cast<uint16_t *>(lds_dyn);
  float *red = reinterpret_cast<float *>(lds_dyn + M * XS / 2);

  // the wave index as a scalar: every per-wave quantity below (tile cursor,
  // share end, read-ahead cursor, trip count) stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, h = lane >> 4;
  // G row groups over P workgroups: the first G % P take one more.  The host
  // passes G / P and G % P, so the first weight loads wait for no division
  // (a per-launch integer division sequence and the x copies' division by
  // their row length, both before those loads, cost 0.1-0.4 us per launch:
  // o 4.88 -> 4.76 us, down 11.0 -> 10.4 us at M = 1); 32-bit arithmetic
  // throughout.
  const uint32_t wg = blockIdx.x;
  const uint32_t gbase = (uint32_t)gbase_, grem = (uint32_t)grem_;
  const int g0 = (int)(wg * gbase + (wg < grem ? wg : grem));
  const int Gw = (int)(gbase + (wg < grem ? 1u : 0u)), T0 = g0 * KT, Twg = Gw * KT;
  const int n = Twg > wave ? (Twg - wave + kFastWaves - 1) / kFastWaves : 0;
  const char *qbase = reinterpret_cast<const char *>(qw);
  const char *sbase = reinterpret_cast<const char *>(am);
  const uint32_t tile_end = (uint32_t)(T0 + Twg);
  // Refills past the end of a wave's share read ahead into the next launch's
  // matrix when one is named (nq): the tiles this wave index of this
  // workgroup index loads first in that launch, so they are in the caches
  // when it starts.  Otherwise, and past that share, they re-read the
  // workgroup's first tile.  Their data is never used.

  // The lane's scales of tile lt: two block scales, or (affine) the params
  // dword in .x.
  auto load_scales = [&](const char *src, uint32_t lt) -> float2 {
    if constexpr (AFF)
      return make_float2(
          __uint_as_float(*reinterpret_cast<const uint32_t *>(src + (lt * 64u + r * 4u))), 0.0f);
    else
      return *reinterpret_cast<const float2 *>(src + (lt * 128u + r * 8u));
  };
  // x rows straight into LDS, issued before the weight loads below so that
  // they can be waited for without waiting for those: one copy is 64 lanes
  // x 16 bytes of one row (1 KB); lanes at or past K copy nothing, their
  // chunks are zeroed below.
  const int chunks = M * KP / 8, cpr = KP / 8;
  if constexpr (!AFF) {
    const int segs = (cpr + 63) / 64;
    const uint32_t xs_base = lds_addr(xs);
#pragma unroll
    for (int m = 0; m < M; ++m)
    for (int seg = wave; seg < segs; seg += kFastWaves) {
      const int c = seg * 64 + lane, k = c * 8;
      if (c < cpr && k < K)
        copy16_to_lds(xs_base + (uint32_t)(m * XS + seg * 512) * 2u, x,
                      (uint32_t)(((int64_t)m * K + k) * 2));
    }
  }
  // Prefetch cursor; steps past the wave's share re-read the workgroup's
  // first tile so that every step issues the same loads.
  uint32_t ptau = (uint32_t)(T0 + wave);
  uint4 wb[D];
  float2 sb[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const uint32_t lt = ptau < tile_end ? ptau : (uint32_t)T0;
    wb[d] = *reinterpret_cast<const uint4 *>(qbase + (lt * 1024u + lane * 16u));
    sb[d] = load_scales(sbase, lt);
    ptau += kFastWaves;
  }
  // every load above is issued before the set-up below starts (the
  // scheduler would otherwise pull the table's selects, which wait for the
  // codebook argument, in between the loads)
  __builtin_amdgcn_sched_barrier(0);
  uint32_t pn = 0, ntile_end = 0;
  if (nq != nullptr && (int)blockIdx.x < nP) {
    const uint32_t nbase = (uint32_t)nG / (uint32_t)nP, nrem = (uint32_t)nG % (uint32_t)nP;
    const int ng0 = (int)(wg * nbase + (wg < nrem ? wg : nrem));
    const int ng1 = ng0 + (int)(nbase + (wg < nrem ? 1u : 0u));
    pn = (uint32_t)(ng0 * nKT + wave);
    ntile_end = (uint32_t)(ng1 * nKT);
  }

  // Setup, one barrier in all, everything in it overlapping the first
  // tiles' flight.  The x copies are waited for just before the barrier.
  // The table entries take the 16 codes from the
  // kernel argument by compile-time index (scalar reads) and pick with
  // selects: an index varying by lane into the argument block would be a
  // vector memory read, waited for behind the tiles above.  Affine: x goes
  // through registers, since a row has a whole number of 128-k tiles and the
  // 16 lanes of a DPP row hold the 16 chunks of one tile row of x, whose sum
  // goes to X as x is stored (the chunk sums in k order, then row16_sum).
  constexpr int kStage = 4;
  float *Xl = red + Gw * kFastWaves * 16 * M;  // affine: X[t][m], 8 floats per tile
  auto store_xsum = [&](int c, uint4 v) {
    if constexpr (AFF) {
      const float sum = row16_sum(chunk_sum8(v));
      if ((lane & 15) == 0 && c < chunks) {
        const int m = c / cpr;
        Xl[((c - m * cpr) >> 4) * 8 + m] = sum;
      }
    }
  };
  uint4 xv0[kStage];
  if constexpr (AFF) {
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int c = (int)threadIdx.x + u * kFastThreads;
    const int m = c / cpr, k = (c - m * cpr) * 8;
    xv0[u] = make_uint4(0u, 0u, 0u, 0u);
    if (c < chunks && k < K) xv0[u] = *reinterpret_cast<const uint4 *>(x + (int64_t)m * K + k);
  }
  }
  if constexpr (!AFF) {
    // Pair table, copies 0 .. 31 of every entry: 16-byte chunk c (four
    // copies) of entry c / 8, for c = threadIdx.x + 512 i.  Its low code
    // index (c / 8) % 16 = (threadIdx.x / 8) % 16 is fixed per lane, its
    // high one c / 128 = threadIdx.x / 128 + 4 i fixed per wave and step.
    static_assert(kFastTableWords / 8 == 4 * kFastWaves * 64, "four chunks per thread");
    const uint32_t lo = pick_code(cw0, cw1, cw2, cw3, ((int)threadIdx.x >> 3) & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = lo | pick_code(cw0, cw1, cw2, cw3, (wave >> 1) + 4 * i) << 16;
      const int c = (int)threadIdx.x + i * kFastWaves * 64;
      reinterpret_cast<uint4 *>(table)[(c >> 3) * 16 + (c & 7)] = make_uint4(v, v, v, v);
    }
    // the zero padding k in [K, KP) of every row
    const int padc = (KP - K) / 8, kc0 = K / 8;
    for (int c = threadIdx.x; c < M * padc; c += kFastThreads) {
      const int m = c / (padc ? padc : 1), k = (kc0 + c - m * padc) * 8;
      *reinterpret_cast<uint4 *>(&xs[m * XS + k]) = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int c = (int)threadIdx.x + u * kFastThreads;
    const int m = c / cpr, k = (c - m * cpr) * 8;
    if (c < chunks) *reinterpret_cast<uint4 *>(&xs[m * XS + k]) = xv0[u];
    store_xsum(c, xv0[u]);
  }
  }
  for (int c0 = (int)threadIdx.x + kStage * kFastThreads; c0 < (AFF ? chunks : 0);
       c0 += kStage * kFastThreads) {
    uint4 v[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int c = c0 + u * kFastThreads;
      const int m = c / cpr, k = (c - m * cpr) * 8;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (c < chunks && k < K) v[u] = *reinterpret_cast<const uint4 *>(x + (int64_t)m * K + k);
    }
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int c = c0 + u * kFastThreads;
      const int m = c / cpr, k = (c - m * cpr) * 8;
      if (c < chunks) *reinterpret_cast<uint4 *>(&xs[m * XS + k]) = v[u];
      store_xsum(c, v[u]);
    }
  }
  // Partial slots start at zero (a wave may touch no tile of a row group
  // when a row group has fewer than 8 tiles).
  for (int c = threadIdx.x; c < Gw * kFastWaves * 16 * M; c += kFastThreads) red[c] = 0.0f;
  // the x sums of rows M .. 7 (read by lanes whose output rows are dropped;
  // store_xsum writes rows below M only)
  if constexpr (AFF && M < 8) {
    for (int c = threadIdx.x; c < KT * 8; c += kFastThreads)
      if ((c & 7) >= M) Xl[c] = 0.0f;
  }
  // The copies of x have landed before the barrier: at least 2 D vector
  // memory instructions (the D tiles' code and scale loads) were issued after
  // the last copy, and they complete in order, so at most D outstanding
  // means every copy is done (the tiles may still be in flight).
  if constexpr (!AFF) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory");
  __syncthreads();

  const uint32_t lane4 = ((uint32_t)lane & 31u) << 2;  // copy lane % 32
  const char *tabc = reinterpret_cast<const char *>(table);
  const uint32_t magic = 0x3F803F80u;  // bf16 pair (1.0, 1.0), affine B operands
  // D rows 4h + i (i < NA) of the lane that can be real output rows
  constexpr int NA = M < 4 ? M : 4;
  float acc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i] = 0.0f;
  // operand A: x row lane % 16 (clamped), k = 128t + 32jj + 8h + 0..7
  const uint16_t *xrow = xs + (M == 1 ? 0 : (r < M ? r : M - 1) * XS) + 8 * h;
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

  // consumed-tile position: local row group j, tile t within it
  const int q8 = kFastWaves / KT, r8 = kFastWaves % KT;
  int j = wave / KT, t = wave % KT;
  const int nsteps = (n + D - 1) / D * D;
  for (int base = 0; base < nsteps; base += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = base + d;
      const bool live = i < n;
      // ---- one 16-row x 128-k tile: lane holds weight row r, k = 128t + 32jj + 8h + 0..7
      // The 16 lookup addresses and the two scales are all the slot's words
      // are needed for, so the slot is refilled (D tiles ahead) as soon as
      // they are formed, and the lookups and products run while that load
      // is in flight.  The empty asm pins the addresses before the refill
      // and the barrier keeps the scheduler from hoisting the global loads
      // above them (either would rotate the slot registers and force a full
      // wait per step); ALU and LDS instructions may still cross it.
      // Affine: no table; the slot's four code words are kept (pinned like
      // the addresses) and the B pairs are formed next to their products.
      uint32_t ad[AFF ? 4 : 16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t wd = jj == 0 ? wb[d].x : jj == 1 ? wb[d].y : jj == 2 ? wb[d].z : wb[d].w;
        if constexpr (AFF) {
          ad[jj] = wd;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ad[4 * jj + q] = __builtin_amdgcn_perm(wd, lane4, 0x0c0c0400u + (q << 8));
        }
      }
      // block scales, or (affine) 16 s and -(16 + z) / 16: P sums x (1 + q/16)
      float s0, s1;
      if constexpr (AFF) {
        const uint32_t pv = __float_as_uint(sb[d].x);
        s0 = live ? 16.0f * (float)__builtin_bit_cast(_Float16, (uint16_t)(pv & 0xFFFFu)) : 0.0f;
        s1 = -(float)(16u + (pv >> 16)) * 0.0625f;
      } else {
        s0 = live ? sb[d].x : 0.0f;
        s1 = live ? sb[d].y : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < (AFF ? 4 : 16); ++u) asm volatile("" ::"v"(ad[u]));
      asm volatile("" ::"v"(s0), "v"(s1));
      __builtin_amdgcn_sched_barrier(kSchedAllButGlobalLoads);
      {
        const bool dead = ptau >= tile_end;
        const bool ahead = dead && pn < ntile_end;
        const uint32_t lt = ahead ? pn : dead ? (uint32_t)T0 : ptau;
        const char *qsrc = ahead ? nq : qbase;
        const char *ssrc = ahead ? nsb : sbase;
        wb[d] = *reinterpret_cast<const uint4 *>(qsrc + (lt * 1024u + lane * 16u));
        sb[d] = load_scales(ssrc, lt);
        ptau += kFastWaves;
        pn += dead ? kFastWaves : 0u;
      }
      const uint16_t *xt = xrow + t * kTileK;
      f32x4 P[2];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint4 xa = *reinterpret_cast<const uint4 *>(xt + 32 * jj);
        uint32_t bb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (AFF) {
            // bf16 (1 + c/16) of codes 2q and 2q + 1: their nibbles sit at
            // bits 4q and 16 + 4q of the interleaved code word
            bb[q] = awq_pair(ad[jj], q, magic);
          } else {
            bb[q] = *reinterpret_cast<const uint32_t *>(tabc + ad[4 * jj + q]);
          }
        }
        const bf16x8 A = __builtin_bit_cast(bf16x8, xa);
        const bf16x8 B = __builtin_bit_cast(bf16x8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
        P[jj >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, (jj & 1) ? P[jj >> 1] : zero,
                                                             0, 0, 0);
      }
      if constexpr (AFF) {
        // D rows 4h + e: x sums of rows 4 (h & 1) + e (rows past M are dropped)
        const f32x4 xz = *reinterpret_cast<const f32x4 *>(Xl + t * 8 + 4 * (h & 1));
#pragma unroll
        for (int e = 0; e < NA; ++e)
          acc[e] = fmaf(s0, fmaf(s1, xz[e], P[0][e] + P[1][e]), acc[e]);
      } else {
#pragma unroll
        for (int e = 0; e < NA; ++e) {
          acc[e] = fmaf(s0, P[0][e], acc[e]);
          acc[e] = fmaf(s1, P[1][e], acc[e]);
        }
      }
      // ---- advance; when the row group changes (or the share ends), leave
      // this wave's partial for it in LDS
      int tn = t + r8, jn = j + q8;
      if (tn >= KT) {
        tn -= KT;
        ++jn;
      }
      if (live && (jn != j || i == n - 1)) {
#pragma unroll
        for (int e = 0; e < NA; ++e) {
          const int m = 4 * h + e;
          if (m < M) red[((j * kFastWaves + wave) * 16 + r) * M + m] = acc[e];
          acc[e] = 0.0f;
        }
      }
      j = jn;
      t = tn;
    }
  }

  // ---- every row group of the workgroup: sum the waves' partials in order
  __syncthreads();
  float bv[M];
  int bn[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    bv[m] = -INFINITY;
    bn[m] = INT_MAX;
  }
  for (int c = threadIdx.x; c < Gw * 16; c += kFastThreads) {
    const int jj = c >> 4, rr = c & 15;
    const int n = (g0 + jj) * 16 + rr;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kFastWaves; ++w) sum += red[((jj * kFastWaves + w) * 16 + rr) * M + m];
      y[(int64_t)m * N + n] = sum;
      if (ARGMAX && amax::better(sum, n, bv[m], bn[m])) {
        bv[m] = sum;
        bn[m] = n;
      }
    }
  }
  if constexpr (ARGMAX) {
    // the table is no longer read: its first bytes hold the reduction
    uint64_t *scratch = reinterpret_cast<uint64_t *>(table);
    amax::finish<M>(bv, bn, blockIdx.x, (int)gridDim.x, counter, cand, index, scratch,
                    reinterpret_cast<int *>(table) + 2 * kFastWaves * M);
  }
}

struct FastPlan {
  int P;
  size_t lds;
};

// dynamic LDS bytes (x, partials and, affine, the x sums); the 64 KB table
// is static
size_t fast_dyn_bytes(int M, int64_t K, int64_t Gw, bool aff) {
  return (size_t)M * (tiles_k(K) * kTileK + kFastSkew) * 2 + (size_t)Gw * kFastWaves * 16 * M * 4 +
         (aff ? (size_t)tiles_k(K) * 8 * 4 : 0);
}
constexpr size_t kDynMax = (size_t)kLdsBytes - (size_t)kFastTableWords * 4;
constexpr size_t kDynMaxAff = (size_t)kLdsBytes - 256;  // no pair table
inline size_t dyn_max(bool aff) { return aff ? kDynMaxAff : kDynMax; }

FastPlan fast_plan(int M, int64_t N, int64_t K, bool aff = false) {
  const int64_t G = N / kTileRows;
  int64_t P = device_cu_count();
  if (P > G) P = G;
  // more workgroups when the partial slots of ceil(G/P) row groups do not fit
  while (fast_dyn_bytes(M, K, (G + P - 1) / P, aff) > dyn_max(aff) && P < G) P += P / 4 + 1;
  if (P > G) P = G;
  return FastPlan{(int)P, fast_dyn_bytes(M, K, (G + P - 1) / P, aff)};
}

bool fast_eligible(int M, int64_t N, int64_t K, int nterm, bool aff = false) {
  // 32-bit tile indices and byte offsets into the code buffer, and LDS room
  // for x plus one row group's partials
  const int64_t qbytes = (N / kTileRows) * tiles_k(K) * kTileBytes;
  return nterm == 1 && qbytes < (int64_t(1) << 32) && fast_dyn_bytes(M, K, 1, aff) <= dyn_max(aff);
}

template <int M, bool ARGMAX, bool AFF = false>
hipError_t launch_fast(const uint16_t *x, const uint4 *qw, const float2 *am, const CodeTerms &ct,
                       int64_t N, int64_t K, float *y, uint32_t *counter, uint64_t *cand,
                       int32_t *index, hipStream_t s, const NextMatrix *next) {
  static std::atomic<bool> attr_set{false};
  if (!attr_set.load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_fast_kernel<M, ARGMAX, AFF>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_max(AFF));
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  const FastPlan p = fast_plan(M, N, K, AFF);
  // the next launch's partition, if it takes this fast path with the same M
  const char *nq = nullptr, *nsb = nullptr;
  int nG = 0, nKT = 0, nP = 0;
  if (next != nullptr && next->qw != nullptr && fast_eligible(M, next->N, next->K, 1, AFF)) {
    nq = reinterpret_cast<const char *>(next->qw);
    nsb = reinterpret_cast<const char *>(next->am);
    nG = (int)(next->N / kTileRows);
    nKT = (int)tiles_k(next->K);
    nP = fast_plan(M, next->N, next->K, AFF).P;
  }
  // the first term's 16 codes as four 8-byte arguments ahead of the rest
  // (code 4 j + i in bits 16 i .. 16 i + 15 of argument j)
  uint64_t cw[4];
  for (int j = 0; j < 4; ++j) {
    cw[j] = 0;
    for (int i = 0; i < 4; ++i) cw[j] |= (uint64_t)ct.t[0][4 * j + i] << (16 * i);
  }
  hipLaunchKernelGGL((gemv_fast_kernel<M, ARGMAX, AFF>), dim3(p.P), dim3(kFastWaves * 64), p.lds, s,
                     qw, am, x, (int)tiles_k(K), (int)((N / kTileRows) / p.P),
                     (int)((N / kTileRows) % p.P), (int)K, (int)N,
                     cw[0], cw[1], cw[2], cw[3], y,
                     counter, cand, index, nq, nsb, nG, nKT, nP);
  return hipGetLastError();
}

template <int M, int NTERM>
hipError_t launch_m(const uint16_t *x, const uint4 *qw, const float2 *am, const CodeTerms &ct,
                    int64_t N, int64_t K, float *y, hipStream_t s) {
  constexpr int W = generic_waves<M>(), TTM = generic_tt_max<M, NTERM>();
  const int64_t KT = tiles_k(K);
  int nw = KT < W ? (int)KT : W;
  const int T = (int)((KT + nw - 1) / nw);
  nw = (int)((KT + T - 1) / T);
  const dim3 grid((unsigned)(N / kTileRows)), block(nw * 64);
  const int tt = T < TTM ? T : TTM;
  if (tt >= 8)
    hipLaunchKernelGGL((gemv_generic_kernel<M, NTERM, (TTM < 8 ? TTM : 8), W>), grid, block, 0, s,
                       x, qw, am, ct, N, K, KT, T, y);
  else if (tt >= 4)
    hipLaunchKernelGGL((gemv_generic_kernel<M, NTERM, (TTM < 4 ? TTM : 4), W>), grid, block, 0, s,
                       x, qw, am, ct, N, K, KT, T, y);
  else if (tt >= 2)
    hipLaunchKernelGGL((gemv_generic_kernel<M, NTERM, (TTM < 2 ? TTM : 2), W>), grid, block, 0, s,
                       x, qw, am, ct, N, K, KT, T, y);
  else
    hipLaunchKernelGGL((gemv_generic_kernel<M, NTERM, 1, W>), grid, block, 0, s, x, qw, am, ct,
                       N, K, KT, T, y);
  return hipGetLastError();
}

template <int NTERM>
hipError_t launch_t(const uint16_t *x, int M, const uint4 *qw, const float2 *am,
                    const CodeTerms &ct, int64_t N, int64_t K, float *y, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1, NTERM>(x, qw, am, ct, N, K, y, s);
    case 2: return launch_m<2, NTERM>(x, qw, am, ct, N, K, y, s);
    case 3: return launch_m<3, NTERM>(x, qw, am, ct, N, K, y, s);
    case 4: return launch_m<4, NTERM>(x, qw, am, ct, N, K, y, s);
    case 5: return launch_m<5, NTERM>(x, qw, am, ct, N, K, y, s);
    case 6: return launch_m<6, NTERM>(x, qw, am, ct, N, K, y, s);
    case 7: return launch_m<7, NTERM>(x, qw, am, ct, N, K, y, s);
    case 8: return launch_m<8, NTERM>(x, qw, am, ct, N, K, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gemv_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

namespace {
int argmax_grid(int64_t N) {
  const int64_t cus = device_cu_count();
  const int64_t want = (N + 1023) / 1024;
  return (int)(want < cus ? want : cus);
}
template <int M>
hipError_t launch_argmax_m(const uint16_t *x, const uint4 *q, const float2 *a, const CodeTerms &ct,
                           int nterm, int64_t N, int64_t K, float *y, uint32_t *counter,
                           uint64_t *cand, int32_t *index, hipStream_t s) {
  if (fast_eligible(M, N, K, nterm))
    return launch_fast<M, true>(x, q, a, ct, N, K, y, counter, cand, index, s, nullptr);
  const hipError_t e =
      skinny_eligible(M, N, K, nterm)
          ? launch_skinny(x, M, reinterpret_cast<const uint8_t *>(q),
                          reinterpret_cast<const float *>(a), ct, N, K, y, s)
      : nterm == 1 ? launch_m<M, 1>(x, q, a, ct, N, K, y, s)
                   : launch_m<M, 3>(x, q, a, ct, N, K, y, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_kernel<M>, dim3(argmax_grid(N)), dim3(256), 0, s, y, (int)N, counter,
                     cand, index);
  return hipGetLastError();
}
}  // namespace

size_t gemv_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // candidates for the larger of the two possible grids
  int64_t P = argmax_grid(N);
  const FastPlan fp = fast_plan((int)M, N, K);
  if (fp.P > P) P = fp.P;
  return amax::kCandOffset + (size_t)P * (size_t)M * sizeof(uint64_t);
}

hipError_t launch_gemv_argmax(const uint16_t *x, int M, const uint8_t *qw, const float *am,
                              const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y,
                              int32_t *index, void *ws, hipStream_t s) {
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const float2 *a = reinterpret_cast<const float2 *>(am);
  uint32_t *counter = reinterpret_cast<uint32_t *>(ws);
  uint64_t *cand = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(ws) + amax::kCandOffset);
  switch (M) {
    case 1: return launch_argmax_m<1>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    case 2: return launch_argmax_m<2>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    case 3: return launch_argmax_m<3>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    case 4: return launch_argmax_m<4>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    case 5: return launch_argmax_m<5>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    case 6: return launch_argmax_m<6>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    case 7: return launch_argmax_m<7>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    case 8: return launch_argmax_m<8>(x, q, a, ct, nterm, N, K, y, counter, cand, index, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const uint16_t *x, int M, const uint8_t *qw, const float *am,
                       const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y, void *ws,
                       hipStream_t s, const NextMatrix *next) {
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const float2 *a = reinterpret_cast<const float2 *>(am);
  if (fast_eligible(M, N, K, nterm)) {
    switch (M) {
      case 1: return launch_fast<1, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      case 2: return launch_fast<2, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      case 3: return launch_fast<3, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      case 4: return launch_fast<4, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      case 5: return launch_fast<5, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      case 6: return launch_fast<6, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      case 7: return launch_fast<7, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      case 8: return launch_fast<8, false>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
      default: return hipErrorInvalidValue;
    }
  }
  // x too long for the LDS of the fast path: the skinny GEMM streams the
  // weights the same way and stages x in chunks
  if (skinny_eligible(M, N, K, nterm)) return launch_skinny(x, M, qw, am, ct, N, K, y, s);
  if (nterm == 1) return launch_t<1>(x, M, q, a, ct, N, K, y, s);
  return launch_t<3>(x, M, q, a, ct, N, K, y, s);
}

bool awq_gemv_fast_eligible(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 8 && fast_eligible((int)M, N, K, 1, true);
}

hipError_t launch_awq_gemv_fast(const uint16_t *x, int M, const uint8_t *qw, const uint32_t *pr,
                                int64_t N, int64_t K, float *y, hipStream_t s,
                                const NextMatrix *next) {
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const float2 *a = reinterpret_cast<const float2 *>(pr);
  const CodeTerms ct = identity_terms();
  switch (M) {
    case 1: return launch_fast<1, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    case 2: return launch_fast<2, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    case 3: return launch_fast<3, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    case 4: return launch_fast<4, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    case 5: return launch_fast<5, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    case 6: return launch_fast<6, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    case 7: return launch_fast<7, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    case 8: return launch_fast<8, false, true>(x, q, a, ct, N, K, y, nullptr, nullptr, nullptr, s, next);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nf4
