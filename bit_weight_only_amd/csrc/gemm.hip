// gemm.hip -- prefill GEMM y = x . dequant(W)^T for any M on bf16 MFMA.
//
// Method (vibevoice.c README, "Quantization" > "Weights", M > 1 bullet): a
// matrix-core GEMM keeps the weights 4-bit through on-chip memory and
// expands them next to the matrix instruction.
//
// Precision on gfx950: a bf16 operand cannot hold c*s exactly, so the codes
// themselves (bf16 values) are the B operand and the fp32 scale is applied
// outside the matrix product: for every 64-block the MFMA sums
// P = sum_k x*c in fp32 (exact products), then acc += s * P.
//
// Kernels:
//   gemm_wide_kernel<WAVES, RG, SPLIT>  codebooks whose values are bf16 (the
//     default one) on grids of 16 (or 14) row groups per workgroup: 128 x
//     16 RG outputs, each wave owning all 128 rows of its own row groups,
//     a pipeline of one barrier per 64-k step;
//   gemm_tile_kernel<RG, AFF, MB, SPLIT>  the asymmetric int4 format (AFF),
//     and the codebook format on 8-row-group grids: 128 x 16 RG outputs per
//     workgroup, waves of 16 MB x 32, copies straight from global memory
//     into LDS rings, each wave expanding the code words of its own columns;
//   gemm_skinny_kernel<MB, D, AFF, SPLIT, OCC>  few rows (below);
//   gemm_narrow_kernel<AFF, SPLIT, LEAD>  up to 32 rows on a matrix of few row
//     groups, both formats: the waves of a workgroup share one row group;
//   gemm_stream_kernel<SPLIT, PG>  up to 16 rows on a matrix whose row groups
//     fit the CUs once (codebook format): as the narrow kernel, with x and the
//     code words loaded straight into registers and K's two parts folded
//     side by side;
//   xsum_kernel           the int4 format's per-group sums of x (pre-pass);
//   gemm_kernel<3>        any finite codebook (each value split into three
//     bf16 terms), and shapes whose byte offsets exceed 32 bits.
// Within each kernel every output is the same sequence of operations
// whatever the tile shape or M: the K order, the MFMA k-split and the
// per-block fold never depend on the launch, so a row of y does not depend on
// the other rows in the batch, and a column slice of a fused matrix equals
// the separate matrix's output when both have the same parts of K.  The
// parts are fixed by (N, K) alone (k_parts: two halves for K >= 8192, more
// for narrow N), each folded from zero, then added in part order: the tiled
// kernel runs the parts on separate workgroups that meet through the
// workspace, the skinny, narrow and generic kernels one after the other in
// the K order of each output.
#include <type_traits>

#include "nf4_internal.h"


namespace nf4 {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int BM = 128, BN = 128;
constexpr int XS = kTileK + 8;  // LDS row stride of the x tile in bf16

template <int NTERM>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                   const uint4 *__restrict__ qw,
                                                   const float2 *__restrict__ am, CodeTerms ct,
                                                   int64_t N, int64_t K, int64_t KT,
                                                   float *__restrict__ y, int np) {
  __shared__ uint32_t table[NTERM * kPairWords];
  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * XS];

  for (int e = threadIdx.x; e < NTERM * kPairWords; e += blockDim.x) {
    const int term = e / kPairWords;
    const int entry = (e % kPairWords) / kPairCopies;
    table[e] = (uint32_t)ct.t[term][entry & 15] | ((uint32_t)ct.t[term][entry >> 4] << 16);
  }

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, h = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t g0 = ((int64_t)blockIdx.x * BN) / kTileRows + wn * 4;
  const int64_t G = N / kTileRows;
  const uint32_t *tab = table + (lane & (kPairCopies - 1));

  // K in np parts: tot adds the sums of the finished parts in part order;
  // the next part starts at tile `cut`
  f32x4 acc[4][4], tot[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = tot[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  int jn = 1, cut = np > 1 ? part_begin(1, KT, np) : -1;

  for (int64_t t = 0; t < KT; ++t) {
    if (t == cut) {  // the next part of K starts from zero
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          tot[a][b] = jn == 1 ? acc[a][b] : tot[a][b] + acc[a][b];
          acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      ++jn;
      cut = jn < np ? part_begin(jn, KT, np) : -1;
    }
    __syncthreads();  // previous x tile fully consumed (and table built)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int idx = tid + 256 * c;
      const int row = idx >> 4, col = (idx & 15) * 8;
      const int64_t gm = m0 + row, k = t * kTileK + col;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (gm < M && k < K) v = *reinterpret_cast<const uint4 *>(x + gm * K + k);
      *reinterpret_cast<uint4 *>(&xs[row * XS + col]) = v;
    }
    uint4 bq[4];
    float2 bs[4];
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int64_t g = g0 + nn;
      if (g < G) {
        bq[nn] = qw[(g * KT + t) * 64 + lane];
        bs[nn] = am[(g * KT + t) * 16 + r];
      } else {
        bq[nn] = make_uint4(0u, 0u, 0u, 0u);
        bs[nn] = make_float2(0.f, 0.f);
      }
    }
    __syncthreads();

#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 p[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) p[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * blk + jj;
        bf16x8 A[4];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
          A[mm] = *reinterpret_cast<const bf16x8 *>(&xs[(wm * 64 + mm * 16 + r) * XS + 32 * j + 8 * h]);
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          const uint32_t wd = j == 0 ? bq[nn].x : j == 1 ? bq[nn].y : j == 2 ? bq[nn].z : bq[nn].w;
#pragma unroll
          for (int term = 0; term < NTERM; ++term) {
            uint32_t b4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              b4[q] = tab[term * kPairWords + ((wd >> (8 * q)) & 0xFFu) * kPairCopies];
            const bf16x8 B = __builtin_bit_cast(bf16x8, b4);
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
              p[mm][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mm], B, p[mm][nn], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) {
        const float s = blk == 0 ? bs[nn].x : bs[nn].y;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mm][nn][i] = fmaf(s, p[mm][nn][i], acc[mm][nn][i]);
      }
    }
  }

  // Output tile of a 16x16x32 MFMA: lane l holds rows 4(l/16)+i, column l%16.
#pragma unroll
  for (int mm = 0; mm < 4; ++mm)
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int64_t col = (g0 + nn) * kTileRows + r;
      if (g0 + nn >= G) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 64 + mm * 16 + 4 * h + i;
        const float v = np > 1 ? tot[mm][nn][i] + acc[mm][nn][i] : acc[mm][nn][i];
        if (row < M) y[row * N + col] = v;
      }
    }
}


constexpr int kBK = 64;  // k per step of the pipelined kernel (one scale block)
// 16-row m-blocks per wave of the tiled kernel: 8 waves per workgroup either
// way, of 128 x 32 outputs for 16 row groups (each B fragment feeds 8
// MFMAs: half the lookup-address VALU per MFMA of 64-row waves) and of
// 64 x 32 for 8 row groups (two waves per SIMD keep latency hidden there)
constexpr int kTileMB = 8, kTileMB8 = 4;

// ---------------------------------------------------------------------------
// Copies straight from global memory into LDS, shared by the tiled and the
// skinny kernels, and the copies of the skinny kernel's pair table.
namespace pipe {
constexpr int kHalfRow = 64;                    // bytes of one row in one 32-k half
constexpr int kCopies = 32;                     // pair-table copies (lane % 32)

// Wait until at most N of this wave's copies are in flight and its LDS
// operations are done, then meet the other waves.
template <int N>
__device__ inline void wait_copies_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
}  // namespace pipe

// ---------------------------------------------------------------------------
// Tiled kernel: a workgroup computes 128 rows x 16 RG columns (RG row groups,
// 8 or 16) with 4 RG / MB waves, each 16 MB rows x 32 columns (MB x 2 MFMA
// blocks; MB = 8 for RG = 16 and 4 for RG = 8, so 8 waves, 2 per SIMD).  Each wave expands the B fragments of its
// own two row groups straight from code words in LDS (no expanded copy of B
// is stored), and the pair table has one copy per lane at a 256-byte stride:
// the lookup address (code byte << 8) | (lane << 2) is one v_perm_b32 and the
// 64 lanes hit 64 banks.  The 64-k step is split into two 32-k halves, each a
// separate LDS block laid out [row][32 bf16], with the four 16-byte chunks of
// a row stored at chunk ^ ((row >> 1) & 3), which makes a fragment read free
// of bank conflicts (the swizzle (row >> 2) & 3 measured 2-5 % slower on the
// int4 GEMMs at 1024 rows).  LDS (bytes): table 64 K at address
// 0, x 2 stages x 2 halves x 8 K, and per row group 2 device tiles of code
// words (1 K each) and of scales (128 each).  Rings, filled by global->LDS
// copies issued right after the barrier of step t: x of step t+1 (into the
// stage step t-1 read); at odd t = 2k+1 also device tile k+2 of every row
// group, code words and scales (into the slot of tile k, which step 2k read
// into registers for both of its steps).  Sources past the end are clamped,
// x is copied first, and a barrier waits until x of the coming step has
// landed.  Every output gets the operations of the other kernels: per
// 64-block P = MFMA(kk=0, zero), MFMA(kk=1, P), acc = fmaf(s, P, acc), in K
// order.
//
// Affine variant (AFF, the asymmetric int4 format in groups of 128 k): no
// pair table (x starts at LDS 0); a B pair is a shift and a mask of the
// interleaved code word, bf16 (1 + c/16, 1 + c'/16).  The scale ring holds
// the params dword per row (binary16 s | z << 16, 64 bytes per tile) and a
// 2-slot ring the x sums X[t][m0 .. m0 + 127] of a tile (512 bytes of the
// pre-pass result; every wave copies 512 / RG bytes of it), tile T + 1's
// copied at the even step of tile T into the slot tile T - 1 used.  Per
// device tile and output: P = four MFMAs over the tile's 32-k quarters from
// zero (two steps; P = sum x (1 + q/16)), g = fmaf(-(16 + z)/16, X, P),
// acc = fmaf(16 s, g, acc).
//
// K in np parts (SPLIT: long K, or narrow N): the grid holds np workgroups
// per output tile, one per part of K, each summing its part from zero; they
// meet through the workspace (sums stored, arrival counted, the last adds
// all parts in part order and stores y), which costs an extra write and read
// of the tile per part but fills the CUs where N alone would not.
namespace tile {
constexpr int kBM = 128;
constexpr int kTable = 256 * 64 * 4;            // one copy per lane
constexpr int kAHalf = kBM * pipe::kHalfRow;    // 8 KB: 128 rows x 32 k

constexpr int kXSum = kBM * 4;                  // x sums of one tile, bytes
template <int RG, bool AFF, int MB>
struct Map {
  // MB 16-row m-blocks per wave: waves of 16 MB x 32, 8 / MB along M and
  // RG / 2 along N
  static constexpr int kWaves = 4 * RG / MB, kThreads = 64 * kWaves, kWN = RG / 2;
  static constexpr int kRGW = RG / kWaves;  // row groups each wave copies (1 or 2)
  // the affine variant has no pair table
  static constexpr int kOffA = AFF ? 0 : kTable, kOffC = kOffA + 4 * kAHalf;
  static constexpr int kOffS = kOffC + RG * 2 * kTileBytes,
                       kOffX = kOffS + RG * 2 * kTileScales * 4,
                       kBytes = kOffX + (AFF ? 2 * kXSum : 0);
  static constexpr int kACopies = 16 / kWaves;  // x copies per wave per step
  static constexpr int kXLanes = kXSum / 16 / kWaves;  // lanes per wave copying x sums
  // copies a wave may leave in flight past the barrier of an even step: the
  // tile copies of the step before
  static constexpr int kTileCopies = 2 * kRGW;
  // bytes of scales (params) per device tile in global memory; the LDS slot
  // keeps 128
  static constexpr int kScaleBytes = AFF ? kTileRows * 4 : kTileScales * 4;
};
}  // namespace tile

template <int RG, bool AFF, int MB, bool SPLIT>
__global__ __launch_bounds__(256 * RG / MB) void gemm_tile_kernel(
    const uint16_t *__restrict__ x, int64_t M, const uint8_t *__restrict__ qw,
    const float *__restrict__ am, CodeTerms ct, int64_t N, int64_t K, int64_t KT,
    float *__restrict__ y, int ntn, int ntm, const float *__restrict__ xsum, int64_t Mp,
    int np_arg, uint32_t *__restrict__ cnt, uint64_t *__restrict__ part) {
  using L = tile::Map<RG, AFF, MB>;
  // K in np parts (SPLIT) or in one
  const int np = SPLIT ? np_arg : 1;
  // the only static LDS array, so the table sits at LDS address 0
  __shared__ __attribute__((aligned(16))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, h = lane >> 4;
  const int wm = wave / L::kWN, wn = wave % L::kWN;
  // Tile order for the 8 XCDs, each with its own L2: consecutive workgroups
  // go to consecutive XCDs, so workgroup b runs on XCD b % 8.  A unit is an
  // N tile and a part of K (u = nt np + kc, the weight tile one workgroup
  // expands); XCD k takes the units k, k+8, ... and, for each, all M tiles
  // one after the other, so the workgroups that expand one weight tile share
  // an L2.  Workgroups past the last unit (the grid is padded to a multiple
  // of 8 units) leave before any barrier.
  const int xcd = (int)(blockIdx.x & 7), slot = (int)(blockIdx.x >> 3);
  const int u = (slot / ntm) * 8 + xcd, mt = slot % ntm;
  if (u >= ntn * np) return;
  const int nt = u / np, kc = u - nt * np;
  const int64_t m0 = (int64_t)mt * tile::kBM;
  const int64_t gblk = (int64_t)nt * RG;
  const int64_t G = N / kTileRows;
  // this workgroup's part of K: device tiles [t0, t1), S 64-k steps (the
  // last part may end in a half tile); every source is addressed from the
  // part's first tile
  const int t0 = SPLIT ? part_begin(kc, KT, np) : 0;
  const int t1 = SPLIT ? part_begin(kc + 1, KT, np) : (int)KT;
  const int64_t KTp = t1 - t0;
  const int S = (int)(2 * (int64_t)t1 < K / kBK ? 2 * (int64_t)t1 : K / kBK) - 2 * t0;
  x += (int64_t)t0 * kTileK;
  qw += (int64_t)t0 * kTileBytes;
  am += (int64_t)t0 * (L::kScaleBytes / 4);
  if (AFF) xsum += (int64_t)t0 * Mp;
  const uint32_t base = lds_addr(lds);
  const char *ldsA = lds + L::kOffA, *ldsC = lds + L::kOffC, *ldsS = lds + L::kOffS;

  // Copy assignment (W waves).  x: copy i (16 per step, 1 KB each) fills
  // rows 16 (i % 8) .. + 15 of half i / 8; wave w issues i = w, w + W, ...
  // Lane l fills chunk slot l % 4 of row 16 (i % 8) + l / 4, i.e. logical
  // chunk (l % 4) ^ ((l >> 3) & 3).  Code words and scales: wave w copies
  // those of row groups w, w + W, ...  Rows past M and row groups past N
  // re-read the last valid one; their outputs are never stored.
  uint32_t aoff[L::kACopies], mA[L::kACopies];
#pragma unroll
  for (int v = 0; v < L::kACopies; ++v) {
    const int i = wave + v * L::kWaves, blk = i % 8, half = i / 8;
    const int64_t R = m0 + 16 * blk + (lane >> 2);
    const int64_t gm = R < M ? R : M - 1;
    const int c = (lane & 3) ^ ((lane >> 3) & 3);
    aoff[v] = (uint32_t)((gm * K + half * 32 + c * 8) * 2);
    mA[v] = base + L::kOffA + half * tile::kAHalf + blk * 1024;
  }
  uint32_t coff[L::kRGW], soff[L::kRGW], mC[L::kRGW], mS[L::kRGW];
#pragma unroll
  for (int u = 0; u < L::kRGW; ++u) {
    const int q = wave + u * L::kWaves;  // row group of the tile
    const int64_t rg = gblk + q;
    const int64_t g = rg < G ? rg : G - 1;
    coff[u] = (uint32_t)(g * KT * kTileBytes + lane * 16);
    soff[u] = (uint32_t)(g * KT * L::kScaleBytes + lane * 16);  // lanes 0..7 (0..3) copy
    mC[u] = base + L::kOffC + q * 2 * kTileBytes;
    mS[u] = base + L::kOffS + q * 2 * kTileScales * 4;
  }
  // x sums (affine): wave w copies bytes [w, w + 1) * 512 / W of a tile's 512
  const uint32_t mX = base + L::kOffX + wave * (tile::kXSum / L::kWaves);
  const uint32_t xoff = (uint32_t)(m0 * 4) + (uint32_t)(wave * L::kXLanes + lane) * 16u;
  auto copy_x = [&](int step) {
    const uint32_t sc = (uint32_t)(step < S ? step : S - 1) * (kBK * 2);
#pragma unroll
    for (int v = 0; v < L::kACopies; ++v)
      copy16_to_lds(mA[v] + (step & 1) * 2 * tile::kAHalf, x, aoff[v] + sc);
  };
  // device tile T (steps 2T, 2T+1) of the wave's row group: 1 KB of code
  // words and 128 bytes of scales, into ring slot T & 1
  auto copy_tile = [&](int T) {
    const uint32_t tc = (uint32_t)(T < KTp ? T : KTp - 1);
#pragma unroll
    for (int u = 0; u < L::kRGW; ++u) {
      copy16_to_lds(mC[u] + (T & 1) * kTileBytes, qw, coff[u] + tc * kTileBytes);
      if (lane < L::kScaleBytes / 16)
        copy16_to_lds(mS[u] + (T & 1) * kTileScales * 4, am, soff[u] + tc * L::kScaleBytes);
    }
  };
  // x sums of device tile T (affine) into ring slot T & 1
  auto copy_xsum = [&](int T) {
    if constexpr (AFF) {
      const uint32_t tc = (uint32_t)(T < KTp ? T : KTp - 1);
      if (lane < L::kXLanes)
        copy16_to_lds(mX + (T & 1) * tile::kXSum, xsum, xoff + tc * (uint32_t)(Mp * 4));
    }
  };

  // the pair table, from the codebook staged in the scale ring (filled only
  // after the second barrier)
  uint16_t *codes16 = reinterpret_cast<uint16_t *>(lds + L::kOffS);
  if (!AFF && tid < 16) codes16[tid] = ct.t[0][tid];
  __syncthreads();
  for (int c = tid; c < (AFF ? 0 : tile::kTable / 16); c += L::kThreads) {
    const int e = c >> 4;  // 16 chunks of 4 copies per entry
    const uint32_t v = (uint32_t)codes16[e & 15] | ((uint32_t)codes16[e >> 4] << 16);
    reinterpret_cast<uint4 *>(lds)[c] = make_uint4(v, v, v, v);
  }
  __syncthreads();
  copy_x(0);
  copy_tile(0);
  copy_tile(1);
  copy_xsum(0);
  pipe::wait_copies_and_barrier<0>();

  const uint32_t lane4 = (uint32_t)lane << 2;
  // fragments: lane (r, h) holds row r of a 16-row block, bf16 8h .. 8h+7 of the half
  const uint32_t afr = (uint32_t)(wm * 16 * MB * pipe::kHalfRow + r * pipe::kHalfRow +
                                  ((h ^ ((r >> 1) & 3)) * 16));
  // this wave's two row groups: code words (16 bytes per lane) and scales
  const char *cw = ldsC + (wn * 2) * 2 * kTileBytes + lane * 16;
  const char *sw = ldsS + (wn * 2) * 2 * kTileScales * 4 + r * (AFF ? 4 : 8);
  // x sums of D rows wm 64 + mm 16 + 4h + i (affine)
  const char *xw = lds + L::kOffX + (wm * 16 * MB + 4 * h) * 4;
  f32x4 acc[MB][2];
#pragma unroll
  for (int a2 = 0; a2 < MB; ++a2)
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) acc[a2][b2] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // Two steps per iteration: the x stage is a constant, and the code words
  // and scales of device tile k = t / 2 are read once, at the even step, for
  // both steps.  Every source offset grows with the step, so min(offset,
  // last offset) is the clamped one.
  const uint32_t xlast = (uint32_t)(S - 1) * (kBK * 2);
  uint4 cv[2];
  float2 sv[2];
  f32x4 pz[MB][2];  // affine: the tile's product, carried from the even step to the odd one
  auto step = [&](auto phc, int t) {
    constexpr int PH = decltype(phc)::value;
    // Landed: x of step t (copied in step t-1; at an even step the tile
    // copies of step t-1 may still be in flight), and device tile t / 2 (two
    // or more steps ago).  Past the barrier no wave reads x of step t-1, and
    // at an odd step no wave reads device tile t / 2 from LDS any more.
    // (the wait and barrier order every memory access; arithmetic may move
    // across them: a scheduling barrier here measured 1.5-4 % slower)
    pipe::wait_copies_and_barrier<PH == 0 ? L::kTileCopies : 0>();
    {
      const uint32_t xo = min((uint32_t)(t + 1) * (kBK * 2), xlast);
#pragma unroll
      for (int v = 0; v < L::kACopies; ++v)
        copy16_to_lds(mA[v] + ((PH + 1) & 1) * 2 * tile::kAHalf, x, aoff[v] + xo);
      if (PH == 1) copy_tile((t >> 1) + 2);
      if (PH == 0) copy_xsum((t >> 1) + 1);
    }
    if (PH == 0) {
      const int sl = (t >> 1) & 1;
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        cv[nn] = *reinterpret_cast<const uint4 *>(cw + (nn * 2 + sl) * kTileBytes);
        if constexpr (AFF)
          sv[nn] = make_float2(__uint_as_float(*reinterpret_cast<const uint32_t *>(
                                   sw + (nn * 2 + sl) * kTileScales * 4)),
                               0.0f);
        else
          sv[nn] = *reinterpret_cast<const float2 *>(sw + (nn * 2 + sl) * kTileScales * 4);
      }
    }
    // block scales, or (affine) 16 s from the params dword: P sums x (1 + q/16)
    auto f16lo = [](float v) {
      return 16.0f * (float)__builtin_bit_cast(_Float16, (uint16_t)(__float_as_uint(v) & 0xFFFFu));
    };
    const float s0 = AFF ? f16lo(sv[0].x) : PH ? sv[0].y : sv[0].x;
    const float s1 = AFF ? f16lo(sv[1].x) : PH ? sv[1].y : sv[1].x;
    f32x4 p[MB][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const char *pa = ldsA + (PH * 2 + hf) * tile::kAHalf + afr;
      bf16x8 A[MB], B[2];
#pragma unroll
      for (int mm = 0; mm < MB; ++mm) A[mm] = *reinterpret_cast<const bf16x8 *>(pa + mm * 1024);
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        // quarter 2 PH + hf of the tile: code dword 2 PH + hf of the lane
        const uint32_t wd = (2 * PH + hf) == 0 ? cv[nn].x : (2 * PH + hf) == 1 ? cv[nn].y
                          : (2 * PH + hf) == 2 ? cv[nn].z : cv[nn].w;
        uint32_t bb[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          if constexpr (AFF) {
            // bf16 (1 + c/16) of codes 2qq, 2qq + 1 (interleaved nibbles)
            bb[qq] = awq_pair(wd, qq, 0x3F803F80u);
          } else {
            const uint32_t a = __builtin_amdgcn_perm(wd, lane4, 0x0c0c0400u + (qq << 8));
            bb[qq] = *reinterpret_cast<const uint32_t *>(lds + a);
          }
        }
        B[nn] = __builtin_bit_cast(bf16x8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
      }
#pragma unroll
      for (int mm = 0; mm < MB; ++mm)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
          if constexpr (AFF)
            pz[mm][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                A[mm], B[nn], (PH == 0 && hf == 0) ? zero : pz[mm][nn], 0, 0, 0);
          else
            p[mm][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mm], B[nn],
                                                                hf ? p[mm][nn] : zero, 0, 0, 0);
        }
    }
    if constexpr (AFF) {
      if (PH == 1) {
        const int sl = (t >> 1) & 1;
        // -(16 + z) / 16, exact
        const float nz0 = -(float)(16u + (__float_as_uint(sv[0].x) >> 16)) * 0.0625f;
        const float nz1 = -(float)(16u + (__float_as_uint(sv[1].x) >> 16)) * 0.0625f;
#pragma unroll
        for (int mm = 0; mm < MB; ++mm) {
          const f32x4 xz = *reinterpret_cast<const f32x4 *>(xw + sl * tile::kXSum + mm * 64);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[mm][0][i] = fmaf(s0, fmaf(nz0, xz[i], pz[mm][0][i]), acc[mm][0][i]);
            acc[mm][1][i] = fmaf(s1, fmaf(nz1, xz[i], pz[mm][1][i]), acc[mm][1][i]);
          }
        }
      }
    } else {
#pragma unroll
      for (int mm = 0; mm < MB; ++mm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[mm][0][i] = fmaf(s0, p[mm][0][i], acc[mm][0][i]);
          acc[mm][1][i] = fmaf(s1, p[mm][1][i], acc[mm][1][i]);
        }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // The workspace pointers are first needed after the loop; taking them into
  // scalar registers here keeps their loads from being in flight through the
  // loop, where the waits for LDS reads would otherwise have to wait for
  // everything (scalar loads return out of order).
  if constexpr (SPLIT) asm volatile("" ::"s"(cnt), "s"(part));
  int t = 0;
  for (; t + 1 < S; t += 2) {
    step(P0{}, t);
    step(P1{}, t + 1);
  }
  if (t < S) step(P0{}, t);
  // the clamped copies of the last steps must land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (SPLIT) {
    // K in np parts: each workgroup of the output tile stores its sums
    // (thread-major, 8 bytes per lane and store) device-wide, then counts its
    // arrival; the last to arrive adds the parts' sums in part order (its
    // own from registers), stores y and sets the counter back to zero.
    constexpr int NV = MB * 4;  // 8-byte pairs of sums per thread
    const int64_t tile_id = (int64_t)nt * ntm + mt;
    const int64_t slot_u64 = (int64_t)L::kThreads * NV;
    uint64_t *mine = part + (tile_id * np + kc) * slot_u64 + tid;
#pragma unroll
    for (int mm = 0; mm < MB; ++mm)
#pragma unroll
      for (int nn = 0; nn < 2; ++nn)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const uint64_t v = (uint64_t)__float_as_uint(acc[mm][nn][2 * i2]) |
                             ((uint64_t)__float_as_uint(acc[mm][nn][2 * i2 + 1]) << 32);
          __hip_atomic_store(mine + ((mm * 2 + nn) * 2 + i2) * L::kThreads, v, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
    // Release/acquire through the arrival counter: every wave's stores of
    // its sums have completed (agent-scope atomic stores, waited for), the
    // barrier orders them before the counting read-modify-write, which is
    // acquire-release at agent scope, and the barrier after it orders that
    // acquire before every wave's loads of the other parts.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // also: no wave reads LDS any more
    int *flag = reinterpret_cast<int *>(lds);
    if (tid == 0)
      *flag = (int)__hip_atomic_fetch_add(cnt + tile_id, 1u, __ATOMIC_ACQ_REL,
                                          __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*flag != np - 1) return;
    f32x4 tot[MB][2], pj[MB][2];
    for (int j = 0; j < np; ++j) {
      if (j == kc) {
#pragma unroll
        for (int mm = 0; mm < MB; ++mm)
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) pj[mm][nn] = acc[mm][nn];
      } else {
        // one batch of loads per part
        const uint64_t *src = part + (tile_id * np + j) * slot_u64 + tid;
#pragma unroll
        for (int mm = 0; mm < MB; ++mm)
#pragma unroll
          for (int nn = 0; nn < 2; ++nn)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
              const uint64_t v = __hip_atomic_load(src + ((mm * 2 + nn) * 2 + i2) * L::kThreads,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              pj[mm][nn][2 * i2] = __uint_as_float((uint32_t)v);
              pj[mm][nn][2 * i2 + 1] = __uint_as_float((uint32_t)(v >> 32));
            }
      }
#pragma unroll
      for (int mm = 0; mm < MB; ++mm)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) tot[mm][nn] = j ? tot[mm][nn] + pj[mm][nn] : pj[mm][nn];
    }
#pragma unroll
    for (int mm = 0; mm < MB; ++mm)
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) acc[mm][nn] = tot[mm][nn];
    if (tid == 0) __hip_atomic_store(cnt + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

#pragma unroll
  for (int mm = 0; mm < MB; ++mm)
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int64_t g = gblk + wn * 2 + nn;
      if (g >= G) continue;
      const int64_t col = g * kTileRows + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 16 * MB + mm * 16 + 4 * h + i;
        if (row < M) y[row * N + col] = acc[mm][nn][i];
      }
    }
}

// ---------------------------------------------------------------------------
// Pipelined tiled kernel (codebook format, 128 x 16 RG outputs per
// workgroup): WAVES waves, each owning all 128 rows and RG / WAVES row
// groups (RG 16, 8 waves: 128 x 32 each, two per SIMD in one workgroup per
// CU; RG 16, 4 waves: 128 x 64 each, one per SIMD, two workgroups per CU;
// RG 14, 7 waves: 128 x 32 each, one workgroup per CU).
//
// What shaped it (measured on MI355X, LDS read rates per CU):
//  - A fragments: a 16-byte read per lane is conflict free when the four
//    16-byte chunks of row r sit at chunk ^ ((r >> 1) & 3); the swizzle
//    (r >> 2) & 3 halves the rate.
//  - Lookups of code bytes: 4-byte reads of random entries cost about eight
//    cycles per wave whatever the table's replication (the LDS serves a
//    limited number of distinct 16-byte lines per cycle), so the pair table
//    is one copy of 256 entries (1 KB) at byte << 2, which leaves LDS for
//    two workgroups per CU.
//  - Two workgroups per CU (4 waves each) are not held in step by each
//    other's barriers; on matrices with enough output tiles this is 8-10 %
//    faster than one workgroup of 8 waves, on few tiles slower.
//
// Pipeline.  x sits in two LDS stages of one 64-k step (16 KB, the two
// 32-k halves each laid out [row][32 bf16] in 16-row blocks of 1 KB).  Step
// t opens with the workgroup's barrier: every wave has landed its copies of
// x(t) (waited for with vmcnt) and no wave reads stage (t - 1) % 2 any
// more, so right after it each wave copies its share of x(t + 1) into that
// stage.  Code words and scales are wave-private: each wave copies the
// device tiles of its own row groups into a two-slot ring (tile T + 1 at
// step 2T - 1) and only waits for its own copies.  A fragments are read
// PD blocks ahead within the step; the B fragments (table lookups) and
// block scales of step t + 1 are formed during step t.  Items (16-row
// block, row group) run in order, each its two products and then the fold
// of the item two before it, whose products have finished: the fold's
// vector FMAs run beside the matrix instructions and only three products
// are live.
// Every output gets the operations of the other kernels: per 64-block
// P = MFMA(kk=0, zero), MFMA(kk=1, P), acc = fmaf(s, P, acc), in K order.
// K in np parts (SPLIT) as gemm_tile_kernel.
namespace wide {
constexpr int kBM = 128, kMB = 8;
constexpr int kXStage = 2 * tile::kAHalf;       // 16 KB: both halves of a step
constexpr int kStages = 2;
constexpr int kTable = 256 * 4;                 // pairs of bf16 codes by code byte
constexpr int kOffX = kTable;
constexpr int kPrefetch = 3;                    // A blocks read ahead
// LDS of a workgroup of RG row groups (69 KB for 16)
template <int RG>
struct Lay {
  static constexpr int kOffC = kOffX + kStages * kXStage;
  static constexpr int kOffS = kOffC + RG * 2 * kTileBytes;
  static constexpr int kBytes = kOffS + RG * 2 * kTileScales * 4;
};
template <int WAVES, int RG>
struct Geo {
  static_assert(RG % WAVES == 0, "row groups split evenly over the waves");
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kRGW = RG / WAVES;                // row groups per wave
  static constexpr int kXCopies = (16 + WAVES - 1) / WAVES;  // 1 KB copies of x per wave and step (at most)
  static constexpr int kTileCopies = 2 * kRGW;           // code + scale copies per wave and tile
  static constexpr int kItems = kMB * kRGW;              // items per step
  static constexpr int kWordItem = 2 * kRGW;             // code words of step t + 1
  static constexpr int kLookItem = 3 * kRGW + 4;         // first B lookup of step t + 1
  static_assert(kMB % (kPrefetch + 1) == 0, "A ring slots repeat per step");
  static_assert(kLookItem + 2 * kRGW <= kItems, "lookups within the step");
};
}  // namespace wide

template <int WAVES, int RG, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void gemm_wide_kernel(
    const uint16_t *__restrict__ x, int64_t M, const uint8_t *__restrict__ qw,
    const float *__restrict__ am, CodeTerms ct, int64_t N, int64_t K, int64_t KT,
    float *__restrict__ y, int ntn, int ntm, int np_arg, uint32_t *__restrict__ cnt,
    uint64_t *__restrict__ part) {
  namespace W = wide;
  using Gm = W::Geo<WAVES, RG>;
  using L = W::Lay<RG>;
  constexpr int RGW = Gm::kRGW, PD = W::kPrefetch;
  const int np = SPLIT ? np_arg : 1;
  // the only static LDS array, so the table sits at LDS address 0
  __shared__ __attribute__((aligned(16))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, h = lane >> 4;
  // tile order for the 8 XCDs as in gemm_tile_kernel
  const int xcd = (int)(blockIdx.x & 7), slot = (int)(blockIdx.x >> 3);
  const int u = (slot / ntm) * 8 + xcd, mt = slot % ntm;
  if (u >= ntn * np) return;
  const int nt = u / np, kc = u - nt * np;
  const int64_t m0 = (int64_t)mt * W::kBM;
  const int64_t gblk = (int64_t)nt * RG;
  const int64_t G = N / kTileRows;
  const int t0 = SPLIT ? part_begin(kc, KT, np) : 0;
  const int t1 = SPLIT ? part_begin(kc + 1, KT, np) : (int)KT;
  const int KTp = t1 - t0;
  const int S = (int)(2 * (int64_t)t1 < K / kBK ? 2 * (int64_t)t1 : K / kBK) - 2 * t0;
  x += (int64_t)t0 * kTileK;
  qw += (int64_t)t0 * kTileBytes;
  am += (int64_t)t0 * kTileScales;
  const uint32_t base = lds_addr(lds);

  // x copies: copy i (16 per step, 1 KB each) fills rows 16 (i % 8) .. + 15
  // of half i / 8; wave w issues i = w, w + WAVES, ...  Lane l fills chunk
  // slot l % 4 of row 16 (i % 8) + l / 4, i.e. logical chunk
  // (l % 4) ^ ((l >> 3) & 3).  The row block and half go into the scalar
  // base, the lane's row and chunk into one offset shared by the copies; in
  // the last, ragged row tile rows past M re-read row M - 1 (never stored),
  // with offsets from x formed per copy (M K 2 < 2^32).
  const int cx = (lane & 3) ^ ((lane >> 3) & 3);
  const uint32_t xl = (uint32_t)(((lane >> 2) * K + cx * 8) * 2);
  const bool ragged = m0 + W::kBM > M;
  const uint32_t lane16 = (uint32_t)lane * 16;
  auto copy_x = [&](int step, int stage) {
    const int64_t sc = (int64_t)(step < S ? step : S - 1) * kBK;
#pragma unroll
    for (int v = 0; v < Gm::kXCopies; ++v) {
      const int i = wave + v * WAVES, blk = i % 8, half = i / 8;
      if (Gm::kXCopies * WAVES != 16 && i >= 16) break;  // uneven split: scalar branch
      const int64_t r0 = m0 + 16 * blk;
      const uint32_t dst = base + W::kOffX + stage * W::kXStage + half * tile::kAHalf + blk * 1024;
      if (!ragged) {
        copy16_to_lds(dst, x + r0 * K + half * 32 + sc, xl);
      } else {
        // offsets from x itself (a block may lie wholly past M)
        const int64_t R = r0 + (lane >> 2);
        const uint32_t off = (uint32_t)(((R < M ? R : M - 1) * K + cx * 8) * 2);
        copy16_to_lds(dst, x + half * 32 + sc, off);
      }
    }
  };
  // code words and scales of this wave's row groups (past N: the last row
  // group, never stored), one scalar base per row group
  auto copy_tile = [&](int T) {
    const int64_t tc = T < KTp ? T : KTp - 1;
#pragma unroll
    for (int q = 0; q < RGW; ++q) {
      const int64_t rg = gblk + wave * RGW + q;
      const int64_t g = rg < G ? rg : G - 1;
      const int dst = (q * 2 + (T & 1));
      copy16_to_lds(base + L::kOffC + (wave * RGW * 2 + dst) * kTileBytes,
                    qw + (g * KT + tc) * kTileBytes, lane16);
      if (lane < kTileScales * 4 / 16)
        copy16_to_lds(base + L::kOffS + (wave * RGW * 2 + dst) * kTileScales * 4,
                      am + (g * KT + tc) * kTileScales, lane16);
    }
  };

  // table entry e: the bf16 pair of codes e & 15 (low half) and e >> 4
  for (int e = tid; e < 256; e += Gm::kThreads)
    reinterpret_cast<uint32_t *>(lds)[e] =
        (uint32_t)ct.t[0][e & 15] | ((uint32_t)ct.t[0][e >> 4] << 16);
  copy_x(0, 0);
  copy_tile(0);
  copy_tile(1);
  pipe::wait_copies_and_barrier<0>();

  // A fragment: lane (r, h) holds row r of a 16-row block, bf16 8h .. 8h+7
  // of the half
  const char *pa0 = lds + W::kOffX + r * pipe::kHalfRow + ((h ^ ((r >> 1) & 3)) * 16);
  const char *pc0 = lds + L::kOffC + wave * RGW * 2 * kTileBytes + lane * 16;
  const char *ps0 = lds + L::kOffS + wave * RGW * 2 * kTileScales * 4 + r * 8;

  // B fragments (both 32-k halves of the wave's column blocks) and block
  // scales of step t: tile t / 2 in ring slot (t / 2) & 1, quarter 2 (t % 2)
  // + hf.  Two sets, by the parity of the step they serve.
  bf16x8 B[2][2][RGW];
  float sc[2][RGW];
  uint2 cw[RGW];  // code words of the coming step
  auto read_words = [&](int t) {
    const int slt = (t >> 1) & 1, par = t & 1;
#pragma unroll
    for (int q = 0; q < RGW; ++q)
      cw[q] = *reinterpret_cast<const uint2 *>(pc0 + (q * 2 + slt) * kTileBytes + par * 8);
  };
  auto read_scales = [&](int t, float (&so)[RGW]) {
    const int slt = (t >> 1) & 1, par = t & 1;
#pragma unroll
    for (int q = 0; q < RGW; ++q)
      so[q] = *reinterpret_cast<const float *>(ps0 + (q * 2 + slt) * kTileScales * 4 + par * 4);
  };
  // fragment f = hf * RGW + q from the code words: byte qq of the code word
  // (codes 2qq, 2qq + 1) is the table entry of B dword qq
  auto look = [&](int f, bf16x8 (&Bo)[2][RGW]) {
    const int hf = f / RGW, q = f % RGW;
    const uint32_t w = hf ? cw[q].y : cw[q].x;
    uint32_t bb[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      bb[qq] = *reinterpret_cast<const uint32_t *>(lds + 4 * ((w >> (8 * qq)) & 0xFFu));
    Bo[hf][q] = __builtin_bit_cast(bf16x8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
  };
  auto read_a = [&](int stage, int mm, bf16x8 &a0, bf16x8 &a1) {
    const char *p = pa0 + stage * W::kXStage + mm * 1024;
    a0 = *reinterpret_cast<const bf16x8 *>(p);
    a1 = *reinterpret_cast<const bf16x8 *>(p + tile::kAHalf);
  };

  f32x4 acc[W::kMB][RGW];
#pragma unroll
  for (int a2 = 0; a2 < W::kMB; ++a2)
#pragma unroll
    for (int b2 = 0; b2 < RGW; ++b2) acc[a2][b2] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // A fragments in flight: block mm is read PD blocks before its products,
  // into ring slot mm % (PD + 1)
  bf16x8 A0[PD + 1], A1[PD + 1];
  read_words(0);
  read_scales(0, sc[0]);
#pragma unroll
  for (int f = 0; f < 2 * RGW; ++f) look(f, B[0]);

  // step t, x in stage st = t % 2; PH = t % 2 fixes the copy wait: the
  // copies of x(t) that the barrier waits for were followed, when t - 1 was
  // odd, by the copies of a device tile, which may stay in flight
  auto step = [&](auto phc, int t) {
    constexpr int PH = decltype(phc)::value;
    constexpr int st = PH;
    constexpr int kLag = 2;
    f32x4 pr[kLag + 1];
    auto fold = [&](int item) {
      const int fm = item / RGW, fq = item % RGW;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[fm][fq][i] = fmaf(sc[PH][fq], pr[item % (kLag + 1)][i], acc[fm][fq][i]);
      // keeps the fold here: the compiler would otherwise sink it towards the
      // next use of acc, a step later, with every product of the step live
      asm volatile("" : "+v"(acc[fm][fq]));
    };
#pragma unroll
    for (int item = 0; item < Gm::kItems; ++item) {
      const int mm = item / RGW, q = item % RGW;
      if (item == 0) {
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PH == 0 ? Gm::kTileCopies : 0)
                     : "memory");
        copy_x(t + 1, st ^ 1);
        if (PH == 1) copy_tile((t >> 1) + 2);
#pragma unroll
        for (int i = 0; i < PD; ++i) read_a(st, i, A0[i], A1[i]);
      }
      if (item == Gm::kWordItem) {
        read_words(t + 1);
        read_scales(t + 1, sc[PH ^ 1]);
      }
      if (q == 0 && mm + PD < W::kMB) read_a(st, mm + PD, A0[(mm + PD) % (PD + 1)],
                                             A1[(mm + PD) % (PD + 1)]);
      if (item >= Gm::kLookItem && item < Gm::kLookItem + 2 * RGW)
        look(item - Gm::kLookItem, B[PH ^ 1]);
      f32x4 &p = pr[item % (kLag + 1)];
      const int sa = mm % (PD + 1);
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[sa], B[PH][0][q], zero, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[sa], B[PH][1][q], p, 0, 0, 0);
      if (item >= kLag) fold(item - kLag);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int item = Gm::kItems - kLag; item < Gm::kItems; ++item) fold(item);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if constexpr (SPLIT) asm volatile("" ::"s"(cnt), "s"(part));
  int t = 0;
  for (; t + 1 < S; t += 2) {
    step(P0{}, t);
    step(P1{}, t + 1);
  }
  if (t < S) step(P0{}, t);
  // the clamped copies of the last steps must land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (SPLIT) {
    // as gemm_tile_kernel: sums stored, arrival counted, the last workgroup
    // of the output tile adds the parts in part order
    constexpr int NV = W::kMB * RGW * 2;  // 8-byte pairs of sums per thread
    const int64_t tile_id = (int64_t)nt * ntm + mt;
    const int64_t slot_u64 = (int64_t)Gm::kThreads * NV;
    uint64_t *mine = part + (tile_id * np + kc) * slot_u64 + tid;
#pragma unroll
    for (int mm = 0; mm < W::kMB; ++mm)
#pragma unroll
      for (int q = 0; q < RGW; ++q)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const uint64_t v = (uint64_t)__float_as_uint(acc[mm][q][2 * i2]) |
                             ((uint64_t)__float_as_uint(acc[mm][q][2 * i2 + 1]) << 32);
          __hip_atomic_store(mine + ((mm * RGW + q) * 2 + i2) * Gm::kThreads, v,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    // Release/acquire through the arrival counter (see gemm_tile_kernel)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // also: no wave reads LDS any more
    int *flag = reinterpret_cast<int *>(lds);
    if (tid == 0)
      *flag = (int)__hip_atomic_fetch_add(cnt + tile_id, 1u, __ATOMIC_ACQ_REL,
                                          __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*flag != np - 1) return;
    // one 16-row block at a time, every part (this one's too) read back from
    // its slot: the registers hold one block's sums, not all parts' at once
#pragma unroll
    for (int mm = 0; mm < W::kMB; ++mm) {
      f32x4 tot[RGW];
      for (int j = 0; j < np; ++j) {
        const uint64_t *src = part + (tile_id * np + j) * slot_u64 + tid;
        f32x4 pj[RGW];
#pragma unroll
        for (int q = 0; q < RGW; ++q)
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            const uint64_t v = __hip_atomic_load(src + ((mm * RGW + q) * 2 + i2) * Gm::kThreads,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pj[q][2 * i2] = __uint_as_float((uint32_t)v);
            pj[q][2 * i2 + 1] = __uint_as_float((uint32_t)(v >> 32));
          }
#pragma unroll
        for (int q = 0; q < RGW; ++q) tot[q] = j ? tot[q] + pj[q] : pj[q];
      }
#pragma unroll
      for (int q = 0; q < RGW; ++q) acc[mm][q] = tot[q];
    }
    if (tid == 0) __hip_atomic_store(cnt + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

#pragma unroll
  for (int mm = 0; mm < W::kMB; ++mm)
#pragma unroll
    for (int q = 0; q < RGW; ++q) {
      const int64_t g = gblk + wave * RGW + q;
      if (g >= G) continue;
      const int64_t col = g * kTileRows + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + mm * 16 + 4 * h + i;
        if (row < M) y[row * N + col] = acc[mm][q][i];
      }
    }
}

// ---------------------------------------------------------------------------
// Skinny path, M <= 64, and up to 256 rows on narrow N (a decode batch, a
// short prefill chunk or the tail of a long one).  There the weights
// dominate: the job is to stream them at the memory rate, which a K loop
// synchronised at every step cannot do with few tiles across N.  Instead
// each wave owns one row group and streams all of its K on its own, like the
// decode GEMV, keeping D weight tiles in flight in registers; only x is
// shared, staged in LDS in 16 KB chunks (double buffered, one barrier per
// chunk).  Per tile the lane's 16 code bytes become the B fragments of four
// 32-k MFMA steps through the pair table, and the MB m-blocks of x (one or
// two 16-row blocks; more rows as further workgroups along the grid's y)
// supply the A fragments.
// Every output is computed with exactly the operations of gemm_tile_kernel:
// per 64-block P = MFMA(kk=0, zero) then MFMA(kk=1, P), acc = fmaf(s, P, acc)
// in K order, with the same operand values in the same lanes, so the two
// kernels give bit-identical rows and the choice between them (by M) does
// not change any row.  Affine variant (AFF): no table (B pairs from the
// interleaved code words by shift and mask), the x sums of a chunk's tiles
// and rows (TC x XR floats from the pre-pass) staged in LDS with the x
// chunk, and per tile P = four MFMAs from zero, g = fmaf(-(16 + z)/16, X,
// P), acc = fmaf(16 s, g, acc), as in the tiled kernel's affine variant.
// ---------------------------------------------------------------------------
namespace skinny {
constexpr int kWaves = 4;        // row groups per workgroup
constexpr int kXBuf = 16 * 1024; // bytes of one x chunk buffer (2 or 3 workgroups per CU fit)
}  // namespace skinny
// OCC workgroups per CU.  Two (the launch bound caps a lane at 256
// registers): at one wave per SIMD each wave's chain of lookups, products
// and folds is exposed; the 32-row instance keeps 4 tiles in flight per wave
// (8 do not fit in 256 registers).  Three, for grids of more than two rounds
// of two (gate|up at up to 64 rows: 592 or 1184 workgroups on 256 CUs): 168
// registers, so half the tiles in flight (4 and 2), and a pair table of 16
// copies (48 KB of LDS with x); one round of three measured 5-14 % faster
// than two rounds of two, and slower on grids of one round.

template <int MB, int D, bool AFF, bool SPLIT, int OCC>
__global__ __launch_bounds__(64 * skinny::kWaves, OCC) void gemm_skinny_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ qw,
    const float *__restrict__ am, CodeTerms ct, int N, int K, int KT, int G,
    float *__restrict__ y, const float *__restrict__ xsum, int Mp, int np_arg) {
  // K in np parts (SPLIT) or in one
  const int np = SPLIT ? np_arg : 1;
  constexpr int XR = 16 * MB;                  // x rows held (m-blocks of 16)
  constexpr int KX = skinny::kXBuf / (XR * 2); // k per chunk: 512 (MB 1), 256 (MB 2)
  constexpr int TC = KX / kTileK;              // tiles per chunk: 4, 2
  constexpr int CPR = KX / 8;                  // 16-byte chunks per x row
  constexpr int XV = skinny::kXBuf / 16 / (64 * skinny::kWaves);  // loads per thread per chunk
  static_assert(D % TC == 0, "the prefetch ring is a whole number of chunks");
  constexpr int XSB = TC * XR * 4;             // x sums of a chunk, bytes (512)
  static_assert(XSB / 16 <= 64 * skinny::kWaves, "one 16-byte load per thread");
  constexpr int SKC = OCC == 3 ? 16 : pipe::kCopies;  // pair-table copies
  constexpr int TB = AFF ? 0 : 256 * SKC * 4;  // the affine variant has no table
  __shared__ __attribute__((aligned(16))) char lds[2 * skinny::kXBuf + TB + (AFF ? 2 * XSB : 0)];
  char *ldsT = lds + 2 * skinny::kXBuf;
  char *ldsX = ldsT + TB;  // affine: x sums [buffer][tile][row]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, h = lane >> 4;
  const int g = blockIdx.x * skinny::kWaves + wave;
  const int gc = g < G ? g : G - 1;  // a wave past N re-reads the last row group, stores nothing
  const int m0 = blockIdx.y * XR;    // first x row of this workgroup
  const int NC = (KT + TC - 1) / TC;  // chunks
  const bool half_tail = (K & (kTileK - 1)) != 0;  // last tile holds one 64-block

  // ---- x chunk c -> registers (rows past M re-read row M-1; k past K is 0);
  // affine: also 16 bytes of the chunk's x sums per thread below XSB / 16
  // (thread i: tile i / (XR / 4), rows m0 + 4 (i % (XR / 4)) .. + 3)
  uint4 xsv = make_uint4(0u, 0u, 0u, 0u);
  auto load_x = [&](int c, uint4 (&xv)[XV]) {
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int q = tid + u * 64 * skinny::kWaves;
      const int R = q / CPR, cr = q - R * CPR;
      const int k = c * KX + cr * 8;
      const int m = m0 + R < M ? m0 + R : M - 1;
      xv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (c < NC && k < K) xv[u] = *reinterpret_cast<const uint4 *>(x + (int64_t)m * K + k);
    }
    if constexpr (AFF) {
      xsv = make_uint4(0u, 0u, 0u, 0u);
      const int tl = tid / (XR / 4), part = tid % (XR / 4), t = c * TC + tl;
      if (tid < XSB / 16 && c < NC && t < KT)
        xsv = *reinterpret_cast<const uint4 *>(xsum + (int64_t)t * Mp + m0 + part * 4);
    }
  };
  // row R, 16-byte chunk cr stored at chunk cr ^ (R & 15): the 16 rows of an
  // A fragment fall in 16 different bank groups
  auto store_x = [&](int buf, const uint4 (&xv)[XV]) {
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int q = tid + u * 64 * skinny::kWaves;
      const int R = q / CPR, cr = q - R * CPR;
      *reinterpret_cast<uint4 *>(lds + buf * skinny::kXBuf + R * (KX * 2) +
                                 ((cr ^ (R & 15)) * 16)) = xv[u];
    }
    if constexpr (AFF) {
      if (tid < XSB / 16) *reinterpret_cast<uint4 *>(ldsX + buf * XSB + tid * 16) = xsv;
    }
  };

  // ---- pair table (32 copies), the codebook staged in x buffer 1 first
  uint16_t *codes16 = reinterpret_cast<uint16_t *>(lds + skinny::kXBuf);
  if (!AFF && tid < 16) codes16[tid] = ct.t[0][tid];
  // weight prefetch: tile i of this wave's row group
  const char *qrow = reinterpret_cast<const char *>(qw) + (int64_t)gc * KT * kTileBytes + lane * 16;
  // scales of a tile: two block scales, or (affine) the params dword in .x
  constexpr int SB = AFF ? kTileRows * 4 : kTileScales * 4;  // bytes per tile
  const char *srow = reinterpret_cast<const char *>(am) + (int64_t)gc * KT * SB + r * (AFF ? 4 : 8);
  auto load_s = [&](int i) -> float2 {
    if constexpr (AFF)
      return make_float2(
          __uint_as_float(*reinterpret_cast<const uint32_t *>(srow + (int64_t)i * SB)), 0.0f);
    else
      return *reinterpret_cast<const float2 *>(srow + (int64_t)i * SB);
  };
  uint4 wb[D];
  float2 sb[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int i = d < KT ? d : KT - 1;
    wb[d] = *reinterpret_cast<const uint4 *>(qrow + (int64_t)i * kTileBytes);
    sb[d] = load_s(i);
  }
  uint4 xv[XV];
  load_x(0, xv);
  __syncthreads();
  for (int c = tid; c < TB / 16; c += 64 * skinny::kWaves) {
    const int e = c / (SKC / 4);
    const uint32_t v = (uint32_t)codes16[e & 15] | ((uint32_t)codes16[e >> 4] << 16);
    reinterpret_cast<uint4 *>(ldsT)[c] = make_uint4(v, v, v, v);
  }
  store_x(0, xv);
  load_x(1, xv);
  __syncthreads();

  const uint32_t tcopy = (uint32_t)(lane & (SKC - 1)) * 4;
  // K in parts: tot adds the sums of the finished parts in part order; the
  // next part starts at tile `cut`
  f32x4 acc[MB], tot[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = tot[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  int jn = 1, cut = SPLIT ? part_begin(1, KT, np) : -1;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // A fragment of row mb*16 + r, logical chunk `cl` of the chunk's row
  const uint32_t arow = (uint32_t)(r * (KX * 2));
  // B fragments of the four 32-k steps of a tile, from the lane's 16 code bytes
  auto lookups = [&](const uint4 &w, bf16x8 (&B)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t wd = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
      uint32_t bb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (AFF) {
          bb[q] = awq_pair(wd, q, 0x3F803F80u);
        } else {
          const uint32_t e = (wd >> (8 * q)) & 0xFFu;
          bb[q] = *reinterpret_cast<const uint32_t *>(ldsT + e * (SKC * 4) + tcopy);
        }
      }
      B[j] = __builtin_bit_cast(bf16x8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
    }
  };
  // The lookups run one tile ahead of the products (two sets chosen by tile
  // parity, D even), so their LDS latency overlaps the matrix instructions.
  static_assert(D % 2 == 0, "B sets alternate by tile parity");
  bf16x8 Bs[2][4];
  lookups(wb[0], Bs[0]);

  for (int base = 0; base < NC * TC; base += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = base + d;                // tile
      const int tl = d % TC, cbuf = (i / TC) & 1;
      // Tiles past K and the empty second block of a half tile run on
      // clamped codes and scales and on x that is zero past K, so their
      // products are exact zeros; they are folded with a zero scale, which
      // leaves every accumulator as it is (an accumulator is never -0: it
      // starts at +0 and a zero sum rounds to +0).
      const bool live0 = i < KT, live1 = live0 && !(half_tail && i == KT - 1);
      if (SPLIT && i == cut) {  // the next part of K starts from zero
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          tot[mb] = jn == 1 ? acc[mb] : tot[mb] + acc[mb];
          acc[mb] = zero;
        }
        ++jn;
        cut = jn < np ? part_begin(jn, KT, np) : -1;
      }
      lookups(wb[(d + 1) % D], Bs[(d + 1) & 1]);
      const bf16x8 (&B)[4] = Bs[d & 1];
      const char *xc = lds + cbuf * skinny::kXBuf + arow;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const char *xm = xc + mb * 16 * (KX * 2);
        bf16x8 A[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          A[j] = *reinterpret_cast<const bf16x8 *>(xm + (((tl * 16 + j * 4 + h) ^ r) * 16));
        if constexpr (AFF) {
          const uint32_t pv = __float_as_uint(sb[d].x);
          const float sc = 16.0f * (float)__builtin_bit_cast(_Float16, (uint16_t)(pv & 0xFFFFu));
          const float nz = -(float)(16u + (pv >> 16)) * 0.0625f;
          const f32x4 xz = *reinterpret_cast<const f32x4 *>(ldsX + cbuf * XSB +
                                                            (tl * XR + mb * 16 + 4 * h) * 4);
          f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], B[0], zero, 0, 0, 0);
#pragma unroll
          for (int j = 1; j < 4; ++j)
            P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[j], B[j], P, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[mb][e] = fmaf(live0 ? sc : 0.0f, fmaf(nz, xz[e], P[e]), acc[mb][e]);
          continue;
        }
        f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], B[0], zero, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], B[1], p, 0, 0, 0);
        f32x4 q2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2], B[2], zero, 0, 0, 0);
        q2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[3], B[3], q2, 0, 0, 0);
        if constexpr (MB == 1 && OCC == 3) {
          // selects on the accumulators: the zero-scale form spills here
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float f0 = fmaf(sb[d].x, p[e], acc[mb][e]);
            const float a0 = live0 ? f0 : acc[mb][e];
            const float f1 = fmaf(sb[d].y, q2[e], a0);
            acc[mb][e] = live1 ? f1 : a0;
          }
        } else {
          const float s0 = live0 ? sb[d].x : 0.0f, s1 = live1 ? sb[d].y : 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[mb][e] = fmaf(s1, q2[e], fmaf(s0, p[e], acc[mb][e]));
        }
      }
      // ---- refill this slot D tiles ahead (clamped: same loads every step)
      {
        const int ni = i + D < KT ? i + D : KT - 1;
        wb[d] = *reinterpret_cast<const uint4 *>(qrow + (int64_t)ni * kTileBytes);
        sb[d] = load_s(ni);
      }
      // ---- chunk boundary: x of the next chunk into the other buffer (it
      // held the chunk before this one, which every wave finished before the
      // previous barrier), the loads of the chunk after, then the barrier
      // that makes the next chunk visible
      if (tl == TC - 1) {
        const int cn = i / TC + 1;
        store_x(cn & 1, xv);
        load_x(cn + 1, xv);
        __syncthreads();
      }
      // (no scheduling barrier between tiles: letting the compiler overlap
      // consecutive tiles measured 1-3 % faster on most shapes)
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + mb * 16 + 4 * h + e;
      const float v = SPLIT ? tot[mb][e] + acc[mb][e] : acc[mb][e];
      if (g < G && m < M) y[(int64_t)m * N + (int64_t)g * 16 + r] = v;
    }
}

// ---------------------------------------------------------------------------
// Narrow kernel (short M, few row groups, both formats).  The skinny kernel
// gives each row group one wave, so q|k|v, o and down (224 to 288 row groups)
// run on that many waves, each bound by its own chain of lookups, products
// and folds: with every weight load hitting the caches it is no faster.
// Here the kWaves waves of a workgroup share one row group and one 16-row
// block of x and take its tiles in turn: window j is tiles kWaves j .. +
// kWaves - 1, wave w computing tile w of each window.  Per tile a wave forms
// the block products of its two 64-blocks as the other kernels do
// (P = MFMA(kk=0, zero), MFMA(kk=1, P)) and parks them in LDS with the
// tile's block scales; one window later, past the next barrier, wave e folds
// outputs 16 e .. 16 e + 15 of the lane order (lane l: output lane
// 16 e + l / 4, element l % 4) through the window's tiles in K order,
// acc = fmaf(s, P, acc).  Every output gets the other kernels' operations
// in their order, so its rows are bit-identical to theirs.
// x (16 rows x 512 k per window), code words and scales all arrive by copies
// into LDS rings LEAD windows ahead; there are no register loads in the
// loop, so one explicit count waits for exactly the window about to be used.
// x row R is copied with its 16-byte chunk c stored at c ^ R, so the 16 rows
// of an A fragment read fall in 16 bank groups.
// LDS (bytes): pair table, x ring (LEAD + 1) x 16 K, code ring (LEAD + 1) x
// kWaves x 1 K, scale ring (LEAD + 1) x kWaves x 128, block products 2 x
// kWaves x 2 K and their scales 2 x kWaves x 128.  LEAD 2 with a one-copy
// table (1 K): 79.5 K, so two workgroups share a CU (8 waves), for grids of
// more workgroups than CUs; with one per CU the waves, one per SIMD, sat
// mostly waiting on their chain of LDS reads, products and barriers, and two
// per CU measured 1.25-1.35 x faster on 29- and 32-row batches.  LEAD 3 with
// 32 copies (32 K, lane % 32 reads its own) at one workgroup per CU for
// grids that fit the CUs once: there the replicated table measured 8 %
// faster on long K than the single copy.
// Affine variant (AFF, int4 in groups of 128): no pair table (B pairs from
// the interleaved code words by shift and mask), one product per tile (four
// MFMAs from zero), 64 bytes of params per tile, and the x sums X[t][m0 ..
// m0 + 15] of the pre-pass copied with each window; the computing wave moves
// its tile's 16 sums next to the product, and the fold takes
// g = fmaf(-(16 + z)/16, X, P), acc = fmaf(16 s, g, acc), as the tiled and
// skinny kernels' affine variants do.
// ---------------------------------------------------------------------------
namespace narrow {
constexpr int kWaves = 4;                            // waves per row group = tiles per window
constexpr int kKW = kWaves * kTileK;                 // k per window: 512
constexpr int kXSlot = 16 * kKW * 2;                 // 16 K
constexpr int kCSlot = kWaves * kTileBytes;          // 4 K
constexpr int kCuLds = 160 * 1024;                   // LDS per CU
static_assert(16 % kWaves == 0, "x rows split evenly over the waves");
// LDS layout; the affine variant has no pair table, one block product per
// tile, 64 bytes of params per tile and a ring of the x sums (16 rows per tile)
template <bool AFF, int LEAD>
struct Lay {
  static constexpr int kSlots = LEAD + 1;             // ring slots
  // pair-table copies (lane % kCopiesT): 32 at one workgroup per CU, one at two
  static constexpr int kCopiesT = AFF ? 0 : LEAD == 2 ? 1 : 32;
  static constexpr int kTable = 256 * 4 * kCopiesT;
  static constexpr int kSBytes = AFF ? kTileRows * 4 : kTileScales * 4;  // scales of a tile
  static constexpr int kSSlot = kWaves * kSBytes;
  static constexpr int kXSSlot = AFF ? kWaves * 16 * 4 : 0;
  static constexpr int kBlocks = AFF ? 1 : 2;         // block products per tile
  static constexpr int kPBuf = kWaves * kBlocks * 1024;
  static constexpr int kSBuf = kWaves * 16 * 8;     // one float2 per weight row
  static constexpr int kXBuf = AFF ? kWaves * 16 * 4 : 0;
  static constexpr int kOffX = kTable;
  static constexpr int kOffC = kOffX + kSlots * kXSlot;
  static constexpr int kOffS = kOffC + kSlots * kCSlot;
  static constexpr int kOffXS = kOffS + kSlots * kSSlot;
  static constexpr int kOffP = kOffXS + kSlots * kXSSlot;
  static constexpr int kOffSB = kOffP + 2 * kPBuf;
  static constexpr int kOffXB = kOffSB + 2 * kSBuf;
  static constexpr int kBytes = kOffXB + 2 * kXBuf;
  // per wave and window: x rows, code words, scales (and x sums)
  static constexpr int kCopies = 16 / kWaves + 2 + (AFF ? 1 : 0);
  static_assert(LEAD != 2 || 2 * kBytes <= kCuLds, "LDS of two workgroups");
  static_assert(kBytes <= kCuLds, "LDS of one workgroup");
  static_assert((LEAD - 1) * kCopies <= 63, "vmcnt range");
};
}  // namespace narrow

template <bool AFF, bool SPLIT, int LEAD>
__global__ __launch_bounds__(64 * narrow::kWaves, LEAD == 2 ? 2 : 1) void gemm_narrow_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ qw,
    const float *__restrict__ am, CodeTerms ct, int N, int K, int KT, int G,
    float *__restrict__ y, const float *__restrict__ xsum, int Mp, int np_arg) {
  using namespace narrow;
  using L = Lay<AFF, LEAD>;
  constexpr int kSlots = L::kSlots;
  const int np = SPLIT ? np_arg : 1;
  // the only static LDS array: the pair table sits at LDS address 0
  __shared__ __attribute__((aligned(16))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, h = lane >> 4;
  const int g = blockIdx.x;           // row group
  const int m0 = blockIdx.y * 16;     // first x row
  const int NW = (KT + kWaves - 1) / kWaves;
  const bool half_tail = (K & (kTileK - 1)) != 0;  // last tile holds one 64-block
  const uint32_t base = lds_addr(lds);

  // copy sources: x rows kRows w .. of the 16-row block (rows past M re-read
  // row M - 1, k past K re-reads the row's last chunk: such values only
  // reach products that are never folded)
  constexpr int kRows = 16 / kWaves;
  uint32_t xrow[kRows];
  int xc[kRows];
#pragma unroll
  for (int v = 0; v < kRows; ++v) {
    const int R = wave * kRows + v;
    const int m = m0 + R < M ? m0 + R : M - 1;
    xrow[v] = (uint32_t)m * (uint32_t)K * 2u;
    xc[v] = lane ^ R;  // logical chunk copied into chunk slot `lane`
  }
  const uint32_t gtile = (uint32_t)g * (uint32_t)KT;
  auto copy_window = [&](int jw) {
    const int sl = jw % kSlots;
    if (!AFF && (jw + 1) * kKW <= K) {
      // whole window inside K: the window's k goes into the scalar base
      // (codebook format; the affine instances measured no faster)
      const char *xw = reinterpret_cast<const char *>(x) + (size_t)jw * (kKW * 2);
#pragma unroll
      for (int v = 0; v < kRows; ++v)
        copy16_to_lds(base + L::kOffX + sl * kXSlot + (wave * kRows + v) * (kKW * 2), xw,
                      xrow[v] + (uint32_t)xc[v] * 16u);
    } else {
#pragma unroll
      for (int v = 0; v < kRows; ++v) {
        const int k = jw * kKW + xc[v] * 8;
        const uint32_t kk = (uint32_t)(k < K ? k : K - 8);
        copy16_to_lds(base + L::kOffX + sl * kXSlot + (wave * kRows + v) * (kKW * 2), x,
                      xrow[v] + kk * 2u);
      }
    }
    const int i = jw * kWaves + wave;
    const int tl = i < KT ? i : KT - 1;
    const uint32_t ti = gtile + (uint32_t)tl;
    copy16_to_lds(base + L::kOffC + sl * kCSlot + wave * kTileBytes, qw,
                  ti * (uint32_t)kTileBytes + (uint32_t)lane * 16u);
    if (lane < L::kSBytes / 16)
      copy16_to_lds(base + L::kOffS + sl * L::kSSlot + wave * L::kSBytes, am,
                    ti * (uint32_t)L::kSBytes + (uint32_t)lane * 16u);
    if constexpr (AFF) {
      // x sums X[tile][m0 .. m0 + 15] (rows up to Mp, a multiple of 128)
      if (lane < 4)
        copy16_to_lds(base + L::kOffXS + sl * L::kXSSlot + wave * 64, xsum,
                      ((uint32_t)tl * (uint32_t)Mp + (uint32_t)m0) * 4u + (uint32_t)lane * 16u);
    }
  };
#pragma unroll
  for (int jw = 0; jw < LEAD; ++jw) copy_window(jw);

  // pair table, from the codebook staged in the (not yet used) product buffers
  if constexpr (!AFF) {
    uint16_t *codes16 = reinterpret_cast<uint16_t *>(lds + L::kOffP);
    if (tid < 16) codes16[tid] = ct.t[0][tid];
    __syncthreads();
    // entry e, copy c at 4 (e kCopiesT + c); with copies, four per 16-byte
    // store (each thread's chain of codebook reads stays short)
    constexpr int kPer = L::kCopiesT >= 4 ? 4 : 1;  // copies per store
    for (int i = tid; i < 256 * L::kCopiesT / kPer; i += 64 * kWaves) {
      const int e = i / (L::kCopiesT / kPer);
      const uint32_t v = (uint32_t)codes16[e & 15] | ((uint32_t)codes16[e >> 4] << 16);
      if constexpr (kPer == 4)
        reinterpret_cast<uint4 *>(lds)[i] = make_uint4(v, v, v, v);
      else
        reinterpret_cast<uint32_t *>(lds)[i] = v;
    }
  }
  const uint32_t tcopy = (uint32_t)(lane % (L::kCopiesT > 0 ? L::kCopiesT : 1)) * 4;

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // products of this wave's tile of window j into buffer j & 1, with the
  // tile's scales (and, affine, its x sums)
  auto compute = [&](int j) {
    const int sl = j % kSlots;
    const uint4 w = *reinterpret_cast<const uint4 *>(lds + L::kOffC + sl * kCSlot + wave * kTileBytes +
                                                     lane * 16);
    float2 sv;
    if constexpr (AFF)
      sv = make_float2(*reinterpret_cast<const float *>(lds + L::kOffS + sl * L::kSSlot +
                                                        wave * L::kSBytes + r * 4),
                       0.0f);
    else
      sv = *reinterpret_cast<const float2 *>(lds + L::kOffS + sl * L::kSSlot + wave * L::kSBytes +
                                             r * 8);
    bf16x8 A[4], B[4];
    const char *xr = lds + L::kOffX + sl * kXSlot + r * (kKW * 2);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      A[jj] = *reinterpret_cast<const bf16x8 *>(xr + (((wave * 16 + jj * 4 + h) ^ r) * 16));
      const uint32_t wd = jj == 0 ? w.x : jj == 1 ? w.y : jj == 2 ? w.z : w.w;
      uint32_t bb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (AFF) {
          // bf16 (1 + c/16) of codes 2q, 2q + 1 (interleaved nibbles)
          bb[q] = awq_pair(wd, q, 0x3F803F80u);
        } else {
          const uint32_t e = (wd >> (8 * q)) & 0xFFu;
          bb[q] = *reinterpret_cast<const uint32_t *>(lds + e * (L::kCopiesT * 4) + tcopy);
        }
      }
      B[jj] = __builtin_bit_cast(bf16x8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
    }
    char *pb = lds + L::kOffP + (j & 1) * L::kPBuf + wave * (L::kBlocks * 1024) + lane * 16;
    if constexpr (AFF) {
      // one group of 128: four MFMAs from zero
      f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], B[0], zero, 0, 0, 0);
#pragma unroll
      for (int jj = 1; jj < 4; ++jj) p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[jj], B[jj], p, 0, 0, 0);
      *reinterpret_cast<f32x4 *>(pb) = p;
      if (lane < 16)
        *reinterpret_cast<float *>(lds + L::kOffXB + (j & 1) * L::kXBuf + wave * 64 + lane * 4) =
            *reinterpret_cast<const float *>(lds + L::kOffXS + sl * L::kXSSlot + wave * 64 + lane * 4);
    } else {
      f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], B[0], zero, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], B[1], p, 0, 0, 0);
      f32x4 q2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2], B[2], zero, 0, 0, 0);
      q2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[3], B[3], q2, 0, 0, 0);
      *reinterpret_cast<f32x4 *>(pb) = p;
      *reinterpret_cast<f32x4 *>(pb + 1024) = q2;
    }
    // the scales of weight row r, once per row
    if (lane < 16)
      *reinterpret_cast<float2 *>(lds + L::kOffSB + (j & 1) * L::kSBuf + wave * 128 + lane * 8) = sv;
  };
  // fold window jf: this lane's output is element lane % 4 of output lane
  // 16 wave + lane / 4 (x row m0 + 4 wave + lane % 4, weight row lane / 4)
  float acc = 0.0f, tot = 0.0f;
  int jn = 1, cut = SPLIT ? part_begin(1, KT, np) : -1;
  auto fold = [&](int jf) {
    const char *pb = lds + L::kOffP + (jf & 1) * L::kPBuf + wave * 256 + lane * 4;
    const char *sb = lds + L::kOffSB + (jf & 1) * L::kSBuf + (lane >> 2) * 8;
    const char *xb = lds + L::kOffXB + (jf & 1) * L::kXBuf + (4 * wave + (lane & 3)) * 4;
    // WHOLE: four whole tiles inside K, folded without selects (codebook
    // format; the affine instances measured no faster)
    auto body = [&](auto wc) {
      constexpr bool WHOLE = decltype(wc)::value;
#pragma unroll
      for (int tw = 0; tw < kWaves; ++tw) {
        const int i = jf * kWaves + tw;
        if (SPLIT && i == cut) {  // the next part of K starts from zero
          tot = jn == 1 ? acc : tot + acc;
          acc = 0.0f;
          ++jn;
          cut = jn < np ? part_begin(jn, KT, np) : -1;
        }
        const bool live0 = i < KT, live1 = live0 && !(half_tail && i == KT - 1);
        const float2 s = *reinterpret_cast<const float2 *>(sb + tw * 128);
        if constexpr (AFF) {
          // 16 s and -(16 + z)/16 from the params dword (binary16 s | z << 16)
          const uint32_t pv = __float_as_uint(s.x);
          const float sc = 16.0f * (float)__builtin_bit_cast(_Float16, (uint16_t)(pv & 0xFFFFu));
          const float nz = -(float)(16u + (pv >> 16)) * 0.0625f;
          const float P = *reinterpret_cast<const float *>(pb + tw * 1024);
          const float xz = *reinterpret_cast<const float *>(xb + tw * 64);
          const float f = fmaf(sc, fmaf(nz, xz, P), acc);
          acc = WHOLE || live0 ? f : acc;
        } else {
          const float p0 = *reinterpret_cast<const float *>(pb + tw * 2048);
          const float p1 = *reinterpret_cast<const float *>(pb + tw * 2048 + 1024);
          const float f0 = fmaf(s.x, p0, acc);
          const float a0 = WHOLE || live0 ? f0 : acc;
          const float f1 = fmaf(s.y, p1, a0);
          acc = WHOLE || live1 ? f1 : a0;
        }
      }
    };
    if (!AFF && (jf + 1) * kWaves <= KT - (half_tail ? 1 : 0))
      body(std::true_type{});
    else
      body(std::false_type{});
  };

  for (int j = 0; j < NW; ++j) {
    // window j's copies have landed for every wave, and the products of
    // window j - 1 are in LDS
    pipe::wait_copies_and_barrier<(LEAD - 1) * L::kCopies>();
    copy_window(j + LEAD);  // into the slot window j - 1 used
    compute(j);
    if (j > 0) fold(j - 1);
  }
  // every copy has landed (the clamped ones past the end too) before the
  // workgroup can end, and the last window's products are in LDS
  pipe::wait_copies_and_barrier<0>();
  fold(NW - 1);

  const int m = m0 + 4 * wave + (lane & 3);
  if (m < M) y[(int64_t)m * N + (int64_t)g * 16 + (lane >> 2)] = SPLIT ? tot + acc : acc;
}

// ---------------------------------------------------------------------------
// Stream kernel (codebook format, up to 16 rows, few row groups).  As in the
// narrow kernel, the four waves of a group share one row group and take its
// tiles in turn (window j = tiles 4 j .. 4 j + 3 of the group's range, wave w
// computing tile w), park the block products in LDS and fold them in K order
// one window later.  What differs:
//  - a wave reads only its own tile's 128 k of x, so its A fragments, code
//    words and block scales come straight from global memory into registers,
//    two windows ahead (a ring of three register slots; the window loop is
//    unrolled by the ring), and no x is staged in LDS;
//  - with K in two parts (PG = 2) the workgroup holds two such groups, waves
//    0-3 folding part 0 and waves 4-7 part 1 side by side, and the group of
//    part 0 adds the two sums in part order at the end: a long-K matrix of
//    few row groups (down, N = 3584, K = 18944) runs twice the waves per
//    row group with no workspace.  With one part (PG = 1) a workgroup is one
//    group.
// LDS holds the pair table (32 copies, lane % 32 reads its own) and, per
// group, the block products and scales of two windows.  Every output gets
// the other kernels' operations in their order (P = MFMA(kk=0, zero),
// MFMA(kk=1, P), acc = fmaf(s, P, acc) in K order, parts added in part
// order), so its rows are bit-identical to theirs.
// ---------------------------------------------------------------------------
namespace stream {
constexpr int kW = 4;     // waves per group = tiles per window
constexpr int kLead = 2;  // windows loaded ahead
constexpr int kTable = 256 * 4 * 32;  // pair table, 32 copies
constexpr int kPBuf = kW * 2 * 1024;  // block products of one window (two 64-blocks per tile)
constexpr int kSBuf = kW * 16 * 8;    // their scales, a float2 per weight row
template <int PG>
struct Lay {
  static constexpr int kOffP = kTable;                  // [group][window parity]
  static constexpr int kOffSB = kOffP + PG * 2 * kPBuf;  // [group][window parity]
  static constexpr int kBytes = kOffSB + PG * 2 * kSBuf;
};
}  // namespace stream

template <bool SPLIT, int PG>
__global__ __launch_bounds__(64 * stream::kW * PG, PG == 1 ? 2 : 1) void gemm_stream_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ qw,
    const float *__restrict__ am, CodeTerms ct, int N, int K, int KT, float *__restrict__ y,
    int np_arg) {
  using L = stream::Lay<PG>;
  constexpr int W = stream::kW, LEAD = stream::kLead;
  constexpr int S = LEAD + 1;  // register ring slots
  static_assert(PG == 1 || SPLIT, "two part groups need K in two parts");
  const int np = SPLIT ? np_arg : 1;
  // the only static LDS array: the pair table sits at LDS address 0
  __shared__ __attribute__((aligned(16))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pg = PG == 1 ? 0 : wave / W;      // part group
  const int ww = PG == 1 ? wave : wave % W;   // wave within the group
  const int r = lane & 15, h = lane >> 4;
  const int g = blockIdx.x;                   // row group
  const int m0 = blockIdx.y * 16;             // first x row
  const bool half_tail = (K & (kTileK - 1)) != 0;  // last tile holds one 64-block
  // this group's tiles [t0, t1); part 0 is the longer of two, so both groups
  // run its number of windows (the other's last window may hold no tile of
  // its own: it reloads its last tile and folds nothing)
  const int t0 = PG == 1 ? 0 : part_begin(pg, KT, 2);
  const int t1 = PG == 1 ? KT : part_begin(pg + 1, KT, 2);
  const int NW = ((PG == 1 ? KT : part_begin(1, KT, 2)) + W - 1) / W;

  // sources: the lane's x row (rows past M re-read row M - 1, k past K the
  // row's last chunk: such values only reach products that are never folded
  // or stored), the row group's code tiles and scales; byte offsets fit 32
  // bits (checked on the host)
  const uint32_t xro = (uint32_t)(m0 + r < M ? m0 + r : M - 1) * (uint32_t)K * 2u;
  const char *xb = reinterpret_cast<const char *>(x);
  const char *qb = reinterpret_cast<const char *>(qw) + (size_t)g * (size_t)KT * kTileBytes;
  const char *sb = reinterpret_cast<const char *>(am) + (size_t)g * (size_t)KT * (kTileScales * 4);

  uint4 cw[S];
  float2 sv[S];
  bf16x8 A[S][4];
  // window j of this wave into ring slot SL: tile t0 + W j + ww (past the
  // group's last tile: that tile again, never folded)
  auto load = [&](int j, auto slc) {
    constexpr int SL = decltype(slc)::value;
    const int i = t0 + j * W + ww;
    const uint32_t tl = (uint32_t)(i < t1 ? i : t1 - 1);
    cw[SL] = *reinterpret_cast<const uint4 *>(qb + tl * (uint32_t)kTileBytes + (uint32_t)lane * 16u);
    sv[SL] = *reinterpret_cast<const float2 *>(sb + tl * (uint32_t)(kTileScales * 4) + (uint32_t)r * 8u);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int k = (int)tl * kTileK + 32 * jj + 8 * h;
      A[SL][jj] = *reinterpret_cast<const bf16x8 *>(xb + xro + (uint32_t)(k < K ? k : K - 8) * 2u);
    }
  };

  // pair table (entry e, copy c at 4 (32 e + c)), from the codebook staged
  // in the (not yet used) product buffers; built before the first loads are
  // issued, since the codebook is a vector read of the argument block whose
  // wait would wait for them too
  {
    uint16_t *codes16 = reinterpret_cast<uint16_t *>(lds + L::kOffP);
    if (tid < 16) codes16[tid] = ct.t[0][tid];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int i = tid; i < stream::kTable / 16; i += 64 * W * PG) {
      const int e = i >> 3;  // four copies per 16-byte store
      const uint32_t v = (uint32_t)codes16[e & 15] | ((uint32_t)codes16[e >> 4] << 16);
      reinterpret_cast<uint4 *>(lds)[i] = make_uint4(v, v, v, v);
    }
  }
  const uint32_t tcopy = (uint32_t)(lane & 31) * 4u;
  load(0, std::integral_constant<int, 0>{});
  load(1, std::integral_constant<int, 1>{});

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  char *const pgrp = lds + L::kOffP + pg * 2 * stream::kPBuf;
  char *const sgrp = lds + L::kOffSB + pg * 2 * stream::kSBuf;
  // products of this wave's tile of window j (ring slot SL) into buffer j & 1
  auto compute = [&](int j, auto slc) {
    constexpr int SL = decltype(slc)::value;
    const uint4 w = cw[SL];
    bf16x8 B[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t wd = jj == 0 ? w.x : jj == 1 ? w.y : jj == 2 ? w.z : w.w;
      uint32_t bb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bb[q] = *reinterpret_cast<const uint32_t *>(lds + ((wd >> (8 * q)) & 0xFFu) * 128u + tcopy);
      B[jj] = __builtin_bit_cast(bf16x8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
    }
    char *pb = pgrp + (j & 1) * stream::kPBuf + ww * 2048 + lane * 16;
    f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[SL][0], B[0], zero, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[SL][1], B[1], p, 0, 0, 0);
    f32x4 q2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[SL][2], B[2], zero, 0, 0, 0);
    q2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[SL][3], B[3], q2, 0, 0, 0);
    *reinterpret_cast<f32x4 *>(pb) = p;
    *reinterpret_cast<f32x4 *>(pb + 1024) = q2;
    // the scales of weight row r, once per row
    if (lane < 16)
      *reinterpret_cast<float2 *>(sgrp + (j & 1) * stream::kSBuf + ww * 128 + lane * 8) = sv[SL];
  };
  // fold: this thread's output is element lane % 4 of output lane
  // 16 ww + lane / 4 (x row m0 + 4 ww + lane % 4, weight row lane / 4)
  float acc = 0.0f, tot = 0.0f;
  int jn = 1, cut = (SPLIT && PG == 1) ? part_begin(1, KT, np) : -1;
  auto fold_any = [&](int jf, auto wc) {
    constexpr bool WHOLE = decltype(wc)::value;  // W whole tiles of the group: no selects
    const char *pb = pgrp + (jf & 1) * stream::kPBuf + ww * 256 + lane * 4;
    const char *sbp = sgrp + (jf & 1) * stream::kSBuf + (lane >> 2) * 8;
#pragma unroll
    for (int tw = 0; tw < W; ++tw) {
      const int i = t0 + jf * W + tw;
      if (SPLIT && PG == 1 && i == cut) {  // the next part of K starts from zero
        tot = jn == 1 ? acc : tot + acc;
        acc = 0.0f;
        ++jn;
        cut = jn < np ? part_begin(jn, KT, np) : -1;
      }
      const bool live0 = i < t1, live1 = live0 && !(half_tail && i == KT - 1);
      const float2 s = *reinterpret_cast<const float2 *>(sbp + tw * 128);
      const float p0 = *reinterpret_cast<const float *>(pb + tw * 2048);
      const float p1 = *reinterpret_cast<const float *>(pb + tw * 2048 + 1024);
      const float f0 = fmaf(s.x, p0, acc);
      const float a0 = WHOLE || live0 ? f0 : acc;
      const float f1 = fmaf(s.y, p1, a0);
      acc = WHOLE || live1 ? f1 : a0;
    }
  };
  // windows of this group whose fold is of W whole tiles
  const int NWW = (t1 - (half_tail && t1 == KT ? 1 : 0) - t0) / W;
  auto fold = [&](int jf) {
    if (jf < NWW)
      fold_any(jf, std::true_type{});
    else
      fold_any(jf, std::false_type{});
  };

  // window j (ring slot j % S): the products of window j - 1 are in LDS for
  // every wave, and no wave still folds window j - 2, whose buffer window j
  // fills.  The steady loop runs whole groups of S windows with nothing but
  // whole folds and no branch between them, so the compiler's count of the
  // loads in flight survives the loop's back edge and each window waits only
  // for its own loads (a loop with branches between the windows waited for
  // nearly every load in flight).  Every wave meets the same barriers.
  auto window = [&](int j, auto slc, auto whole) {
    constexpr int SL = decltype(slc)::value;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load(j + LEAD, std::integral_constant<int, (SL + LEAD) % S>{});
    compute(j, slc);
    if constexpr (decltype(whole)::value)
      fold_any(j - 1, std::true_type{});
    else if (j > 0)
      fold(j - 1);
  };
  using T = std::true_type;
  using F = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  static_assert(S == 3, "the steady loop is unrolled by three ring slots");
  window(0, I0{}, F{});
  int j = 1;
  // windows j, j + 1, j + 2 fold windows j - 1, j, j + 1
  for (; j + S <= NW && j + 2 <= NWW; j += S) {
    window(j, I1{}, T{});
    window(j + 1, I2{}, T{});
    window(j + 2, I0{}, T{});
  }
  // the rest, one window at a time, slot by j % S
  for (; j < NW; ++j) {
    const int sl = j % S;
    if (sl == 0)
      window(j, I0{}, F{});
    else if (sl == 1)
      window(j, I1{}, F{});
    else
      window(j, I2{}, F{});
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  fold(NW - 1);

  float v = (SPLIT && PG == 1) ? tot + acc : acc;
  if constexpr (PG == 2) {
    // part 1's sums through LDS (the product buffers are free once every
    // wave has folded), added to part 0's in part order
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float *xch = reinterpret_cast<float *>(lds + L::kOffP);
    const int gt = tid - pg * 64 * W;  // thread within the group
    if (pg == 1) xch[gt] = v;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (pg == 1) return;
    v = v + xch[gt];
  }
  const int m = m0 + 4 * ww + (lane & 3);
  if (m < M) y[(int64_t)m * N + (int64_t)g * 16 + (lane >> 2)] = v;
}

// ---------------------------------------------------------------------------
// Pre-pass of the affine GEMM: X[t][m] = sum of x[m][128 t .. 128 t + 127]
// for m < Mp (zero past M), 16 lanes (a DPP row) per (t, m): each lane adds
// its 8 values in k order, then row16_sum; the GEMV sums the same way.
// Consecutive 16-lane groups take consecutive m, so a wave writes 16
// consecutive bytes of X.  Also sets the ncnt arrival counters of a tiled
// launch with K in parts to zero.
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                   int64_t K, int64_t Mp, int64_t ngroups,
                                                   float *__restrict__ X, uint32_t *__restrict__ cnt,
                                                   int64_t ncnt) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < ncnt; i += (int64_t)gridDim.x * 256)
    cnt[i] = 0u;
  const int64_t gi = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int q = threadIdx.x & 15;
  const bool ok = gi < ngroups;
  const int64_t g = ok ? gi : ngroups - 1;
  const int64_t t = g / Mp, m = g - t * Mp;
  const int64_t mr = m < M ? m : M - 1;
  const uint4 c = *reinterpret_cast<const uint4 *>(x + mr * K + t * kTileK + 8 * q);
  const float v = row16_sum(chunk_sum8(c));
  if (ok && q == 0) X[g] = m < M ? v : 0.0f;
}

// Arrival counters of a tiled launch with K in parts set to zero before the
// launch (the int4 format's pre-pass does the same): a workspace shared by
// calls of other shapes holds part sums where this call keeps counters.
__global__ __launch_bounds__(256) void zero_counters_kernel(uint32_t *__restrict__ cnt,
                                                            int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    cnt[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launch choices, shared by both formats.

// 32-bit byte offsets into x and the code buffer for the copies into LDS
bool tile_dma_ok(int64_t M, int64_t N, int64_t K) {
  return M * K * 2 < (int64_t(1) << 32) &&
         (N / kTileRows) * tiles_k(K) * kTileBytes < (int64_t(1) << 32);
}

// The narrow kernel rather than the skinny one (bit-identical rows): short M
// on a matrix of few row groups, where one wave per row group leaves most
// SIMDs idle.
constexpr int64_t kNarrowMaxG = 1024;
constexpr int64_t kNarrowMaxM = 32;
bool prefer_narrow(int64_t M, int64_t N, int64_t K) {
  return M <= kNarrowMaxM && N / kTileRows <= kNarrowMaxG && tile_dma_ok(M, N, K);
}
// Narrow launches: three windows ahead at one workgroup per CU when the grid
// fits the CUs once, else two windows ahead at two per CU.
inline bool narrow_long_lead(int64_t blocks) { return blocks <= device_cu_count(); }
// The stream kernel rather than the narrow one (codebook format, same rows):
// up to 16 rows on a grid that fits the CUs once, with K in one part or in
// two (then two part groups per workgroup).  Measured per launch (rows
// bit-identical): down (N = 3584, K = 18944) at 3-12 rows 28.2-28.5 ->
// 17.8-21.2 us, at 16 rows 28.0 -> 24.6 us; Voxtral's w2 (3072 x 9216) at 4
// rows 15.6 -> 10.6 us; o (3584 x 3584) at 4 rows 8.1 -> 7.1 us.  q|k|v
// (288 row groups, more than the CUs) was slower (10.7 -> 12.3 us at 16
// rows), as were 29- and 32-row batches in 32-row workgroups on the same
// design (down at 32 rows 40.6 -> 41.3 us).
inline bool prefer_stream(int64_t M, int64_t G, int np, int cus) {
  return M <= 16 && np <= 2 && G <= cus;
}

// The skinny kernel rather than the tiled one (bit-identical rows, so the
// choice is about speed only): up to 64 rows, and up to 256 rows when the
// tiled grid would occupy less than half of the CUs (narrow N).
bool prefer_skinny(int64_t M, int64_t N, int64_t K, int nterm, int cus) {
  if (!skinny_eligible(M, N, K, nterm)) return false;
  return M <= 64 || ((N + BN - 1) / BN) * ((M + tile::kBM - 1) / tile::kBM) < cus / 2;
}

// Tiled launch: 16 row groups per workgroup unless that grid would leave
// more than half of the CUs idle, then 8 (one workgroup per CU on twice as
// many CUs); np parts of K multiply the grid by np.  In the codebook format,
// with K in parts, a 16-row-group grid of fewer workgroups than CUs takes 14
// row groups per workgroup (7 waves) when that grid fits the CUs once: down
// at 1024 rows (224 row groups, K in two parts) then runs 256 workgroups
// instead of 224, 169 -> 163 us.  The waves of a workgroup share the CU's
// four SIMDs (2, 2, 2 and 1 of them), so a workgroup of 7 waves takes about
// as long as one of 8: on q|k|v (K in one part) 14 or 12 row groups gave no
// gain, and gate|up at 113 rows was 59.3 -> 60.8 us.
struct TilePlan {
  int rg;
  int64_t nt, mt;
  int np;
};
TilePlan tile_plan(int64_t M, int64_t N, int64_t K, int cus, bool wide = false) {
  const int64_t G = N / kTileRows, mt = (M + tile::kBM - 1) / tile::kBM;
  const int np = k_parts(N, K);
  const int64_t w16 = ((G + 15) / 16) * mt * np, w14 = ((G + 13) / 14) * mt * np;
  // codebook format, K in parts, fewer wide workgroups than CUs: tiles of 14
  // row groups (7 waves) when their grid still fits the CUs once
  if (wide && np > 1 && w16 >= cus / 2 && w16 < cus && w14 <= cus)
    return {14, (G + 13) / 14, mt, np};
  if (w16 >= cus / 2) return {16, (G + 15) / 16, mt, np};
  return {8, (G + 7) / 8, mt, np};
}

// Workspace of a tiled launch with K in np > 1 parts: one 4-byte arrival
// counter per output tile (a 256-byte aligned block), then per output tile
// the sums of every part (128 x 16 RG floats each).
size_t split_counter_bytes(int64_t ntiles) { return (size_t)((ntiles * 4 + 255) / 256 * 256); }
size_t split_bytes(int rg, int64_t ntiles, int np) {
  return split_counter_bytes(ntiles) +
         (size_t)ntiles * np * (size_t)(tile::kBM * kTileRows * rg) * sizeof(float);
}
// the larger of the two widths (the choice between them depends on the CU count)
size_t split_bytes_max(int64_t M, int64_t N, int64_t K) {
  const int np = k_parts(N, K);
  if (np == 1) return 0;
  const int64_t G = N / kTileRows, mt = (M + tile::kBM - 1) / tile::kBM;
  size_t best = 0;
  for (int rg : {16, 14, 8}) {
    const size_t b = split_bytes(rg, ((G + rg - 1) / rg) * mt, np);
    if (b > best) best = b;
  }
  return best;
}

template <bool AFF>
void launch_tile(const TilePlan &p, const uint16_t *x, int64_t M, const uint8_t *qw,
                 const float *am, const CodeTerms &ct, int64_t N, int64_t K, float *y,
                 const float *xsum, int64_t Mp, void *split_ws, hipStream_t s) {
  const int64_t KT = tiles_k(K);
  // one-dimensional grid, units (N tile, part of K) padded to a multiple of 8
  // (see the kernel)
  const bool split = p.np > 1;
  const unsigned grid = (unsigned)((p.nt * p.np + 7) / 8 * 8 * p.mt);
  uint32_t *cnt = split ? reinterpret_cast<uint32_t *>(split_ws) : nullptr;
  uint64_t *part = split ? reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(split_ws) +
                                                        split_counter_bytes(p.nt * p.mt))
                         : nullptr;
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, x, M, qw, am, ct, N, K, KT, y,
                       (int)p.nt, (int)p.mt, xsum, Mp, p.np, cnt, part);
  };
  if constexpr (!AFF) {
    if (p.rg == 16) {
      // two 4-wave workgroups per CU when the grid holds more workgroups
      // than CUs, else one workgroup of 8 waves (gate|up at 200 rows, 296
      // workgroups: 119 us in two rounds of 8 waves, 111 us in one of two
      // 4-wave workgroups per CU; at 113 rows, 148 workgroups, 8 waves per
      // CU 64 us, 4 waves 76 us)
      const bool two = (int64_t)grid > (int64_t)device_cu_count();
      auto gw = [&](auto kern, int threads) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, x, M, qw, am, ct, N, K,
                           KT, y, (int)p.nt, (int)p.mt, p.np, cnt, part);
      };
      if (two)
        split ? gw(gemm_wide_kernel<4, 16, true>, 256) : gw(gemm_wide_kernel<4, 16, false>, 256);
      else
        split ? gw(gemm_wide_kernel<8, 16, true>, 512) : gw(gemm_wide_kernel<8, 16, false>, 512);
      return;
    }
    if (p.rg == 14) {
      // 128 x 224 tiles, 7 waves of two row groups, one workgroup per CU (the
      // plan takes them only with K in parts)
      hipLaunchKernelGGL((gemm_wide_kernel<7, 14, true>), dim3(grid), dim3(448), 0, s, x, M, qw,
                         am, ct, N, K, KT, y, (int)p.nt, (int)p.mt, p.np, cnt, part);
      return;
    }
  } else if (p.rg == 16) {
    split ? go(gemm_tile_kernel<16, AFF, kTileMB, true>, 256 * 16 / kTileMB)
          : go(gemm_tile_kernel<16, AFF, kTileMB, false>, 256 * 16 / kTileMB);
    return;
  }
  split ? go(gemm_tile_kernel<8, AFF, kTileMB8, true>, 256 * 8 / kTileMB8)
        : go(gemm_tile_kernel<8, AFF, kTileMB8, false>, 256 * 8 / kTileMB8);
}

}  // namespace

int k_parts(int64_t N, int64_t K) {
  const int64_t KT = tiles_k(K);
  // two halves for long K
  int64_t P = K >= kSplitK ? 2 : 1;
  // narrow N: the 128 x 128 output tiles of a 1024-row batch would cover
  // less than half of a 256-CU device; then as many parts as fill it once,
  // of at least four device tiles each
  const int64_t tiles = (N / kTileRows + 7) / 8 * 8;
  if (tiles * P < 128) {
    const int64_t want = 256 / tiles, cap = KT / 4;
    const int64_t q = want < cap ? want : cap;
    if (q > P) P = q;
  }
  return (int)P;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // only the tiled kernel with K in parts needs one; the skinny kernel (up
  // to 64 rows) and the generic kernel do not
  if (k_parts(N, K) == 1 || !tile_dma_ok(M, N, K)) return 0;
  if (M <= 64 && skinny_eligible(M, N, K, 1)) return 0;
  return split_bytes_max(M, N, K);
}

namespace {
int64_t awq_rows_padded(int64_t M) { return (M + tile::kBM - 1) / tile::kBM * tile::kBM; }
size_t awq_xsum_bytes(int64_t M, int64_t K) {
  return (size_t)(K / kTileK) * (size_t)awq_rows_padded(M) * sizeof(float);
}
}  // namespace

bool awq_gemm_supported(int64_t M, int64_t N, int64_t K) {
  // 32-bit byte offsets for the copies into LDS: x, code words, x sums
  const int64_t KT = K / kTileK, Mp = awq_rows_padded(M);
  return M >= 1 && K % kTileK == 0 && tile_dma_ok(M, N, K) && KT * Mp * 4 < (int64_t(1) << 32);
}

size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // the x sums, then what a tiled launch with K in parts needs
  const bool skinny_only = M <= 64 && skinny_eligible(M, N, K, 1);
  return awq_xsum_bytes(M, K) + (skinny_only ? 0 : split_bytes_max(M, N, K));
}

hipError_t launch_awq_gemm(const uint16_t *x, int64_t M, const uint8_t *qw, const uint32_t *pr,
                           int64_t N, int64_t K, float *y, void *ws, hipStream_t s) {
  const int64_t KT = K / kTileK, Mp = awq_rows_padded(M);
  float *X = reinterpret_cast<float *>(ws);
  char *split_ws = reinterpret_cast<char *>(ws) + awq_xsum_bytes(M, K);
  const int cus = device_cu_count();
  // the codebook GEMM's choices: skinny for few rows, else the tiled kernel
  const bool skinny = prefer_skinny(M, N, K, 1, cus);
  const TilePlan p = tile_plan(M, N, K, cus);
  const int64_t ngroups = KT * Mp;
  hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)((ngroups * 16 + 255) / 256)), dim3(256), 0, s,
                     x, M, K, Mp, ngroups, X, reinterpret_cast<uint32_t *>(split_ws),
                     (!skinny && p.np > 1) ? p.nt * p.mt : (int64_t)0);
  const CodeTerms ct = identity_terms();
  const int64_t G = N / kTileRows;
  const float *prf = reinterpret_cast<const float *>(pr);
  if (skinny) {
    const int np = k_parts(N, K);
    if (prefer_narrow(M, N, K)) {
      const dim3 grid((unsigned)G, (unsigned)((M + 15) / 16)), block(64 * narrow::kWaves);
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, s, x, (int)M, qw, prf, ct, (int)N, (int)K,
                           (int)KT, (int)G, y, X, (int)Mp, np);
      };
      if (narrow_long_lead((int64_t)grid.x * grid.y))
        np > 1 ? go(gemm_narrow_kernel<true, true, 3>) : go(gemm_narrow_kernel<true, false, 3>);
      else
        np > 1 ? go(gemm_narrow_kernel<true, true, 2>) : go(gemm_narrow_kernel<true, false, 2>);
      return hipGetLastError();
    }
    const unsigned gx = (unsigned)((G + skinny::kWaves - 1) / skinny::kWaves);
    const dim3 block(64 * skinny::kWaves);
    auto go = [&](auto kern, dim3 grid) {
      hipLaunchKernelGGL(kern, grid, block, 0, s, x, (int)M, qw, prf, ct, (int)N, (int)K, (int)KT,
                         (int)G, y, X, (int)Mp, np);
    };
    const dim3 g2(gx, (unsigned)((M + 31) / 32));
    // three workgroups per CU for grids of more than two rounds (32-row
    // instance; the 16-row one of this format does not fit 168 registers)
    const bool three = M > 16 && (int64_t)gx * g2.y > 2 * (int64_t)cus;
    if (M <= 16)
      np > 1 ? go(gemm_skinny_kernel<1, 8, true, true, 2>, dim3(gx))
             : go(gemm_skinny_kernel<1, 8, true, false, 2>, dim3(gx));
    else if (three)
      np > 1 ? go(gemm_skinny_kernel<2, 2, true, true, 3>, g2)
             : go(gemm_skinny_kernel<2, 2, true, false, 3>, g2);
    else
      np > 1 ? go(gemm_skinny_kernel<2, 4, true, true, 2>, g2)
             : go(gemm_skinny_kernel<2, 4, true, false, 2>, g2);
    return hipGetLastError();
  }
  launch_tile<true>(p, x, M, qw, prf, ct, N, K, y, X, Mp, split_ws, s);
  return hipGetLastError();
}

bool skinny_eligible(int64_t M, int64_t N, int64_t K, int nterm) {
  // 32-bit tile indices and element offsets
  return nterm == 1 && M >= 1 && M <= kSkinnyMaxM && M * K < (int64_t(1) << 31) &&
         (N / kTileRows) * tiles_k(K) < (int64_t(1) << 31);
}

hipError_t launch_skinny(const uint16_t *x, int64_t M, const uint8_t *qw, const float *am,
                         const CodeTerms &ct, int64_t N, int64_t K, float *y, hipStream_t s) {
  const int64_t G = N / kTileRows;
  if (prefer_narrow(M, N, K)) {
    const int np = k_parts(N, K);
    if (prefer_stream(M, G, np, device_cu_count())) {
      const dim3 grid((unsigned)G, (unsigned)((M + 15) / 16)), block(np == 2 ? 512 : 256);
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, s, x, (int)M, qw, am, ct, (int)N, (int)K,
                           (int)tiles_k(K), y, np);
      };
      np == 2 ? go(gemm_stream_kernel<true, 2>) : go(gemm_stream_kernel<false, 1>);
      return hipGetLastError();
    }
    const dim3 grid((unsigned)G, (unsigned)((M + 15) / 16)), block(64 * narrow::kWaves);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, s, x, (int)M, qw, am, ct, (int)N, (int)K,
                         (int)tiles_k(K), (int)G, y, nullptr, 0, np);
    };
    if (narrow_long_lead((int64_t)grid.x * grid.y))
      np > 1 ? go(gemm_narrow_kernel<false, true, 3>) : go(gemm_narrow_kernel<false, false, 3>);
    else
      np > 1 ? go(gemm_narrow_kernel<false, true, 2>) : go(gemm_narrow_kernel<false, false, 2>);
    return hipGetLastError();
  }
  const unsigned gx = (unsigned)((G + skinny::kWaves - 1) / skinny::kWaves);
  const dim3 block(64 * skinny::kWaves);
  const int KT = (int)tiles_k(K);
  const int np = k_parts(N, K);
  // up to 16 rows: one m-block per wave; otherwise 32-row groups of x along
  // the grid's y (workgroups of one row-group block run side by side and
  // share the weights through the caches)
  auto go = [&](auto kern, dim3 grid) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, x, (int)M, qw, am, ct, (int)N, (int)K, KT, (int)G, y,
                       nullptr, 0, np);
  };
  const dim3 g2(gx, (unsigned)((M + 31) / 32));
  const int64_t cus = device_cu_count();
  // three workgroups per CU (half the tiles in flight, a 16-copy table) for
  // grids of more than two rounds
  const bool three = (int64_t)gx * (M <= 16 ? 1 : g2.y) > 2 * cus;
  // 16-row blocks past 16 rows when their grid fits the CUs once, or twice
  // on long K: twice the waves per row group, each with half the products
  // per tile (the lookups are repeated per block)
  const int64_t g16 = (int64_t)gx * ((M + 15) / 16);
  if (M > 16 && (g16 <= cus || (g16 <= 2 * cus && K >= kSplitK))) {
    const dim3 g1(gx, (unsigned)((M + 15) / 16));
    np > 1 ? go(gemm_skinny_kernel<1, 8, false, true, 2>, g1)
           : go(gemm_skinny_kernel<1, 8, false, false, 2>, g1);
    return hipGetLastError();
  }
  if (M <= 16) {
    if (three)
      np > 1 ? go(gemm_skinny_kernel<1, 4, false, true, 3>, dim3(gx))
             : go(gemm_skinny_kernel<1, 4, false, false, 3>, dim3(gx));
    else
      np > 1 ? go(gemm_skinny_kernel<1, 8, false, true, 2>, dim3(gx))
             : go(gemm_skinny_kernel<1, 8, false, false, 2>, dim3(gx));
  } else if (three)
    np > 1 ? go(gemm_skinny_kernel<2, 2, false, true, 3>, g2)
           : go(gemm_skinny_kernel<2, 2, false, false, 3>, g2);
  else
    np > 1 ? go(gemm_skinny_kernel<2, 4, false, true, 2>, g2)
           : go(gemm_skinny_kernel<2, 4, false, false, 2>, g2);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint16_t *x, int64_t M, const uint8_t *qw, const float *am,
                       const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y, void *ws,
                       size_t ws_bytes, hipStream_t s) {
  const int64_t KT = tiles_k(K);
  const int cus = device_cu_count();
  if (prefer_skinny(M, N, K, nterm, cus)) return launch_skinny(x, M, qw, am, ct, N, K, y, s);
  if (nterm == 1 && tile_dma_ok(M, N, K)) {
    const TilePlan p = tile_plan(M, N, K, cus, true);
    if (p.np > 1 && (!ws || ws_bytes < split_bytes(p.rg, p.nt * p.mt, p.np)))
      return hipErrorInvalidValue;
    if (p.np > 1) {
      const int64_t n = p.nt * p.mt;
      hipLaunchKernelGGL(zero_counters_kernel, dim3((unsigned)((n + 255) / 256 < 64 ? (n + 255) / 256 : 64)),
                         dim3(256), 0, s, reinterpret_cast<uint32_t *>(ws), n);
    }
    launch_tile<false>(p, x, M, qw, am, ct, N, K, y, nullptr, 0, ws, s);
    return hipGetLastError();
  }
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const float2 *a = reinterpret_cast<const float2 *>(am);
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(256);
  hipLaunchKernelGGL(gemm_kernel<3>, grid, block, 0, s, x, M, q, a, ct, N, K, KT, y,
                     k_parts(N, K));
  return hipGetLastError();
}

}  // namespace nf4
