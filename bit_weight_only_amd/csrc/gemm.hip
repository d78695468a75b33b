// gemm.hip -- prefill GEMM y = x . dequant(W)^T for any M on bf16 MFMA.
//
// Method (vibevoice.c README, "Quantization" > "Weights", M > 1 bullet): a
// matrix-core GEMM keeps the weights 4-bit through on-chip memory and
// expands them next to the matrix instruction; split over K when the tile
// grid would not cover the GPU.
//
// Precision on gfx950: a bf16 operand cannot hold c*s exactly, so the codes
// themselves (bf16 values) are the B operand and the fp32 scale is applied
// outside the matrix product: for every 64-block the MFMA sums
// P = sum_k x*c in fp32 (exact products), then acc += s * P.
//
// Tiling: 128 x 128 outputs per 256-thread workgroup, four waves in 2 x 2,
// each wave 64 x 64 = 4 x 4 v_mfma_f32_16x16x32_bf16 tiles.  Per 128-k
// device tile the workgroup stages the x tile in LDS; each wave loads its
// four 1 KB code tiles straight into registers (lane l's 16 bytes are its B
// fragments for the four k-steps), maps each code byte through the LDS pair
// table to two bf16 values, and feeds the MFMA.
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
                                                   float *__restrict__ y) {
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

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t = 0; t < KT; ++t) {
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
        if (row < M) y[row * N + col] = acc[mm][nn][i];
      }
    }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm(const uint16_t *x, int64_t M, const uint8_t *qw, const float *am,
                       const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y, void *,
                       size_t, hipStream_t s) {
  const int64_t KT = tiles_k(K);
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(256);
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const float2 *a = reinterpret_cast<const float2 *>(am);
  if (nterm == 1)
    hipLaunchKernelGGL(gemm_kernel<1>, grid, block, 0, s, x, M, q, a, ct, N, K, KT, y);
  else
    hipLaunchKernelGGL(gemm_kernel<3>, grid, block, 0, s, x, M, q, a, ct, N, K, KT, y);
  return hipGetLastError();
}

}  // namespace nf4
