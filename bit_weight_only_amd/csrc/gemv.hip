// gemv.hip -- decode GEMV for 1 <= M <= 8 activation rows.
//
// Method (vibevoice.c README, "The kernels that matter" and "Quantization" >
// "Weights", decode GEMV bullet): single-token decode reads every packed
// weight once and is bound by memory bandwidth, so dequantization is fused
// into the multiply-accumulate and the weights stay 4-bit up to the product;
// 128-bit loads; split over K when the rows alone would not cover the GPU.
//
// Mapping on gfx950: one workgroup per 16-row group, its waves splitting the
// K tiles.  A lane's 16-byte load holds 32 codes of one row.  Each byte (two
// codes) indexes a replicated LDS table of bf16 code pairs, and
// v_dot2_f32_bf16 multiplies that pair by the matching pair of bf16
// activations with fp32 accumulation (the codes are bf16 values, so every
// product is exact).  The fp32 block scale multiplies each 64-block's sum.
// Lanes sharing a row combine with cross-lane shuffles, waves through LDS in
// a fixed order, so the result is reproducible bit for bit.
#include "nf4_internal.h"

namespace nf4 {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

constexpr int kMaxWaves = 16;

template <int M, int NTERM, int TT>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw,
    const float2 *__restrict__ am, CodeTerms ct, int64_t N, int64_t K, int64_t KT, int T,
    float *__restrict__ y) {
  __shared__ uint32_t table[NTERM * kPairWords];
  __shared__ float red[kMaxWaves][16][M];

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

template <int M, int NTERM>
hipError_t launch_m(const uint16_t *x, const uint4 *qw, const float2 *am, const CodeTerms &ct,
                    int64_t N, int64_t K, float *y, hipStream_t s) {
  const int64_t KT = tiles_k(K);
  int nw = KT < kMaxWaves ? (int)KT : kMaxWaves;
  const int T = (int)((KT + nw - 1) / nw);
  nw = (int)((KT + T - 1) / T);
  const dim3 grid((unsigned)(N / kTileRows)), block(nw * 64);
  if (T >= 8)
    hipLaunchKernelGGL((gemv_kernel<M, NTERM, 8>), grid, block, 0, s, x, qw, am, ct, N, K, KT, T, y);
  else if (T >= 4)
    hipLaunchKernelGGL((gemv_kernel<M, NTERM, 4>), grid, block, 0, s, x, qw, am, ct, N, K, KT, T, y);
  else if (T >= 2)
    hipLaunchKernelGGL((gemv_kernel<M, NTERM, 2>), grid, block, 0, s, x, qw, am, ct, N, K, KT, T, y);
  else
    hipLaunchKernelGGL((gemv_kernel<M, NTERM, 1>), grid, block, 0, s, x, qw, am, ct, N, K, KT, T, y);
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

hipError_t launch_gemv(const uint16_t *x, int M, const uint8_t *qw, const float *am,
                       const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y,
                       hipStream_t s) {
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const float2 *a = reinterpret_cast<const float2 *>(am);
  if (nterm == 1) return launch_t<1>(x, M, q, a, ct, N, K, y, s);
  return launch_t<3>(x, M, q, a, ct, N, K, y, s);
}

}  // namespace nf4
