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


// ---------------------------------------------------------------------------
// Main path (codebook of bf16 values).  Workgroup tile (64*WM) x 128
// outputs: WM x 2 waves, each 64 x 64 (4 x 4 MFMA tiles; the per-block sum P
// and the running sum both in VGPRs).  The K loop steps one 64-block at a
// time (one scale per output column per step):
//   - global fetch runs two steps ahead into registers (x rows, the codes of
//     the step, the lane's scales), so its latency hides behind two steps of
//     MFMAs;
//   - each step writes step t+1 into LDS stage (t+1)&1 from registers (codes
//     expanded once per workgroup to bf16 through the LDS pair table), then
//     runs the MFMAs of step t from stage t&1;
//   - rows of the A and B stages are padded to 72 bf16 (144 bytes), so the
//     16 rows a ds_read_b128 touches start in 16 different 16-byte bank
//     groups;
//   - one barrier per step.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;                         // k per step (one scale block)
constexpr int kRS = kBK + 8;                    // padded LDS row stride in bf16

template <int WM>
struct MainCfg {
  static constexpr int kBM = 64 * WM;
  static constexpr int kThreads = 128 * WM;     // WM x 2 waves
  static constexpr int kCopies = WM == 4 ? 32 : 8;
  static constexpr int kXChunks = kBM * kBK / 8 / kThreads;   // 16-byte x chunks per thread
  static constexpr int kCodeSlots = 8 * 64 / kThreads;         // (row group, lane) per thread
};

template <int WM>
__global__ __launch_bounds__(128 * WM) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_main_kernel(const uint16_t *__restrict__ x,
                                                            int64_t M,
                                                            const uint32_t *__restrict__ qw32,
                                                            const float *__restrict__ am,
                                                            CodeTerms ct, int64_t N, int64_t K,
                                                            int64_t KT, float *__restrict__ y) {
  using C = MainCfg<WM>;
  constexpr int BMW = C::kBM, NT = C::kThreads, CP = C::kCopies;
  __shared__ __attribute__((aligned(16))) uint32_t table[256 * CP];
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BMW * kRS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kRS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, h = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BMW;
  const int64_t gblk = ((int64_t)blockIdx.x * BN) / kTileRows;  // first row group of the tile
  const int64_t G = N / kTileRows;
  const int64_t nsteps = K / kBK;

  // ---- registers holding one fetched step
  struct Fetch {
    uint4 x[C::kXChunks];
    uint2 q[C::kCodeSlots];
    float s[4];
  };
  auto fetch = [&](Fetch &f, int64_t t) {
    const int64_t dt = t >> 1, half = t & 1;
#pragma unroll
    for (int u = 0; u < C::kXChunks; ++u) {
      const int c = tid + NT * u, row = c >> 3, col = (c & 7) * 8;
      const int64_t gm = m0 + row;
      f.x[u] = make_uint4(0u, 0u, 0u, 0u);
      if (gm < M) f.x[u] = *reinterpret_cast<const uint4 *>(x + gm * K + t * kBK + col);
    }
#pragma unroll
    for (int u = 0; u < C::kCodeSlots; ++u) {
      const int c = tid + NT * u, gt = c >> 6, ln = c & 63;
      f.q[u] = make_uint2(0u, 0u);
      if (gblk + gt < G)
        f.q[u] = *reinterpret_cast<const uint2 *>(qw32 + ((gblk + gt) * KT + dt) * 256 + ln * 4 +
                                                  half * 2);
    }
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int64_t g = gblk + wn * 4 + nn;
      f.s[nn] = g < G ? am[(g * KT + dt) * 32 + 2 * r + half] : 0.0f;
    }
  };
  // ---- write a fetched step into LDS stage st; codes expanded to bf16
  auto stage = [&](const Fetch &f, int st) {
#pragma unroll
    for (int u = 0; u < C::kXChunks; ++u) {
      const int c = tid + NT * u, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<uint4 *>(&As[st][row * kRS + col]) = f.x[u];
    }
    const uint32_t copy4 = (uint32_t)(lane & (CP - 1)) << 2;
#pragma unroll
    for (int u = 0; u < C::kCodeSlots; ++u) {
      const int c = tid + NT * u, gt = c >> 6, ln = c & 63;
      const int n = gt * 16 + (ln & 15), kh = 8 * (ln >> 4);
      const uint32_t wd[2] = {f.q[u].x, f.q[u].y};
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        uint32_t bb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t e = (wd[jj] >> (8 * q)) & 0xFFu;
          bb[q] = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(table) +
                                                        e * (CP * 4) + copy4);
        }
        *reinterpret_cast<uint4 *>(&Bs[st][n * kRS + 32 * jj + kh]) =
            make_uint4(bb[0], bb[1], bb[2], bb[3]);
      }
    }
  };

  // fA and fB swap roles every step (the loop is unrolled by two), so no
  // register set is ever copied while its loads are in flight.
  Fetch fA, fB;
  fetch(fA, 0);
  if (nsteps > 1) fetch(fB, 1);
  // the codes go through LDS once (in the B stage) before the table is built
  uint16_t *codes_lds = &Bs[1][0];
  if (tid < 16) codes_lds[tid] = ct.t[0][tid];
  __syncthreads();
  for (int c = tid; c < 256 * CP / 4; c += NT) {
    const int e = c / (CP / 4);
    const uint32_t v = (uint32_t)codes_lds[e & 15] | ((uint32_t)codes_lds[e >> 4] << 16);
    reinterpret_cast<uint4 *>(table)[c] = make_uint4(v, v, v, v);
  }
  __syncthreads();
  stage(fA, 0);
  float sc[4] = {fA.s[0], fA.s[1], fA.s[2], fA.s[3]};
  if (nsteps > 2) fetch(fA, 2);

  f32x4 acc[4][4];
#pragma unroll
  for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
    for (int b2 = 0; b2 < 4; ++b2) acc[a2][b2] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int arow = (wm * 64 + r) * kRS + 8 * h;
  const int brow = (wn * 64 + r) * kRS + 8 * h;
  // One step: stage `nxt` (step t+1) into LDS stage st^1, run the MFMAs of
  // step t from stage st, fold with this step's scales, refetch `nxt` with
  // step t+3.
  auto step = [&](int64_t t, Fetch &nxt) {
    const int st = (int)(t & 1);
    __syncthreads();  // stage st written by all; stage st^1 no longer read
    float sn[4] = {nxt.s[0], nxt.s[1], nxt.s[2], nxt.s[3]};
    if (t + 1 < nsteps) stage(nxt, st ^ 1);
    if (t + 3 < nsteps) fetch(nxt, t + 3);
    f32x4 p[4][4];
#pragma unroll
    for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
      for (int b2 = 0; b2 < 4; ++b2) p[a2][b2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 A[4], B[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
        A[mm] = *reinterpret_cast<const bf16x8 *>(&As[st][arow + mm * 16 * kRS + 32 * kk]);
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
        B[nn] = *reinterpret_cast<const bf16x8 *>(&Bs[st][brow + nn * 16 * kRS + 32 * kk]);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
#pragma unroll
        for (int nn = 0; nn < 4; ++nn)
          p[mm][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mm], B[nn], p[mm][nn], 0, 0, 0);
    }
#pragma unroll
    for (int nn = 0; nn < 4; ++nn)
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mm][nn][i] = fmaf(sc[nn], p[mm][nn][i], acc[mm][nn][i]);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) sc[nn] = sn[nn];
  };
  // step t stages step t+1, which sits in fB for even t and in fA for odd t
  for (int64_t t = 0; t < nsteps; t += 2) {
    step(t, fB);
    if (t + 1 < nsteps) step(t + 1, fA);
  }

  // Output tile of a 16x16x32 MFMA: lane l holds rows 4(l/16)+i, column l%16.
#pragma unroll
  for (int mm = 0; mm < 4; ++mm)
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int64_t g = gblk + wn * 4 + nn;
      if (g >= G) continue;
      const int64_t col = g * kTileRows + r;
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
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const float2 *a = reinterpret_cast<const float2 *>(am);
  if (nterm == 1) {
    // Tall tiles (256 rows, 8 waves) when they still give every CU a
    // workgroup; otherwise 128-row tiles, two workgroups per CU.
    const int64_t ntile = (N + BN - 1) / BN;
    const int64_t tall = ntile * ((M + 255) / 256);
    if (tall >= device_cu_count()) {
      const dim3 grid((unsigned)ntile, (unsigned)((M + 255) / 256));
      hipLaunchKernelGGL(gemm_main_kernel<4>, grid, dim3(512), 0, s, x, M,
                         reinterpret_cast<const uint32_t *>(qw), am, ct, N, K, KT, y);
    } else {
      const dim3 grid((unsigned)ntile, (unsigned)((M + 127) / 128));
      hipLaunchKernelGGL(gemm_main_kernel<2>, grid, dim3(256), 0, s, x, M,
                         reinterpret_cast<const uint32_t *>(qw), am, ct, N, K, KT, y);
    }
  } else {
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(256);
    hipLaunchKernelGGL(gemm_kernel<3>, grid, block, 0, s, x, M, q, a, ct, N, K, KT, y);
  }
  return hipGetLastError();
}

}  // namespace nf4
