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
// Two kernels:
//   gemm_pipe_kernel<WM>  codebooks whose values are bf16 (the default one):
//     (64 WM) x 128 outputs per workgroup, WM x 2 waves of 64 x 64, copies
//     straight from global memory into LDS rings, codes expanded once per
//     workgroup;
//   gemm_kernel<3>        any finite codebook (each value split into three
//     bf16 terms), and shapes whose byte offsets exceed 32 bits.
// Within each kernel every output is the same sequence of operations
// whatever the tile shape or M: the K order, the MFMA k-split and the
// per-block fold never depend on the launch, so a row of y does not depend on
// the other rows in the batch, and a column slice of a fused matrix equals
// the separate matrix's output.  K is therefore never split across
// workgroups.
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


constexpr int kBK = 64;  // k per step of the pipelined kernel (one scale block)

// ---------------------------------------------------------------------------
// Pipelined kernel.  The 64-k step is split into two 32-k halves (kk = 0, 1),
// each a separate LDS block laid out [row][32 bf16].  The four 16-byte chunks
// of a row are stored at chunk ^ ((row >> 2) & 3): LDS serves 16 lanes at a
// time, and a fragment's 16 lanes (16 rows, one chunk) then hit 16 different
// bank groups instead of 4.  Rings:
//   A (x)        2 stages x 2 halves, copied global->LDS one step ahead;
//   B (codes)    2 stages x 2 halves, expanded by the workgroup one step ahead;
//   code words   per-wave ring of 8 quarter-slots, copied two steps ahead;
//   scales       ring of 4 steps, copied two steps ahead.
// In step t every wave runs the kk=0 products of step t from fragments it
// loaded during step t-1, loads the kk=0 fragments of step t+1 meanwhile, then
// runs the kk=1 products; so the matrix unit starts right after the barrier.
// One barrier per step.  All copies issued after barrier t land before
// barrier t+1, except the code and scale copies, which may stay in flight one
// more step: they are issued last, and each barrier waits until at most that
// many copies are outstanding.  Copy sources past the end are clamped, so
// every step issues the same number of copies.
namespace pipe {
constexpr int kHalfRow = 64;                    // bytes of one row in one 32-k half
constexpr int kCopies = 32;                     // pair-table copies (lane % 32)
constexpr int kTableBytes = 256 * kCopies * 4;
constexpr int kCodeSlots = 8;                   // quarter-slots per row group
constexpr int kScaleSlots = 4;
template <int WM>
struct Map {
  static constexpr int kWaves = 2 * WM, kThreads = 64 * kWaves, kBM = 64 * WM;
  static constexpr int kRgPerWave = 8 / kWaves;  // row groups each wave copies and expands
  static constexpr int kAHalf = kBM * kHalfRow, kBHalf = 128 * kHalfRow;
  static constexpr int kOffA = 0, kOffB = kOffA + 4 * kAHalf, kOffC = kOffB + 4 * kBHalf,
                       kOffS = kOffC + 8 * kCodeSlots * 256, kOffT = kOffS + kScaleSlots * 512,
                       kBytes = kOffT + kTableBytes;
  // copies per step that may still be in flight at the next barrier
  static constexpr int kLate = 3 * kRgPerWave;
};

typedef __attribute__((address_space(3))) void lds_void;
__device__ inline uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const lds_void *)p;
}
// One copy from global memory (uniform base + per-lane 32-bit byte offset)
// straight into LDS: 16 bytes per lane land at m0 + 16 * lane (copy16), or 4
// bytes at m0 + 4 * lane (copy4).  Issued from inline assembly, so the
// compiler neither waits for them nor knows what they write: every use is
// ordered by an explicit vmcnt wait and a barrier.
__device__ inline void copy16(uint32_t m0, const void *base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(base)
               : "memory");
}
// Wait until at most N of this wave's copies are in flight and its LDS
// operations are done, then meet the other waves.
template <int N>
__device__ inline void wait_copies_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ inline void copy4(uint32_t m0, const void *base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(m0), "v"(voff), "s"(base)
               : "memory");
}
}  // namespace pipe

template <int WM>
__global__ __launch_bounds__(128 * WM) void gemm_pipe_kernel(
    const uint16_t *__restrict__ x, int64_t M, const uint8_t *__restrict__ qw,
    const float *__restrict__ am, CodeTerms ct, int64_t N, int64_t K, int64_t KT,
    float *__restrict__ y) {
  using L = pipe::Map<WM>;
  __shared__ __attribute__((aligned(16))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, h = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * L::kBM;
  const int64_t gblk = (int64_t)blockIdx.x * 8;
  const int64_t G = N / kTileRows;
  const int S = (int)(K / kBK), U = 2 * S;  // steps, 32-k quarters
  const uint32_t base = pipe::lds_addr(lds);
  char *ldsA = lds + L::kOffA, *ldsB = lds + L::kOffB, *ldsC = lds + L::kOffC;
  char *ldsS = lds + L::kOffS, *ldsT = lds + L::kOffT;

  // ---- per-lane copy offsets (bytes).  Rows past M and row groups past N
  // re-read the last valid one; their outputs are never stored.
  // A: copy i = 2 * wave + v fills rows 16i .. 16i+15 of a half block; lane l
  // fills chunk slot l % 4 of row 16i + l/4, i.e. logical chunk
  // (l % 4) ^ ((row >> 2) & 3) = (l % 4) ^ ((l >> 4) & 3).
  uint32_t aoff[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int R = 16 * (2 * wave + v) + (lane >> 2);
    const int64_t gm = m0 + R < M ? m0 + R : M - 1;
    const int c = (lane & 3) ^ ((lane >> 4) & 3);
    aoff[v] = (uint32_t)((gm * K + c * 8) * 2);
  }
  uint32_t coff[L::kRgPerWave], soff[L::kRgPerWave];
#pragma unroll
  for (int v = 0; v < L::kRgPerWave; ++v) {
    const int64_t rg = gblk + wave * L::kRgPerWave + v;
    const int64_t g = rg < G ? rg : G - 1;
    coff[v] = (uint32_t)(g * KT * kTileBytes + lane * 16);
    soff[v] = (uint32_t)((g * KT * kTileScales + 2 * r) * 4);
  }
  // half `half` of x columns [64 step, 64 step + 64) -> A stage step & 1
  auto issue_a = [&](int step, int half) {
    const int sc = step < S ? step : S - 1;
    const uint16_t *src = x + (int64_t)sc * kBK + half * 32;
    const uint32_t dst = base + L::kOffA + ((step & 1) * 2 + half) * L::kAHalf;
#pragma unroll
    for (int v = 0; v < 2; ++v) pipe::copy16(dst + (2 * wave + v) * 1024, src, aoff[v]);
  };
  // quarter u = code dword u & 3 of device tile u >> 2 (k in [32u, 32u + 32))
  auto issue_codes = [&](int u) {
    const int uc = u < U ? u : U - 1;
    const uint8_t *src = qw + (int64_t)(uc >> 2) * kTileBytes + (uc & 3) * 4;
#pragma unroll
    for (int v = 0; v < L::kRgPerWave; ++v)
      pipe::copy4(base + L::kOffC + ((wave * L::kRgPerWave + v) * pipe::kCodeSlots + (u & 7)) * 256,
                  src, coff[v]);
  };
  // scales of step `step` (one per row of each row group)
  auto issue_scales = [&](int step) {
    const int sc = step < S ? step : S - 1;
    const float *src = am + (int64_t)(sc >> 1) * kTileScales + (sc & 1);
    if (lane < 16) {
#pragma unroll
      for (int v = 0; v < L::kRgPerWave; ++v)
        pipe::copy4(base + L::kOffS + (step & 3) * 512 + (wave * L::kRgPerWave + v) * 64, src,
                    soff[v]);
    }
  };
  // expand quarter u of this wave's row groups into B stage (u >> 1) & 1, half u & 1
  const uint32_t tcopy = (uint32_t)(lane & (pipe::kCopies - 1)) * 4;
  // row r, logical chunk h within a 16-row block (rows differ by multiples of
  // 16, so the swizzle only depends on r)
  const uint32_t bsw = (uint32_t)(r * pipe::kHalfRow + ((h ^ ((r >> 2) & 3)) * 16));
  auto dequant = [&](int u) {
#pragma unroll
    for (int v = 0; v < L::kRgPerWave; ++v) {
      const int rgl = wave * L::kRgPerWave + v;
      const uint32_t wd = *reinterpret_cast<const uint32_t *>(
          ldsC + (rgl * pipe::kCodeSlots + (u & 7)) * 256 + lane * 4);
      uint32_t bb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t e = (wd >> (8 * q)) & 0xFFu;
        bb[q] = *reinterpret_cast<const uint32_t *>(ldsT + e * (pipe::kCopies * 4) + tcopy);
      }
      *reinterpret_cast<uint4 *>(ldsB + (((u >> 1) & 1) * 2 + (u & 1)) * L::kBHalf + rgl * 1024 +
                                 bsw) = make_uint4(bb[0], bb[1], bb[2], bb[3]);
    }
  };
  // fragments: lane (r, h) holds row r of a 16-row block, bf16 8h .. 8h+7 of the half
  const uint32_t afr = (uint32_t)(wm * 64 * pipe::kHalfRow) + bsw;
  const uint32_t bfr = (uint32_t)(wn * 64 * pipe::kHalfRow) + bsw;
  auto load_frags = [&](int st, int half, bf16x8(&A)[4], bf16x8(&B)[4]) {
    const char *pa = ldsA + (st * 2 + half) * L::kAHalf + afr;
    const char *pb = ldsB + (st * 2 + half) * L::kBHalf + bfr;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) A[mm] = *reinterpret_cast<const bf16x8 *>(pa + mm * 1024);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) B[nn] = *reinterpret_cast<const bf16x8 *>(pb + nn * 1024);
  };

  // ---- prologue: pair table (from the codebook staged in B stage 1 half 1,
  // which the prologue does not expand into), then the first copies
  uint16_t *codes16 = reinterpret_cast<uint16_t *>(ldsB + 3 * L::kBHalf);
  if (tid < 16) codes16[tid] = ct.t[0][tid];
  __syncthreads();
  for (int c = tid; c < pipe::kTableBytes / 16; c += L::kThreads) {
    const int e = c / (pipe::kCopies / 4);
    const uint32_t v = (uint32_t)codes16[e & 15] | ((uint32_t)codes16[e >> 4] << 16);
    reinterpret_cast<uint4 *>(ldsT)[c] = make_uint4(v, v, v, v);
  }
  issue_a(0, 0);
  issue_a(0, 1);
  issue_a(1, 0);
#pragma unroll
  for (int u = 0; u < 7; ++u) issue_codes(u);
  issue_scales(0);
  issue_scales(1);
  pipe::wait_copies_and_barrier<0>();
  dequant(0);
  dequant(1);
  dequant(2);
  pipe::wait_copies_and_barrier<0>();

  bf16x8 A0[4], B0[4], A1[4], B1[4];
  load_frags(0, 0, A0, B0);
  f32x4 acc[4][4];
#pragma unroll
  for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
    for (int b2 = 0; b2 < 4; ++b2) acc[a2][b2] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < S; ++t) {
    // A copies of step t-1 have landed and B halves expanded in step t-1 are
    // visible; every wave is done reading what this step's copies overwrite.
    pipe::wait_copies_and_barrier<L::kLate>();
    issue_a(t + 1, 1);
    issue_a(t + 2, 0);
    issue_codes(2 * t + 7);
    issue_codes(2 * t + 8);
    issue_scales(t + 2);

    load_frags(t & 1, 1, A1, B1);
    f32x4 p[4][4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
        p[mm][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[mm], B0[nn], zero, 0, 0, 0);
    load_frags((t + 1) & 1, 0, A0, B0);
    dequant(2 * t + 3);
    dequant(2 * t + 4);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
        p[mm][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[mm], B1[nn], p[mm][nn], 0, 0, 0);
    const char *sp = ldsS + (t & 3) * 512 + wn * 4 * 64 + r * 4;
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const float s = *reinterpret_cast<const float *>(sp + nn * 64);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mm][nn][i] = fmaf(s, p[mm][nn][i], acc[mm][nn][i]);
    }
  }
  // the clamped copies of the last steps must land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
  // 32-bit byte offsets into x and the code buffer for the copies
  const bool dma_ok = M * K * 2 < (int64_t(1) << 32) &&
                      (N / kTileRows) * KT * kTileBytes < (int64_t(1) << 32);
  if (nterm == 1 && dma_ok) {
    // 256-row tiles (8 waves) unless 128-row tiles (4 waves) need no more
    // rounds of workgroups over the CUs: a 128-row tile takes nearly as long
    // as a 256-row one, so the short tiles only pay off when they fill CUs
    // that would otherwise idle.
    const int64_t ntile = (N + BN - 1) / BN;
    const int64_t cus = device_cu_count();
    const int64_t rounds_tall = (ntile * ((M + 255) / 256) + cus - 1) / cus;
    const int64_t rounds_short = (ntile * ((M + 127) / 128) + cus - 1) / cus;
    if (rounds_tall < rounds_short) {
      const dim3 grid((unsigned)ntile, (unsigned)((M + 255) / 256));
      hipLaunchKernelGGL(gemm_pipe_kernel<4>, grid, dim3(512), 0, s, x, M, qw, am, ct, N, K, KT,
                         y);
    } else {
      const dim3 grid((unsigned)ntile, (unsigned)((M + 127) / 128));
      hipLaunchKernelGGL(gemm_pipe_kernel<2>, grid, dim3(256), 0, s, x, M, qw, am, ct, N, K, KT,
                         y);
    }
  } else {
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(256);
    hipLaunchKernelGGL(gemm_kernel<3>, grid, block, 0, s, x, M, q, a, ct, N, K, KT, y);
  }
  return hipGetLastError();
}

}  // namespace nf4
