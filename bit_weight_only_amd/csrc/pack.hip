// pack.hip -- load-time kernels: quantize fp32 weights into the device
// layout, the debug dequant, and the canonical <-> device layout copies, for
// the NF4 format and the asymmetric int4 format; and the activation gather
// of act-order checkpoints.
//
// Method (vibevoice.c README, "Quantization" > "Weights"): every projection
// is quantized once as it is loaded, before placement, deterministically;
// blocks of 64 weights along K share one absmax scale.  The nearest-code rule
// with ties to the lower code is the reading taken where the page is silent.
//
// Each wavefront owns one 16-row x 128-k device tile; lane l handles row
// l % 16 and the four 8-element runs k = 128t + 32j + 8(l/16) + 0..7.
#include "nf4_internal.h"

#pragma clang fp contract(off)

namespace nf4 {
namespace {

constexpr int kWavesPerBlock = 4;

struct TileCoord {
  int64_t tile, g;
  int t, lane, r, h;
};

__device__ inline bool tile_coord(int64_t ntiles, int64_t KT, TileCoord &c) {
  c.tile = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (c.tile >= ntiles) return false;
  c.lane = threadIdx.x & 63;
  c.g = c.tile / KT;
  c.t = (int)(c.tile - c.g * KT);
  c.r = c.lane & 15;
  c.h = c.lane >> 4;
  return true;
}

// Quantizer: s = max |w| over the block (exact); s == 0 -> zero code;
// else code = #{ i : (double)w > mid_i * (double)s }.  The max over a block
// combines the four lanes that share a row (lanes r, r+16, r+32, r+48).
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ W, int64_t K,
                                                   int64_t KT, int64_t ntiles, PackConsts pc,
                                                   uint4 *__restrict__ qw,
                                                   float *__restrict__ am) {
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const float *row = W + (c.g * kTileRows + c.r) * K;
  float w[4][8];
  bool valid[4];
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = (int64_t)c.t * kTileK + 32 * j + 8 * c.h;
    valid[j] = k0 < K;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (valid[j]) {
      a = *reinterpret_cast<const float4 *>(row + k0);
      b = *reinterpret_cast<const float4 *>(row + k0 + 4);
    }
    w[j][0] = a.x; w[j][1] = a.y; w[j][2] = a.z; w[j][3] = a.w;
    w[j][4] = b.x; w[j][5] = b.y; w[j][6] = b.z; w[j][7] = b.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float m = fabsf(w[j][i]);
      if (j < 2)
        s0 = fmaxf(s0, m);
      else
        s1 = fmaxf(s1, m);
    }
  }
  s0 = fmaxf(s0, __shfl_xor(s0, 16));
  s0 = fmaxf(s0, __shfl_xor(s0, 32));
  s1 = fmaxf(s1, __shfl_xor(s1, 16));
  s1 = fmaxf(s1, __shfl_xor(s1, 32));

  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float s = j < 2 ? s0 : s1;
    const double sd = (double)s;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t code;
      if (!valid[j]) {
        code = 0;
      } else if (s == 0.0f) {
        code = (uint32_t)pc.zero_index;
      } else {
        const double wd = (double)w[j][i];
        code = 0;
#pragma unroll
        for (int q = 0; q < 15; ++q) code += (wd > pc.mid[q] * sd) ? 1u : 0u;
      }
      word |= code << (4 * i);
    }
    out[j] = word;
  }
  qw[c.tile * 64 + c.lane] = make_uint4(out[0], out[1], out[2], out[3]);
  if (c.h == 0) {
    am[c.tile * kTileScales + 2 * c.r] = s0;
    am[c.tile * kTileScales + 2 * c.r + 1] = s1;
  }
}

// Debug dequant: W'[n][k] = fl32(c[code] * s), one binary32 multiply.
__global__ __launch_bounds__(256) void dequant_kernel(const uint4 *__restrict__ qw,
                                                      const float *__restrict__ am, Codebook cb,
                                                      int64_t K, int64_t KT, int64_t ntiles,
                                                      float *__restrict__ out) {
  __shared__ float cbs[16];
  if (threadIdx.x < 16) cbs[threadIdx.x] = cb.c[threadIdx.x];
  __syncthreads();
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const uint4 q = qw[c.tile * 64 + c.lane];
  const float s0 = am[c.tile * kTileScales + 2 * c.r];
  const float s1 = am[c.tile * kTileScales + 2 * c.r + 1];
  const uint32_t words[4] = {q.x, q.y, q.z, q.w};
  float *row = out + (c.g * kTileRows + c.r) * K;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = (int64_t)c.t * kTileK + 32 * j + 8 * c.h;
    if (k0 >= K) continue;
    const float s = j < 2 ? s0 : s1;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = cbs[(words[j] >> (4 * i)) & 15u] * s;
    *reinterpret_cast<float4 *>(row + k0) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(row + k0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Canonical -> device layout.  A device dword holds exactly the four
// canonical bytes of its 8-k run, so this is a permutation of dwords.
__global__ __launch_bounds__(256) void repack_kernel(const uint32_t *__restrict__ codes,
                                                     const float *__restrict__ scales, int64_t K,
                                                     int64_t KT, int64_t ntiles,
                                                     uint4 *__restrict__ qw,
                                                     float *__restrict__ am) {
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const int64_t n = c.g * kTileRows + c.r;
  const uint32_t *row = codes + n * (K / 8);  // K/2 bytes = K/8 dwords
  uint32_t wd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = (int64_t)c.t * kTileK + 32 * j + 8 * c.h;
    wd[j] = k0 < K ? row[k0 / 8] : 0u;
  }
  qw[c.tile * 64 + c.lane] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  if (c.h == 0) {
    const int64_t nb = K / kBlock, b0 = 2 * (int64_t)c.t;
    am[c.tile * kTileScales + 2 * c.r] = scales[n * nb + b0];
    am[c.tile * kTileScales + 2 * c.r + 1] = b0 + 1 < nb ? scales[n * nb + b0 + 1] : 0.0f;
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint4 *__restrict__ qw,
                                                     const float *__restrict__ am, int64_t K,
                                                     int64_t KT, int64_t ntiles,
                                                     uint32_t *__restrict__ codes,
                                                     float *__restrict__ scales) {
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const int64_t n = c.g * kTileRows + c.r;
  uint32_t *row = codes + n * (K / 8);
  const uint4 q = qw[c.tile * 64 + c.lane];
  const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = (int64_t)c.t * kTileK + 32 * j + 8 * c.h;
    if (k0 < K) row[k0 / 8] = wd[j];
  }
  if (c.h == 0) {
    const int64_t nb = K / kBlock, b0 = 2 * (int64_t)c.t;
    scales[n * nb + b0] = am[c.tile * kTileScales + 2 * c.r];
    if (b0 + 1 < nb) scales[n * nb + b0 + 1] = am[c.tile * kTileScales + 2 * c.r + 1];
  }
}

// ---------------------------------------------------------------------------
// Second format: asymmetric int4, one group per device tile row (128 k):
// w = (q - z) * s with a binary16 scale s and an integer zero point z per
// group (vibevoice.c README, "Quantization" > "Weights", the AWQ/GPTQ
// paragraph).  The codes use the device layout above with the nibbles of
// every dword interleaved: code i (k = k0 + i) sits at nibble position
// (i >> 1) + 4 (i & 1), so codes 2p and 2p + 1 share the bit positions of
// the two halves of a bf16 pair (the pages permute nibbles inside 16-byte
// runs for the same reason: one logic operation with a magic constant
// yields the pair).  A tile's params are 16 dwords, dword r = binary16 bits
// of s | z << 16 for row r (s is a binary16 value by construction, so
// nothing is lost).
__device__ inline int awq_nibble_pos(int i) { return (i >> 1) + 4 * (i & 1); }
// canonical dword (code i at nibble i) <-> interleaved dword
__device__ inline uint32_t awq_interleave(uint32_t w) {
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) o |= ((w >> (4 * i)) & 15u) << (4 * awq_nibble_pos(i));
  return o;
}
__device__ inline uint32_t awq_deinterleave(uint32_t w) {
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) o |= ((w >> (4 * awq_nibble_pos(i))) & 15u) << (4 * i);
  return o;
}

// Nearest binary16 value of a positive finite double, ties to even, as a
// double: the significand is cut to 11 bits (10 stored) by integer
// arithmetic on the binary64 encoding; below 2^-14 the quantum is 2^-24.
__device__ inline double awq_fp16_of_positive(double a) {
  if (a < 0x1p-14) return rint(a * 0x1p24) * 0x1p-24;  // exact scaling; rint ties to even
  const uint64_t u = (uint64_t)__double_as_longlong(a);
  const uint64_t drop = 42;                             // 52 - 10 fraction bits
  const uint64_t keep = u >> drop, rest = u & ((1ull << drop) - 1), half = 1ull << (drop - 1);
  const uint64_t up = (rest > half || (rest == half && (keep & 1))) ? 1u : 0u;
  const double r = __longlong_as_double((long long)((keep + up) << drop));
  return r >= 65520.0 ? __longlong_as_double(0x7FF0000000000000ll) : r;
}

// Quantizer of the second format, one group per (tile, row): lanes r, r+16,
// r+32, r+48 share the row; min and max over their 32 values each.
__global__ __launch_bounds__(256) void awq_pack_kernel(const float *__restrict__ W, int64_t K,
                                                       int64_t KT, int64_t ntiles,
                                                       uint4 *__restrict__ qw,
                                                       uint32_t *__restrict__ pr) {
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const float *row = W + (c.g * kTileRows + c.r) * K;
  float w[4][8];
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = (int64_t)c.t * kTileK + 32 * j + 8 * c.h;
    const float4 a = *reinterpret_cast<const float4 *>(row + k0);
    const float4 b = *reinterpret_cast<const float4 *>(row + k0 + 4);
    w[j][0] = a.x; w[j][1] = a.y; w[j][2] = a.z; w[j][3] = a.w;
    w[j][4] = b.x; w[j][5] = b.y; w[j][6] = b.z; w[j][7] = b.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo = fminf(lo, w[j][i]);
      hi = fmaxf(hi, w[j][i]);
    }
  }
  lo = fminf(lo, __shfl_xor(lo, 16));
  lo = fminf(lo, __shfl_xor(lo, 32));
  hi = fmaxf(hi, __shfl_xor(hi, 16));
  hi = fmaxf(hi, __shfl_xor(hi, 32));
  double range = (double)hi - (double)lo;
  if (range < 1e-5) range = 1e-5;
  const double sd = awq_fp16_of_positive(range / 15.0);
  const double zd = fmin(fmax(rint(-(double)lo / sd), 0.0), 15.0);
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double v = fmin(fmax(rint((double)w[j][i] / sd) + zd, 0.0), 15.0);
      word |= (uint32_t)v << (4 * awq_nibble_pos(i));
    }
    out[j] = word;
  }
  qw[c.tile * 64 + c.lane] = make_uint4(out[0], out[1], out[2], out[3]);
  if (c.h == 0)
    pr[c.tile * kTileRows + c.r] =
        (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)sd) | ((uint32_t)zd << 16);
}

// Canonical codes [N][K/2], scales [N][K/128] (binary16 bits) and zero
// points [N][K/128] (bytes) -> device layout.
__global__ __launch_bounds__(256) void awq_repack_kernel(const uint32_t *__restrict__ codes,
                                                         const uint16_t *__restrict__ scales,
                                                         const uint8_t *__restrict__ zeros,
                                                         int64_t K, int64_t KT, int64_t ntiles,
                                                         uint4 *__restrict__ qw,
                                                         uint32_t *__restrict__ pr) {
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const int64_t n = c.g * kTileRows + c.r;
  const uint32_t *row = codes + n * (K / 8);
  uint32_t wd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wd[j] = awq_interleave(row[((int64_t)c.t * kTileK + 32 * j + 8 * c.h) / 8]);
  qw[c.tile * 64 + c.lane] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  if (c.h == 0)
    pr[c.tile * kTileRows + c.r] =
        (uint32_t)scales[n * KT + c.t] | ((uint32_t)(zeros[n * KT + c.t] & 15) << 16);
}

// Device layout -> canonical codes, scales (binary16 bits) and zero points.
__global__ __launch_bounds__(256) void awq_unpack_kernel(const uint4 *__restrict__ qw,
                                                         const uint32_t *__restrict__ pr,
                                                         int64_t K, int64_t KT, int64_t ntiles,
                                                         uint32_t *__restrict__ codes,
                                                         uint16_t *__restrict__ scales,
                                                         uint8_t *__restrict__ zeros) {
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const int64_t n = c.g * kTileRows + c.r;
  const uint4 q = qw[c.tile * 64 + c.lane];
  uint32_t *row = codes + n * (K / 8);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    row[((int64_t)c.t * kTileK + 32 * j + 8 * c.h) / 8] =
        awq_deinterleave(j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w);
  if (c.h == 0) {
    const uint32_t v = pr[c.tile * kTileRows + c.r];
    scales[n * KT + c.t] = (uint16_t)(v & 0xFFFFu);
    zeros[n * KT + c.t] = (uint8_t)(v >> 16);
  }
}

// Debug dequant of the second format: W'[n][k] = fl32((q - z) * s).
__global__ __launch_bounds__(256) void awq_dequant_kernel(const uint4 *__restrict__ qw,
                                                          const uint32_t *__restrict__ pr,
                                                          int64_t K, int64_t KT, int64_t ntiles,
                                                          float *__restrict__ out) {
  TileCoord c;
  if (!tile_coord(ntiles, KT, c)) return;
  const uint32_t v = pr[c.tile * kTileRows + c.r];
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
  const float z = (float)(v >> 16);
  const uint4 q = qw[c.tile * 64 + c.lane];
  float *row = out + (c.g * kTileRows + c.r) * K;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t word = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
    const int64_t k0 = (int64_t)c.t * kTileK + 32 * j + 8 * c.h;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ((float)((word >> (4 * awq_nibble_pos(i))) & 15u) - z) * s;
    *reinterpret_cast<float4 *>(row + k0) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(row + k0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Activation gather of act-order checkpoints (vibevoice.c README,
// "Quantization" > "Weights", the GPTQ act-order bullet: the loader sorts
// the input channels by group and the decoder gathers x through that order
// before the product): out[m][j] = x[m][perm[j]].  One thread writes 8
// consecutive outputs as one 16-byte store; perm values outside [0, K) are
// clamped into it.
__global__ __launch_bounds__(256) void gather_columns_kernel(const uint16_t *__restrict__ x,
                                                             int64_t K,
                                                             const int32_t *__restrict__ perm,
                                                             uint16_t *__restrict__ out,
                                                             int64_t nchunks) {
  const int64_t kc = K / 8;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * 256) {
    const int64_t m = c / kc, j0 = (c - m * kc) * 8;
    const int4 p0 = *reinterpret_cast<const int4 *>(perm + j0);
    const int4 p1 = *reinterpret_cast<const int4 *>(perm + j0 + 4);
    const int p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const uint16_t *row = x + m * K;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t a = p[2 * i] < 0 ? 0 : p[2 * i] >= K ? K - 1 : p[2 * i];
      const int64_t b = p[2 * i + 1] < 0 ? 0 : p[2 * i + 1] >= K ? K - 1 : p[2 * i + 1];
      w[i] = (uint32_t)row[a] | ((uint32_t)row[b] << 16);
    }
    *reinterpret_cast<uint4 *>(out + m * K + j0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

inline dim3 tile_grid(int64_t ntiles) {
  return dim3((unsigned)((ntiles + kWavesPerBlock - 1) / kWavesPerBlock));
}

}  // namespace

hipError_t launch_pack(const float *W, int64_t N, int64_t K, const PackConsts &pc, uint8_t *qw,
                       float *am, hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(pack_kernel, tile_grid(ntiles), dim3(256), 0, s, W, K, KT, ntiles, pc,
                     reinterpret_cast<uint4 *>(qw), am);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *qw, const float *am, const Codebook &cb, int64_t N,
                          int64_t K, float *out, hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(dequant_kernel, tile_grid(ntiles), dim3(256), 0, s,
                     reinterpret_cast<const uint4 *>(qw), am, cb, K, KT, ntiles, out);
  return hipGetLastError();
}

hipError_t launch_repack(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                         uint8_t *qw, float *am, hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(repack_kernel, tile_grid(ntiles), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t *>(codes), scales, K, KT, ntiles,
                     reinterpret_cast<uint4 *>(qw), am);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *qw, const float *am, int64_t N, int64_t K, uint8_t *codes,
                         float *scales, hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(unpack_kernel, tile_grid(ntiles), dim3(256), 0, s,
                     reinterpret_cast<const uint4 *>(qw), am, K, KT, ntiles,
                     reinterpret_cast<uint32_t *>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_awq_pack(const float *W, int64_t N, int64_t K, uint8_t *qw, uint32_t *pr,
                           hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(awq_pack_kernel, tile_grid(ntiles), dim3(256), 0, s, W, K, KT, ntiles,
                     reinterpret_cast<uint4 *>(qw), pr);
  return hipGetLastError();
}

hipError_t launch_awq_repack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                             int64_t N, int64_t K, uint8_t *qw, uint32_t *pr, hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(awq_repack_kernel, tile_grid(ntiles), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t *>(codes), scales, zeros, K, KT, ntiles,
                     reinterpret_cast<uint4 *>(qw), pr);
  return hipGetLastError();
}

hipError_t launch_awq_unpack(const uint8_t *qw, const uint32_t *pr, int64_t N, int64_t K,
                             uint8_t *codes, uint16_t *scales, uint8_t *zeros, hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(awq_unpack_kernel, tile_grid(ntiles), dim3(256), 0, s,
                     reinterpret_cast<const uint4 *>(qw), pr, K, KT, ntiles,
                     reinterpret_cast<uint32_t *>(codes), scales, zeros);
  return hipGetLastError();
}

hipError_t launch_awq_dequant(const uint8_t *qw, const uint32_t *pr, int64_t N, int64_t K,
                              float *out, hipStream_t s) {
  const int64_t KT = tiles_k(K), ntiles = (N / kTileRows) * KT;
  hipLaunchKernelGGL(awq_dequant_kernel, tile_grid(ntiles), dim3(256), 0, s,
                     reinterpret_cast<const uint4 *>(qw), pr, K, KT, ntiles, out);
  return hipGetLastError();
}

hipError_t launch_gather_columns(const uint16_t *x, int64_t M, int64_t K, const int32_t *perm,
                                 uint16_t *out, hipStream_t s) {
  const int64_t nchunks = M * (K / 8);
  int64_t blocks = (nchunks + 255) / 256;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;  // grid-stride beyond
  hipLaunchKernelGGL(gather_columns_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, K, perm,
                     out, nchunks);
  return hipGetLastError();
}

}  // namespace nf4
