// nf4_internal.h -- device layout geometry, kernel argument blocks and the
// launchers shared by the entry points in nf4_abi.hip.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace nf4 {

// Quantization block along K (vibevoice.c README, "Quantization" >
// "Weights": blocks of 64 with one absmax scale each).
constexpr int kBlock = 64;
// Device tile: 16 rows x 128 k = 1024 bytes of codes, one 16-byte run per
// lane of a 64-wide wavefront.  Lane l owns row l % 16 and, in dword j,
// k = 32j + 8(l / 16) + 0..7: the bf16 B operand of
// v_mfma_f32_16x16x32_bf16 for k-step j.
constexpr int kTileRows = 16;
constexpr int kTileK = 128;
constexpr int kTileBytes = 1024;
constexpr int kTileScales = 32;  // 16 rows x 2 blocks

// Replicated lookup table of code pairs: entry e (a packed byte holding the
// codes of k and k+1) maps to (bf16 c[e & 15]) | (bf16 c[e >> 4]) << 16.
// kPairCopies copies interleave so that lane l reads copy l % 32 and the
// dword address is e * 32 + copy: 32 lanes of a half-wave hit 32 banks.
constexpr int kPairCopies = 32;
constexpr int kPairWords = 256 * kPairCopies;

// Codebook split into bf16 terms c = t0 + t1 + t2 (exact for binary32 when
// the host check passes); the GEMV/GEMM products with each term are exact in
// fp32.  Passed by value as a kernel argument; the 16-byte alignment lets a
// kernel read it with scalar loads (a 2-byte aligned block is read with
// vector loads, which wait in line behind the kernel's other vector loads).
struct alignas(16) CodeTerms {
  uint16_t t[3][16];
};

// Quantizer constants: midpoints of neighbouring codes in double, and the
// index of the +0.0 code.
struct PackConsts {
  double mid[15];
  int zero_index;
};

struct Codebook {
  float c[16];
};

inline int64_t tiles_k(int64_t K) { return (K + kTileK - 1) / kTileK; }

// K is summed in P parts fixed by (N, K) alone (k_parts): device tiles
// [part_begin(j), part_begin(j + 1)) for j = 0 .. P-1, each part folded from
// zero in K order, then the parts' sums added in part order.  Every GEMM path
// (skinny, tiled, generic) uses the same parts, so a row of y never depends
// on M.  P = 1: one part.
constexpr int64_t kSplitK = 8192;
int k_parts(int64_t N, int64_t K);
__host__ __device__ inline int part_begin(int j, int64_t KT, int P) {
  return (int)((j * KT + P - 1) / P);
}

// The codebook 0, 1, ..., 15 as bf16 (exact): the codes of the asymmetric
// int4 format enter the products as their integer values.
inline CodeTerms identity_terms() {
  CodeTerms ct{};
  for (int i = 0; i < 16; ++i) ct.t[0][i] = (uint16_t)(__builtin_bit_cast(uint32_t, (float)i) >> 16);
  return ct;
}

hipError_t launch_pack(const float *W, int64_t N, int64_t K, const PackConsts &pc, uint8_t *qw,
                       float *am, hipStream_t s);
hipError_t launch_dequant(const uint8_t *qw, const float *am, const Codebook &cb, int64_t N,
                          int64_t K, float *out, hipStream_t s);
hipError_t launch_repack(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                         uint8_t *qw, float *am, hipStream_t s);
hipError_t launch_unpack(const uint8_t *qw, const float *am, int64_t N, int64_t K, uint8_t *codes,
                         float *scales, hipStream_t s);
// Second format (asymmetric int4, group 128 = one device tile row): codes in
// the device layout; params 16 dwords per tile, dword r = binary16 bits of s
// | z << 16 for row r.  K % 128 == 0.
constexpr int kAwqParamBytes = kTileRows * 4;  // params of one tile
hipError_t launch_awq_pack(const float *W, int64_t N, int64_t K, uint8_t *qw, uint32_t *pr,
                           hipStream_t s);
hipError_t launch_awq_repack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                             int64_t N, int64_t K, uint8_t *qw, uint32_t *pr, hipStream_t s);
hipError_t launch_awq_unpack(const uint8_t *qw, const uint32_t *pr, int64_t N, int64_t K,
                             uint8_t *codes, uint16_t *scales, uint8_t *zeros, hipStream_t s);
hipError_t launch_awq_dequant(const uint8_t *qw, const uint32_t *pr, int64_t N, int64_t K,
                              float *out, hipStream_t s);
// out[m][j] = x[m][perm[j]] (bf16 bits), K % 8 == 0; perm clamped to [0, K).
hipError_t launch_gather_columns(const uint16_t *x, int64_t M, int64_t K, const int32_t *perm,
                                 uint16_t *out, hipStream_t s);
// The packed matrix of the next GEMV launch, named so that the current
// launch can read its first tiles ahead (a hint: results never depend on it).
struct NextMatrix {
  const uint8_t *qw = nullptr;
  const float *am = nullptr;
  int64_t N = 0, K = 0;
};
hipError_t launch_gemv(const uint16_t *x, int M, const uint8_t *qw, const float *am,
                       const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y, void *ws,
                       hipStream_t s, const NextMatrix *next = nullptr);
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K);
// GEMV followed by the row-wise argmax of y (fused into the fast kernel).
hipError_t launch_gemv_argmax(const uint16_t *x, int M, const uint8_t *qw, const float *am,
                              const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y,
                              int32_t *index, void *ws, hipStream_t s);
size_t gemv_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Compute units of the current device (queried once per device).
int device_cu_count();
hipError_t launch_gemm(const uint16_t *x, int64_t M, const uint8_t *qw, const float *am,
                       const CodeTerms &ct, int nterm, int64_t N, int64_t K, float *y,
                       void *ws, size_t ws_bytes, hipStream_t s);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Skinny path of the GEMM (M <= kSkinnyMaxM, codebook of bf16 values): one
// wave per row group streams all of K; also serves nf4_gemv when x does not
// fit the GEMV's LDS.  Bit-identical to the tiled GEMM.
constexpr int64_t kSkinnyMaxM = 256;
bool skinny_eligible(int64_t M, int64_t N, int64_t K, int nterm);
hipError_t launch_skinny(const uint16_t *x, int64_t M, const uint8_t *qw, const float *am,
                         const CodeTerms &ct, int64_t N, int64_t K, float *y, hipStream_t s);


// LDS byte address of a pointer into LDS.
typedef __attribute__((address_space(3))) void lds_void;
__device__ inline uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_void *)p; }
// One copy from global memory (uniform base + per-lane 32-bit byte offset)
// straight into LDS: 16 bytes per active lane land at m0 + 16 * lane.
// Issued from inline assembly, so the compiler neither waits for it nor
// knows what it writes: every use is ordered by an explicit vmcnt wait and a
// barrier.  m0 is an input operand of the statement ("{m0}"): the compiler
// sets it and knows that it holds the destination, so no value of its own
// is kept in m0 across the copy.
__device__ inline void copy16_to_lds(uint32_t m0, const void *base, uint32_t voff) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

// Sum of the 8 bf16 values of a 16-byte chunk, in k order.
__device__ inline float chunk_sum8(uint4 c) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float v = __uint_as_float(w[0] << 16);
  v += __uint_as_float(w[0] & 0xFFFF0000u);
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    v += __uint_as_float(w[i] << 16);
    v += __uint_as_float(w[i] & 0xFFFF0000u);
  }
  return v;
}

// Sum over the 16 lanes of a row (lanes 16i .. 16i + 15) left in every lane
// of it: neighbours (lane ^ 1), then pairs (lane ^ 2), then quads (lane i of
// a half-row with lane 7 - i), then halves (lane i with 15 - i), each step a
// DPP add.  A balanced tree, so every lane of the row gets the same bits.
// Every lane of the wave must execute it.
__device__ inline float row16_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      0xF, 0xF, false));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
  return v;
}

// B pair of the asymmetric int4 format: bf16 (1 + c/16) of codes 2q and
// 2q + 1 of an interleaved code word (nibble positions q and q + 4), i.e.
// the nibbles moved to mantissa bits 3..6 of each half and or-ed with bf16
// 1.0 (0x3F80).  One shift and one v_and_or_b32 whose mask comes from a
// scalar register and whose magic word from a vector register (the
// three-operand encoding takes neither a literal nor two scalar operands).
__device__ inline uint32_t awq_pair(uint32_t wd, int q, uint32_t magic_v) {
  const uint32_t sh = q ? wd >> (4 * q - 3) : wd << 3;
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(sh), "s"(0x00780078u), "v"(magic_v));
  return d;
}

// Linear layers of the asymmetric int4 format.  The GEMV keeps x and its
// per-tile sums in LDS (M <= 8 and x small enough); the GEMM sums x per tile
// in a pre-pass into the workspace ([K/128][M rounded up to 128] floats) and
// runs the tiled kernel with the affine fold.
bool awq_gemv_fast_eligible(int64_t M, int64_t N, int64_t K);
hipError_t launch_awq_gemv_fast(const uint16_t *x, int M, const uint8_t *qw, const uint32_t *pr,
                                int64_t N, int64_t K, float *y, hipStream_t s,
                                const NextMatrix *next = nullptr);
bool awq_gemm_supported(int64_t M, int64_t N, int64_t K);
size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_awq_gemm(const uint16_t *x, int64_t M, const uint8_t *qw, const uint32_t *pr,
                           int64_t N, int64_t K, float *y, void *ws, hipStream_t s);

}  // namespace nf4
