// nf4_abi.hip -- the exported C entry points declared in include/nf4.h:
// host-side validation, codebook preparation, launch on the caller's stream.
//
// Conventions follow the vibevoice.c README: a kernel call is launches on the
// caller's stream and nothing else (no allocation, free or sync; "The speech
// front end"), never the legacy default stream by the library's own choice
// ("The decode step is one submission"), split-K partials live in the
// caller's scratch ("Quantization" > "Weights", M > 1 bullet), and failures
// are named status codes.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/nf4.h"
#include "nf4_internal.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxGemvM = 8;
constexpr int64_t kMaxGemmM = int64_t(1) << 23;

bool shape_ok(int64_t N, int64_t K) {
  if (N < nf4::kTileRows || N % nf4::kTileRows != 0) return false;
  if (K < nf4::kBlock || K % nf4::kBlock != 0) return false;
  if (N > kMaxDim || K > kMaxDim) return false;
  return N * K <= kMaxElems;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// fp32 -> bf16 with ties to even (inputs are finite).
uint16_t bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float bf16_value(uint16_t h) { return bits_f32((uint32_t)h << 16); }

// Split every code into up to three bf16 terms whose sum is the fp32 value
// exactly.  Returns the number of terms needed (1 or 3), or 0 when a code is
// not finite or cannot be split exactly.
int split_codebook(const float *cb, nf4::CodeTerms &ct) {
  int nterm = 1;
  for (int i = 0; i < 16; ++i) {
    const float c = cb[i];
    if (!isfinite(c)) return 0;
    const uint16_t t0 = bf16_rne(c);
    const float r0 = c - bf16_value(t0);
    const uint16_t t1 = bf16_rne(r0);
    const float r1 = r0 - bf16_value(t1);
    const uint16_t t2 = bf16_rne(r1);
    const double sum = (double)bf16_value(t0) + (double)bf16_value(t1) + (double)bf16_value(t2);
    if (!isfinite(bf16_value(t0)) || sum != (double)c) return 0;
    ct.t[0][i] = t0;
    ct.t[1][i] = t1;
    ct.t[2][i] = t2;
    if (bf16_value(t1) != 0.0f || bf16_value(t2) != 0.0f) nterm = 3;
  }
  return nterm;
}

// bfloat16 activations as their bit patterns (hip_bfloat16 is a 2-byte
// standard-layout wrapper of them).
const uint16_t *bf16_bits(const hip_bfloat16 *x) { return reinterpret_cast<const uint16_t *>(x); }

nf4_status from_hip(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_HIP; }

// Shapes of the asymmetric int4 format: one group of 128 k per tile row.
bool awq_shape_ok(int64_t N, int64_t K) { return shape_ok(N, K) && K % nf4::kTileK == 0; }

nf4_status check_linear_args(const uint16_t *x, int64_t M, const uint8_t *qw, const float *am,
                             const float *cb, int64_t N, int64_t K, const float *y,
                             int64_t max_m) {
  if (!x || !qw || !am || !cb || !y) return NF4_ERR_NULL;
  if (M < 1 || M > max_m || !shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(qw) || !aligned16(am) || !aligned16(y)) return NF4_ERR_ALIGN;
  return NF4_OK;
}

}  // namespace

namespace nf4 {

// A device property, cached per device id after the first query.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace nf4

extern "C" {

const char *nf4_status_string(nf4_status status) {
  switch (status) {
    case NF4_OK: return "NF4_OK";
    case NF4_ERR_NULL: return "NF4_ERR_NULL: a required pointer is NULL";
    case NF4_ERR_SHAPE: return "NF4_ERR_SHAPE: M, N or K outside the supported limits";
    case NF4_ERR_ALIGN: return "NF4_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case NF4_ERR_CODEBOOK: return "NF4_ERR_CODEBOOK: codebook not usable by this entry point";
    case NF4_ERR_WORKSPACE: return "NF4_ERR_WORKSPACE: workspace smaller than nf4_workspace_bytes()";
    case NF4_ERR_HIP: return "NF4_ERR_HIP: the HIP runtime rejected a launch";
    case NF4_ERR_SCRATCH:
      return "NF4_ERR_SCRATCH: the call needs more than the library's static scratch (64 KiB)";
  }
  return "NF4 unknown status";
}

namespace {
// Standard normal CDF through the complementary error function of libm.
double phi_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

// Inverse standard normal CDF for p in (1/2, 1): Newton's method on
// Phi(z) - p from z = 0.  Phi is increasing and concave on z > 0, so every
// tangent step lands at or below the root and the iterates rise to it
// monotonically (quadratically near it); stop when a step no longer moves z.
double phi_inv_upper(double p) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  double z = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double step = (p - phi_cdf(z)) / (inv_sqrt_2pi * exp(-0.5 * z * z));
    const double zn = z + step;
    if (!(zn > z)) break;
    z = zn;
  }
  return z;
}

// Nearest bfloat16 (8 significant bits, ties to even) of a finite double in
// the normal range, as a float: v = q * 2^(e - 8) rounded to an integer q.
float round_to_bf16(double v) {
  if (v == 0.0) return 0.0f;
  int e = 0;
  frexp(v, &e);  // |v| = f 2^e, f in [1/2, 1)
  const double scaled = ldexp(v, 8 - e);
  return (float)ldexp(nearbyint(scaled), e - 8);
}
}  // namespace

nf4_status nf4_codebook(double delta, float codebook[16]) {
  if (!codebook) return NF4_ERR_NULL;
  if (!(delta > 0.75 && delta <= 0.9999)) return NF4_ERR_CODEBOOK;
  const double d = phi_inv_upper(delta);
  double v[16];
  v[7] = 0.0;
  for (int j = 1; j <= 7; ++j) v[7 - j] = -phi_inv_upper(0.5 + (delta - 0.5) * j / 7.0) / d;
  for (int j = 1; j <= 8; ++j) v[7 + j] = phi_inv_upper(0.5 + (delta - 0.5) * j / 8.0) / d;
  // the end points are exactly -1 and +1 (each level j = 7 or 8 is Phi^-1(delta) / d)
  v[0] = -1.0;
  v[15] = 1.0;
  for (int i = 0; i < 16; ++i) codebook[i] = round_to_bf16(v[i]);
  return NF4_OK;
}

size_t nf4_qweight_bytes(int64_t N, int64_t K) {
  if (!shape_ok(N, K)) return 0;
  return (size_t)(N / nf4::kTileRows) * (size_t)nf4::tiles_k(K) * nf4::kTileBytes;
}

size_t nf4_absmax_bytes(int64_t N, int64_t K) {
  if (!shape_ok(N, K)) return 0;
  return (size_t)(N / nf4::kTileRows) * (size_t)nf4::tiles_k(K) * nf4::kTileScales * sizeof(float);
}

size_t nf4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxGemmM || !shape_ok(N, K)) return 0;
  size_t need = nf4::gemm_workspace_bytes(M, N, K);
  if (M <= kMaxGemvM) {
    const size_t v = nf4::gemv_workspace_bytes(M, N, K);
    need = v > need ? v : need;
  }
  return need;
}

nf4_status nf4_pack(const float *W, int64_t N, int64_t K, const float codebook[16],
                    uint8_t *qweight, float *absmax, hipStream_t stream) {
  if (!W || !codebook || !qweight || !absmax) return NF4_ERR_NULL;
  if (!shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(qweight) || !aligned16(absmax)) return NF4_ERR_ALIGN;
  nf4::PackConsts pc;
  pc.zero_index = -1;
  for (int i = 0; i < 16; ++i) {
    if (!isfinite(codebook[i])) return NF4_ERR_CODEBOOK;
    if (i > 0 && !(codebook[i] > codebook[i - 1])) return NF4_ERR_CODEBOOK;
    if (codebook[i] == 0.0f && !signbit(codebook[i])) pc.zero_index = i;
  }
  if (pc.zero_index < 0) return NF4_ERR_CODEBOOK;
  for (int i = 0; i < 15; ++i) pc.mid[i] = ((double)codebook[i] + (double)codebook[i + 1]) / 2.0;
  return from_hip(nf4::launch_pack(W, N, K, pc, qweight, absmax, stream));
}

nf4_status nf4_dequant(const uint8_t *qweight, const float *absmax, const float codebook[16],
                       int64_t N, int64_t K, float *W_out, hipStream_t stream) {
  if (!qweight || !absmax || !codebook || !W_out) return NF4_ERR_NULL;
  if (!shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(qweight) || !aligned16(absmax) || !aligned16(W_out)) return NF4_ERR_ALIGN;
  nf4::Codebook cb;
  for (int i = 0; i < 16; ++i) {
    if (!isfinite(codebook[i])) return NF4_ERR_CODEBOOK;
    cb.c[i] = codebook[i];
  }
  return from_hip(nf4::launch_dequant(qweight, absmax, cb, N, K, W_out, stream));
}

nf4_status nf4_repack(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                      uint8_t *qweight, float *absmax, hipStream_t stream) {
  if (!codes || !scales || !qweight || !absmax) return NF4_ERR_NULL;
  if (!shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(qweight) || !aligned16(absmax))
    return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_repack(codes, scales, N, K, qweight, absmax, stream));
}

nf4_status nf4_unpack(const uint8_t *qweight, const float *absmax, int64_t N, int64_t K,
                      uint8_t *codes, float *scales, hipStream_t stream) {
  if (!codes || !scales || !qweight || !absmax) return NF4_ERR_NULL;
  if (!shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(qweight) || !aligned16(absmax))
    return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_unpack(qweight, absmax, N, K, codes, scales, stream));
}

nf4_status nf4_gemv(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight, const float *absmax,
                    const float codebook[16], int64_t N, int64_t K, float *y, void *workspace,
                    size_t ws_bytes, hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_linear_args(x, M, qweight, absmax, codebook, N, K, y, kMaxGemvM);
  if (st != NF4_OK) return st;
  const size_t need = nf4::gemv_workspace_bytes(M, N, K);
  if (need > 0 && !workspace) return NF4_ERR_NULL;
  if (need > ws_bytes) return NF4_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return NF4_ERR_ALIGN;
  nf4::CodeTerms ct;
  const int nterm = split_codebook(codebook, ct);
  if (nterm == 0) return NF4_ERR_CODEBOOK;
  return from_hip(
      nf4::launch_gemv(x, (int)M, qweight, absmax, ct, nterm, N, K, y, workspace, stream));
}

nf4_status nf4_gemv_prefetch(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight,
                             const float *absmax, const float codebook[16], int64_t N, int64_t K,
                             float *y, void *workspace, size_t ws_bytes,
                             const uint8_t *next_qweight, const float *next_absmax,
                             int64_t next_N, int64_t next_K, hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_linear_args(x, M, qweight, absmax, codebook, N, K, y, kMaxGemvM);
  if (st != NF4_OK) return st;
  nf4::NextMatrix next;
  if (next_qweight != nullptr) {
    if (!next_absmax) return NF4_ERR_NULL;
    if (!aligned16(next_qweight) || !aligned16(next_absmax)) return NF4_ERR_ALIGN;
    if (!shape_ok(next_N, next_K)) return NF4_ERR_SHAPE;
    next.qw = next_qweight;
    next.am = next_absmax;
    next.N = next_N;
    next.K = next_K;
  }
  const size_t need = nf4::gemv_workspace_bytes(M, N, K);
  if (need > 0 && !workspace) return NF4_ERR_NULL;
  if (need > ws_bytes) return NF4_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return NF4_ERR_ALIGN;
  nf4::CodeTerms ct;
  const int nterm = split_codebook(codebook, ct);
  if (nterm == 0) return NF4_ERR_CODEBOOK;
  return from_hip(nf4::launch_gemv(x, (int)M, qweight, absmax, ct, nterm, N, K, y, workspace,
                                   stream, next_qweight ? &next : nullptr));
}

size_t nf4_gemv_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxGemvM || !shape_ok(N, K)) return 0;
  return nf4::gemv_argmax_workspace_bytes(M, N, K);
}

nf4_status nf4_gemv_argmax(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight,
                           const float *absmax, const float codebook[16], int64_t N, int64_t K,
                           float *y, int32_t *index, void *workspace, size_t ws_bytes,
                           hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_linear_args(x, M, qweight, absmax, codebook, N, K, y, kMaxGemvM);
  if (st != NF4_OK) return st;
  if (!index || !workspace) return NF4_ERR_NULL;
  if (!aligned16(index) || !aligned16(workspace)) return NF4_ERR_ALIGN;
  if (nf4::gemv_argmax_workspace_bytes(M, N, K) > ws_bytes) return NF4_ERR_WORKSPACE;
  nf4::CodeTerms ct;
  const int nterm = split_codebook(codebook, ct);
  if (nterm == 0) return NF4_ERR_CODEBOOK;
  return from_hip(nf4::launch_gemv_argmax(x, (int)M, qweight, absmax, ct, nterm, N, K, y, index,
                                          workspace, stream));
}

}  // extern "C"

// Scratch of nf4_gemv_argmax_noalloc: the arrival counter (first 256 bytes)
// and the per-workgroup candidates of the argmax that nf4_gemv_argmax keeps
// in the caller's workspace.  Each device the library runs on holds its own
// copy until the process ends; every call on a device shares it.
static constexpr size_t kStaticScratchBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

// Device address of `scratch` on the current device, taken once per device
// with that device current (the array's name is not a device address in
// host code).
hipError_t scratch_address(void **out) {
  static std::atomic<void *> addr[64];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// Zero the first `words` dwords of p (a kernel, not a memset, so that a
// captured graph clears it on every replay).
__global__ void zero_words_kernel(uint32_t *p, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0u;
}
}  // namespace

extern "C" {

nf4_status nf4_gemv_argmax_noalloc(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight,
                                   const float *absmax, const float codebook[16], int64_t N,
                                   int64_t K, float *y, int32_t *index, hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_linear_args(x, M, qweight, absmax, codebook, N, K, y, kMaxGemvM);
  if (st != NF4_OK) return st;
  if (!index) return NF4_ERR_NULL;
  if (!aligned16(index)) return NF4_ERR_ALIGN;
  if (nf4::gemv_argmax_workspace_bytes(M, N, K) > kStaticScratchBytes) return NF4_ERR_SCRATCH;
  nf4::CodeTerms ct;
  const int nterm = split_codebook(codebook, ct);
  if (nterm == 0) return NF4_ERR_CODEBOOK;
  void *ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return NF4_ERR_HIP;
  // the arrival counter starts at zero whatever an earlier call left
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream,
                     reinterpret_cast<uint32_t *>(ws), 64);
  e = hipGetLastError();
  if (e != hipSuccess) return NF4_ERR_HIP;
  return from_hip(nf4::launch_gemv_argmax(x, (int)M, qweight, absmax, ct, nterm, N, K, y, index,
                                          ws, stream));
}

nf4_status nf4_gemm(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight, const float *absmax,
                    const float codebook[16], int64_t N, int64_t K, float *y, void *workspace,
                    size_t ws_bytes, hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_linear_args(x, M, qweight, absmax, codebook, N, K, y, kMaxGemmM);
  if (st != NF4_OK) return st;
  const size_t need = nf4::gemm_workspace_bytes(M, N, K);
  if (need > 0 && !workspace) return NF4_ERR_NULL;
  if (need > ws_bytes) return NF4_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return NF4_ERR_ALIGN;
  nf4::CodeTerms ct;
  const int nterm = split_codebook(codebook, ct);
  if (nterm == 0) return NF4_ERR_CODEBOOK;
  return from_hip(nf4::launch_gemm(x, M, qweight, absmax, ct, nterm, N, K, y, workspace,
                                   ws_bytes, stream));
}

// ---------------------------------------------------------------------------
// Asymmetric int4, groups of 128 along K: w = (q - z) * s.

size_t nf4_awq_params_bytes(int64_t N, int64_t K) {
  if (!awq_shape_ok(N, K)) return 0;
  return (size_t)(N / nf4::kTileRows) * (size_t)nf4::tiles_k(K) * nf4::kAwqParamBytes;
}

size_t nf4_awq_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxGemmM || !awq_shape_ok(N, K) || !nf4::awq_gemm_supported(M, N, K))
    return 0;
  return nf4::awq_gemm_workspace_bytes(M, N, K);
}

nf4_status nf4_awq_pack(const float *W, int64_t N, int64_t K, uint8_t *qweight,
                        uint32_t *params, hipStream_t stream) {
  if (!W || !qweight || !params) return NF4_ERR_NULL;
  if (!awq_shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(qweight) || !aligned16(params)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_awq_pack(W, N, K, qweight, params, stream));
}

nf4_status nf4_awq_repack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                          int64_t N, int64_t K, uint8_t *qweight, uint32_t *params,
                          hipStream_t stream) {
  if (!codes || !scales || !zeros || !qweight || !params) return NF4_ERR_NULL;
  if (!awq_shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(zeros) || !aligned16(qweight) ||
      !aligned16(params))
    return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_awq_repack(codes, scales, zeros, N, K, qweight, params, stream));
}

nf4_status nf4_awq_unpack(const uint8_t *qweight, const uint32_t *params, int64_t N, int64_t K,
                          uint8_t *codes, uint16_t *scales, uint8_t *zeros, hipStream_t stream) {
  if (!codes || !scales || !zeros || !qweight || !params) return NF4_ERR_NULL;
  if (!awq_shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(zeros) || !aligned16(qweight) ||
      !aligned16(params))
    return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_awq_unpack(qweight, params, N, K, codes, scales, zeros, stream));
}

nf4_status nf4_awq_dequant(const uint8_t *qweight, const uint32_t *params, int64_t N, int64_t K,
                           float *W_out, hipStream_t stream) {
  if (!qweight || !params || !W_out) return NF4_ERR_NULL;
  if (!awq_shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(qweight) || !aligned16(params) || !aligned16(W_out)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_awq_dequant(qweight, params, N, K, W_out, stream));
}

nf4_status nf4_gather_columns(const hip_bfloat16 *xb, int64_t M, int64_t K, const int32_t *perm,
                              hip_bfloat16 *x_out_bf16, hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  uint16_t *x_out = reinterpret_cast<uint16_t *>(x_out_bf16);
  if (!x || !perm || !x_out) return NF4_ERR_NULL;
  if (M < 1 || M > kMaxGemmM || K < 8 || K % 8 != 0 || K > kMaxDim || M * K > kMaxElems)
    return NF4_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(perm) || !aligned16(x_out)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_gather_columns(x, M, K, perm, x_out, stream));
}

}  // extern "C"

namespace {
nf4_status check_awq_linear(const uint16_t *x, int64_t M, const uint8_t *qw, const uint32_t *pr,
                            int64_t N, int64_t K, const float *y, int64_t max_m) {
  if (!x || !qw || !pr || !y) return NF4_ERR_NULL;
  if (M < 1 || M > max_m || !awq_shape_ok(N, K)) return NF4_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(qw) || !aligned16(pr) || !aligned16(y)) return NF4_ERR_ALIGN;
  return NF4_OK;
}
nf4_status check_awq_workspace(int64_t M, int64_t N, int64_t K, const void *ws, size_t ws_bytes) {
  if (!nf4::awq_gemm_supported(M, N, K)) return NF4_ERR_SHAPE;
  if (!ws) return NF4_ERR_NULL;
  if (nf4::awq_gemm_workspace_bytes(M, N, K) > ws_bytes) return NF4_ERR_WORKSPACE;
  if (!aligned16(ws)) return NF4_ERR_ALIGN;
  return NF4_OK;
}
}  // namespace

extern "C" {

nf4_status nf4_awq_gemv(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight,
                        const uint32_t *params, int64_t N, int64_t K, float *y, void *workspace,
                        size_t ws_bytes, hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_awq_linear(x, M, qweight, params, N, K, y, kMaxGemvM);
  if (st != NF4_OK) return st;
  if (nf4::awq_gemv_fast_eligible(M, N, K))
    return from_hip(nf4::launch_awq_gemv_fast(x, (int)M, qweight, params, N, K, y, stream));
  // x too long for LDS: the tiled GEMM, which sums x in the workspace
  st = check_awq_workspace(M, N, K, workspace, ws_bytes);
  if (st != NF4_OK) return st;
  return from_hip(nf4::launch_awq_gemm(x, M, qweight, params, N, K, y, workspace, stream));
}

nf4_status nf4_awq_gemv_prefetch(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight,
                                 const uint32_t *params, int64_t N, int64_t K, float *y,
                                 void *workspace, size_t ws_bytes, const uint8_t *next_qweight,
                                 const uint32_t *next_params, int64_t next_N, int64_t next_K,
                                 hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_awq_linear(x, M, qweight, params, N, K, y, kMaxGemvM);
  if (st != NF4_OK) return st;
  nf4::NextMatrix next;
  if (next_qweight != nullptr) {
    if (!next_params) return NF4_ERR_NULL;
    if (!aligned16(next_qweight) || !aligned16(next_params)) return NF4_ERR_ALIGN;
    if (!awq_shape_ok(next_N, next_K)) return NF4_ERR_SHAPE;
    next.qw = next_qweight;
    next.am = reinterpret_cast<const float *>(next_params);
    next.N = next_N;
    next.K = next_K;
  }
  if (nf4::awq_gemv_fast_eligible(M, N, K))
    return from_hip(nf4::launch_awq_gemv_fast(x, (int)M, qweight, params, N, K, y, stream,
                                              next_qweight ? &next : nullptr));
  st = check_awq_workspace(M, N, K, workspace, ws_bytes);
  if (st != NF4_OK) return st;
  return from_hip(nf4::launch_awq_gemm(x, M, qweight, params, N, K, y, workspace, stream));
}

nf4_status nf4_awq_gemm(const hip_bfloat16 *xb, int64_t M, const uint8_t *qweight,
                        const uint32_t *params, int64_t N, int64_t K, float *y, void *workspace,
                        size_t ws_bytes, hipStream_t stream) {
  const uint16_t *x = bf16_bits(xb);
  nf4_status st = check_awq_linear(x, M, qweight, params, N, K, y, kMaxGemmM);
  if (st != NF4_OK) return st;
  st = check_awq_workspace(M, N, K, workspace, ws_bytes);
  if (st != NF4_OK) return st;
  return from_hip(nf4::launch_awq_gemm(x, M, qweight, params, N, K, y, workspace, stream));
}

}  // extern "C"
