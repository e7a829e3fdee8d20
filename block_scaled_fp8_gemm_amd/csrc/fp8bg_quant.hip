// gfx950 kernels of the operand quantisers.  First the per-token 1x128
// activation quantiser, the producer of the GEMM's A and a_s:  bf16 x [M,K]
// ->  OCP E4M3 codes A [M,K] and fp32 scales a_s [M, K/128]; then the
// 128x128 weight-block quantiser (below), the producer of B and b_s.  (FlagGems-vllm PR #693, "feat: optimize w8a8 block
// fp8 matmul for Hopper", section "Description": per-token FP8 E4M3
// activations with de-quant scales.)
//
//   a_s[m,g] = max(max_{k in group g} |x[m,k]|, 1e-12) / 448
//   A[m,k]   = E4M3 round-to-nearest-even of clamp(x[m,k] / a_s[m,g], -448, 448)
//
// 448 is E4M3's largest finite value.  The scale is an IEEE fp32 division;
// the codes are those of the IEEE fp32 quotients x / a_s.  The quotient is
// formed as y = 1/a_s (one correctly rounded division per group), q = x*y,
// then one correction step q' = fma(fma(-q, a_s, x), y, q) (Markstein's),
// with x's sign: 3 VALU operations instead of a full division per element
// (the division sequence took a fifth of the kernel's time).  For every
// possible pair of a bf16 x and a bf16 group maximum (about 1.07e9 pairs)
// q' has the same E4M3 code as x / a_s; the quotients differ only below
// 2^-80, where both codes are zero of x's sign.
//
// HBM-bound: 2 bytes read and 1 byte written per element, 4 bytes per
// 128-wide group.  With K % 128 == 0 the groups are contiguous in memory, so
// the matrix is a flat run of M*K/128 groups; a wave takes kQuads runs of 4
// consecutive groups (16 lanes per group, 8 elements = one 16-byte load per
// lane), issues every load before any arithmetic, and writes 8 codes per lane
// with one 8-byte store.  The group maximum is a 16-lane butterfly.
#include "fp8bg_internal.h"

namespace fbg {

namespace {

constexpr int kQuads = 2;  // 4-group runs per wave

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Four fp32 values -> four E4M3 codes in one dword (byte i = value i), by the
// gfx950 conversion instruction (OCP E4M3, round to nearest even).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Streaming accesses: the input is read once and the codes written once, so
// both carry the non-temporal hint (activation quantiser 16384 x 4096: 38.9
// -> 35.7 us, interleaved runs).  The weight quantiser takes the hint on its
// stores only (4096 x 4096: 14.1 -> 10.5 us); on its loads, 256-byte block
// rows read 16 to a wave, the hint cost 13% (10.6 -> 12.0 us).
__device__ __forceinline__ uint4 ldg_stream(const uint16_t* p) {
  typedef unsigned int U4 __attribute__((ext_vector_type(4)));
  const U4 t = __builtin_nontemporal_load(reinterpret_cast<const U4*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void stg_stream(uint8_t* p, uint32_t lo, uint32_t hi) {
  typedef unsigned int U2 __attribute__((ext_vector_type(2)));
  const U2 t = {lo, hi};
  __builtin_nontemporal_store(t, reinterpret_cast<U2*>(p));
}

__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                       float* __restrict__ a_s, int64_t groups) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4, part = lane & 15;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  uint4 raw[kQuads];
#pragma unroll
  for (int u = 0; u < kQuads; ++u) {
    const int64_t g = (wave * kQuads + u) * 4 + sub;
    raw[u] = g < groups ? ldg_stream(x + g * 128 + part * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kQuads; ++u) {
    const int64_t g = (wave * kQuads + u) * 4 + sub;
    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // Maximum over the group's 16 lanes (lanes 16*sub .. 16*sub + 15).
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const float s = fmaxf(amax, 1e-12f) / 448.0f;
    const float y = 1.0f / s;
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = v[i] * y;
      const float e = __builtin_fmaf(-t, s, v[i]);
      r[i] = clamp448(__builtin_copysignf(__builtin_fmaf(e, y, t), v[i]));
    }
    if (g < groups) {
      stg_stream(q + g * 128 + part * 8, e4m3x4(r[0], r[1], r[2], r[3]), e4m3x4(r[4], r[5], r[6], r[7]));
      if (part == 0) a_s[g] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Weight quantisation, the producer of B and b_s: w [N,K] bf16 -> E4M3 codes
// B [N,K] and one fp32 scale per 128 x 128 block, b_s [ceil(N/128), K/128]
// (section "Description": [block_n, block_k] = [128, 128] weight scales).
//
//   b_s[nb,g] = max(max over the block of |w|, 1e-12) / 448
//   B[n,k]    = E4M3 round-to-nearest-even of clamp(w[n,k] / b_s, -448, 448)
//
// One 256-thread workgroup per block: 16 lanes cover one 256-byte block row,
// so the workgroup reads 16 rows per pass and 8 passes cover the block, all
// 8 loads per lane in flight at once (rows past N read as zero and are not
// stored).  The block maximum is a wave butterfly, then 4 values through LDS;
// the quotient is formed as in the row quantiser (per-block reciprocal and
// one correction step, the same E4M3 codes as the IEEE division).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_blocks(const uint16_t* __restrict__ w, uint8_t* __restrict__ q,
                                                         float* __restrict__ b_s, int N, int K) {
  constexpr int kPasses = 8;
  __shared__ float s_max[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = K / 128;
  const int nb = blockIdx.x / G, g = blockIdx.x - nb * G;
  const int row_in = tid >> 4, col = 128 * g + 8 * (tid & 15);
  uint4 raw[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int n = 128 * nb + 16 * p + row_in;
    raw[p] = n < N ? *reinterpret_cast<const uint4*>(w + (int64_t)n * K + col) : make_uint4(0, 0, 0, 0);
  }
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const uint32_t v4[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v4[i])), fabsf(bf16_hi(v4[i]))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = fmaxf(amax, 1e-12f) / 448.0f;
  const float y = 1.0f / s;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int n = 128 * nb + 16 * p + row_in;
    const uint32_t v4[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = (i & 1) ? bf16_hi(v4[i >> 1]) : bf16_lo(v4[i >> 1]);
      const float t = v * y;
      const float e = __builtin_fmaf(-t, s, v);
      r[i] = clamp448(__builtin_copysignf(__builtin_fmaf(e, y, t), v));
    }
    if (n < N)
      stg_stream(q + (int64_t)n * K + col, e4m3x4(r[0], r[1], r[2], r[3]), e4m3x4(r[4], r[5], r[6], r[7]));
  }
  if (tid == 0) b_s[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_quantize_blocks(const uint16_t* w, uint8_t* q, float* b_s, int N, int K, hipStream_t stream) {
  const int64_t blocks = (int64_t)((N + 127) / 128) * (K / 128);
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quantize_blocks, dim3((unsigned)blocks), dim3(256), 0, stream, w, q, b_s, N, K);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* x, uint8_t* q, float* a_s, int64_t groups, hipStream_t stream) {
  const int64_t waves = (groups + 4 * kQuads - 1) / (4 * kQuads);
  const int64_t blocks = (waves + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, a_s, groups);
  return hipGetLastError();
}

}  // namespace fbg
