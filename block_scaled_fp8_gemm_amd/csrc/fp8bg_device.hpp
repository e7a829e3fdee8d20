// Device building blocks shared by the gfx950 kernels of the block-scaled FP8
// GEMM: the FP8 MFMA that forms one 128-wide group's partial, operand
// fragments (from global memory or from swizzled LDS tiles), the per-group
// scale fold, and output conversion / stores.
//
// Operation (FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul for
// Hopper", section "Description"):
//   C[m,n] = sum_g a_s[m,g] * b_s[n/128,g] * sum_{k in g} A[m,k] * B[n,k]
// Every path accumulates in FP32 and casts to the output dtype (section
// "Numerical safety").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fbg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;  // K elements (= bytes) per scale group
constexpr int kWave = 64;

enum OutKind { kOutBF16 = 0, kOutFP16 = 1, kOutFP32 = 2 };

// ---------------------------------------------------------------------------
// One 16x16 output block of one group: P[i][j] = sum_{k<128} X[i][k] * Y[j][k]
// on v_mfma_f32_16x16x128_f8f6f4 (format code 0 = FP8 E4M3 for both operands;
// scale operands 0 select the unscaled instruction).  The accumulator input is
// zero, so P is a fresh FP32 partial of exactly one group.
//
// Fragment layout (both operands alike, so the 128-term dot pairs X[i][k]
// with Y[j][k] whatever order the unit sums in): lane l holds row (l & 15) of
// its 16-row block; with h = l >> 4, dwords 0..3 hold bytes [16h, 16h+16) and
// dwords 4..7 hold bytes [64+16h, 64+16h+16) of that row's group slice.
// Result: lane l, element r holds P[4*(l>>4) + r][l & 15].
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_group(const v8i& x, const v8i& y) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i join(const v4i& lo, const v4i& hi) {
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Fragment of a 16-row block straight from global memory.  `row_ptr` points
// at this lane's row (already clamped in range) at the group's first byte.
__device__ __forceinline__ v8i load_frag_global(const uint8_t* row_ptr, int lane) {
  const int h = lane >> 4;
  const v4i lo = *reinterpret_cast<const v4i*>(row_ptr + 16 * h);
  const v4i hi = *reinterpret_cast<const v4i*>(row_ptr + 64 + 16 * h);
  return join(lo, hi);
}

// ---------------------------------------------------------------------------
// LDS tiles: one group slice per row, 128 bytes = 8 chunks of 16 bytes.
// Chunk c of row r is stored at slot 8r + (c ^ swz(r)).  swz is a bijection
// on every 8 consecutive rows and keeps even and odd rows apart, so the 16
// lanes that read chunk c of 16 consecutive rows touch 16 distinct 16-byte
// bank groups (64 banks) and every 8 of them distinct groups (32 banks).
// Writers fill slots linearly (thread t -> slot t), which is conflict-free,
// and read global chunk (t & 7) ^ swz(t >> 3) of row t >> 3: 8 consecutive
// threads cover one 128-byte row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return (r + (r >> 3)) & 7; }

__device__ __forceinline__ v8i load_frag_lds(const uint8_t* tile, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int h = lane >> 4;
  const int s = swz(r);
  const v4i lo = *reinterpret_cast<const v4i*>(tile + 128 * r + 16 * (h ^ s));
  const v4i hi = *reinterpret_cast<const v4i*>(tile + 128 * r + 16 * ((h + 4) ^ s));
  return join(lo, hi);
}

// Global source of LDS slot t of a tile whose rows start at global row `row0`
// (rows at or past `rows` are clamped to the last valid row: they only feed
// outputs that are never stored).
__device__ __forceinline__ const uint8_t* slot_src(const uint8_t* X, int64_t ld, int row0, int rows,
                                                   int t, int k0) {
  const int r = t >> 3;
  int gr = row0 + r;
  gr = gr < rows ? gr : rows - 1;
  const int c = (t & 7) ^ swz(r);
  return X + (int64_t)gr * ld + k0 + 16 * c;
}

// ---------------------------------------------------------------------------
// Output conversion (round to nearest even) and stores.
// ---------------------------------------------------------------------------
template <int OUT> struct Out;
template <> struct Out<kOutBF16> {
  typedef __bf16 T;
  static __device__ __forceinline__ T cvt(float x) { return (__bf16)x; }
};
template <> struct Out<kOutFP16> {
  typedef _Float16 T;
  static __device__ __forceinline__ T cvt(float x) { return (_Float16)x; }
};
template <> struct Out<kOutFP32> {
  typedef float T;
  static __device__ __forceinline__ T cvt(float x) { return x; }
};

// Stores C[row][n .. n+count) from v[0 .. count), count <= 4.  `vec` says the
// four addresses are in range and aligned for one vector store.
template <int OUT>
__device__ __forceinline__ void store4(void* C, int64_t idx, const v4f& v, int count, bool vec) {
  typedef typename Out<OUT>::T T;
  T* p = reinterpret_cast<T*>(C) + idx;
  if (vec && count >= 4) {
    if constexpr (OUT == kOutFP32) {
      *reinterpret_cast<v4f*>(p) = v;
    } else {
      typedef T T4 __attribute__((ext_vector_type(4)));
      T4 o;
      o[0] = Out<OUT>::cvt(v[0]); o[1] = Out<OUT>::cvt(v[1]);
      o[2] = Out<OUT>::cvt(v[2]); o[3] = Out<OUT>::cvt(v[3]);
      *reinterpret_cast<T4*>(p) = o;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < count) p[r] = Out<OUT>::cvt(v[r]);
  }
}

template <int OUT>
__device__ __forceinline__ void store1(void* C, int64_t idx, float v) {
  reinterpret_cast<typename Out<OUT>::T*>(C)[idx] = Out<OUT>::cvt(v);
}

// ---------------------------------------------------------------------------
// Workgroup -> tile mapping.  Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup i runs on XCD i % 8), each with its own L2.  xcd_remap
// gives every XCD a contiguous run of logical tile ids, so that tiles which
// share operand rows (neighbours in the raster below) share an L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total / kXcds, rem = total % kXcds;
  const int x = bid % kXcds, i = bid / kXcds;
  return x * q + (x < rem ? x : rem) + i;
}

// Grouped raster: tiles are walked column by column inside bands of
// `band` tile-rows, so consecutive tiles reuse the same B columns and the
// band's A rows.
__device__ __forceinline__ void raster(int lid, int tiles_m, int tiles_n, int band, int& tm, int& tn) {
  const int per_band = band * tiles_n;
  const int b = lid / per_band;
  const int first = b * band;
  const int rows = (tiles_m - first) < band ? (tiles_m - first) : band;
  const int w = lid - b * per_band;
  tm = first + w % rows;
  tn = w / rows;
}

}  // namespace fbg
