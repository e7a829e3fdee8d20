// Device building blocks shared by the gfx950 kernels of the block-scaled FP8
// GEMM: the FP8 MFMA that forms one 128-wide group's partial, operand
// fragments (from global memory or from swizzled LDS tiles), the per-group
// scale fold, and output conversion / stores.
//
// Operation (FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul for
// Hopper", section "Description"):
//   C[m,n] = sum_g a_s[m,g] * b_s[n/128,g] * sum_{k in g} A[m,k] * B[n,k]
// FP32 accumulation throughout, one rounding to the output type (section
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
// Swizzled LDS tiles (generic kernel).  A tile holds one 128-byte group
// slice per row; 16-byte chunk c of row r sits at slot r*128 + 16*(c ^ s(r))
// with s(r) = (r' ^ (r' >> 3)) & 7, r' = r mod 16.
//  - The direct-to-LDS loads fill slots linearly (lane t of a 1 KB load ->
//    slot t: 8 adjacent lanes cover one row, reading its 128 bytes).
//  - A fragment read (lane l: row l & 15 of a 16-row block, chunks 2h and
//    2h+1 with h = l >> 4, i.e. bytes 32h .. 32h+31 of the group) touches
//    LDS banks without conflicts: the SQ_LDS_BANK_CONFLICT counter reads zero
//    for this pattern on gfx950, and ds_read_b128 runs ~1.5x faster than
//    with a linear (fragment-major) or row-plus-row/8 layout, which count 4
//    conflict cycles per read.
// Both MFMA operands of the generic kernel are read this way, so their K
// order (lane group h holds bytes 32h .. 32h+31) matches.
__device__ __forceinline__ int swz_row(int r) {
  const int rr = r & 15;
  return (rr ^ (rr >> 3)) & 7;
}

__device__ __forceinline__ v8i load_frag_lds_sw(const uint8_t* tile, int row0, int lane) {
  const int r = row0 + (lane & 15), h = lane >> 4, s = swz_row(r);
  const uint8_t* p = tile + 128 * r;
  const v4i lo = *reinterpret_cast<const v4i*>(p + 16 * ((2 * h) ^ s));
  const v4i hi = *reinterpret_cast<const v4i*>(p + 16 * ((2 * h + 1) ^ s));
  return join(lo, hi);
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

// Direct global -> LDS loads through a buffer resource: lane l's `size`
// bytes, read at base + voff + soff, land at lds + l * size; `lds` and `soff`
// are wave-uniform.  The resource spans 4 GiB from `base` with no stride;
// callers keep every access inside its operand (rows are clamped), so the
// range check never decides a result.  A tile base in SGPRs plus 32-bit
// per-lane offsets replaces 64-bit per-lane addresses.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
// A resource of `bytes` bytes: loads at or past the end (voff, not soff,
// counts) read zeros and touch no memory.
__device__ __forceinline__ buf_rsrc make_rsrc_n(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(buf_rsrc r, uint32_t voff, int soff, lds_u8* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voff, soff, 0, 0);
}
// The same with the non-temporal hint, for bytes that one workgroup reads
// once and no later workgroup reads again.
__device__ __forceinline__ void lds_dma16_nt(buf_rsrc r, uint32_t voff, int soff, lds_u8* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voff, soff, 0, 2);
}
__device__ __forceinline__ void lds_dma4(buf_rsrc r, uint32_t voff, int soff, lds_u8* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, (int)voff, soff, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory loads of this
// wave are outstanding and leaves the other counters alone (gfx9 layout:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_only(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

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
