// gfx950 kernels of the block-scaled FP8 GEMM and their launchers.
//
//   C[m,n] = sum_g a_s[m,g] * b_s[n/128,g] * sum_{k in g} A[m,k] * B[n,k]
//
// (FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul for Hopper",
// sections "Description" and "Specialized kernels and the optimization
// idea".)  The pages' kernels were Hopper/Triton designs; these are written
// for CDNA4: 64-lane waves, the 16x16x128 FP8 MFMA (one MFMA consumes exactly
// one 128-wide scale group, so its output is the group's fresh partial),
// swizzled LDS tiles, and XCD-aware workgroup placement.
//
// Every kernel computes, per output element, the same FP32 chain
//   acc = 0; for g in its group range: acc = fma(P_g, a_s[m,g] * b_s[n/128,g], acc)
// and casts once (round to nearest even).
#include "fp8bg_device.hpp"
#include "fp8bg_configs.h"
#include "fp8bg_internal.h"

namespace fbg {

// Grouped form of the generic kernel: row tile t (in expert order, expert e
// holding ceil(rows_e / BM) tiles) -> (expert, tile within the expert),
// written to out[0..1] by one wave; out[0] = -1 if t is past the last tile.
// The wave scans the experts' tile counts 64 at a time (offsets clamped into
// [0, M] as everywhere else), so no host step or extra launch is needed.
template <int BM>
__device__ __forceinline__ void find_expert_tile(const int* offsets, int E, int M, int t, int lane, int* out) {
  int carry = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int tiles = 0;
    if (e < E) {
      int lo = offsets[e], hi = offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > M ? M : lo);
      hi = hi < lo ? lo : (hi > M ? M : hi);
      tiles = (hi - lo + BM - 1) / BM;
    }
    int incl = tiles;  // inclusive prefix sum over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int first = carry + incl - tiles;
    const bool mine = tiles > 0 && t >= first && t < first + tiles;
    if (mine) {
      out[0] = e;
      out[1] = t - first;
    }
    if (__any(mine)) return;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) out[0] = -1;
}

// ===========================================================================
// Generic kernel: LDS-staged A and B tiles, STAGES-deep ring, one 128-wide
// group per step.  (The pages' generic tuned GEMM and its GROUP_M raster,
// section "Specialized kernels and the optimization idea".)
//
// Loads go straight from global memory into LDS (buffer_load_dwordx4 ... lds):
// no staging registers and no LDS store instructions.  Every thread issues
// the same LPG loads per group (A images, B images, one a_s load -- the
// group's row scales, or with SCH = 1 a part of a later chunk of them -- and
// one b_s load), so one vmcnt bound says "this wave's loads of group g have
// landed";
// a barrier then makes the whole tile visible.  The one barrier per group
// sits in the group's last row block, once every LDS read of the group has
// been issued: past it, the slot is refilled with the group STAGES ahead,
// and the next group's scales and fragments are read while the last
// block's MFMAs run, so a group starts with its operands in registers.
//
// Operand order: weight rows n on the MFMA's first operand, activation rows
// m on the second, so a lane ends with ONE output row m and 4 consecutive
// columns n of each 16x16 block.  The block's scale a_s[m,g] * b_s[n/128,g]
// is then one value per lane (a wave's columns share one b_s block), the
// a_s of a lane's rows are a few short LDS reads per group, and the epilogue
// stores 4 outputs per lane at once.
//
// Each MFMA writes a fresh FP32 partial; its fold acc = fma(P, s, acc) is
// issued two MFMAs later, in their shadow.
//
// GRP = 1 is the grouped (mixture-of-experts) form: the grid enumerates
// (row tile, column tile) with the row tiles of all experts in expert order,
// each workgroup finds its expert with find_expert_tile, offsets B and b_s to
// that expert's weight, and clamps its rows to the expert's range instead of
// to M.  Everything after the tile's placement is shared with the dense form.
// ===========================================================================
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int SCH, int MID, int OUT, int GRP>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void k_generic(
    const uint8_t* __restrict__ A, const float* __restrict__ a_s, const uint8_t* __restrict__ B,
    const float* __restrict__ b_s, void* __restrict__ C, int M, int N, int K, int band, int vec_ok,
    const int* __restrict__ offsets, int E) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int IB = WM / 16, JB = WN / 16;
  constexpr int A_PER_T = BM * 8 / NT, B_PER_T = BN * 8 / NT;
  constexpr int LPG = A_PER_T + B_PER_T + 2;         // vector-memory loads per group per thread
  // A ring slot holds a group's A and B tiles, its b_s (64 floats) and, with
  // SCH = 0, its row scales a_s (BM floats).
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, S_BYTES = 64 * 4 + (SCH ? 0 : BM * 4 + (NW > BM / 64 ? 64 * 4 : 0));
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES, RING_BYTES = STAGES * STAGE_BYTES;
  // With SCH = 1 the row scales travel in chunks of CH groups per row (CH * 4
  // contiguous bytes of a_s), three chunk buffers deep, outside the ring.  A
  // chunk is NQ load images of 256 bytes (one 4-byte load per lane each), 268
  // bytes apart.  CH = 8 where the workgroups per CU that the LDS allows stay
  // those of the SCH = 0 ring, else 4.
  constexpr int QSTRIDE = 256 + 12;
  constexpr int LDS_CU = 160 * 1024, PER_CU = LDS_CU / (STAGES * (A_BYTES + B_BYTES + 64 * 4 + BM * 4));
  constexpr int CH = LDS_CU / (RING_BYTES + 3 * (BM * 8 / 64) * QSTRIDE) >= PER_CU ? 8 : 4;
  constexpr int NQ = BM * CH / 64, CB_BYTES = SCH ? NQ * QSTRIDE : 0;
  constexpr int NBI = 64 / (CH * IB);                // row classes per load image
  constexpr int RF = 64 * NW / BM;                   // loads of each image per chunk
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile images must split evenly over waves");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must share one b_s block");
  static_assert(BM % 64 == 0 && (!SCH || RF == 1 || RF == 2) && CH % RF == 0, "a chunk's images must split evenly over the waves");
  static_assert(CH * IB <= 64 && 64 % (CH * IB) == 0, "a load image holds whole row classes");
  static_assert(SCH || IB == 2 || IB == 4 || IB == 8, "a lane reads its row scales of a slot as 8 or 16-byte words");
  static_assert(STAGES >= 2 && STAGES <= 8 && LDS_CU / (RING_BYTES + 3 * CB_BYTES) >= PER_CU, "LDS ring must fit in 160 KB");
  static_assert((STAGES - 1) * LPG + CH / RF < 64, "vmcnt counts at most 63 outstanding loads");
  // MID = 1: a group's refill is split at a second barrier in the middle of
  // the group.  By then every wave holds the group's B fragments (read at the
  // previous switch point) and has read the A rows of its first IB/2 row
  // blocks, so the B images, the b_s load and the A images covering those
  // rows (A load i covers rows 64i .. 64i + 63, those of the first half of a
  // wave row when i is even) refill the slot for group g + 2, spread over the
  // next row blocks; only the other A images and the a_s load wait for the
  // switch point.  Issuing all of a group's loads right after one barrier
  // stalls the waves behind the address unit (prefill 288 -> 276 us bf16,
  // 305 -> 294 us fp32, interleaved runs on one box).
  // LATE_REFILL (2- and 3-slot rings): the switch point's refill is issued
  // after the last row block's MFMAs and next-group B fragment reads rather
  // than right after the barrier, so those LDS reads do not queue behind the
  // refill's LDS writes.  Same loads in the same order; the slot is free from
  // the barrier on.  (Interleaved runs: prefill 282.5 -> 279.3 and 278.2 ->
  // 274.8 us bf16, 292.4 -> 288.3 us fp32; MoE 4096 tokens 248.8 -> 240.8
  // us; 3 slots: 1024 x 8192 x 4096 48.1 -> 47.2 us, 4096 x 1536 x 1024
  // 14.29 -> 14.20, MoE 2048 tokens 203.6 -> 201.0.  On the 4-slot 64 x 64
  // tiles at K <= 1024 the later issue cost 1-2%, so they keep the early
  // one.)
  constexpr bool LATE_REFILL = STAGES <= 3;
  constexpr int A_EARLY = MID ? A_PER_T / 2 : 0;
  constexpr int N_MID = MID ? B_PER_T + 1 + A_EARLY : 0;  // loads per wave issued in the group's second half
  static_assert(!MID || (SCH == 1 && STAGES == 2 && IB >= 6 && A_PER_T % 2 == 0 && WM == 64 * NW / 4 && NW == 8),
                "the mid-group refill assumes the 256 x 256 tile's image-to-row-block mapping");

  __shared__ __attribute__((aligned(16))) uint8_t smem[RING_BYTES + 3 * CB_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int G = K / kGroup;
  const int tiles_n = (N + BN - 1) / BN;
  const int nblk = (N + 127) / 128;
  int m0, n0, m_end;  // the tile's first row, first column, and the end of its rows
  if constexpr (GRP) {
    // Grouped: the grid enumerates (row tile t, column tile tn) with t over
    // the experts' row tiles in expert order, ceil(rows_e / BM) per expert.
    __shared__ int sTile[2];
    const int lid = xcd_remap(blockIdx.x, (int)gridDim.x);
    const int t = lid / tiles_n, tn = lid - t * tiles_n;
    if (wave == 0) find_expert_tile<BM>(offsets, E, M, t, lane, sTile);
    __syncthreads();
    const int e = sTile[0];
    if (e < 0) return;  // past the last row tile (uniform over the workgroup)
    int lo = offsets[e], hi = offsets[e + 1];
    lo = lo < 0 ? 0 : (lo > M ? M : lo);
    hi = hi < lo ? lo : (hi > M ? M : hi);
    m0 = lo + sTile[1] * BM;
    m_end = hi;
    n0 = tn * BN;
    B += (int64_t)e * N * K;
    b_s += (int64_t)e * nblk * G;
  } else {
    const int tiles_m = (M + BM - 1) / BM;
    int tm, tn;
    raster(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, band, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    m_end = M;
  }
  const int nb = ((n0 + wn * WN) >> 7) < nblk ? ((n0 + wn * WN) >> 7) : nblk - 1;

  // Per-lane 32-bit source offsets inside the tile's rows (rows past the
  // matrix are clamped to its last row: they feed outputs never stored).
  // Load q (q = i*NW + wave) fills LDS bytes [1024q, 1024q + 1024) of the
  // tile: rows 8q .. 8q+7; lane l writes row 8q + (l >> 3), slot l & 7, so it
  // reads the row's chunk (l & 7) ^ s(row).
  const uint8_t* Atile = A + (int64_t)m0 * K;
  const uint8_t* Btile = B + (int64_t)n0 * K;
  uint32_t aoff[A_PER_T], boff[B_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int r = 8 * (i * NW + wave) + (lane >> 3);
    const int gr = (m0 + r) < m_end ? r : (m_end - 1 - m0);
    aoff[i] = (uint32_t)gr * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ swz_row(r));
  }
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int r = 8 * (i * NW + wave) + (lane >> 3);
    const int gr = (n0 + r) < N ? r : (N - 1 - n0);
    boff[i] = (uint32_t)gr * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ swz_row(r));
  }
  // Row scales, SCH = 1: chunk c (groups CH*c .. CH*c + CH-1 of every tile
  // row) sits in chunk buffer c mod 3.  Row class b (b = wm*16 + r: the IB rows
  // wm*WM + 16*i + r that lane r of the waves in wave row wm needs) is stored
  // as [i][group]; image q holds classes q*NBI .. q*NBI + NBI-1.  An image
  // load (lane l: class q*NBI + l / (CH*IB), row i = (l mod CH*IB) / CH,
  // group l mod CH) reads CH consecutive groups of a row with CH adjacent
  // lanes, so it touches 64/CH short runs of a_s where one load per row and
  // group would touch 64 separate rows.  A lane reads its IB scales of a
  // group CH floats apart; the 268-byte image pitch (67 words, 3 mod 64)
  // keeps the 16 lanes of a read, and of a paired read of rows i and i+1, on
  // different banks.  The group loop issues one image load per wave per
  // group, the next chunk's images spread over the current chunk's CH groups
  // (with RF = 2, two waves load each image).  Loads past the end of a_s read
  // zeros (the resource's size is exact); the values of groups past G are
  // never used.
  const int ch_sub = lane / (CH * IB), ch_i = (lane % (CH * IB)) / CH, ch_grp = lane % CH;
  auto as_off = [&](int q, int c) {  // a_s byte offset of this lane's element of image q of chunk c
    const int b = q * NBI + ch_sub;
    const int row = m0 + (b / 16) * WM + 16 * ch_i + (b % 16);
    const int r = row < m_end ? row : (m_end - 1);
    return (uint32_t)r * (uint32_t)G * 4u + 4u * (uint32_t)(c * CH + ch_grp);
  };
  // Row scales, SCH = 0: a_s of a group staged in its ring slot, transposed:
  // slot (w*16 + r)*IB + i holds row w*WM + 16*i + r, so the IB row scales a
  // lane needs (its row r = l & 15 in each of its wave's row blocks) are
  // contiguous.  Waves w < BM/64 stage slots 64w + lane: one load per row
  // and group.  The other waves (their load keeps every wave's count per
  // group equal) read one scale, the tile's first row's, into a spare 256
  // bytes of the slot: one access instead of 64 more rows.
  const bool s_spare = wave >= BM / 64;
  const int slot = (wave * 64) % BM + lane;
  const int srow = (slot / (16 * IB)) * WM + 16 * (slot % IB) + (slot / IB) % 16;
  const int sr = s_spare ? m0 : ((m0 + srow) < m_end ? (m0 + srow) : (m_end - 1));
  const uint32_t soff = (uint32_t)sr * (uint32_t)G * 4u;
  // b_s of the tile's column blocks (lane l holds block n0/128 + l, clamped to
  // the tile's last block), so the loop issues no scalar-memory loads.
  const int bl = lane < (BN + 127) / 128 ? lane : (BN + 127) / 128 - 1;
  const int bblk = ((n0 >> 7) + bl) < nblk ? ((n0 >> 7) + bl) : (nblk - 1);
  const uint32_t bsoff = (uint32_t)bblk * (uint32_t)G * 4u;

  // LDS destinations are formed in the LDS address space from the array
  // itself (the load writes lane l's bytes at dst + l * size).
  lds_u8* const lds = (lds_u8*)smem;
  lds_u8* const cbuf = lds + RING_BYTES;
  const buf_rsrc rA = make_rsrc(Atile), rB = make_rsrc(Btile), rBs = make_rsrc(b_s);
  const buf_rsrc rAs = make_rsrc_n(a_s, (uint32_t)M * (uint32_t)G * 4u);
  (void)ch_sub; (void)ch_i; (void)soff;
  // Group g's tiles, b_s and (SCH = 0) a_s into ring slot st; with SCH = 1,
  // part g mod CH of chunk g / CH + 1 (its images (g mod CH) * BM/64 ..)
  // instead of a_s: by the time group CH * (g / CH + 1) is waited for, every
  // part of its chunk has landed.
  // MID: load j of the mid-group part (B images, b_s, even A images).
  auto issue_mid = [&](int g, int st, int j) {
    lds_u8* base = lds + st * STAGE_BYTES;
    if (j < B_PER_T) lds_dma16(rB, boff[j], g * kGroup, base + A_BYTES + 1024 * (j * NW + wave));
    else if (j == B_PER_T) lds_dma4(rBs, bsoff, 4 * g, base + A_BYTES + B_BYTES);
    else {
      const int i = 2 * (j - B_PER_T - 1);
      lds_dma16(rA, aoff[i], g * kGroup, base + 1024 * (i * NW + wave));
    }
  };
  auto issue = [&](int g, int st) {
    lds_u8* base = lds + st * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i)
      if (!MID || (i & 1)) lds_dma16(rA, aoff[i], g * kGroup, base + 1024 * (i * NW + wave));
    if constexpr (!MID) {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) lds_dma16(rB, boff[i], g * kGroup, base + A_BYTES + 1024 * (i * NW + wave));
    }
    if constexpr (SCH) {
      const int c = g / CH + 1, q = (g % CH) * (BM / 64) + wave % (BM / 64);
      lds_dma4(rAs, as_off(q, c), 0, cbuf + (c % 3) * CB_BYTES + q * QSTRIDE);
    } else {
      lds_dma4(rAs, soff, 4 * g, base + A_BYTES + B_BYTES + 64 * 4 + (s_spare ? 4 * BM : 4 * ((wave * 64) % BM)));
    }
    if constexpr (!MID) lds_dma4(rBs, bsoff, 4 * g, base + A_BYTES + B_BYTES);
  };
  // Both parts (the prologue's full groups).
  auto issue_all = [&](int g, int st) {
    if constexpr (MID) {
#pragma unroll
      for (int j = 0; j < N_MID; ++j) issue_mid(g, st, j);
    }
    issue(g, st);
  };

  v4f acc[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // fold(a, P, s): a = fma(P, s, a) elementwise, the group's contribution.
  auto fold = [](v4f& a, const v4f& P, float s) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = __builtin_fmaf(P[r], s, a[r]);
  };
  // Each MFMA's partial is folded two MFMAs later (pp2: the partial of the
  // MFMA before last, pp1: of the last one, with their scales), so a fold
  // never waits for an MFMA still in the pipe.  The last two partials of a
  // group are folded in the next group (zero partials and zero scales before
  // the first group).
  v4f pp1 = v4f{0.f, 0.f, 0.f, 0.f}, pp2 = pp1;
  float sc1 = 0.f, sc2 = 0.f;

  // Head of a group: what its first MFMAs need, read from its LDS slot --
  // the lane's row scales, the b_s of the wave's columns, the first A
  // fragment (the B fragments are read one by one by the caller).
  float as[IB], bsv;
  v8i bf[JB], af;
  auto read_head = [&](int st, int g, float* as_o, float& bsv_o, v8i& af_o) {
    const uint8_t* base = smem + st * STAGE_BYTES;
    bsv_o = reinterpret_cast<const float*>(base + A_BYTES + B_BYTES)[nb - (n0 >> 7)];
    if constexpr (SCH) {
      const int b = wm * 16 + (lane & 15);
      const float* cs = reinterpret_cast<const float*>(smem + RING_BYTES + ((g / CH) % 3) * CB_BYTES +
                                                       (b / NBI) * QSTRIDE + (b % NBI) * CH * IB * 4) + g % CH;
#pragma unroll
      for (int i = 0; i < IB; ++i) as_o[i] = cs[CH * i];
    } else {
      if constexpr (IB >= 4) {
        const v4f* ps = reinterpret_cast<const v4f*>(base + A_BYTES + B_BYTES + 64 * 4) + (wm * 16 + (lane & 15)) * IB / 4;
#pragma unroll
        for (int q = 0; q < IB / 4; ++q) {
          const v4f v = ps[q];
#pragma unroll
          for (int r = 0; r < 4; ++r) as_o[4 * q + r] = v[r];
        }
      } else {  // two row blocks per wave: the lane's two scales as one 8-byte word
        typedef float v2f __attribute__((ext_vector_type(2)));
        const v2f v = reinterpret_cast<const v2f*>(base + A_BYTES + B_BYTES + 64 * 4)[wm * 16 + (lane & 15)];
        as_o[0] = v[0];
        as_o[1] = v[1];
      }
    }
    af_o = load_frag_lds_sw(base, wm * WM, lane);
  };
  auto read_b = [&](int st, int j) {
    return load_frag_lds_sw(smem + st * STAGE_BYTES + A_BYTES, wn * WN + 16 * j, lane);
  };

  // Slot s holds group s, s + STAGES, ...  Every slot is filled up front;
  // group g's slot is refilled with group g + STAGES at g's switch point.
  // Refills past the last group load the last group again into a slot no
  // wave reads any more: the loop body stays a single basic block (a branch
  // there lets the compiler sink every fold below it), and the number of
  // loads in flight is the same at every switch point.
  auto grp = [&](int g) { return g < G ? g : G - 1; };
  // SCH = 1: chunk 0 up front, wave w loading images j*NW + w.
  if constexpr (SCH) {
#pragma unroll
    for (int j = 0; j < CH / RF; ++j) lds_dma4(rAs, as_off(j * NW + wave, 0), 0, cbuf + (j * NW + wave) * QSTRIDE);
  }
#pragma unroll
  for (int p = 0; p < STAGES; ++p) issue_all(grp(p), p);
  // Chunk 0 and group 0 have landed once at most the later slots' loads are
  // outstanding.
  __builtin_amdgcn_s_waitcnt(vmcnt_only((STAGES - 1) * LPG));
  __builtin_amdgcn_s_barrier();
  read_head(0, 0, as, bsv, af);
#pragma unroll
  for (int j = 0; j < JB; ++j) bf[j] = read_b(0, j);

  // Grouped mode: a wave whose rows all lie past the expert's last row (an
  // expert of at most 128 tokens in a 256-row tile leaves the second wave row
  // idle) issues no MFMAs.  It still loads its share of every group and takes
  // every barrier, in the same order and with the same waits as the full
  // loop, so the ring's accounting is unchanged; its accumulators stay zero
  // and its rows are never stored.  The other wave on its SIMD then has the
  // matrix core to itself (4096 tokens over 256 experts: 257.5 -> 248.2 us;
  // 2048 tokens in 128 x 256 tiles: 210.0 -> 204.6 us).
  bool run_full = true;
  if constexpr (GRP) {
    static_assert(!MID, "grouped tiles use no mid-group refill");
    if (m0 + wm * WM >= m_end) {
      run_full = false;
      for (int g = 0; g < G; ++g) {
        const int st = g % STAGES;
        __builtin_amdgcn_s_waitcnt(vmcnt_only((STAGES - 2) * LPG) & ~(15 << 8));
        __builtin_amdgcn_s_barrier();
        issue(grp(g + STAGES), st);
      }
    }
  }
  if (run_full)
  for (int g = 0; g < G; ++g) {
    const int st = g % STAGES, nst = (g + 1) % STAGES;
    const uint8_t* base = smem + st * STAGE_BYTES;
    float as_n[IB], bsv_n;
    v8i af_n;
    float sc = 0.f;
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      v8i af_next;
      if (i + 1 < IB) af_next = load_frag_lds_sw(base, wm * WM + 16 * (i + 1), lane);
      sc = as[i] * bsv;
      if (i == IB / 2) __builtin_amdgcn_s_setprio(0);
      if constexpr (MID) {
        // Mid-group barrier: the slot's B region and the A rows of the first
        // IB/2 row blocks are no longer read by any wave; their refill for
        // group g + 2 goes out over row blocks IB/2 .. IB-2.
        if (i == IB / 2) __builtin_amdgcn_s_barrier();
        if (i >= IB / 2 && i <= IB - 2) {
          constexpr int NB = IB / 2 - 1;
#pragma unroll
          for (int j = 0; j < N_MID; ++j)
            if (j * NB / N_MID == i - IB / 2) issue_mid(grp(g + STAGES), st, j);
        }
      }
      if (i == IB - 1) {
        // Switch point: every LDS read of this group's slot has been issued.
        // Wait for them and for group g+1's loads (the later groups' loads
        // may stay outstanding), so that past the barrier g+1's tile is
        // visible and no wave reads slot st any more: refill it with group
        // g + STAGES, and read g+1's head while this block's MFMAs run.
        // (After the last group the head reads fetch a stale slot; the
        // values are never used.)
        __builtin_amdgcn_s_waitcnt(vmcnt_only((STAGES - 2) * LPG + N_MID) & ~(15 << 8));
        __builtin_amdgcn_s_barrier();
        // Wave priority 1 from here to the middle of the next group, 0 in its
        // second half: of the two waves sharing a SIMD, one that has fallen
        // behind gets the issue slots, so both reach the next barrier closer
        // together (prefill 267 -> 260 us).
        __builtin_amdgcn_s_setprio(1);
        if constexpr (!LATE_REFILL) issue(grp(g + STAGES), st);
        read_head(nst, g + 1, as_n, bsv_n, af_n);
      }
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        // MFMA, then the fold of the partial two MFMAs back (block k - 2 in
        // the order k = i*JB + j, wrapping into the previous group), in this
        // order: left alone, the scheduler pulls each MFMA's own fold up next
        // to it (to free registers early) and every fold stalls on its MFMA.
        const v4f p = mfma_group(bf[j], af);
        __builtin_amdgcn_sched_barrier(0);
        const int k2 = (i * JB + j + IB * JB - 2) % (IB * JB);
        fold(acc[k2 / JB][k2 % JB], pp2, sc2);
        // In the last block, B fragment j of the next group replaces this
        // one once its MFMA has been issued.
        if (i == IB - 1) bf[j] = read_b(nst, j);
        __builtin_amdgcn_sched_barrier(0);
        pp2 = pp1;
        sc2 = sc1;
        pp1 = p;
        sc1 = sc;
      }
      if (i + 1 < IB) af = af_next;
      if constexpr (LATE_REFILL) {
        if (i == IB - 1) issue(grp(g + STAGES), st);
      }
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) as[i] = as_n[i];
    bsv = bsv_n;
    af = af_n;
  }
  fold(acc[(IB * JB - 2) / JB][(IB * JB - 2) % JB], pp2, sc2);
  fold(acc[IB - 1][JB - 1], pp1, sc1);
  // The refills issued past the last group must land before the workgroup
  // ends and its LDS is handed to another.
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

  // Block (i, j): lane holds row m = 16*i + (lane & 15), columns
  // n = 16*j + 4*(lane >> 4) + r, r = 0..3, of the wave's sub-tile.
  const int m_l = m0 + wm * WM + (lane & 15);
  const int n_l = n0 + wn * WN + 4 * (lane >> 4);
  if ((vec_ok & 2) && n0 + BN <= N) {
    // Whole-row stores through LDS (every column of the tile in range, C rows
    // 16-byte aligned): each wave writes its 16 x WN slab of converted
    // outputs per 16-row block to LDS, then stores the slabs back 16
    // contiguous bytes per lane, so one store instruction writes whole
    // 64-128-byte row segments instead of 16 rows x 8 bytes.  As many row
    // blocks as the LDS ring holds go in one phase (all of them for bf16 and
    // fp16 tiles), with one barrier between a phase's writes and its reads.
    // Slab rows are padded by 16 bytes: with an unpadded 128-byte pitch the 16
    // rows a write instruction touches would all start in the same LDS bank.
    typedef typename Out<OUT>::T T;
    constexpr int ES = (int)sizeof(T), ROWB = WN * ES, ROWP = ROWB + 16, SLAB = 16 * ROWP;
    constexpr int CHUNKS = 16 * ROWB / 16, PER_LANE = (CHUNKS + 63) / 64;
    constexpr int FIT = (STAGES * STAGE_BYTES) / (NW * SLAB);
    constexpr int PB = FIT < IB ? FIT : IB;  // row blocks per phase
    static_assert(PB >= 1, "one row block of slabs must fit in the LDS ring");
#pragma unroll
    for (int i0 = 0; i0 < IB; i0 += PB) {
      __syncthreads();  // the last group's (or the previous phase's) LDS reads are done
#pragma unroll
      for (int ii = 0; ii < PB; ++ii) {
        if (i0 + ii >= IB) break;
        uint8_t* slab = smem + (ii * NW + wave) * SLAB;
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          T* d = reinterpret_cast<T*>(slab + (lane & 15) * ROWP) + 16 * j + 4 * (lane >> 4);
          if constexpr (OUT == kOutFP32) {
            *reinterpret_cast<v4f*>(d) = acc[i0 + ii][j];
          } else {
            typedef T T4 __attribute__((ext_vector_type(4)));
            T4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = Out<OUT>::cvt(acc[i0 + ii][j][r]);
            *reinterpret_cast<T4*>(d) = o;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int ii = 0; ii < PB; ++ii) {
        if (i0 + ii >= IB) break;
        const uint8_t* slab = smem + (ii * NW + wave) * SLAB;
#pragma unroll
        for (int t = 0; t < PER_LANE; ++t) {
          const int q = t * 64 + lane;
          const int row = q / (ROWB / 16), cb = (q % (ROWB / 16)) * 16;
          const int m = m0 + wm * WM + 16 * (i0 + ii) + row;
          // Non-temporal stores: C is written once and not read back here.
          // (Against plain stores, interleaved runs: 184x4096x256 3.93 ->
          // 3.56 us, 264x4096x256 4.89 -> 4.33, 512x8192x1024 11.87 ->
          // 10.64, 1024x8192x1024 19.1 -> 16.4, prefill fp32 299 -> 290,
          // prefill bf16 unchanged; on the skinny kernel's small outputs the
          // same hint was slower, 4.77 -> 4.88 us at 64x512x4096.)
          if ((CHUNKS % 64 == 0 || q < CHUNKS) && m < m_end)
            __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(slab + row * ROWP + cb),
                                        reinterpret_cast<v4i*>(reinterpret_cast<uint8_t*>(C) +
                                                               ((int64_t)m * N + n0 + wn * WN) * ES + cb));
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int m = m_l + 16 * i, n = n_l + 16 * j;
      const int cnt = (N - n) < 4 ? (N - n) : 4;
      if (m < m_end && cnt > 0) store4<OUT>(C, (int64_t)m * N + n, acc[i][j], cnt, vec_ok);
    }
}

// ===========================================================================
// Building blocks of the skinny kernels.
//
// skinny_tile: this wave's FP32 partials of a workgroup tile of NB16 x MB16
// 16x16 blocks (weight rows pb, activation rows pa with their a_s rows pas,
// the tile's b_s block row pbs) over its chunks of the group range
// [g_lo, g_hi).  Every wave loads its own B and A fragments -- through its
// own LDS staging area (DMA = 1) or straight into registers -- all loads of
// a chunk of GPW groups in flight at once and the next chunk prefetched
// while the current one is computed.  The KW waves of a workgroup split the
// range: wave kw takes chunks kw, kw+KW, ...
//
// skinny_reduce: sums the KW waves' partials through LDS in the fixed order
// kw = 0..KW-1; wave w then owns blocks b with b % KW == w.
// ===========================================================================
// Single-stage tiles of one 16-row activation block and 4 groups per wave
// stage their scales through LDS too (skinny_tile's sscl, 80 floats per
// wave, which the kernel provides exactly when this holds).
constexpr bool skinny_scales_in_lds(int DMA, int ONE, int MB16, int GPW, int KFIX) {
  return DMA && ONE != 0 && MB16 == 1 && GPW == 4 && KFIX == 0;
}

template <int NB16, int MB16, int KW, int GPW, int KFIX, int DMA = 0, int ONE = 0>
__device__ __forceinline__ void skinny_tile(const uint8_t* const* pb, const uint8_t* const* pa,
                                            const float* const* pas, const float* pbs, int g_lo, int g_hi, int kw,
                                            int lane, v4f (&acc)[NB16][MB16],
                                            const uint32_t (*pd)[2] = nullptr, const buf_rsrc* rsc = nullptr, uint8_t* stage0 = nullptr,
                                            uint8_t* stage1 = nullptr, int arows = 8, float* sscl = nullptr,
                                            const buf_rsrc* rss = nullptr, uint32_t sc_row_off = 0) {
  struct Chunk {
    v8i bf[GPW][NB16];
    v8i af[GPW][MB16];
    float as[GPW][MB16];
    float bs[GPW];
  };
  // Chunk c of this wave: groups g_lo + (c*KW + kw)*GPW + u, u < GPW.  Only
  // chunks with at least one group in range are loaded; inside the last one,
  // groups past the range are clamped (never computed).  Loads carry no
  // per-group condition, so the compiler counts outstanding loads exactly
  // and waits only for the chunk about to be used.
  // DMA = 1: the fragments travel through this wave's LDS staging areas
  // instead (stage0 with register buffer b0, stage1 with b1: two arrays, so
  // the compiler sees that reading one does not wait for loads into the
  // other; block b of group u -- weight blocks first, then activation blocks
  // -- at u*NBK + b, 2 KB each, in the generic kernel's swizzled row layout).  Eight adjacent lanes then read
  // one row's 128-byte group slice, so a load reaches the L1 as 64-byte
  // accesses; a fragment load straight into registers reads 16 rows with
  // 16 adjacent lanes and costs one access per lane.  pd[b][q] is this
  // lane's offset, in resource rsc[b < NB16 ? 0 : 1], of rows 8q .. 8q+7 of
  // block b (row 8q + lane/8 at its swizzled chunk).  The loads' completion
  // is waited for by count: at most the next chunk's 2*NBK tile loads per
  // group may stay in flight (the scale loads issued after them can only
  // make this wait longer, never shorter).
  constexpr int NBK = NB16 + MB16, LPC = GPW * 2 * NBK;
  // Single-stage tiles of one 16-row activation block and 4 groups per wave
  // stage their scales too: one 4-byte-per-lane DMA brings the 16 rows x 4
  // groups of a_s (lane l: row l / 4, group l % 4, from the 16-byte run of
  // the row's 4 consecutive groups) and one more the 4 groups of b_s, into
  // sscl, in place of 8 scattered loads per wave (the 16x16 single-stage
  // tile at 64x512x4096: 5.63 -> 5.35 us; the 8-row tile unchanged).
  constexpr bool SCL = skinny_scales_in_lds(DMA, ONE, MB16, GPW, KFIX);
  auto load = [&](Chunk& ch, int c, uint8_t* stage) {
    const int g0 = g_lo + (c * KW + kw) * GPW;
    if constexpr (DMA && ONE != 0) {
      // Single-stage tiles issue all of a chunk's weight-row loads (from
      // HBM) before its activation-row loads (mostly L2 hits), rather than
      // group by group (decode 64x512x4096: 4.91 -> 4.84 us; the 16x16 tile
      // 5.30 -> 5.10 us; 32x512x4096 4.83 -> 4.72 us; interleaved runs; the
      // same order in the two-slot tiles measured no different).
      // Weight rows carry the non-temporal hint: the few workgroups that
      // share a weight tile (its m-tiles, on one XCD) read it at about the
      // same time, and nothing reads it later.  (Decode 64x512x4096: 4.93 ->
      // 4.78 us; the same hint on the activation rows, which every n-tile
      // re-reads, 6.2 us.)  With ONE == 2 an activation block holds 8 rows,
      // of which the lanes of the tile's arows real rows load theirs; the
      // other rows in LDS stay stale and feed only MFMA rows that are never
      // stored.
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
          const int g = (g0 + u) < g_hi ? (g0 + u) : (g_hi - 1);
          const int k0 = g * kGroup;
          lds_u8* base = (lds_u8*)(stage + u * NBK * 2048);
#pragma unroll
          for (int b = 0; b < NBK; ++b)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              if (b < NB16) {
                if (pass == 0) lds_dma16_nt(rsc[0], pd[b][q], k0, base + b * 2048 + q * 1024);
              } else if (pass == 1) {
                if (ONE == 2) {
                  if (q == 0 && (lane >> 3) < arows) lds_dma16(rsc[1], pd[b][0], k0, base + b * 2048);
                } else {
                  lds_dma16(rsc[1], pd[b][q], k0, base + b * 2048 + q * 1024);
                }
              }
            }
        }
      }
      if constexpr (!SCL) {
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
          const int g = (g0 + u) < g_hi ? (g0 + u) : (g_hi - 1);
#pragma unroll
          for (int j = 0; j < MB16; ++j) ch.as[u][j] = pas[j][g];
          ch.bs[u] = pbs[g];
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < GPW; ++u) {
        const int g = (g0 + u) < g_hi ? (g0 + u) : (g_hi - 1);
        const int k0 = g * kGroup;
        if constexpr (DMA) {
          lds_u8* base = (lds_u8*)(stage + u * NBK * 2048);
#pragma unroll
          for (int b = 0; b < NBK; ++b)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              // Weight rows carry the non-temporal hint, as in the single-stage
              // tiles above.
              if (b < NB16) {
                lds_dma16_nt(rsc[0], pd[b][q], k0, base + b * 2048 + q * 1024);
              } else {
                lds_dma16(rsc[1], pd[b][q], k0, base + b * 2048 + q * 1024);
              }
            }
        } else {
#pragma unroll
          for (int i = 0; i < NB16; ++i) ch.bf[u][i] = load_frag_global(pb[i] + k0, lane);
#pragma unroll
          for (int j = 0; j < MB16; ++j) ch.af[u][j] = load_frag_global(pa[j] + k0, lane);
        }
        if constexpr (!SCL) {
#pragma unroll
          for (int j = 0; j < MB16; ++j) ch.as[u][j] = pas[j][g];
          ch.bs[u] = pbs[g];
        }
      }
    }
    if constexpr (SCL) {
      const int u = lane % GPW;
      const int g = (g0 + u) < g_hi ? (g0 + u) : (g_hi - 1);
      lds_dma4(rss[0], sc_row_off + 4u * (uint32_t)g, 0, (lds_u8*)sscl);
      if (lane < GPW) lds_dma4(rss[1], 4u * (uint32_t)g, 0, (lds_u8*)(sscl + 64));
    }
  };

#pragma unroll
  for (int i = 0; i < NB16; ++i)
#pragma unroll
    for (int j = 0; j < MB16; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // pending: chunk c+1's loads were issued after chunk c's and may stay in
  // flight (DMA form only; the register form is tracked by the compiler).
  auto compute = [&](Chunk& ch, int c, bool pending, const uint8_t* stage) {
    const int g0 = g_lo + (c * KW + kw) * GPW;
    if constexpr (DMA) {
      if (pending) __builtin_amdgcn_s_waitcnt(vmcnt_only(LPC));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
#pragma unroll
      for (int u = 0; u < GPW; ++u) {
        const uint8_t* base = stage + u * NBK * 2048;
#pragma unroll
        for (int i = 0; i < NB16; ++i) ch.bf[u][i] = load_frag_lds_sw(base + i * 2048, 0, lane);
#pragma unroll
        for (int j = 0; j < MB16; ++j) ch.af[u][j] = load_frag_lds_sw(base + (NB16 + j) * 2048, 0, lane);
        if constexpr (SCL) {
          ch.as[u][0] = sscl[(lane & 15) * GPW + u];
          ch.bs[u] = sscl[64 + u];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      if (g0 + u < g_hi) {
#pragma unroll
        for (int j = 0; j < MB16; ++j) {
          const float sc = ch.as[u][j] * ch.bs[u];  // a_s * b_s, once per group and lane
#pragma unroll
          for (int i = 0; i < NB16; ++i) {
            const v4f p = mfma_group(ch.bf[u][i], ch.af[u][j]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sc, acc[i][j][r]);
          }
        }
      }
    }
  };

  // Chunks of this wave that hold at least one group of [g_lo, g_hi).
  const int first = g_lo + kw * GPW;
  const int my_chunks = first < g_hi ? (g_hi - first + KW * GPW - 1) / (KW * GPW) : 0;
  if constexpr (KFIX != 0) {
    if (my_chunks > 0) {
      Chunk ch;
      load(ch, 0, stage0);
      compute(ch, 0, false, stage0);
    }
  } else if constexpr (ONE) {
    // One staging area: each chunk's loads all in flight, one wait, then its
    // MFMAs (the configurations are chosen so one chunk covers the range).
    // The area is refilled only after the previous chunk's fragments are in
    // registers (its MFMAs consumed them).
    for (int c = 0; c < my_chunks; ++c) {
      Chunk ch;
      load(ch, c, stage0);
      compute(ch, c, false, stage0);
    }
  } else if (my_chunks > 0) {
    // Two register buffers in ping-pong, no copies between them: chunk c+1
    // is in flight while chunk c is computed.  The steady-state loop runs
    // while two more chunks exist; the last one or two are peeled.
    Chunk b0, b1;
    load(b0, 0, stage0);
    int c = 0;
    for (; c + 2 < my_chunks; c += 2) {
      load(b1, c + 1, stage1);
      compute(b0, c, true, stage0);
      load(b0, c + 2, stage0);
      compute(b1, c + 1, true, stage1);
    }
    if (my_chunks - c == 2) {
      load(b1, c + 1, stage1);
      compute(b0, c, true, stage0);
      compute(b1, c + 1, false, stage1);
    } else {
      compute(b0, c, false, stage0);
    }
  }

}

// row(q, b, r): the 64 floats of wave q's partial of block b, element r, in
// the reduction buffer.
template <int NB16, int MB16, int KW, typename Row>
__device__ __forceinline__ void skinny_reduce(Row&& row, int kw, int lane, v4f (&acc)[NB16][MB16]) {
  constexpr int NBLK = NB16 * MB16;
  if constexpr (KW > 1) {
#pragma unroll
    for (int i = 0; i < NB16; ++i)
#pragma unroll
      for (int j = 0; j < MB16; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) row(kw, i * MB16 + j, r)[lane] = acc[i][j][r];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      if (b % KW != kw) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = row(0, b, r)[lane];
#pragma unroll
        for (int q = 1; q < KW; ++q) v += row(q, b, r)[lane];
        acc[b / MB16][b % MB16][r] = v;
      }
    }
  }
}

// ===========================================================================
// Skinny kernel: swap-AB, optionally split over K, and (KFIX = 2) the
// short-K kernel.  (Section "Specialized kernels and the optimization idea":
// swap_ab, swap_ab_splitk, short_k256.)
//
// Computes tiles of C^T = B A^T: weight rows n sit on the MFMA's first
// operand, activation rows m (small M) on the second, so each lane ends with
// 4 consecutive n of one output row m -- one vector store per block.
//
// Small-M shapes are latency- and bandwidth-bound, so no workgroup-wide
// operand tiles: every wave loads its own B and A fragments, through a
// per-wave LDS staging area (coalesced 128-byte rows, no barriers) or, for
// the largest tiles and the short-K form, straight into registers; all loads
// of a chunk of GPW groups in flight at once and the next chunk prefetched
// while the current one is computed.
// The KW waves of a workgroup split the workgroup's K range (wave kw takes
// chunks kw, kw+KW, ...); their FP32 partials are summed through LDS in the
// fixed order kw = 0..KW-1.
//
// Split-K over workgroups (S > 1): workgroup (tile, s) covers a contiguous
// run of G/S or G/S + 1 groups (the first G%S splits take one more) and
// publishes its FP32 partial at device scope; the last
// of the S workgroups of a tile to arrive (one counter atomic per workgroup,
// no atomics on data) sums the S partials in the fixed order s = 0..S-1,
// casts, stores and resets the counter.  The page's split-K summed partials
// with atomic adds into C (section "Numerical safety"), which is not
// bit-reproducible; this order is.
//
// KFIX = 2 (short-K, K == 256): the group count is a compile-time 2, so the
// loads and the fold are fully unrolled; each lane forms a_s*b_s of both
// groups once per tile (b_s folded into a_s) and the two partials combine as
// fma(P1, s1, fma(P0, s0, 0)).
// ===========================================================================
template <int NB16, int MB16, int KW, int GPW, int KFIX, int ONE, int OUT>
__global__ __launch_bounds__(64 * KW) void k_skinny(
    const uint8_t* __restrict__ A, const float* __restrict__ a_s, const uint8_t* __restrict__ B,
    const float* __restrict__ b_s, void* __restrict__ C, int M, int N, int K, int S,
    float* __restrict__ ws, unsigned* __restrict__ counters, int vec_ok) {
  constexpr int BN = 16 * NB16;   // n rows per workgroup (every wave covers all of them)
  constexpr bool HALF = ONE == 2;  // tiles of 8 activation rows
  constexpr int BMS = HALF ? 8 : 16 * MB16;  // m columns per workgroup
  constexpr int BLK_ELEMS = 16 * BN * MB16;   // FP32 partial elements of a tile (16-row blocks)
  constexpr int NBLK = NB16 * MB16;
  static_assert(128 % BN == 0, "a tile's n rows must share one b_s block");
  static_assert(KFIX == 0 || KW * GPW == KFIX, "the short-K form covers its groups in one chunk");
  static_assert(!HALF || (MB16 == 1 && KFIX == 0), "8-row activation tiles are single 16-row blocks");

  // Fragments through LDS (DMA) where the staging area stays within 96 KB
  // per workgroup for two chunks per wave, or 128 KB for one (ONE, and the
  // short-K form, whose one chunk holds both groups); the other
  // configurations load straight into registers.
  constexpr int STAGE_H = GPW * (NB16 + MB16) * 2048;  // one chunk of one wave
  constexpr int SINGLE = ONE != 0 || KFIX != 0;
  constexpr int DMA = SINGLE ? STAGE_H * KW <= 128 * 1024 : 2 * STAGE_H * KW <= 96 * 1024;
  // With one staging area per wave, the cross-wave sum reuses it: wave q's
  // partials overwrite its own area once its last fragments are in registers
  // (only that wave ever wrote or read it), so no separate buffer is needed.
  constexpr bool RED_ALIAS = SINGLE && DMA && KW > 1 && NBLK * 1024 <= STAGE_H;
  __shared__ __attribute__((aligned(16))) float sRed[KW > 1 && !RED_ALIAS ? KW : 1][RED_ALIAS ? 1 : NBLK][4][64];
  __shared__ __attribute__((aligned(16))) uint8_t sStage0[DMA ? STAGE_H * KW : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sStage1[DMA && !SINGLE ? STAGE_H * KW : 16];
  // Per-wave scale images of the single-stage tiles: 16 rows x 4 groups of
  // a_s, then 4 groups of b_s.
  constexpr bool SCL = skinny_scales_in_lds(DMA, ONE, MB16, GPW, KFIX);
  __shared__ __attribute__((aligned(16))) float sScl[SCL ? KW * 80 : 4];
  __shared__ int sLast;

  const int tid = threadIdx.x, lane = tid & 63;
  const int kw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = KFIX ? KFIX : K / kGroup;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BMS - 1) / BMS;
  const int T = tiles_n * tiles_m;
  const int lid = xcd_remap(blockIdx.x, T * S);
  const int s = lid / T, tile = lid - s * T;
  // The m-tiles of one n-tile are consecutive, so they run on one XCD and
  // the weight rows they share are fetched from HBM once, then hit its L2.
  const int tn = tile / tiles_m, tm = tile - tn * tiles_m;
  const int m0 = tm * BMS, n0 = tn * BN;
  // Split s takes G/S groups, one more for the first G%S splits (32-bit
  // arithmetic: a 64-bit division here costs hundreds of scalar cycles at
  // every workgroup's start).
  const int gq = G / S, gr = G - gq * S;
  const int g_lo = s * gq + (s < gr ? s : gr), g_hi = g_lo + gq + (s < gr ? 1 : 0);
  const int nblk = (N + 127) / 128;
  const int nb = (n0 >> 7) < nblk ? (n0 >> 7) : nblk - 1;
  const int64_t ldk = KFIX ? (int64_t)KFIX * kGroup : (int64_t)K;

  // Row pointers (clamped rows only feed outputs that are never stored).
  const uint8_t* pb[NB16];
#pragma unroll
  for (int i = 0; i < NB16; ++i) {
    const int r = n0 + 16 * i + (lane & 15);
    pb[i] = B + (int64_t)(r < N ? r : N - 1) * ldk;
  }
  const uint8_t* pa[MB16];
  const float* pas[MB16];
#pragma unroll
  for (int j = 0; j < MB16; ++j) {
    int r = m0 + 16 * j + (HALF ? (lane & 7) : (lane & 15));
    r = r < M ? r : M - 1;
    pa[j] = A + (int64_t)r * ldk;
    pas[j] = a_s + (int64_t)r * G;
  }
  const float* pbs = b_s + (int64_t)nb * G;
  // DMA sources: rows 8q + lane/8 of each 16-row block (clamped), at the
  // row's swizzled 16-byte chunk, as 32-bit offsets from the tile's first
  // weight row and first activation row.
  const buf_rsrc rsc[2] = {make_rsrc(B + (int64_t)n0 * ldk), make_rsrc(A + (int64_t)m0 * ldk)};
  uint32_t pd[NB16 + MB16][2];
#pragma unroll
  for (int b = 0; b < NB16 + MB16; ++b)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rr = 8 * q + (lane >> 3);
      const uint32_t chunk = 16u * (uint32_t)((lane & 7) ^ swz_row(rr));
      if (b < NB16) {
        const int r = 16 * b + rr;
        pd[b][q] = (uint32_t)((n0 + r) < N ? r : (N - 1 - n0)) * (uint32_t)ldk + chunk;
      } else {
        const int r = 16 * (b - NB16) + rr;
        pd[b][q] = (uint32_t)((m0 + r) < M ? r : (M - 1 - m0)) * (uint32_t)ldk + chunk;
      }
    }

  // Scale-image sources (SCL): lane l reads row m0 + l / 4 (clamped) of a_s,
  // as an offset from the tile's first row; the group offset is added per
  // chunk.
  const buf_rsrc rss[2] = {make_rsrc(a_s + (int64_t)m0 * G), make_rsrc(pbs)};
  const int srow = m0 + lane / 4;
  const uint32_t sc_row_off = (uint32_t)((srow < M ? srow : M - 1) - m0) * (uint32_t)G * 4u;

  v4f acc[NB16][MB16];
  skinny_tile<NB16, MB16, KW, GPW, KFIX, DMA, ONE>(pb, pa, pas, pbs, g_lo, g_hi, kw, lane, acc, pd, rsc,
                                                   sStage0 + kw * (DMA ? STAGE_H : 0),
                                                   sStage1 + kw * (DMA && !SINGLE ? STAGE_H : 0),
                                                   M - m0 < 8 ? M - m0 : 8, sScl + (SCL ? kw * 80 : 0), rss,
                                                   sc_row_off);
  // The KW waves' partials, summed in the fixed order kw = 0..KW-1; wave w
  // then owns blocks b with b % KW == w for the rest of the epilogue.
  if constexpr (RED_ALIAS)
    skinny_reduce<NB16, MB16, KW>(
        [&](int q, int b, int r) { return reinterpret_cast<float*>(sStage0 + q * STAGE_H) + (b * 4 + r) * 64; },
        kw, lane, acc);
  else
    skinny_reduce<NB16, MB16, KW>([&](int q, int b, int r) { return &sRed[q][b][r][0]; }, kw, lane, acc);

  if (S > 1) {
    // Publish this split's partial at device scope and count the arrival.
    // The ordering contract, in the terms of the gfx950 ISA:
    //  1. the partials are agent-scope atomic stores, which the hardware
    //     performs write-through to the device coherence point (the memory
    //     side of every XCD's L2), and a store leaves the wave's vmcnt only
    //     once it is complete there;
    //  2. every wave waits for all of its stores (s_waitcnt 0) before the
    //     workgroup barrier, so no partial store is outstanding when
    //  3. one wave increments the tile's counter, an agent-scope atomic
    //     performed at the coherence point;
    //  4. the last arrival (the increment that returns S - 1) reads the
    //     partials with agent-scope atomic loads, served from the coherence
    //     point and issued only after that return value reached the wave
    //     (through the barrier), so they see every partial completed before
    //     any earlier increment.
    // The memory model's agent-scope release/acquire (an acq_rel increment
    // and an acquire fence in the last arrival) gives the same order, but on
    // gfx950 it is an L2 writeback and invalidate per workgroup: the decode
    // shape split in 4 ran 16.8 us against 6.2 us, so it is not used.
    constexpr int TILE_ELEMS = BLK_ELEMS;
    float* mine = ws + ((int64_t)s * T + tile) * TILE_ELEMS;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      if (b % KW != kw) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __hip_atomic_store(mine + (b * 4 + r) * 64 + lane, acc[b / MB16][b % MB16][r], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sLast = (prev == (unsigned)(S - 1));
    }
    __syncthreads();
    if (!sLast) return;
    // Last arrival: sum the S partials in the fixed order q = 0..S-1.  The
    // partials are loaded QB splits at a time, every load of a batch issued
    // before its adds (split indices past S-1 reload split S-1 and are not
    // added), so S <= QB costs one memory round trip.
    constexpr int QB = 4;
    const float* wt = ws + (int64_t)tile * TILE_ELEMS;
    const int64_t split_stride = (int64_t)T * TILE_ELEMS;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      if (b % KW != kw) continue;
      v4f v = v4f{0.f, 0.f, 0.f, 0.f};
      for (int q0 = 0; q0 < S; q0 += QB) {
        v4f t[QB];
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int q = (q0 + u) < S ? (q0 + u) : (S - 1);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            t[u][r] = __hip_atomic_load(wt + q * split_stride + (b * 4 + r) * 64 + lane, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          if (q0 + u >= S) break;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (q0 + u == 0) ? t[u][r] : v[r] + t[u][r];
        }
      }
      acc[b / MB16][b % MB16] = v;
    }
    if (tid == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Result block (i, j): lane holds n = 16i + 4*(lane>>4) + r, m = 16j + (lane & 15).
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    if (b % KW != kw) continue;
    const int i = b / MB16, j = b % MB16;
    const int n = n0 + 16 * i + 4 * (lane >> 4);
    const int m = m0 + 16 * j + (lane & 15);
    const int cnt = N - n < 4 ? N - n : 4;
    if ((!HALF || (lane & 15) < 8) && m < M && cnt > 0) store4<OUT>(C, (int64_t)m * N + n, acc[i][j], cnt, vec_ok);
  }
}

// ===========================================================================
// Grouped (mixture-of-experts) kernel: rows offsets[e] .. offsets[e+1]-1 of A
// are the tokens routed to expert e, multiplied by that expert's weight
// B[e] ([N,K]) with its block scales b_s[e].  (MoE-style traffic: the first
// page's section "Description"; per-expert token groups and the decode
// swap-AB path: the MoE kernel page, section "Summary".)
//
// One workgroup per (expert, n-tile): it streams its weight rows once per
// token tile and walks the expert's tokens in tiles of up to 16*MB16 rows
// (decode experts hold a handful of tokens, so usually one tile), in the
// swap-AB orientation and with the skinny kernels' K loop and fixed-order
// cross-wave sum.  A tile computes only its 16-row blocks that hold tokens:
// the count of such blocks selects one of MB16 straight-line instances, so a
// 20-token expert loads and multiplies 2 blocks, not MB16.  An expert with no
// tokens costs one offset read: its weights are never touched.  The offsets
// stay on the device (no host synchronisation); they are clamped into
// [0, M], so malformed offsets can only leave rows unwritten, never address
// outside A or C.
// ===========================================================================
template <int NB16, int MBA, int KW, int GPW, int OUT, typename Red>
__device__ __forceinline__ void grouped_mtile(const uint8_t* const* pb, const float* pbs, const uint8_t* A,
                                              const float* a_s, void* C, Red& sRed, int m0, int hi, int n0, int N,
                                              int K, int G, int kw, int lane, int vec_ok) {
  // Token rows past the expert's last are clamped to it (never stored).
  const uint8_t* pa[MBA];
  const float* pas[MBA];
#pragma unroll
  for (int j = 0; j < MBA; ++j) {
    int r = m0 + 16 * j + (lane & 15);
    r = r < hi ? r : hi - 1;
    pa[j] = A + (int64_t)r * K;
    pas[j] = a_s + (int64_t)r * G;
  }
  v4f acc[NB16][MBA];
  skinny_tile<NB16, MBA, KW, GPW, 0>(pb, pa, pas, pbs, 0, G, kw, lane, acc);
  // The first NB16*MBA blocks of the reduction buffer, in this tile's shape.
  auto& red = *reinterpret_cast<float(*)[KW > 1 ? KW : 1][NB16 * MBA][4][64]>(&sRed[0][0][0][0]);
  skinny_reduce<NB16, MBA, KW>([&](int q, int b, int r) { return &red[q][b][r][0]; }, kw, lane, acc);
  // Block (i, j): lane holds n = 16i + 4*(lane>>4) + r, m = 16j + (lane & 15).
#pragma unroll
  for (int b = 0; b < NB16 * MBA; ++b) {
    if (b % KW != kw) continue;
    const int i = b / MBA, j = b % MBA;
    const int n = n0 + 16 * i + 4 * (lane >> 4);
    const int m = m0 + 16 * j + (lane & 15);
    const int cnt = N - n < 4 ? N - n : 4;
    if (m < hi && cnt > 0) store4<OUT>(C, (int64_t)m * N + n, acc[i][j], cnt, vec_ok);
  }
}

template <int NB16, int MB16, int KW, int GPW, int OUT>
__global__ __launch_bounds__(64 * KW) void k_grouped(
    const uint8_t* __restrict__ A, const float* __restrict__ a_s, const uint8_t* __restrict__ B,
    const float* __restrict__ b_s, void* __restrict__ C, const int* __restrict__ offsets, int E, int M, int N,
    int K, int vec_ok) {
  constexpr int BN = 16 * NB16, BMS = 16 * MB16, NBLK = NB16 * MB16;
  static_assert(128 % BN == 0, "a tile's n rows must share one b_s block");
  static_assert(MB16 >= 1 && MB16 <= 4, "up to 4 token blocks per tile");
  __shared__ __attribute__((aligned(16))) float sRed[KW > 1 ? KW : 1][NBLK][4][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int kw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = K / kGroup;
  const int tiles_n = (N + BN - 1) / BN;
  const int lid = xcd_remap(blockIdx.x, E * tiles_n);
  const int e = lid / tiles_n, tn = lid - e * tiles_n;
  int lo = offsets[e], hi = offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > M ? M : lo);
  hi = hi < lo ? lo : (hi > M ? M : hi);
  if (lo >= hi) return;

  const int n0 = tn * BN;
  const int nblk = (N + 127) / 128;
  const int nb = (n0 >> 7) < nblk ? (n0 >> 7) : nblk - 1;
  const uint8_t* Be = B + (int64_t)e * N * K;
  const float* pbs = b_s + ((int64_t)e * nblk + nb) * G;
  const uint8_t* pb[NB16];
#pragma unroll
  for (int i = 0; i < NB16; ++i) {
    const int r = n0 + 16 * i + (lane & 15);
    pb[i] = Be + (int64_t)(r < N ? r : N - 1) * K;
  }

  for (int m0 = lo; m0 < hi; m0 += BMS) {
    const int rows = hi - m0 < BMS ? hi - m0 : BMS;
    const int mba = __builtin_amdgcn_readfirstlane((rows + 15) >> 4);  // token blocks of this tile
    if (MB16 >= 4 && mba >= 4)
      grouped_mtile<NB16, (MB16 >= 4 ? 4 : 1), KW, GPW, OUT>(pb, pbs, A, a_s, C, sRed, m0, hi, n0, N, K, G, kw,
                                                              lane, vec_ok);
    else if (MB16 >= 3 && mba == 3)
      grouped_mtile<NB16, (MB16 >= 3 ? 3 : 1), KW, GPW, OUT>(pb, pbs, A, a_s, C, sRed, m0, hi, n0, N, K, G, kw,
                                                              lane, vec_ok);
    else if (MB16 >= 2 && mba == 2)
      grouped_mtile<NB16, (MB16 >= 2 ? 2 : 1), KW, GPW, OUT>(pb, pbs, A, a_s, C, sRed, m0, hi, n0, N, K, G, kw,
                                                              lane, vec_ok);
    else
      grouped_mtile<NB16, 1, KW, GPW, OUT>(pb, pbs, A, a_s, C, sRed, m0, hi, n0, N, K, G, kw, lane, vec_ok);
    if (m0 + BMS < hi) __syncthreads();  // the next token tile rewrites sRed
  }
}

// ===========================================================================
// K == 0: the empty sum, C = +0.
// ===========================================================================
template <int OUT>
__global__ void k_fill_zero(void* __restrict__ C, int64_t count) {
  typedef typename Out<OUT>::T T;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    reinterpret_cast<T*>(C)[i] = Out<OUT>::cvt(0.f);
}

// ===========================================================================
// Launchers
// ===========================================================================
template <int BM, int BN, int WM_, int WN_, int ST, int SCH, int MID, int GRP>
static hipError_t launch_generic_t(const GemmArgs& a, int64_t grid, int band, const int* offsets, int E) {
  const dim3 blk(64 * WM_ * WN_);
  switch (a.out) {
    case kOutBF16:
      hipLaunchKernelGGL((k_generic<BM, BN, WM_, WN_, ST, SCH, MID, kOutBF16, GRP>), dim3(grid), blk, 0, a.stream, a.A, a.a_s,
                         a.B, a.b_s, a.C, a.M, a.N, a.K, band, a.vec, offsets, E);
      break;
    case kOutFP16:
      hipLaunchKernelGGL((k_generic<BM, BN, WM_, WN_, ST, SCH, MID, kOutFP16, GRP>), dim3(grid), blk, 0, a.stream, a.A, a.a_s,
                         a.B, a.b_s, a.C, a.M, a.N, a.K, band, a.vec, offsets, E);
      break;
    default:
      hipLaunchKernelGGL((k_generic<BM, BN, WM_, WN_, ST, SCH, MID, kOutFP32, GRP>), dim3(grid), blk, 0, a.stream, a.A, a.a_s,
                         a.B, a.b_s, a.C, a.M, a.N, a.K, band, a.vec, offsets, E);
  }
  return hipGetLastError();
}

hipError_t launch_generic(const GemmArgs& a, int cfg, int64_t grid, int band) {
  switch (cfg) {
#define X(id, bm, bn, wm, wn, st, sch, mid) \
  case id: return launch_generic_t<bm, bn, wm, wn, st, sch, mid, 0>(a, grid, band, nullptr, 0);
    FBG_GENERIC_CFGS(X)
#undef X
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_generic_grouped(const GemmArgs& a, int cfg, int64_t grid, const int* offsets, int E) {
  switch (cfg) {
#define X(id, bm, bn, wm, wn, st, sch, mid) \
  case id:                              \
    if constexpr (id < kNumGroupedGenericCfgs) return launch_generic_t<bm, bn, wm, wn, st, sch, mid, 1>(a, grid, 0, offsets, E);
    FBG_GENERIC_CFGS(X)
#undef X
    default: return hipErrorInvalidValue;
  }
}

template <int NB16, int MB16, int KW, int GPW, int KFIX, int ONE>
static hipError_t launch_skinny_t(const GemmArgs& a, int64_t grid, int S, float* ws, unsigned* cnt) {
  const dim3 blk(64 * KW);
  switch (a.out) {
    case kOutBF16:
      hipLaunchKernelGGL((k_skinny<NB16, MB16, KW, GPW, KFIX, ONE, kOutBF16>), dim3(grid), blk, 0, a.stream, a.A, a.a_s,
                         a.B, a.b_s, a.C, a.M, a.N, a.K, S, ws, cnt, a.vec);
      break;
    case kOutFP16:
      hipLaunchKernelGGL((k_skinny<NB16, MB16, KW, GPW, KFIX, ONE, kOutFP16>), dim3(grid), blk, 0, a.stream, a.A, a.a_s,
                         a.B, a.b_s, a.C, a.M, a.N, a.K, S, ws, cnt, a.vec);
      break;
    default:
      hipLaunchKernelGGL((k_skinny<NB16, MB16, KW, GPW, KFIX, ONE, kOutFP32>), dim3(grid), blk, 0, a.stream, a.A, a.a_s,
                         a.B, a.b_s, a.C, a.M, a.N, a.K, S, ws, cnt, a.vec);
  }
  return hipGetLastError();
}

hipError_t launch_swap(const GemmArgs& a, int cfg, int64_t grid, int S, float* ws, unsigned* counters) {
  switch (cfg) {
#define X(id, nb, mb, kw, gpw, one) \
  case id: return (one == 2 && S > 1) ? hipErrorInvalidValue : launch_skinny_t<nb, mb, kw, gpw, 0, one>(a, grid, S, ws, counters);
    FBG_SWAP_CFGS(X)
#undef X
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_short_k256(const GemmArgs& a, int cfg, int64_t grid) {
  switch (cfg) {
#define X(id, nb, mb, kw, gpw) \
  case id: return launch_skinny_t<nb, mb, kw, gpw, 2, 0>(a, grid, 1, nullptr, nullptr);
    FBG_SHORT_CFGS(X)
#undef X
    default: return hipErrorInvalidValue;
  }
}

template <int NB16, int MB16, int KW, int GPW>
static hipError_t launch_grouped_t(const GemmArgs& a, int64_t grid, const int* offsets, int E) {
  const dim3 blk(64 * KW);
  switch (a.out) {
    case kOutBF16:
      hipLaunchKernelGGL((k_grouped<NB16, MB16, KW, GPW, kOutBF16>), dim3(grid), blk, 0, a.stream, a.A, a.a_s, a.B,
                         a.b_s, a.C, offsets, E, a.M, a.N, a.K, a.vec);
      break;
    case kOutFP16:
      hipLaunchKernelGGL((k_grouped<NB16, MB16, KW, GPW, kOutFP16>), dim3(grid), blk, 0, a.stream, a.A, a.a_s, a.B,
                         a.b_s, a.C, offsets, E, a.M, a.N, a.K, a.vec);
      break;
    default:
      hipLaunchKernelGGL((k_grouped<NB16, MB16, KW, GPW, kOutFP32>), dim3(grid), blk, 0, a.stream, a.A, a.a_s, a.B,
                         a.b_s, a.C, offsets, E, a.M, a.N, a.K, a.vec);
  }
  return hipGetLastError();
}

hipError_t launch_grouped(const GemmArgs& a, int cfg, int64_t grid, const int* offsets, int E) {
  switch (cfg) {
#define X(id, nb, mb, kw, gpw) \
  case id: return launch_grouped_t<nb, mb, kw, gpw>(a, grid, offsets, E);
    FBG_GROUPED_CFGS(X)
#undef X
    default: return hipErrorInvalidValue;
  }
}

// Zeroes `count` 32-bit words with plain vector stores (the split-K arrival
// counters of a fresh workspace).  A kernel rather than hipMemsetAsync, so a
// caller may capture the call in a HIP graph.
__global__ void k_zero_words(uint32_t* __restrict__ p, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) p[i] = 0u;
}

hipError_t launch_zero_words(void* p, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks64 = (count + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 1024 ? blocks64 : 1024);
  hipLaunchKernelGGL(k_zero_words, dim3(blocks), dim3(256), 0, stream, static_cast<uint32_t*>(p), count);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* C, int64_t count, int out, hipStream_t stream) {
  const int64_t blocks64 = (count + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 4096 ? (blocks64 > 0 ? blocks64 : 1) : 4096);
  switch (out) {
    case kOutBF16: hipLaunchKernelGGL(k_fill_zero<kOutBF16>, dim3(blocks), dim3(256), 0, stream, C, count); break;
    case kOutFP16: hipLaunchKernelGGL(k_fill_zero<kOutFP16>, dim3(blocks), dim3(256), 0, stream, C, count); break;
    default: hipLaunchKernelGGL(k_fill_zero<kOutFP32>, dim3(blocks), dim3(256), 0, stream, C, count);
  }
  return hipGetLastError();
}

}  // namespace fbg
