// Device side of the scaled FP8 x FP8 GEMM with fp32 accumulation, per-operand dequantization,
// fused fp32 bias and one bf16 rounding, on gfx950 FP8 MFMA.
//
// Pages: AstrAI commit history of csrc/kernels/fp8/gemm.cuh (@5e76fbd1) and
// of astrai/extension/fp8.py (@f4c44ebf): bf16-only output, bias added in
// fp32 before the single rounding with exact N tails, batched operands with
// stride-0 broadcast, congruous (NT) forward and crosswise dX / dW operands,
// grouped rasterization, a small-tile family for small problems.  Their CUDA
// tiling (cp.async staging, ldmatrix, PRMT transposes) is prior art only.
//
// gfx950 design:
//  * Waves in a WGM x WGN grid each own a block of C made of 32 x 32 tiles of
//    v_mfma_f32_32x32x64_f8f6f4.  The instruction's first source is the B
//    fragment and its second the A fragment, so each lane ends up holding four
//    consecutive n of one row m: 8-byte bf16 stores and 4-wide bias loads in
//    the epilogue.  The per-operand format selectors of the instruction take
//    E4M3 x E4M3 and E5M2 x E4M3 (dX, dW) alike.
//  * Operand tiles go global -> LDS with buffer_load ... lds (no VGPR round
//    trip), 64 K-bytes per stage, several stages in flight.  Loads outside the
//    operand or past K get an offset beyond the buffer's size and land as
//    zeros.
//  * K-contiguous tiles are [rows][64 B] and are read with ds_read_b128;
//    MN-contiguous (crosswise) tiles are [64 k][BM or BN bytes] and are read
//    with ds_read_b64_tr_b8, which transposes 8 x 8-byte blocks across 16
//    lanes, so crosswise operands need no transpose pass.  16-byte chunks are
//    XOR-swizzled per row so both read kinds are free of bank conflicts.
//  * The grid holds as many workgroups as the device runs at once; each runs
//    every G-th output tile, and its stream of K stages runs on across tile
//    boundaries, so the loads of the next tile overlap the end of the current
//    one and its epilogue.
//  * Tile v runs on XCD v mod 8 (workgroups are dealt to XCDs round-robin);
//    each XCD gets a contiguous run of tiles in grouped order, so the tiles
//    sharing A rows and B columns meet in one XCD's L2.
//
// The kernels are templates over the tile, the operand orientations and the
// formats; each gemm_*.hip file instantiates one group of them (so the groups
// compile in parallel) and exposes it through a picker declared below.
// gemm.hip holds the host side: the tile family, its choice and the launch.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace fp8ds {

struct GemmKArgs {
  const uint8_t* a;
  const uint8_t* b;
  uint16_t* c;
  int m, n, k;
  int tiles_m, tiles_n, batch, group_m;
  uint32_t lda, ldb;
  int64_t ldc;
  int64_t stride_a, stride_b, stride_c;
  uint32_t extent_a, extent_b;
  const float* a_scale_inv;
  const float* b_scale_inv;
  const void* bias;
  const float* bias_scale_inv;
  int bias_kind;
  int ldc_small;   // 256 * ldc < 2^31: offsets inside a tile fit 32 bits
};

typedef void (*GemmFn)(GemmKArgs);
typedef void (*GemmPairFn)(GemmKArgs, GemmKArgs, int);

// Kernel pickers, one per translation unit.  tile indexes the family of
// gemm.hip (0: 256x256 four waves, 1: 128x128, 2: 64x64, 3: 256x128,
// 4: 128x256, 5 / 6: 256x256 eight waves as 2x4 / 4x2, 7 / 8: 128x128 /
// 64x64 on 128-byte K units); fa / fb are the operand formats (0 E4M3,
// 1 E5M2).  "large" covers tiles 0, 5 and 6, "small" tiles 1 to 4, 7 and 8.
GemmFn gemm_fn_nt_large(int tile, int fa, int fb);
GemmFn gemm_fn_nt_small(int tile, int fa, int fb);
GemmFn gemm_fn_nn_large(int tile, int fa, int fb);
GemmFn gemm_fn_nn_small(int tile, int fa, int fb);
GemmFn gemm_fn_tn_large(int tile, int fa, int fb);
GemmFn gemm_fn_tn_small(int tile, int fa, int fb);
// The fused NN + TN pair (a layer's dX and dW) on tile 7 or 8.
GemmPairFn gemm_pair_fn(int tile, int fa, int fb);

namespace {

constexpr int kBK = 64;           // K bytes (= elements) per pipeline stage
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;  // offset past every buffer: loads give zero



// K-contiguous tile [rows][64 B]: 16-byte chunk c of row r sits at chunk
// c ^ swz_k(r).  A fragment read (32 consecutive rows, lanes l and l+32
// taking adjacent chunk pairs of one row) is then free of LDS bank conflicts;
// the choice was measured on gfx950 (SQ_LDS_BANK_CONFLICT = 0), where the
// xor of (r >> 1) ^ (r >> 3) still left 4 conflict cycles per ds_read_b128.
__device__ __forceinline__ int swz_k(int r) { return (r >> 2) & 3; }

// MN-contiguous tile [64 k][R chunks]: chunk c of row k sits at c ^ swz_mn(k).
// A transpose read touches 8 consecutive rows x 2 adjacent chunks; the
// swizzle spreads them over distinct bank groups.
template <int R>
__device__ __forceinline__ int swz_mn(int k) {
  if constexpr (R == 16) return ((k & 7) << 1) | ((k >> 2) & 1);
  else if constexpr (R == 8) return k & 7;
  else return ((k >> 2) & 1) << 1;
}

// Tile index v -> (batch, tile row, tile column).  Workgroups are dealt to the
// 8 XCDs round-robin and the grid size is a multiple of 8 whenever a
// workgroup runs more than one tile, so index v runs on XCD v mod 8: each XCD
// gets a contiguous run of tiles in grouped order and the tiles sharing A rows
// and B columns meet in one XCD's L2.
__device__ __forceinline__ void map_tile(const GemmKArgs& p, int v, int& bt, int& tm, int& tn) {
  const int total = p.tiles_m * p.tiles_n * p.batch;
  const int q = total >> 3, r = total & 7;
  const int xcd = v & 7, j = v >> 3;
  const int t = xcd < r ? xcd * (q + 1) + j : r * (q + 1) + (xcd - r) * q + j;
  const int per_batch = p.tiles_m * p.tiles_n;
  bt = t / per_batch;
  const int u = t - bt * per_batch;
  const int in_group = p.group_m * p.tiles_n;
  const int g = u / in_group;
  const int first_m = g * p.group_m;
  const int gsize = min(p.tiles_m - first_m, p.group_m);
  const int w = u - g * in_group;
  tm = first_m + w % gsize;
  tn = w / gsize;
}

// 32 rows x 64 k of a K-contiguous tile: lane l gets row base + l%32,
// k = 32*(l/32) + [0, 32).
__device__ __forceinline__ v8i frag_k(const lds_char_t* tile, int base, int lane) {
  const int row = base + (lane & 31);
  const int c0 = 2 * (lane >> 5);
  const int sw = swz_k(row);
  const v4i lo = *(const lds_v4i_t*)(tile + row * kBK + ((c0 ^ sw) << 4));
  const v4i hi = *(const lds_v4i_t*)(tile + row * kBK + (((c0 + 1) ^ sw) << 4));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The same fragment from an MN-contiguous tile [64 k][R*16 B] through four
// transpose reads: read t hands lane l the bytes k = 32*(l/32) + 8*t + [0, 8)
// of column base + l%32.  Within each 16-lane group, the even lanes address
// rows k..k+7 at the group's first 8 columns and the odd lanes the next 8.
template <int R>
__device__ __forceinline__ v8i frag_mn(const lds_char_t* tile, int base, int lane) {
  const int q = lane & 15;
  const int cl = (base >> 4) + ((lane >> 4) & 1);
  v2i part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kr = 32 * (lane >> 5) + 8 * t + (q >> 1);
    const int addr = kr * (R * 16) + ((cl ^ swz_mn<R>(kr)) << 4) + 8 * (q & 1);
    part[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(tile + addr));
  }
  return v8i{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
}

template <bool KC, int ROWS>
__device__ __forceinline__ v8i load_frag(const lds_char_t* tile, int base, int lane) {
  if constexpr (KC) return frag_k(tile, base, lane);
  else return frag_mn<ROWS / 16>(tile, base, lane);
}

// Per-lane byte offset of load slot `slot` of an operand tile, for k0 = 0;
// kOOB for rows / columns outside the operand.
template <bool KC, int ROWS>
__device__ __forceinline__ uint32_t slot_offset(int slot, int mn0, int mn_lim, uint32_t ld) {
  if constexpr (KC) {
    const int row = slot >> 2, pch = slot & 3, lch = pch ^ swz_k(row);
    return mn0 + row < mn_lim ? (uint32_t)row * ld + (uint32_t)(lch << 4) : kOOB;
  } else {
    constexpr int R = ROWS / 16;
    const int kr = slot / R, pch = slot % R, lch = pch ^ swz_mn<R>(kr);
    return mn0 + (lch << 4) < mn_lim ? (uint32_t)kr * ld + (uint32_t)(lch << 4) : kOOB;
  }
}

// K position, inside its stage, of the bytes load slot `slot` brings in; the
// slot lies past K in a tail stage when this is >= K mod 64.
template <bool KC, int ROWS>
__device__ __forceinline__ int slot_kpos(int slot) {
  if constexpr (KC) {
    const int row = slot >> 2, pch = slot & 3;
    return (pch ^ swz_k(row)) << 4;
  } else {
    return slot / (ROWS / 16);
  }
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most N stages of LPS loads each are still in flight.
template <int LPS, int STAGES, int N>
__device__ __forceinline__ void wait_stages() {
  static_assert(LPS * (STAGES - 1) <= 63, "vmcnt holds at most 63");
  static_assert(N >= 0 && N < STAGES, "stages in flight");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N * LPS));
}

// Workgroup barrier ordering LDS only: outstanding global->LDS prefetches of
// later stages stay in flight across it.  It waits for this wave's own LDS
// operations first (the release half), so LDS written before it is seen by
// every wave after it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The K loop's per-stage barrier: a bare s_barrier that keeps the compiler
// from moving memory operations across it but waits for nothing, so LDS
// reads already issued stay in flight across it.  The callers make the
// data it publishes complete first (they wait for the global -> LDS loads of
// the stage by vmcnt), and never write LDS that another wave may still read
// (see the buffer rotation in gemm_body).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Lanes l and l+32 hold the same row; lane l+32 holds the four columns after
// lane l's in each 8-column group.  This swaps a value between the two lane
// halves (v_permlane32_swap): lane l receives lane l+32's value and the
// other way round.
__device__ __forceinline__ uint32_t swap_lane_halves(uint32_t x, bool hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return hi ? r[0] : r[1];
}

// s_waitcnt immediate that waits until none of this wave's LDS operations is
// outstanding (vmcnt and expcnt left unconstrained).
constexpr int lgkmcnt_zero_imm() { return 15 | (3 << 14) | (7 << 4); }

// Columns a wave stages through LDS at a time in the epilogue: 32 rows of
// them fit the wave's LPS KiB share of a stage buffer, and they divide the
// wave's WN columns.
constexpr int staged_cols(int wn, int lps) {
  int cw = wn;
  while (cw * 64 > lps * 1024) cw /= 2;
  return cw;
}

// Bias of the four consecutive columns n .. n+3, all inside the output, in
// fp32: bf16 and fp32 as stored, an 8-bit bias as fl32(dec(code) *
// bias_scale_inv).  n is a multiple of 4, so each kind is one aligned load.
__device__ __forceinline__ v4f bias4_full(const GemmKArgs& p, int n) {
  if (p.bias_kind == 1) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.bias) + n);
    return v4f{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xFFFF0000u)};
  }
  if (p.bias_kind == 2) return *reinterpret_cast<const v4f*>(static_cast<const float*>(p.bias) + n);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.bias) + n);
  const float bsi = p.bias_scale_inv[0];
  v4f r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = (int)(w >> (8 * e));
    r[e] = (p.bias_kind == 3 ? __builtin_amdgcn_cvt_f32_fp8(c, 0) : __builtin_amdgcn_cvt_f32_bf8(c, 0)) * bsi;
  }
  return r;
}

// Epilogue of one wave for a block inside C, through LDS.  Per pass of SC
// columns (CW, or 64 with a bias) and per band of 32 rows, the wave writes
// y = bf16(acc * alpha + bias) to a staging area (each lane its row's 4-column
// pieces, as the MFMA left them), reads them back row-contiguous and stores 16
// bytes per lane, so every store instruction writes whole rows of SC columns:
// full 128-byte lines.  A pass loads its columns' bias once for all bands.
// The staging area is the wave's own share of `buf`, the stage buffer the
// tile's last stage freed: the 1 KiB pieces t * NW + wave, t < LPS, exactly
// the pieces the wave's next loads into that buffer refill, so no other wave
// touches them until those loads are issued.  Staged rows are RB bytes; their
// 16-byte chunks are XOR-swizzled by row so the row-contiguous reads are free
// of bank conflicts.  LDS operations of one wave run in order, so the reads
// see the writes and later writes wait for earlier reads.
// Global stores one wave issues in store_c_staged without a bias: TN * 32 /
// CW column passes, each TM row bands of 32 rows read back in 16-byte chunks
// (64 lanes cover 64 * 16 / (2 * CW) rows per store).
template <int TM, int TN, int LPS>
constexpr int staged_store_ops() {
  constexpr int cw = staged_cols(TN * 32, LPS), rows_per_store = 64 * 16 / (2 * cw);
  return (TN * 32 / cw) * TM * (32 / rows_per_store);
}

template <int BM, int BN, int TM, int TN, int NW, int LPS>
__device__ __forceinline__ void store_c_staged(const GemmKArgs& p, const v16f (&acc)[TN][TM], int m0, int n0,
                                               uint16_t* cb, int lane, int wave, float alpha, lds_char_t* buf) {
  constexpr uint32_t CW = staged_cols(TN * 32, LPS);
  static_assert(CW >= 32 && (TN * 32) % CW == 0 && 32 * 2 * CW <= LPS * 1024, "staging area");
  uint8_t* base = reinterpret_cast<uint8_t*>(cb + (int64_t)m0 * p.ldc + n0);
  const uint32_t ldc2 = 2u * (uint32_t)p.ldc;
  // The per-lane staging addresses are cheap: compute them here, not once
  // for the whole kernel, where they would hold registers through the K loop.
  uint32_t ul = (uint32_t)lane;
  asm volatile("" : "+v"(ul));
  const uint32_t sbase = lds_address(buf) + (uint32_t)wave * 1024u;
  const uint32_t wr = ul & 31u, wh = ul >> 5;   // write phase: MFMA row l % 32, column half l / 32
  // With a bias, at most 64 columns per pass, so their bias values (8 x 4 per
  // lane) fit the registers the K loop leaves free.
  auto run = [&](auto with_bias) __attribute__((always_inline)) {
    constexpr bool HB = decltype(with_bias)::value;
    constexpr uint32_t SC = HB && CW > 64 ? 64 : CW;   // columns per pass
    constexpr uint32_t RB = 2 * SC, CH = RB / 16, RPP = 1024 / RB, RPI = 64 / CH, NR = 32 / RPI;
    constexpr uint32_t SG = SC / 32 * 4;                // 4-column groups of a lane per staged row
    auto row_at = [&](uint32_t r) __attribute__((always_inline)) {
      return sbase + (r / RPP) * (NW * 1024u) + (r % RPP) * RB;
    };
    const uint32_t wsw = wr % CH, waddr = row_at(wr) + 8u * wh;
    // Read phase: lane l reads chunk l % CH of row l / CH (+ RPI per read).
    const uint32_t rr = ul / CH, rc = ul % CH;
    const uint32_t goff = rr * ldc2 + rc * 16u;
#pragma unroll
    for (uint32_t cc = 0; cc < TN * 32 / SC; ++cc) {
      // Without a bias, fma with +0: a zero product rounds to +0, as with one.
      v4f bias[SG];
#pragma unroll
      for (uint32_t g = 0; g < SG; ++g)
        bias[g] = HB ? bias4_full(p, n0 + (int)(cc * SC + (g / 4) * 32 + 8 * (g % 4) + 4 * wh)) : v4f{};
#pragma unroll
      for (int j = 0; j < TM; ++j) {
#pragma unroll
        for (uint32_t g = 0; g < SG; ++g) {
          const v16f& a = acc[cc * (SC / 32) + g / 4][j];
          const uint32_t rq = g % 4;
          const uint32_t lo = pack_bf16x2(__builtin_fmaf(a[4 * rq + 0], alpha, bias[g][0]),
                                          __builtin_fmaf(a[4 * rq + 1], alpha, bias[g][1]));
          const uint32_t hi = pack_bf16x2(__builtin_fmaf(a[4 * rq + 2], alpha, bias[g][2]),
                                          __builtin_fmaf(a[4 * rq + 3], alpha, bias[g][3]));
          const uint32_t addr = waddr + ((g ^ wsw) << 4);
          *(lds_v2i_t*)((lds_char_t*)(uintptr_t)addr) = v2i{(int)lo, (int)hi};
        }
        v4i val[NR];
#pragma unroll
        for (uint32_t q = 0; q < NR; ++q) {
          const uint32_t r = q * RPI + rr;
          val[q] = *(const lds_v4i_t*)((lds_char_t*)(uintptr_t)(row_at(r) + ((rc ^ (r % CH)) << 4)));
        }
        uint8_t* band = base + (uint32_t)j * 32u * ldc2 + cc * SC * 2u;
        // Streaming stores: written normally, C's lines stay dirty in the
        // Infinity Cache and the next kernel pays for their write-back (the
        // 8192^2 quantize after an 8192^3 GEMM took 73.4 us after plain
        // stores, 68.9 us after streaming ones, 64.7 us after another
        // quantize; the GEMM itself ran 1.3 us faster).  A choice between
        // the two at run time doubles this code and makes the 256x256
        // four-wave kernel spill.
#pragma unroll
        for (uint32_t q = 0; q < NR; ++q)
          __builtin_nontemporal_store(val[q], reinterpret_cast<v4i*>(band + goff + q * RPI * ldc2));
        // One row band at a time: interleaving the bands holds more registers
        // than the K loop leaves free.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if constexpr (TM * TN <= 8) {
    if (p.bias_kind != 0) {
      run(std::true_type{});
      return;
    }
  }
  run(std::false_type{});
}

// Epilogue of one wave for output tile v: y = acc * alpha + bias[n] with one
// bf16 rounding, alpha = sa_inv * sb_inv.  The wave's C block starts at row
// r0 and column c0 of the tile; lane l holds rows +l%32 and four consecutive
// columns per 8-column group of each 32 x 32 MFMA tile.
//
// A block inside C stores through LDS (store_c_staged) when the caller hands
// over a free stage buffer (staged = true; with a bias, only blocks of at most
// 8 MFMA tiles).  The flag is separate from the pointer because the buffer at
// LDS offset 0 is a valid one, and a null test of an LDS pointer compares it
// with 0.  Without a buffer (a launch with K = 0) a block inside
// C with no bias takes the register path: two column groups are combined by
// swapping half of them between the lane halves, so every lane stores 8
// consecutive columns (16 bytes) and each store instruction writes 32 rows x
// 32 contiguous bytes.  Edge blocks go through the guarded path.  A bias load
// makes the wave wait for the next tile's loads already in flight (the
// compiler cannot count those), once per tile.  Returns whether the block went through
// LDS (then it issued exactly staged_store_ops<TM, TN, LPS>() global stores
// and no other memory operation).  DRAIN: the guarded path ends by waiting
// for all of the wave's vector memory operations, so a caller's loop finds
// none of its loads pending (the compiler would otherwise wait for them, and
// for every load in flight, at the loop's next register reuse).
template <int BM, int BN, int TM, int TN, int NW, int LPS, bool DRAIN = false>
__device__ __forceinline__ bool store_c_tile(const GemmKArgs& p, const v16f (&acc)[TN][TM], int v, int r0, int c0,
                                             int lane, int wave, float alpha, bool staged,
                                             lds_char_t* stage_buf) {
  int bt, tmi, tni;
  map_tile(p, v, bt, tmi, tni);
  const int m0 = tmi * BM + r0, n0 = tni * BN + c0;
  uint16_t* cb = p.c + bt * p.stride_c;
  // (Blocks of 16 MFMA tiles, one wave per SIMD, stage no bias: its registers
  // make the compiler spill in the K loop.)
  if (staged && (TM * TN <= 8 || p.bias_kind == 0) && p.ldc_small && m0 + TM * 32 <= p.m &&
      n0 + TN * 32 <= p.n) {
    store_c_staged<BM, BN, TM, TN, NW, LPS>(p, acc, m0, n0, cb, lane, wave, alpha, stage_buf);
    return true;
  }
  // (Blocks of more than 8 MFMA tiles keep their accumulators in AGPRs; for
  // them the fast path's extra registers cost more than it saves.)
  if (TM * TN <= 8 && p.bias_kind == 0 && p.ldc_small && m0 + TM * 32 <= p.m && n0 + TN * 32 <= p.n) {
    uint8_t* base = reinterpret_cast<uint8_t*>(cb + (int64_t)m0 * p.ldc + n0);
    const bool hi = lane >= 32;
    const uint32_t ldc = (uint32_t)p.ldc;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int rq = 0; rq < 4; rq += 2) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const v16f& a = acc[i][j];
          const uint32_t g0a = pack_bf16x2(__builtin_fmaf(a[4 * rq + 0], alpha, 0.f), __builtin_fmaf(a[4 * rq + 1], alpha, 0.f));
          const uint32_t g0b = pack_bf16x2(__builtin_fmaf(a[4 * rq + 2], alpha, 0.f), __builtin_fmaf(a[4 * rq + 3], alpha, 0.f));
          const uint32_t g1a = pack_bf16x2(__builtin_fmaf(a[4 * rq + 4], alpha, 0.f), __builtin_fmaf(a[4 * rq + 5], alpha, 0.f));
          const uint32_t g1b = pack_bf16x2(__builtin_fmaf(a[4 * rq + 6], alpha, 0.f), __builtin_fmaf(a[4 * rq + 7], alpha, 0.f));
          // lane l keeps group rq and gets lane l+32's half of it; lane l+32
          // keeps group rq+1 and gets lane l's half of that one.
          const uint32_t ra = swap_lane_halves(hi ? g0a : g1a, hi);
          const uint32_t rb = swap_lane_halves(hi ? g0b : g1b, hi);
          const u32x4 out = hi ? u32x4{ra, rb, g1a, g1b} : u32x4{g0a, g0b, ra, rb};
          const uint32_t col = (uint32_t)(i * 32 + 8 * (rq + (hi ? 1 : 0)));
          const uint32_t off = ((uint32_t)(j * 32 + (lane & 31)) * ldc + col) * 2u;
          *reinterpret_cast<u32x4*>(base + off) = out;
        }
      }
    }
    return false;
  }
#pragma unroll
  for (int i = 0; i < TN; ++i) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int n = n0 + i * 32 + 8 * rq + 4 * (lane >> 5);
      if (n >= p.n) continue;
      float bias4[4] = {0.f, 0.f, 0.f, 0.f};
      const bool full4 = n + 3 < p.n;
      if (p.bias_kind == 1) {
        const uint16_t* bp = static_cast<const uint16_t*>(p.bias) + n;
        if (full4) {
          const uint2 w = *reinterpret_cast<const uint2*>(bp);
          bias4[0] = __uint_as_float(w.x << 16);
          bias4[1] = __uint_as_float(w.x & 0xFFFF0000u);
          bias4[2] = __uint_as_float(w.y << 16);
          bias4[3] = __uint_as_float(w.y & 0xFFFF0000u);
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < p.n) bias4[e] = __uint_as_float((uint32_t)bp[e] << 16);
        }
      } else if (p.bias_kind == 2) {
        const float* bp = static_cast<const float*>(p.bias) + n;
        if (full4) {
          const float4 w = *reinterpret_cast<const float4*>(bp);
          bias4[0] = w.x; bias4[1] = w.y; bias4[2] = w.z; bias4[3] = w.w;
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < p.n) bias4[e] = bp[e];
        }
      } else if (p.bias_kind >= 3) {
        // 8-bit bias: fl32(dec(code) * bias_scale_inv), added to acc * alpha.
        const uint8_t* bp = static_cast<const uint8_t*>(p.bias) + n;
        const float bsi = p.bias_scale_inv[0];
        uint32_t w = 0;
        for (int e = 0; e < 4; ++e)
          if (n + e < p.n) w |= (uint32_t)bp[e] << (8 * e);
        for (int e = 0; e < 4; ++e) {
          const int c = (int)(w >> (8 * e));
          const float d = p.bias_kind == 3 ? __builtin_amdgcn_cvt_f32_fp8(c, 0) : __builtin_amdgcn_cvt_f32_bf8(c, 0);
          bias4[e] = d * bsi;
        }
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + j * 32 + (lane & 31);
        if (m >= p.m) continue;
        const float y0 = __builtin_fmaf(acc[i][j][4 * rq + 0], alpha, bias4[0]);
        const float y1 = __builtin_fmaf(acc[i][j][4 * rq + 1], alpha, bias4[1]);
        const float y2 = __builtin_fmaf(acc[i][j][4 * rq + 2], alpha, bias4[2]);
        const float y3 = __builtin_fmaf(acc[i][j][4 * rq + 3], alpha, bias4[3]);
        uint16_t* dst = cb + (int64_t)m * p.ldc + n;
        if (full4) {
          *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        } else {
          const uint32_t lo = pack_bf16x2(y0, y1), hi = pack_bf16x2(y2, y3);
          const uint16_t v4[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
          for (int e = 0; e < 4; ++e)
            if (n + e < p.n) dst[e] = v4[e];
        }
      }
    }
  }
  if constexpr (DRAIN) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  return false;
}

template <int TM, int TN>
__device__ __forceinline__ void zero_acc(v16f (&acc)[TN][TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};
}

// Global -> LDS side of a workgroup that runs the output tiles wg, wg + G,
// ... (wg its index among the G workgroups of its problem) as one stream of K
// stages of kBK bytes.
// Stage s lands in LDS buffer s % NBUF as [A tile | B tile]; each of the
// NW waves brings 1 KiB per buffer_load ... lds.  The next stage to issue is
// stage k of the workgroup's tile number it.  Each tile's operand strips get
// one buffer descriptor spanning the rest of the operand from the strip's
// start; a stage adds its K offset as the loads' scalar offset.  Past the
// workgroup's last tile the descriptors are empty: those loads fetch nothing
// and land zeros, so every stage issues the same number of loads and vmcnt
// counts stay fixed.
template <int BM, int BN, int NW, int NBUF, bool A_KC, bool B_KC>
struct TileLoader {
  static constexpr int A_BYTES = BM * kBK, B_BYTES = BN * kBK, STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / NW, B_LOADS = B_BYTES / 1024 / NW;
  static constexpr int LPS = A_LOADS + B_LOADS;   // loads per wave and stage
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small");

  int it = 0, k = 0, wg = 0, G = 1;
  uint32_t s = 0;
  v4i ra, rb;
  uint32_t a_voff[A_LOADS], b_voff[B_LOADS];
  uint32_t tail_oob = 0;   // bit j: this lane's load j lies past K in a tail stage

  struct Ctx {
    uint32_t sa, sb, la, lb;
    bool tail;
  };

  __device__ __forceinline__ void set_tile(const GemmKArgs& p, int v, int wave, int lane) {
    int bt, tmi, tni;
    map_tile(p, v, bt, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const uint32_t a_tile_off = A_KC ? (uint32_t)m0 * p.lda : (uint32_t)m0;
    const uint32_t b_tile_off = B_KC ? (uint32_t)n0 * p.ldb : (uint32_t)n0;
    ra = rsrc_words(p.a + bt * p.stride_a + a_tile_off, p.extent_a - a_tile_off);
    rb = rsrc_words(p.b + bt * p.stride_b + b_tile_off, p.extent_b - b_tile_off);
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j)
      a_voff[j] = slot_offset<A_KC, BM>((j * NW + wave) * 64 + lane, m0, p.m, p.lda);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j)
      b_voff[j] = slot_offset<B_KC, BN>((j * NW + wave) * 64 + lane, n0, p.n, p.ldb);
  }

  __device__ __forceinline__ void init(const GemmKArgs& p, int wave, int lane, int kt_full, int wg_, int G_) {
    wg = wg_;
    G = G_;
    // The same for every tile, as all tiles share K.
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j)
      tail_oob |= (uint32_t)(slot_kpos<A_KC, BM>((j * NW + wave) * 64 + lane) >= p.k - kt_full * kBK) << j;
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j)
      tail_oob |= (uint32_t)(slot_kpos<B_KC, BN>((j * NW + wave) * 64 + lane) >= p.k - kt_full * kBK)
                  << (A_LOADS + j);
    set_tile(p, wg, wave, lane);
  }

  // Scalar part of the next stage's loads: K offsets and LDS bases.
  __device__ __forceinline__ Ctx ctx(const GemmKArgs& p, const lds_char_t* smem, int wave, int kt_full) const {
    const uint32_t k0 = (uint32_t)k * kBK;
    Ctx c;
    c.sa = A_KC ? k0 : k0 * p.lda;
    c.sb = B_KC ? k0 : k0 * p.ldb;
    c.la = lds_address(smem + (s % NBUF) * STAGE) + wave * 1024;
    c.lb = c.la + A_BYTES;
    c.tail = k >= kt_full;
    return c;
  }

  __device__ __forceinline__ void issue_one(const Ctx& c, int j) const {
    const bool oob = c.tail && ((tail_oob >> j) & 1u);
    if (j < A_LOADS)
      load_lds16(ra, c.la + j * NW * 1024, oob ? kOOB : a_voff[j], c.sa);
    else
      load_lds16(rb, c.lb + (j - A_LOADS) * NW * 1024, oob ? kOOB : b_voff[j - A_LOADS], c.sb);
  }

  __device__ __forceinline__ void advance(const GemmKArgs& p, int my_tiles, int kt_total, int wave, int lane) {
    ++s;
    if (++k == kt_total) {
      k = 0;
      if (++it < my_tiles) {
        set_tile(p, wg + it * G, wave, lane);
      } else {
        ra[2] = 0;
        rb[2] = 0;
      }
    }
  }

  __device__ __forceinline__ void issue_next(const GemmKArgs& p, const lds_char_t* smem, int my_tiles, int kt_total,
                                             int kt_full, int wave, int lane) {
    const Ctx c = ctx(p, smem, wave, kt_full);
#pragma unroll
    for (int j = 0; j < LPS; ++j) issue_one(c, j);
    advance(p, my_tiles, kt_total, wave, lane);
  }
};

// The chunk holding K's last bytes also holds the row's padding; zero the
// bytes at or past K in the K-contiguous tiles of a tail stage's LDS buffer
// (one row per thread, at most 15 bytes each).
template <int BM, int BN, bool A_KC, bool B_KC, int kThreads>
__device__ __forceinline__ void zero_k_padding(lds_char_t* stage_buf, int k, int kt_full) {
  constexpr int A_BYTES = BM * kBK;
  const int kin = k - kt_full * kBK;
  const int c_lo = kin & ~15;
  constexpr int ROWS = (A_KC ? BM : 0) + (B_KC ? BN : 0);
  for (int r = threadIdx.x; r < ROWS; r += kThreads) {
    const bool in_a = A_KC && r < BM;
    const int row = in_a || !A_KC ? r : r - BM;
    lds_char_t* rp = stage_buf + (in_a ? 0 : A_BYTES) + row * kBK + (((c_lo >> 4) ^ swz_k(row)) << 4) - c_lo;
#pragma nounroll
    for (int b = kin; b < c_lo + 16; ++b) rp[b] = 0;
  }
}

// One wave's fragments of a stage: TM 32-row A fragments from row r0 and TN
// 32-column B fragments from column c0 of the tile.
template <int BM, int BN, int TM, int TN, bool A_KC, bool B_KC>
__device__ __forceinline__ void read_frags(const lds_char_t* stage_buf, int r0, int c0, int lane, v8i (&fa)[TM],
                                           v8i (&fb)[TN]) {
  const lds_char_t* sb = stage_buf + BM * kBK;
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[i] = load_frag<A_KC, BM>(stage_buf, r0 + i * 32, lane);
#pragma unroll
  for (int i = 0; i < TN; ++i) fb[i] = load_frag<B_KC, BN>(sb, c0 + i * 32, lane);
}

// Items of one kind (global loads, or fragment reads) issued after MFMA q of
// a stage, as the half-open range [slot_items(q), slot_items(q+1)): the n
// items spread evenly over the first nm MFMAs of one parity (q % 2 ==
// parity), so loads and fragment reads take turns after successive MFMAs.  A
// stage of one MFMA issues everything after it.
constexpr int slot_items(int q, int nm, int n, int parity) {
  if (nm == 1) return q == 0 ? 0 : n;
  if (q > nm) q = nm;                         // MFMAs past the first nm issue none
  const int slots = (nm + 1 - parity) / 2;    // MFMAs of this parity
  return (q + 1 - parity) / 2 * n / slots;    // items issued before MFMA q
}

template <int TM, int TN, int FA, int FB>
__device__ __forceinline__ void mfmas(v16f (&acc)[TN][TM], const v8i (&fa)[TM], const v8i (&fb)[TN]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], acc[i][j], FB, FA, 0, 0, 0, 0);
}

// General kernel: any tile of the family, any K.  Waves in a WGM x WGN grid
// each own a (BM/WGM) x (BN/WGN) block of the tile.  The workgroup has NBUF
// LDS stage buffers and keeps D = NBUF - 1 stages of global loads in flight.
// Every wave runs all stages: wait for stage s+1, barrier, then stage s's
// MFMAs interleaved with the loads of stage s+D and the LDS reads of stage
// s+1's fragments.
template <int BM, int BN, int NBUF>
constexpr int smem_bytes() { return NBUF * (BM + BN) * kBK; }

// Workgroup wg of the G that run one problem (a whole launch, or one part of
// a launch shared by two problems); smem: the workgroup's LDS stages.
template <int BM, int BN, int WGM, int WGN, int NBUF, bool A_KC, bool B_KC, int FA, int FB>
__device__ __forceinline__ void gemm_body(const GemmKArgs& p, lds_char_t* smem, int wg, int G) {
  constexpr int NW = WGM * WGN, kThreads = 64 * NW;   // waves in a WGM x WGN grid
  constexpr int WM = BM / WGM, WN = BN / WGN;          // C block of one wave
  constexpr int TM = WM / 32, TN = WN / 32;
  // Stages of global loads in flight.  The loads issued during stage s fill
  // stage s+D's buffer, which held stage s-1: every wave consumed that
  // stage's fragments in its MFMAs before the barrier that opened stage s,
  // so the barrier need not wait for LDS reads still in flight.
  constexpr int D = NBUF - 1;
  static_assert(D >= 2, "at least two stages in flight");
  using Loader = TileLoader<BM, BN, NW, NBUF, A_KC, B_KC>;
  constexpr int STAGE = Loader::STAGE, LPS = Loader::LPS;
  static_assert(TM >= 1 && TN >= 1, "tile too small");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = (wave % WGM) * WM, c0 = (wave / WGM) * WN;

  // The loads of a tile's first stages go out while the previous tile's last
  // stages compute, so the operand pipeline never drains between tiles and
  // the epilogue's stores overlap the loads.
  const int total = p.tiles_m * p.tiles_n * p.batch;
  const int my_tiles = (total - 1 - wg) / G + 1;     // >= 1: launches keep G <= total
  const int kt_total = (p.k + kBK - 1) / kBK;
  const int kt_full = p.k / kBK;
  const bool kfix = (p.k & 15) != 0;

  // The dequantization scales: scalar loads, issued now and first waited for
  // after the prologue's operand loads are in flight (they count on lgkmcnt,
  // so no later wait for them holds back an operand load).
  const float sa_inv = p.a_scale_inv[0], sb_inv = p.b_scale_inv[0];
  auto make_alpha = [&]() __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, sa_inv * sb_inv)));
  };

  v16f acc[TN][TM];
  zero_acc(acc);
  if (kt_total == 0) {          // K = 0: every output is bf16(bias) or zero
    const float alpha = make_alpha();
    for (int it = 0; it < my_tiles; ++it)
      store_c_tile<BM, BN, TM, TN, NW, LPS>(p, acc, wg + it * G, r0, c0, lane, wave, alpha, false, nullptr);
    return;
  }

  Loader ld;
  ld.init(p, wave, lane, kt_full, wg, G);
  auto buf = [&](uint32_t st) __attribute__((always_inline)) { return smem + (st % NBUF) * STAGE; };

  // Stage s+1 is visible to the whole workgroup: zero its K padding first if
  // it is a tail stage (K position next_k) of a K that is not a multiple of 16.
  auto fix_tail = [&](int s, int next_k) __attribute__((always_inline)) {
    if (kfix && next_k == kt_full) {
      zero_k_padding<BM, BN, A_KC, B_KC, kThreads>(buf(s + 1), p.k, kt_full);
      lds_barrier();
    }
  };

  // Fragments of two consecutive stages live in registers: while the MFMAs
  // of stage s run, the LDS reads of stage s+1 and the global loads of stage
  // s+D are in flight.
  v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];

  // One stage s: make stage s+1 visible (its loads have landed for every
  // wave), then issue stage s's MFMAs one by one, each followed, when READ,
  // by its share of the global loads of stage s+D (into the buffer stage s-1
  // freed) and of the LDS reads of stage s+1's fragments into na / nb.  The
  // barrier does not wait for this wave's LDS reads: the fragments of stage
  // s+1 are waited for where its MFMAs use them, the first ones read first.
  // Scheduling barriers keep that interleave: bursts of loads or LDS reads
  // right after the barrier left the matrix cores idle.  The wave runs at
  // raised priority while it issues the MFMA stream.  A tile's last stage
  // (not READ) issues MFMAs only: the buffer its loads would fill stages the
  // epilogue, and those loads go out after it.
  constexpr int NM = TM * TN, NF = TM + TN;
  auto stage = [&](auto read, int s, int next_k, const v8i (&fa)[TM], const v8i (&fb)[TN], v8i (&na)[TM],
                   v8i (&nb)[TN]) __attribute__((always_inline)) {
    constexpr bool READ = decltype(read)::value;
    // Global loads after the even-numbered MFMAs, fragment reads after the
    // odd ones (a stage of one MFMA issues both after it).
    constexpr int LP = 0, FP = NM == 1 ? 0 : 1;
    wait_stages<LPS, NBUF, D - 2>();
    stage_barrier();
    fix_tail(s, next_k);
    const typename Loader::Ctx c = ld.ctx(p, smem, wave, kt_full);
    const lds_char_t* sa = buf(s + 1);
    const lds_char_t* sb = sa + Loader::A_BYTES;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const int i = q / TM, j = q % TM;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], acc[i][j], FB, FA, 0, 0, 0, 0);
      if constexpr (READ) {
#pragma unroll
        for (int l = slot_items(q, NM, LPS, LP); l < slot_items(q + 1, NM, LPS, LP); ++l) ld.issue_one(c, l);
#pragma unroll
        for (int f = slot_items(q, NM, NF, FP); f < slot_items(q + 1, NM, NF, FP); ++f) {
          if (f < TM) na[f] = load_frag<A_KC, BM>(sa, r0 + f * 32, lane);
          else nb[f - TM] = load_frag<B_KC, BN>(sb, c0 + (f - TM) * 32, lane);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (READ) ld.advance(p, my_tiles, kt_total, wave, lane);
  };
  using Read = std::true_type;
  using NoRead = std::false_type;

  // Prologue: stages 0 .. D-1 in flight, stage 0's fragments in set 0.
#pragma unroll
  for (int st = 0; st < D; ++st) ld.issue_next(p, smem, my_tiles, kt_total, kt_full, wave, lane);
  const float alpha = make_alpha();
  wait_stages<LPS, NBUF, D - 1>();
  lds_barrier();
  if (kfix && kt_full == 0) {
    zero_k_padding<BM, BN, A_KC, B_KC, kThreads>(buf(0), p.k, kt_full);
    lds_barrier();
  }
  read_frags<BM, BN, TM, TN, A_KC, B_KC>(buf(0), r0, c0, lane, fa0, fb0);

  // Each tile starts with its first stage's fragments in set 0 and runs its
  // kt_total - 1 leading stages in pairs that alternate the two fragment
  // sets (one single stage first when their count is odd, its fragments
  // moved back to set 0).  Its last stage runs the MFMAs only; then the tile
  // is stored through the buffer that stage's loads fill (stage s0 +
  // kt_total - 1 + D's, free since the barrier that opened the stage), the
  // loads go out, the accumulators are cleared and the next stage's
  // fragments read into set 0, so the epilogue has the registers of both
  // fragment sets to itself.

  for (int it = 0; it < my_tiles; ++it) {
    const int s0 = it * kt_total;
    int kt = 0;
    if ((kt_total - 1) & 1) {
      stage(Read{}, s0, 1, fa0, fb0, fa1, fb1);
#pragma unroll
      for (int i = 0; i < TM; ++i) fa0[i] = fa1[i];
#pragma unroll
      for (int i = 0; i < TN; ++i) fb0[i] = fb1[i];
      kt = 1;
    }
    for (; kt < kt_total - 1; kt += 2) {
      stage(Read{}, s0 + kt, kt + 1, fa0, fb0, fa1, fb1);
      stage(Read{}, s0 + kt + 1, kt + 2, fa1, fb1, fa0, fb0);
    }
    stage(NoRead{}, s0 + kt_total - 1, 0, fa0, fb0, fa1, fb1);
    store_c_tile<BM, BN, TM, TN, NW, LPS>(p, acc, wg + it * G, r0, c0, lane, wave, alpha, true,
                                          buf(s0 + kt_total - 1 + D));
    // The staging reads have returned before the loads refill the area.  (The
    // loads after the last tile fetch nothing; skipping them with an early
    // exit made the compiler wait for every outstanding load in the K loop.)
    __builtin_amdgcn_s_waitcnt(lgkmcnt_zero_imm());
    ld.issue_next(p, smem, my_tiles, kt_total, kt_full, wave, lane);
    zero_acc(acc);
    read_frags<BM, BN, TM, TN, A_KC, B_KC>(buf(s0 + kt_total), r0, c0, lane, fa0, fb0);
  }
  // The loads of the stages past the last tile write this workgroup's LDS:
  // let them land before the workgroup ends.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------------------
// The four-wave 256x256 tile on load units of 128 K bytes (the body is a
// template over the tile size R, which also runs 128x128 and 64x64 tiles;
// the figures below are those of R = 256).
//
// An LDS-direct load that covers 128 contiguous bytes of each of 8 rows moves
// more bytes per cycle through the CU's address unit than one that covers 64
// bytes of 16 rows (measured on gfx950, with the fragment reads of a GEMM
// running beside the loads: 40 against 36 bytes per clock per CU).  At this
// tile the loads take about a third of the CU's load throughput, so queueing
// there stalled the waves' instruction streams, and with them the MFMAs.
//
// Here the operands move through LDS in units of 128 K bytes.  A "load stage"
// brings one operand's 256 rows (or K rows, crosswise) of one unit, 32 KiB, 8
// loads per wave; a unit's A and B are consecutive load stages, A first, and
// load stage j lands in slot j % 5 of a ring of five 32 KiB slots.  The MFMAs
// still run half-stages of 64 K bytes, reading the fragments of each half
// during the half before, and half-stage t issues load stage t + 4, whose
// slot held load stage t - 1.  So:
//  * at an odd half-stage t = 2U - 1 (about to read unit U's first half) the
//    wave waits until only load stage 2U + 2 may be in flight, i.e. unit U
//    has landed, and the workgroup meets at a barrier that also waits for its
//    LDS reads; no other half-stage waits or meets;
//  * the slot load stage t + 4 refills held load stage t - 1, whose last
//    fragment reads were issued in half-stage t - 2 at the latest and are
//    complete at the barrier of t - 1 or t;
//  * unit U's B has one to two half-stages from issue to use, its A two to
//    three.
// The tile's half-stages come in pairs (even: A loads, reads the unit's second
// half; odd: B loads, reads the next unit's first half), so the operand a
// stage loads and the fragment sets are fixed at compile time.  K tails: a
// partial last unit loads whatever lies past K (bytes of the operand, or
// zeros past its end) and, once landed, has its K positions past K zeroed in
// LDS in both operands, so the loads carry no per-lane tail test.

constexpr int kKU = 128;      // K bytes per load unit
constexpr int kUSlots = 5;    // slots of the ring

// K-contiguous slot [rows][128 B]: chunk c (0..7) of row r sits at chunk
// c ^ swz_k128(r).  A ds_read_b128 serves 16 lanes (256 bytes, all 64
// banks) at a time; 16 consecutive rows' reads of one chunk then land in 16
// distinct 16-byte bank groups (the first swizzle tried, (r >> 1) & 3,
// repeated every 8 rows and measured 34M conflict cycles per 8192^3 GEMM).
__device__ __forceinline__ int swz_k128(int r) { return (r >> 1) & 7; }

// 32 rows x 64 k (half h of the unit) of a K-contiguous slot: lane l gets row
// base + l % 32, k = 64 h + 32 (l / 32) + [0, 32).
__device__ __forceinline__ v8i frag_k128(const lds_char_t* slot, int base, int lane, int h) {
  const int row = base + (lane & 31);
  const int c0 = 4 * h + 2 * (lane >> 5);
  const int sw = swz_k128(row);
  const v4i lo = *(const lds_v4i_t*)(slot + row * kKU + ((c0 ^ sw) << 4));
  const v4i hi = *(const lds_v4i_t*)(slot + row * kKU + (((c0 + 1) ^ sw) << 4));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The same fragment from a crosswise slot [128 k][R B]: half h is k rows
// 64 h .. 64 h + 63, read as in the general kernel.
template <bool KC, int R>
__device__ __forceinline__ v8i frag_u128(const lds_char_t* slot, int base, int lane, int h) {
  if constexpr (KC) return frag_k128(slot, base, lane, h);
  else return frag_mn<R / 16>(slot + h * 64 * R, base, lane);
}

// Load l of a wave covers slots i = (l * NW + wave) * 64 + lane: for a
// K-contiguous operand rows 32 l + 8 wave + lane / 8, chunk lane % 8; for a
// crosswise one (R-byte k rows of CH = R / 16 chunks, KR = 64 / CH of them
// per load and wave) k rows NW KR l + KR wave + lane / CH, chunk lane % CH
// (R = 256: 16 l + 4 wave + lane / 16, chunk lane % 16).  The
// swizzle depends only on the row bits that l leaves alone, so a lane's byte
// offset is base + l * step with one per-lane base and a uniform step.
// Rows of a K-contiguous operand past M (N) start past the end of the
// operand, where the buffer descriptor's range check returns zeros; columns
// of a crosswise operand past N (M) are marked kOOB in the base.
template <bool KC, int NW, int R>
__device__ __forceinline__ uint32_t u128_base(int wave, int lane, int mn0, int mn_lim, uint32_t ld) {
  if constexpr (KC) {
    const int row = 8 * wave + (lane >> 3), lch = (lane & 7) ^ swz_k128(row);
    return (uint32_t)row * ld + (uint32_t)(lch << 4);
  } else {
    constexpr int CH = R / 16, KR = 64 / CH;   // chunks of a k row; k rows per wave and load
    const int kr = KR * wave + lane / CH, lch = (lane % CH) ^ swz_mn<CH>(kr);
    return mn0 + (lch << 4) < mn_lim ? (uint32_t)kr * ld + (uint32_t)(lch << 4) : kOOB;
  }
}
template <bool KC, int NW, int R>
__device__ __forceinline__ uint32_t u128_step(uint32_t ld) {
  return KC ? (uint32_t)(8 * NW) * ld : (uint32_t)(NW * 64 / (R / 16)) * ld;
}

template <int NW, bool A_KC, bool B_KC, int R>
struct UnitLoader {
  static constexpr int SLOT = R * kKU;                // bytes of one slot
  static constexpr int LPS = SLOT / 1024 / NW;        // loads per wave and load stage
  static_assert(NW == 4, "the slot mapping assumes four waves");
  int it = 0, j = 0, wg = 0, G = 1, units = 1;
  uint32_t lslot = 0;          // slot of the next load stage
  v4i ra, rb;
  uint32_t a_base = 0, b_base = 0;

  __device__ __forceinline__ void set_tile(const GemmKArgs& p, int v, int wave, int lane) {
    int bt, tmi, tni;
    map_tile(p, v, bt, tmi, tni);
    const int m0 = tmi * R, n0 = tni * R;
    const uint32_t a_tile_off = A_KC ? (uint32_t)m0 * p.lda : (uint32_t)m0;
    const uint32_t b_tile_off = B_KC ? (uint32_t)n0 * p.ldb : (uint32_t)n0;
    ra = rsrc_words(p.a + bt * p.stride_a + a_tile_off, p.extent_a - a_tile_off);
    rb = rsrc_words(p.b + bt * p.stride_b + b_tile_off, p.extent_b - b_tile_off);
    a_base = u128_base<A_KC, NW, R>(wave, lane, m0, p.m, p.lda);
    b_base = u128_base<B_KC, NW, R>(wave, lane, n0, p.n, p.ldb);
  }

  __device__ __forceinline__ void init(const GemmKArgs& p, int wave, int lane, int wg_, int G_) {
    wg = wg_;
    G = G_;
    units = (p.k + kKU - 1) / kKU;
    set_tile(p, wg, wave, lane);
  }

  // Load l of the next load stage (operand OP: 0 = A, 1 = B).
  template <int OP>
  __device__ __forceinline__ void issue_one(const GemmKArgs& p, const lds_char_t* smem, int wave, int l) const {
    const int u = j >> 1;
    const uint32_t lds = lds_address(smem + lslot * SLOT) + (uint32_t)((l * NW + wave) * 1024);
    constexpr bool KC = OP == 0 ? A_KC : B_KC;
    const uint32_t ld = OP == 0 ? p.lda : p.ldb;
    const uint32_t soff = KC ? (uint32_t)(u * kKU) : (uint32_t)(u * kKU) * ld;
    const uint32_t voff = (OP == 0 ? a_base : b_base) + (uint32_t)l * u128_step<KC, NW, R>(ld);
    load_lds16(OP == 0 ? ra : rb, lds, voff, soff);
  }

  __device__ __forceinline__ void advance(const GemmKArgs& p, int my_tiles, int wave, int lane) {
    lslot = lslot == kUSlots - 1 ? 0 : lslot + 1;
    if (++j == 2 * units) {
      j = 0;
      if (++it < my_tiles) {
        set_tile(p, wg + it * G, wave, lane);
      } else {
        ra[2] = 0;
        rb[2] = 0;
      }
    }
  }

  template <int OP>
  __device__ __forceinline__ void issue_stage(const GemmKArgs& p, const lds_char_t* smem, int my_tiles, int wave,
                                              int lane) {
#pragma unroll
    for (int l = 0; l < LPS; ++l) issue_one<OP>(p, smem, wave, l);
    advance(p, my_tiles, wave, lane);
  }
};

// Zero the K positions kin .. 127 (kin = K mod 128 > 0) of a tile's partial
// last unit in one operand's slot, over whatever the loads brought there
// (bytes of the operand past K, or zeros past its end): in a K-contiguous
// slot bytes kin .. 127 of every row (chunk c of row r at c ^ swz_k128(r)),
// in a crosswise slot the R-byte k rows kin .. 127.
template <bool KC, int kThreads, int R>
__device__ __forceinline__ void zero_k_tail_slot(lds_char_t* slot, int kin) {
  const v4i z = v4i{0, 0, 0, 0};
  if constexpr (KC) {
    for (int r = threadIdx.x; r < R; r += kThreads) {
      lds_char_t* rp = slot + r * kKU;
      const int sw = swz_k128(r);
#pragma nounroll
      for (int c = (kin + 15) >> 4; c < kKU / 16; ++c) *(lds_v4i_t*)(rp + ((c ^ sw) << 4)) = z;
      lds_char_t* cp = rp + (((kin >> 4) ^ sw) << 4);
#pragma nounroll
      for (int b = kin & 15; b != 0 && b < 16; ++b) cp[b] = 0;
    }
  } else {
    for (int i = threadIdx.x; i < (kKU - kin) * (R / 16); i += kThreads) *(lds_v4i_t*)(slot + kin * R + i * 16) = z;
  }
}

template <bool A_KC, bool B_KC, int FA, int FB, int R>
__device__ __forceinline__ void gemm_body_u128(const GemmKArgs& p, lds_char_t* smem, int wg, int G) {
  constexpr int BM = R, BN = R, NW = 4, kThreads = 256;
  constexpr int WM = R / 2, WN = R / 2, TM = WM / 32, TN = WN / 32, NM = TM * TN, NF = TM + TN;
  constexpr int kFragMfmas = NM >= 4 ? 3 * NM / 4 : NM;   // (one MFMA per wave: its reads follow it)
  using Loader = UnitLoader<NW, A_KC, B_KC, R>;
  constexpr int SLOT = Loader::SLOT, LPS = Loader::LPS;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = (wave % 2) * WM, c0 = (wave / 2) * WN;
  const int total = p.tiles_m * p.tiles_n * p.batch;
  const int my_tiles = (total - 1 - wg) / G + 1;
  const int units = (p.k + kKU - 1) / kKU;
  const int kt_total = 2 * units;                    // half-stages per tile
  const int kin = p.k % kKU;                         // K bytes of a partial last unit (0: none)
  constexpr int kStoreOps = staged_store_ops<TM, TN, LPS>();
  static_assert(LPS + kStoreOps <= 63, "vmcnt range");

  const float sa_inv = p.a_scale_inv[0], sb_inv = p.b_scale_inv[0];
  auto make_alpha = [&]() __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, sa_inv * sb_inv)));
  };

  v16f acc[TN][TM];
  zero_acc(acc);
  if (units == 0) {
    const float alpha = make_alpha();
    for (int it = 0; it < my_tiles; ++it)
      store_c_tile<BM, BN, TM, TN, NW, LPS>(p, acc, wg + it * G, r0, c0, lane, wave, alpha, false, nullptr);
    return;
  }

  Loader ld;
  ld.init(p, wave, lane, wg, G);
  auto slot = [&](uint32_t i) __attribute__((always_inline)) { return smem + i * SLOT; };
  uint32_t rslot = 0;          // A slot of the unit whose fragments are read next (its B: the next slot)
  auto next_slot = [](uint32_t s) { return s == kUSlots - 1 ? 0u : s + 1; };
  auto read_frags_u = [&](int h, v8i (&fa)[TM], v8i (&fb)[TN]) __attribute__((always_inline)) {
    const lds_char_t* sa = slot(rslot);
    const lds_char_t* sb = slot(next_slot(rslot));
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = frag_u128<A_KC, R>(sa, r0 + i * 32, lane, h);
#pragma unroll
    for (int i = 0; i < TN; ++i) fb[i] = frag_u128<B_KC, R>(sb, c0 + i * 32, lane, h);
  };
  // Zero the K padding of the unit about to be read when it is a partial
  // last unit of a tile (the slots are visible: its loads have landed).
  auto fix_tail_u = [&](bool last_unit) __attribute__((always_inline)) {
    if (kin != 0 && last_unit) {
      zero_k_tail_slot<A_KC, kThreads, R>(slot(rslot), kin);
      zero_k_tail_slot<B_KC, kThreads, R>(slot(next_slot(rslot)), kin);
      lds_barrier();
    }
  };
  // Set when the last epilogue stored through LDS: its kStoreOps stores sit
  // between the load stages the next odd half-stage waits for and the one it
  // leaves in flight.
  bool after_store = false;

  v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];

  // Half-stage t.  ODD: wait for the next unit, barrier, advance the read
  // slot to it.  The MFMAs of fa / fb, each followed by its share of
  // load stage t + 4 (operand A for even t, B for odd) and of the fragment
  // reads of half-stage t + 1 (the same unit's second half for even t, the
  // next unit's first half for odd t).
  auto stage = [&](auto odd, auto first, bool next_last_unit, const v8i (&fa)[TM], const v8i (&fb)[TN],
                   v8i (&na)[TM], v8i (&nb)[TN]) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(odd)::value, FIRST = decltype(first)::value;
    constexpr int OP = ODD ? 1 : 0, H = ODD ? 0 : 1;
    if constexpr (ODD) {
      if (after_store) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS + kStoreOps));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
      after_store = false;
      lds_barrier();
      rslot = next_slot(next_slot(rslot));
      fix_tail_u(next_last_unit);
    }
    const lds_char_t* sa = slot(rslot);
    const lds_char_t* sb = slot(next_slot(rslot));
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const int i = q / TM, j = q % TM;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], FIRST ? v16f{} : acc[i][j], FB,
                                                                 FA, 0, 0, 0, 0);
#pragma unroll
      for (int l = slot_items(q, NM, LPS, 0); l < slot_items(q + 1, NM, LPS, 0); ++l)
        ld.template issue_one<OP>(p, smem, wave, l);
      // Fragment reads only after the first three quarters of the MFMAs, so
      // they have landed when the next half-stage starts.
#pragma unroll
      for (int f = slot_items(q, kFragMfmas, NF, 1); f < slot_items(q + 1, kFragMfmas, NF, 1); ++f) {
        if (f < TM) na[f] = frag_u128<A_KC, R>(sa, r0 + f * 32, lane, H);
        else nb[f - TM] = frag_u128<B_KC, R>(sb, c0 + (f - TM) * 32, lane, H);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    ld.advance(p, my_tiles, wave, lane);
  };
  using T = std::true_type;
  using F = std::false_type;

  // Prologue: load stages 0 .. 3 (units 0 and 1) in flight; unit 0 read.
  ld.template issue_stage<0>(p, smem, my_tiles, wave, lane);
  ld.template issue_stage<1>(p, smem, my_tiles, wave, lane);
  ld.template issue_stage<0>(p, smem, my_tiles, wave, lane);
  ld.template issue_stage<1>(p, smem, my_tiles, wave, lane);
  const float alpha = make_alpha();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPS));
  lds_barrier();
  fix_tail_u(units == 1);
  read_frags_u(0, fa0, fb0);

  // The last half-stage of a tile loads and reads ahead into the next tile
  // like any other (past the last tile its loads fetch nothing and its reads
  // are never used).  A tile's first half-stage starts its accumulators from
  // zero in the MFMAs themselves, so they carry nothing from tile to tile.
  for (int it = 0; it < my_tiles; ++it) {
    const bool next_tile_one_unit = units == 1 && it + 1 < my_tiles;
    stage(F{}, T{}, false, fa0, fb0, fa1, fb1);
    stage(T{}, F{}, units == 2 || next_tile_one_unit, fa1, fb1, fa0, fb0);
    for (int kt = 2; kt < kt_total; kt += 2) {
      stage(F{}, F{}, false, fa0, fb0, fa1, fb1);
      stage(T{}, F{}, kt + 2 == kt_total - 2, fa1, fb1, fa0, fb0);   // (units > 1 here)
    }
    // The tile goes out through the slot of its last B, which the next
    // half-stage's loads refill (free since the barrier of the last
    // half-stage; each wave stages in the pieces its own loads fill, and its
    // staging reads have returned before its stores issue).  The stores
    // trail the loads the next odd half-stage waits for, and its wait lets
    // them stay in flight.
    after_store = store_c_tile<BM, BN, TM, TN, NW, LPS, true>(p, acc, wg + it * G, r0, c0, lane, wave, alpha,
                                                              true, slot(ld.lslot));
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// One problem per launch: workgroup blockIdx.x of gridDim.x.
template <int BM, int BN, int WGM, int WGN, int NBUF, int OCC, bool A_KC, bool B_KC, int FA, int FB>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void gemm_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[smem_bytes<BM, BN, NBUF>()];
  gemm_body<BM, BN, WGM, WGN, NBUF, A_KC, B_KC, FA, FB>(p, (lds_char_t*)smem_raw, (int)blockIdx.x,
                                                       (int)gridDim.x);
}

// The four-wave 256x256 tile on 128-byte load units (one problem per launch).
template <bool A_KC, bool B_KC, int FA, int FB>
__global__ __launch_bounds__(256, 1) void gemm_u128_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kUSlots * 256 * kKU];
  gemm_body_u128<A_KC, B_KC, FA, FB, 256>(p, (lds_char_t*)smem_raw, (int)blockIdx.x, (int)gridDim.x);
}

// The same body on a 128x128 tile (each wave a 64x64 block; five 16 KiB
// slots, two workgroups per CU).
template <bool A_KC, bool B_KC, int FA, int FB>
__global__ __launch_bounds__(256, 2) void gemm_u128s_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kUSlots * 128 * kKU];
  gemm_body_u128<A_KC, B_KC, FA, FB, 128>(p, (lds_char_t*)smem_raw, (int)blockIdx.x, (int)gridDim.x);
}

// And on a 64x64 tile (each wave a 32x32 block; five 8 KiB slots, four
// workgroups per CU).
template <bool A_KC, bool B_KC, int FA, int FB>
__global__ __launch_bounds__(256, 4) void gemm_u128t_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kUSlots * 64 * kKU];
  gemm_body_u128<A_KC, B_KC, FA, FB, 64>(p, (lds_char_t*)smem_raw, (int)blockIdx.x, (int)gridDim.x);
}

// Two independent problems in one launch (a layer's dX and dW) on that tile:
// workgroups [0, g0) run the first, the rest the second, each as a grid of
// its own.  The two share the tile, the formats and the LDS of a workgroup;
// only the operand orientations differ.  g0 is a multiple of 8 whenever the
// first problem's workgroups run more than one tile each, so the second keeps
// the tile-to-XCD mapping of a launch of its own.
template <bool A_KC0, bool B_KC0, bool A_KC1, bool B_KC1, int FA, int FB>
__global__ __launch_bounds__(256, 2) void gemm_pair_u128s_kernel(GemmKArgs p0, GemmKArgs p1, int g0) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kUSlots * 128 * kKU];
  const int wg = (int)blockIdx.x;
  if (wg < g0)
    gemm_body_u128<A_KC0, B_KC0, FA, FB, 128>(p0, (lds_char_t*)smem_raw, wg, g0);
  else
    gemm_body_u128<A_KC1, B_KC1, FA, FB, 128>(p1, (lds_char_t*)smem_raw, wg - g0, (int)gridDim.x - g0);
}

// The same on the 64x64 unit tile.
template <bool A_KC0, bool B_KC0, bool A_KC1, bool B_KC1, int FA, int FB>
__global__ __launch_bounds__(256, 4) void gemm_pair_u128t_kernel(GemmKArgs p0, GemmKArgs p1, int g0) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kUSlots * 64 * kKU];
  const int wg = (int)blockIdx.x;
  if (wg < g0)
    gemm_body_u128<A_KC0, B_KC0, FA, FB, 64>(p0, (lds_char_t*)smem_raw, wg, g0);
  else
    gemm_body_u128<A_KC1, B_KC1, FA, FB, 64>(p1, (lds_char_t*)smem_raw, wg - g0, (int)gridDim.x - g0);
}

// ---------------------------------------------------------------------------
// Instantiation helpers of the picker files.  The template arguments of each
// tile (waves as WGM x WGN, LDS stages, workgroups per CU) live here, next to
// the kernels; gemm.hip's tile table gives the same tiles' sizes and waves.

template <int BM, int BN, int WGM, int WGN, int ST, int OCC, bool AKC, bool BKC>
GemmFn pick_fmt(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_kernel<BM, BN, WGM, WGN, ST, OCC, AKC, BKC, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_kernel<BM, BN, WGM, WGN, ST, OCC, AKC, BKC, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_kernel<BM, BN, WGM, WGN, ST, OCC, AKC, BKC, 0, 1>;
  return gemm_kernel<BM, BN, WGM, WGN, ST, OCC, AKC, BKC, 1, 1>;
}

template <bool AKC, bool BKC>
GemmFn pick_u128(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_u128_kernel<AKC, BKC, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_u128_kernel<AKC, BKC, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_u128_kernel<AKC, BKC, 0, 1>;
  return gemm_u128_kernel<AKC, BKC, 1, 1>;
}

template <bool AKC, bool BKC>
GemmFn pick_u128s(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_u128s_kernel<AKC, BKC, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_u128s_kernel<AKC, BKC, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_u128s_kernel<AKC, BKC, 0, 1>;
  return gemm_u128s_kernel<AKC, BKC, 1, 1>;
}

template <bool AKC, bool BKC>
GemmFn pick_u128t(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_u128t_kernel<AKC, BKC, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_u128t_kernel<AKC, BKC, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_u128t_kernel<AKC, BKC, 0, 1>;
  return gemm_u128t_kernel<AKC, BKC, 1, 1>;
}

template <bool AKC, bool BKC>
GemmFn pick_large(int tile, int fa, int fb) {
  switch (tile) {
    case 5: return pick_fmt<256, 256, 2, 4, 4, 1, AKC, BKC>(fa, fb);
    case 6: return pick_fmt<256, 256, 4, 2, 4, 1, AKC, BKC>(fa, fb);
    default: return pick_u128<AKC, BKC>(fa, fb);
  }
}

// The 256x128 / 128x256 tiles with both operands crosswise (TN) run one
// workgroup per CU: at two, the transposed fragment reads leave too few
// registers and the compiler spills hundreds of them.
template <bool AKC, bool BKC>
GemmFn pick_small(int tile, int fa, int fb) {
  constexpr int kOccRect = AKC || BKC ? 2 : 1;
  switch (tile) {
    case 1: return pick_fmt<128, 128, 2, 2, 4, 2, AKC, BKC>(fa, fb);
    case 2: return pick_fmt<64, 64, 2, 2, 4, 4, AKC, BKC>(fa, fb);
    case 3: return pick_fmt<256, 128, 2, 2, 3, kOccRect, AKC, BKC>(fa, fb);
    case 7: return pick_u128s<AKC, BKC>(fa, fb);
    case 8: return pick_u128t<AKC, BKC>(fa, fb);
    default: return pick_fmt<128, 256, 2, 2, 3, kOccRect, AKC, BKC>(fa, fb);
  }
}

}  // namespace
}  // namespace fp8ds
