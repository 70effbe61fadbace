// The fused kernel of libmoegg for gfx950 (CDNA4): contiguous grouped
// block-scaled GEMM with fused epilogue.  Included by one translation unit
// per operand family (inst_*.hip), which instantiate it.
//
// Method ("Grouped GEMM + Quant (SM100)", "Grouped GEMM + SwiGLU (SM100)",
// "Grouped GEMM + sReLU (SM100)", "Grouped GEMM + dGLU (SM100)", §Equations):
// rows m of A in [padded_offsets[g-1], padded_offsets[g]) are multiplied by
// expert g's weight B[g] (N x K, K-major) with per-32-element E8M0 block
// scales on both operands, scaled by alpha_g (alpha_g^2 for the dSwiGLU
// backward), then the activation / gating / output-formatting epilogue.
//
// Mapping onto CDNA4:
//  * persistent workgroups, one per CU (8 wave64s, about 140 KB of LDS),
//    walk a list of 256 x 256 output tiles.  A tile never straddles two
//    experts: expert g's padded rows are cut into 256-row tiles plus one
//    128-row tile when its row count is an odd number of 128-row blocks.
//    Each workgroup builds the per-expert tile prefix sums in LDS from
//    padded_offsets once and maps a linear tile index to (expert, first row,
//    first column) by binary search.  Linear tile indices are handed out so
//    that the workgroups resident on one XCD (one L2) work on a compact patch
//    of neighbouring tiles at any time.
//  * the contraction runs on the block-scaled matrix cores:
//    v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, E5M2 or E2M1 operands, one E8M0 byte
//    per lane and operand selects the scale of that lane's 32 K-elements) or
//    v_mfma_f32_32x32x16_bf16.  The weight tile is the instruction's first
//    operand and the token tile the second, so an accumulator lane holds one
//    token row and 16 output columns (4 runs of 4 contiguous columns): row
//    reductions are lane-local.
//  * K advances in steps of 128 bytes per row (128 E4M3 or E5M2, 256 E2M1 or
//    64 BF16 elements).  Two LDS stages (A, B and their scale words) are
//    filled by direct global -> LDS loads issued up to two steps ahead,
//    spread over the clusters of the ping-pong schedule (see the tile loop).
//    With an even step count the next tile's first stage is loaded during
//    the tile's last two steps, otherwise while its epilogue runs.
//  * the epilogue works on the fp32 accumulators in registers; column
//    blocks of the FP8 output are reduced through a per-wave LDS transpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moegg_internal.h"

namespace moegg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));   // native vectors (HIP's uint4
typedef uint32_t v2u __attribute__((ext_vector_type(2)));   // struct defeats SROA)

constexpr int kBK = 128;          // bytes of K per row and pipeline stage (one cache line)
constexpr int kBandM = 8;         // m-tiles per raster band (L2 reuse of B)
constexpr int kTPitch = 36;       // floats per row of the epilogue transpose (see quant_codes)
constexpr int kScratch = 8192;    // bytes of epilogue scratch per wave

// Unrolled loop whose index is a compile-time constant (instruction
// immediates such as the MFMA scale byte selectors need one).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRcp448 = 1.0f / 448.0f;   // rcp_max of E4M3, rounded to fp32

// ---------------------------------------------------------------------------
// device codecs
// ---------------------------------------------------------------------------

// Two fp32 -> two bf16 (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
}

// E8M0 byte of the smallest power of two >= sf (sf >= 0), clamped to [0, 254].
__device__ __forceinline__ uint32_t e8m0_ceil(float sf) {
  const uint32_t u = __float_as_uint(sf);
  const uint32_t e = u >> 23, m = u & 0x7FFFFFu;
  uint32_t b = (e == 0) ? (m > 0x400000u ? 1u : 0u) : e + (m != 0u ? 1u : 0u);
  return b > 254u ? 254u : b;
}

// 2^(127 - byte), exact.
__device__ __forceinline__ float e8m0_inverse(uint32_t byte) {
  return byte < 254u ? __uint_as_float((254u - byte) << 23) : __uint_as_float(0x00400000u);
}

// E8M0 byte -> its value 2^(byte - 127) as fp32 (byte 0 is the subnormal
// 2^-127), the form the scaled conversions take.
__device__ __forceinline__ float e8m0_value(uint32_t byte) {
  return __uint_as_float(byte ? byte << 23 : 0x00400000u);
}

// Four fp32 -> four E4M3 codes, RNE by the conversion unit, packed
// little-endian (a is the lowest byte).  The inputs are block-scaled values,
// |x| <= 448 (1 + 2^-22) for finite D, which the conversion rounds to +-448;
// non-finite D gives the E4M3 NaN code.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// Same for x / 2^(byte - 127) with the block scale folded into the conversion
// (v_cvt_scalef32_pk_fp8_f32 takes the exponent of `scale`): equal to
// e4m3x4(x * 2^(127 - byte)) for every finite x.
__device__ __forceinline__ uint32_t e4m3x4_scaled(float a, float b, float c, float d, float scale) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, a, b, scale, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, scale, true);
  return static_cast<uint32_t>(static_cast<uint16_t>(w.x)) | (static_cast<uint32_t>(static_cast<uint16_t>(w.y)) << 16);
}

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)); saturates to 0 / 1 at the extremes.
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// tanh(x) for x >= 0: odd Taylor series below 1/8 (error < 2e-10), else
// 1 - 2 / (1 + e^2x) (one reciprocal and one fused multiply-add; e^2x
// overflowing to infinity gives exactly 1).  Result in [0, 1] by
// construction, so that the clamp min(tanh, 1) needs no instruction.
__device__ __forceinline__ float tanh_nonneg(float x) {
  const float x2 = x * x;
  const float series = x * (1.0f + x2 * (-1.0f / 3.0f + x2 * (2.0f / 15.0f + x2 * (-17.0f / 315.0f))));
  const float big = fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(2.0f * kLog2e * x)), 1.0f);
  return x < 0.125f ? series : big;
}

// tanh(x) and sech(x)^2 / 4 = (1 - tanh(x)^2) / 4 for x >= 0, the latter
// free of the cancellation of 1 - t*t as t approaches 1: with e = e^-2x and
// r = 1 / (1 + e), t = (1 - e) / (1 + e) = 1 - 2 e r (in [0, 1]; below 1/8
// the odd series, as in tanh_nonneg) and sech^2 / 4 = e / (1 + e)^2 = e r^2
// for every x (no subtraction; the caller folds the 4 into its factors).
__device__ __forceinline__ void tanh_sech2_nonneg(float x, float& t, float& sech2_4) {
  const float x2 = x * x;
  const float series = x * (1.0f + x2 * (-1.0f / 3.0f + x2 * (2.0f / 15.0f + x2 * (-17.0f / 315.0f))));
  const float e = __builtin_amdgcn_exp2f(-2.0f * kLog2e * x);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  const float er = e * r;
  t = x < 0.125f ? series : fmaf(-2.0f, er, 1.0f);
  sech2_4 = er * r;
}

// Cross-lane helpers on the VALU (DPP and the gfx950 permlane swaps), no LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max over the 32 lanes of each half-wave (lanes 0-31 and 32-63 separately):
// pairs, quads, 8-lane halves of a row (mirror), 16-lane rows (mirror), then
// rows 0/1 and 2/3 exchanged by v_permlane16_swap.
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));     // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));     // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));    // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));    // row_mirror
  const v2u sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw.x), __uint_as_float(sw.y));
}

__device__ __forceinline__ float wave_max(float v) {
  v = half_max(v);
  const v2u sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw.x), __uint_as_float(sw.y));
}

// Sum of the two halves' values (lane l and lane l ^ 32), in every lane.
__device__ __forceinline__ float halves_sum(float v) {
  const v2u sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw.x) + __uint_as_float(sw.y);
}

// Max of the two halves' values, in every lane.
__device__ __forceinline__ float halves_max(float v) {
  const v2u sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw.x), __uint_as_float(sw.y));
}

// The value lane l ^ 32 holds, in every lane.
__device__ __forceinline__ uint32_t other_half(uint32_t v, int hi) {
  const v2u sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return hi ? sw.x : sw.y;
}

// max(|a|, |b|, c) (one v_max3_f32 with abs modifiers).
__device__ __forceinline__ float max_abs2(float c, float a, float b) {
  return fmaxf(fmaxf(fabsf(a), fabsf(b)), c);
}

// Epilogue addressing: every output address is a wave-uniform base (the
// wave's first row and the block's first column) plus a 32-bit per-lane byte
// offset.  Offsets stay below 2^32: 128 rows of at most 2^21 two-byte
// elements.
// The integer round trip keeps the compiler from carrying extra 64-bit
// pointers through the epilogue (plain byte-pointer arithmetic measured
// 2-7 % slower: more scalar registers live, more spills); the cast to the
// global address space then makes the accesses global_* rather than flat_*:
// a flat store also counts on the LDS counter, so the LDS waits of the next
// output block would wait for it (measured 1-3 % faster on every workload).
template <typename T>
__device__ __forceinline__ T* at(T* base, uint32_t byte_off) {
  typedef __attribute__((address_space(1))) T GT;
  GT* const g = (GT*)(reinterpret_cast<uintptr_t>(base) + static_cast<uint64_t>(byte_off));
  return (T*)g;
}

// Element i of read-only kernel data at a wave-uniform index, read through
// the scalar cache (s_load): it waits on the scalar-memory counter only, not
// behind vector stores still in flight.
template <typename T>
__device__ __forceinline__ T sload(const T* base, int i) {
  return ((const __attribute__((address_space(4))) T*)base)[i];
}

// 16 values of one row (one 32-column tile) as bf16, in 16-byte pieces.
// This lane holds columns 8j + 4*hi + [0, 4) (8 bytes each);
// v_permlane32_swap(x, y) exchanges x of lanes 32-63 with y of lanes 0-31, so
// swapping the runs of j = 2i and 2i + 1 leaves lane hi = 0 with columns
// 16i + [0, 8) and lane hi = 1 with 16i + [8, 16): piece q[i] is the row's
// bytes [32 i + 16 hi, +16).
__device__ __forceinline__ void bf16_pieces(const float* v, v4u* q) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t a0 = bf16x2(v[8 * i + 0], v[8 * i + 1]), a1 = bf16x2(v[8 * i + 2], v[8 * i + 3]);
    const uint32_t b0 = bf16x2(v[8 * i + 4], v[8 * i + 5]), b1 = bf16x2(v[8 * i + 6], v[8 * i + 7]);
    const v2u s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
    const v2u s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
    q[i] = v4u{s0.x, s1.x, s0.y, s1.y};
  }
}

// One row's 32 bf16 of a 32-column tile into this lane's layout, runs of 4
// at columns 8j + 4*hi (w[j], 8 bytes each): the inverse of bf16_pieces.
// q[i] holds the row's bytes [32 i + 16 hi, + 16) (two 16-byte reads per
// lane cover 32 contiguous bytes of every row); the runs are exchanged with
// lane ^ 32.
__device__ __forceinline__ void unpack_bf16(const v4u* q, v2u* w) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const v2u s0 = __builtin_amdgcn_permlane32_swap(q[i].x, q[i].z, false, false);
    const v2u s1 = __builtin_amdgcn_permlane32_swap(q[i].y, q[i].w, false, false);
    w[2 * i] = v2u{s0.x, s1.x};
    w[2 * i + 1] = v2u{s0.y, s1.y};
  }
}

// One row's 32 E4M3 codes of a 32-column tile as this lane's 16-byte piece.
// This lane holds the codes of columns 8j + 4*hi + [0, 4) (w[j]).
// v_permlane32_swap(x, y) exchanges x of lanes 32-63 with y of lanes 0-31:
// with x = w[j], y = w[j+2] lane hi = 0 ends with (own w[j], partner's w[j])
// = columns 8j + [0, 8) and lane hi = 1 with (partner's w[j+2], own w[j+2])
// = columns 16 + 8j + [0, 8): the piece is the row's bytes [16 hi, +16).
__device__ __forceinline__ v4u e4m3_piece(const uint32_t* w) {
  const v2u s0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  const v2u s1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  return v4u{s0.x, s0.y, s1.x, s1.y};
}

// Whole-segment stores of one 32-row block of output bytes.  Lane (row l32,
// half hi) holds, for each 32-byte column piece b < W / 32 of the block, the
// row's bytes [32 b + 16 hi, +16) (q[b]: the layout of the pieces above).
// Stored as they are, one instruction writes 32 rows x 32 bytes; here they
// pass through the wave's LDS scratch `lds` (32 x W bytes) and come back so
// that each instruction writes 1024 / W whole W-byte row segments (W / 16
// lanes per row): the memory system takes 2x (W = 64) or 4x (W = 128) fewer,
// larger requests.  Chunk c of row r sits at chunk slot c ^ swz(r), so that
// the 16-lane groups of the writes (16 rows, one chunk) and of the reads
// (whole rows) hit 16 distinct bank quads.  Only chunks below `valid` bytes
// of a row are stored.  `base`: the block's first byte; `pitch`: bytes per
// row.  Lanes read what other lanes wrote: wave-scope fences around a wave
// barrier (no instructions: the LDS serves one wave's accesses in order) make
// the compiler keep every write ahead of the reads, and this call's accesses
// after the scratch's earlier uses and before its later ones; without them it
// may treat a write that its own lane never reads back as dead on some paths.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
template <int W>
__device__ __forceinline__ void store_rows(uint8_t* base, uint32_t pitch, const v4u* q, float* lds, int lid,
                                           uint32_t valid = W) {
  static_assert(W == 64 || W == 128, "segment width");
  constexpr int CPR = W / 16;                      // 16-byte chunks per row
  auto slot = [](int r, int c) __attribute__((always_inline)) {
    return W == 128 ? c ^ ((r >> 1) & 7) : c ^ ((r >> 2) & 3);
  };
  const int l32 = lid & 31, hi = lid >> 5;
  wave_sync_lds();
#pragma unroll
  for (int b = 0; b < W / 32; ++b)
    *reinterpret_cast<v4f*>(lds + l32 * (W / 4) + slot(l32, 2 * b + hi) * 4) = __builtin_bit_cast(v4f, q[b]);
  wave_sync_lds();
  const int c = lid % CPR;
  // all reads in flight together (pinned here, not sunk into the store
  // condition), then the stores
  v4f v[W / 32];
#pragma unroll
  for (int k = 0; k < W / 32; ++k) {
    const int r = k * (64 / CPR) + lid / CPR;
    v[k] = *reinterpret_cast<const v4f*>(lds + r * (W / 4) + slot(r, c) * 4);
  }
#pragma unroll
  for (int k = 0; k < W / 32; ++k) asm volatile("" : "+v"(v[k]));
  if (static_cast<uint32_t>(c * 16) < valid) {
#pragma unroll
    for (int k = 0; k < W / 32; ++k) {
      const int r = k * (64 / CPR) + lid / CPR;
      *at(reinterpret_cast<v4u*>(base), r * pitch + c * 16) = __builtin_bit_cast(v4u, v[k]);
    }
  }
  wave_sync_lds();
}

// FP8 row + column quantisation of one 32 x 32 output tile ("Grouped GEMM +
// Quant (SM100)", §Equations Step 3 and §Diagram Row/Col Quantize).
// dn[v] = D * norm_const for row m (this lane's row) and column
// 8*(v/4) + 4*hi + v%4 of the tile.  A row block is one row's 32 values
// (this lane and lane ^ 32); a column block is one column over the tile's 32
// rows, reduced through the wave's LDS scratch:
//   T: 32 rows x kTPitch floats, row r at T + r * kTPitch (16-byte writes of
//      4 columns; the pitch keeps every 16-lane group of writes on distinct
//      banks),
//   S: 32 floats, the inverse column scales.
// Lanes 0-31 read rows 0-15 of column l, lanes 32-63 rows 24-31 then 16-23,
// so that both halves of a 64-lane read hit complementary bank ranges.
// Outputs: this lane's 16-byte pieces of its row of D (prow) and of D_col
// (pcol), see e4m3_piece; the row block's scale byte at sfW + sfoff.
// Returns the E8M0 byte of this lane's column (l % 32) block.
__device__ __forceinline__ uint32_t quant_codes(float* T, float* S, uint8_t* sfW, uint32_t sfoff, int hi, int l32,
                                                const float* dn, v4u& prow, v4u& pcol) {
  // the previous call's cross-lane reads of T and S stay ahead of this
  // call's writes
  __builtin_amdgcn_wave_barrier();
  // ---- row block ----
  float ra = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; v += 2) ra = max_abs2(ra, dn[v], dn[v + 1]);
  ra = halves_max(ra);
  const uint32_t br = e8m0_ceil(ra * kRcp448);
  const float sr = e8m0_value(br);

  // ---- column blocks through LDS ----
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<v4f*>(T + l32 * kTPitch + 8 * j + 4 * hi) = v4f{dn[4 * j], dn[4 * j + 1], dn[4 * j + 2], dn[4 * j + 3]};
  // lanes read what other lanes of the wave wrote: keep the compiler from
  // moving LDS accesses across this point (the LDS executes one wave's
  // accesses in order)
  __builtin_amdgcn_wave_barrier();
  float cm = 0.0f;
  const float* c0 = T + l32 + (hi ? 24 * kTPitch : 0);      // rows [0, 8) / [24, 32)
  const float* c1 = T + l32 + (hi ? 8 * kTPitch : 0);       // rows [8, 16) / [16, 24) at r + 8
  // all sixteen reads in flight together, then one wait
  float cv[16];
#pragma unroll
  for (int r = 0; r < 8; ++r) cv[r] = c0[r * kTPitch];
#pragma unroll
  for (int r = 8; r < 16; ++r) cv[r] = c1[r * kTPitch];
  asm volatile("" : "+v"(cv[0]), "+v"(cv[1]), "+v"(cv[2]), "+v"(cv[3]), "+v"(cv[4]), "+v"(cv[5]), "+v"(cv[6]),
               "+v"(cv[7]), "+v"(cv[8]), "+v"(cv[9]), "+v"(cv[10]), "+v"(cv[11]), "+v"(cv[12]), "+v"(cv[13]),
               "+v"(cv[14]), "+v"(cv[15]));
#pragma unroll
  for (int r = 0; r < 16; r += 2) cm = max_abs2(cm, cv[r], cv[r + 1]);
  cm = halves_max(cm);
  const uint32_t bc = e8m0_ceil(cm * kRcp448);
  if (hi == 0) S[l32] = e8m0_inverse(bc);
  __builtin_amdgcn_wave_barrier();
  v4f sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sc[j] = *reinterpret_cast<const v4f*>(S + 8 * j + 4 * hi);

  uint32_t wr[4], wc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wr[j] = e4m3x4_scaled(dn[4 * j], dn[4 * j + 1], dn[4 * j + 2], dn[4 * j + 3], sr);
    wc[j] = e4m3x4(dn[4 * j] * sc[j].x, dn[4 * j + 1] * sc[j].y, dn[4 * j + 2] * sc[j].z, dn[4 * j + 3] * sc[j].w);
  }
  prow = e4m3_piece(wr);
  pcol = e4m3_piece(wc);
  if (hi == 0) *at(sfW, sfoff) = static_cast<uint8_t>(br);
  return bc;
}


// ---------------------------------------------------------------------------
// the fused kernel
// ---------------------------------------------------------------------------

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane i of the wave writes lds_base + 16 i.  `lds_base` must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
// Same with 4 bytes per lane (global_load_lds_dword).
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}
// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// One output tile: rows [row0, row0 + rows) of expert g, GEMM columns
// [n0, n0 + 256).  rows is 0 (nothing to store), 128 or 256.
struct Tile {
  int g, row0, rows, n0;
  const uint8_t* bg;    // expert g's weights (row 0) and SFB bytes (row 0)
  const uint8_t* sg;
};

template <int AB, int ACT, int OUT>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(KernelArgs p) {
  constexpr int BM = kBM, BN = kBN, BK = kBK;
  constexpr int NW = kThreads / 64;  // 8 waves: 2 (m) x 4 (n), waves w and w+4 share a SIMD
  constexpr int WM = BM / 2;         // rows per wave (128)
  constexpr int WN = BN / 4;         // GEMM columns per wave (64)
  constexpr int TM = WM / 32;        // 32-row MFMA tiles per wave (4)
  constexpr int TN = WN / 32;        // 32-column MFMA tiles per wave (2)
  constexpr bool MX = AB != AB_BF16;
  constexpr bool F8 = AB == AB_E4M3 || AB == AB_E5M2;   // 8-bit operands (one layout, two MFMA formats)
  constexpr int FMT8 = AB == AB_E5M2 ? 1 : 0;           // MFMA operand format: E4M3 0, E5M2 1
  constexpr int SW = AB == AB_E2M1 ? 2 : 1;          // scale words per row per step
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  constexpr int AH_BYTES = A_BYTES / 2;              // one of the two A row halves
  constexpr int SA_WORDS = MX ? SW * BM : 1, SB_WORDS = MX ? SW * BN : 1;
  static_assert(NW == 8 && TM == 4 && TN == 2, "tile shape");
  static_assert(2 * kScratch <= AH_BYTES && 4 * kScratch <= B_BYTES, "epilogue scratch lives in stage 1");

  // Two LDS stages (about 66 KB each), one distinct array per stage, operand
  // and A row half: the compiler can then tell them apart and adds no
  // conservative waits for the direct-to-LDS loads (the explicit waits below
  // order them).  A's rows are split by bit 6 of the tile row: rows with it
  // clear (the first two 32-row MFMA tiles of each wave row) sit in sAl,
  // the others in sAh, each half at index (r & 63) | ((r >> 1) & 64).
  // Rows are BK = 128 bytes, a whole cache line, so every load instruction
  // moves whole lines; the 16-byte chunk c of array row i sits at chunk slot
  // c ^ ((i >> 1) & 7).  The LDS has 64 four-byte banks (256 bytes), so two
  // consecutive 128-byte rows fill one bank window and a 16-lane group of
  // 16-byte reads (16 consecutive rows, one chunk each) hits 16 distinct bank
  // quads.  Stage 1's A and B areas double as the epilogue scratch.
  __shared__ __attribute__((aligned(16))) uint8_t sAl0[AH_BYTES], sAh0[AH_BYTES], sAl1[AH_BYTES], sAh1[AH_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[B_BYTES], sB1[B_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t sSA0[SA_WORDS], sSA1[SA_WORDS];
  __shared__ __attribute__((aligned(16))) uint32_t sSB0[SB_WORDS], sSB1[SB_WORDS];
  __shared__ int32_t sTiles[1025];   // m-tiles before expert g, g = 0..L
  __shared__ uint32_t sAmax[2];      // the current tile's amax (float bits), see flush_amax
  __shared__ float sPr[kThreads / 64][kBM / 2];   // prob of each wave's 128 rows (epilogue)
  // backward epilogues: rows 16-31 of the second staged C_in block (1 KB per wave)
  __shared__ __attribute__((aligned(16))) uint8_t sCin[kThreads / 64][1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, hi = lane >> 5;
  const int L = p.num_groups;
  const int vm = static_cast<int>(p.valid_m);

  // ---- per-expert tile prefix sums (once per workgroup) ----
  // expert g owns P_g = (po[g] - po[g-1]) / 128 row blocks -> ceil(P_g / 2)
  // m-tiles.  Counts are clamped so that inconsistent offsets can neither
  // overflow the sums nor address rows outside [0, valid_m).
  if (wave == 0) {
    int base = 0;
    for (int c0 = 0; c0 < L; c0 += 64) {
      const int gi = c0 + lane;
      int cnt = 0;
      if (gi < L) {
        const int end = p.po[gi], beg = gi ? p.po[gi - 1] : 0;
        const int blocks = min(max(end - beg, 0) >> 7, vm >> 7);
        cnt = (blocks + 1) >> 1;
      }
      int x = cnt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
      }
      if (gi < L) sTiles[gi + 1] = min(base + x, 1 << 30);
      base = min(base + __shfl(x, 63), 1 << 30);
    }
    if (lane == 0) sTiles[0] = 0;
  }
  if (tid < 2) sAmax[tid] = 0;
  __syncthreads();
  const int m_tiles = sTiles[L];
  const int n_tiles = p.n_tiles;
  // the host guarantees (valid_m / 128 + L) / 2 * n_tiles < 2^31
  const int total = __builtin_amdgcn_readfirstlane(m_tiles * n_tiles);

  // Linear tile index -> tile.  Workgroups are dispatched round-robin over
  // the 8 XCDs (each with its own L2): workgroup w runs on XCD w % 8.  The
  // workgroups of XCD x take the contiguous slots [x*q + min(x, r), ...) of
  // the nwg slots, and pass i of slot s handles linear tile i * nwg + s, so
  // the tiles in flight on one XCD are consecutive.  Linear tiles run in
  // bands of kBandM m-tiles, m fastest, so consecutive tiles share B (same
  // expert and columns) or A (same rows) through L2.
  const int nwg = static_cast<int>(gridDim.x);
  const int wg = static_cast<int>(blockIdx.x);
  const int slot = [&] {
    const int xcd = wg & 7, j = wg >> 3, q = nwg >> 3, r = nwg & 7;
    return xcd * q + min(xcd, r) + j;
  }();
  auto tile_of = [&](int t) __attribute__((always_inline)) -> Tile {
    const int band_size = kBandM * n_tiles;
    const int band = t / band_size;
    const int in_band = t - band * band_size;
    const int band_rows = min(kBandM, m_tiles - band * kBandM);
    const int nt = in_band / band_rows;
    const int mt = band * kBandM + (in_band - nt * band_rows);
    // expert: the largest g < L with sTiles[g] <= mt (empty experts
    // skipped).  sTiles is non-decreasing, so that is the number of entries
    // <= mt less one: counted 64 entries per LDS read with a ballot, up to
    // the first chunk holding an entry above mt.
    int cnt = 0;
    for (int c0 = 0; c0 < L; c0 += 64) {
      const int i = c0 + lane;
      const int v = i < L ? sTiles[i] : 0x7FFFFFFF;
      cnt += __popcll(__ballot(v <= mt));
      if (cnt < c0 + 64) break;
    }
    const int lo = cnt - 1;
    Tile tl;
    tl.g = __builtin_amdgcn_readfirstlane(lo);
    // first row: a multiple of 128 in [0, valid_m - 128] whatever the offsets
    // hold (valid_m is a positive multiple of 128 here); rows past the
    // expert's end or valid_m are not stored
    const int64_t beg = tl.g ? sload(p.po, tl.g - 1) : 0, end = sload(p.po, tl.g);
    const int64_t jt = min(mt - sTiles[lo], vm >> 8);
    const int r0 = static_cast<int>(min((max(beg, int64_t{0}) + jt * BM) & ~int64_t{127}, int64_t{vm - 128}));
    const int64_t rows = min(min(int64_t{BM}, end - r0), int64_t{vm - r0});
    tl.row0 = __builtin_amdgcn_readfirstlane(r0);
    tl.rows = __builtin_amdgcn_readfirstlane(static_cast<int>(max(rows, int64_t{0})) & ~127);
    tl.n0 = __builtin_amdgcn_readfirstlane(nt * BN);
    // dense weights: expert g's rows follow the previous experts'; discrete
    // weights: its own allocations (low 4 bits cleared: 16-byte aligned
    // loads).  Resolved here, at tile set-up, so that the operand loads of
    // the K loop need no branch.
    if (p.b_ptrs) {
      tl.bg = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(sload(p.b_ptrs, tl.g)) & ~uintptr_t{15});
      tl.sg = p.sfb_ptrs ? reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(sload(p.sfb_ptrs, tl.g)) &
                                                            ~uintptr_t{15})
                         : nullptr;
    } else {
      tl.bg = p.b + static_cast<int64_t>(tl.g) * p.n * p.row_bytes;
      tl.sg = p.sfb ? p.sfb + static_cast<int64_t>(tl.g) * p.n * p.sf_row_b : nullptr;
    }
    return tl;
  };

  // ---- direct global -> LDS staging ----
  // One wave instruction fills 8 rows (1 KB): lane i writes row 8j + i/8 of
  // its group, chunk slot i%8, i.e. logical chunk (i%8) ^ ((row >> 1) & 7).
  // Wave w fills B rows [32w, 32w+32) (4 instructions) and rows
  // [16w, 16w+16) of each A half (2 + 2).  A rows past the tile's valid rows
  // repeat its last row and B rows past N repeat row N-1 (loaded, never
  // stored).  Scale dwords ride along, one per lane: 8-bit operands (one dword per row
  // and step): waves 0-3 load A rows, waves 4-7 B rows; E2M1 (two dwords):
  // two loads per wave; BF16 has none.
  // A stage's loads come in two sets: the early set (B, the low A half and
  // all scale words: everything the first operand cluster of a step reads)
  // and the late set (the high A half, read by the second cluster).
  constexpr int S_LOADS = F8 ? 1 : AB == AB_E2M1 ? 2 : 0;
  constexpr int SL = S_LOADS > 0 ? S_LOADS : 1;
  constexpr int S_HALF = F8 ? 4 : 8;                 // scale jobs of A (the rest are B's)
  constexpr int N_EA = 2 + S_LOADS, N_EB = 4, N_EARLY = N_EA + N_EB, N_LATE = 2;

  struct Src {
    const uint8_t* a;    // wave-uniform bases
    const uint8_t* b;
    uint32_t oa[4];      // per-lane byte offsets: low half j = 0, 1; high half 2, 3
    uint32_t ob[4];
    const uint8_t* s[SL];   // scale words: wave-uniform bases ...
    uint32_t so[SL];         // ... and per-lane byte offsets
  };
  auto make_src = [&](const Tile& tl) __attribute__((always_inline)) {
    // per-lane values are rebuilt from an opaque copy of the lane id instead
    // of being kept live (and spilled) across the K loop
    int lid = lane;
    asm volatile("" : "+v"(lid));
    const int lrow = lid >> 3;
    Src s;
    s.a = p.a + static_cast<int64_t>(tl.row0) * p.row_bytes;
    s.b = tl.bg + static_cast<int64_t>(tl.n0) * p.row_bytes;
    const int alast = max(min(tl.rows, vm - tl.row0), 1) - 1;   // last loadable row of the tile
    const int blast = p.n - 1 - tl.n0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = wave * 16 + (j & 1) * 8 + lrow;              // row within the half
      const int r = (i & 63) | ((j >> 1) << 6) | ((i & 64) << 1);
      s.oa[j] = static_cast<uint32_t>(min(r, alast) * p.row_bytes + (((lid & 7) ^ ((i >> 1) & 7)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wave * 32 + j * 8 + lrow;
      s.ob[j] = static_cast<uint32_t>(min(r, blast) * p.row_bytes + (((lid & 7) ^ ((r >> 1) & 7)) * 16));
    }
    if constexpr (MX) {
#pragma unroll
      for (int u = 0; u < S_LOADS; ++u) {
        // job (wave * S_LOADS + u): 8-bit operands: jobs 0-3 A rows, 4-7 B rows;
        // E2M1 jobs 0-7 A (word, quarter), 8-15 B (word, quarter)
        const int job = wave * S_LOADS + u;
        const bool isA = job < S_HALF;
        const int jj = isA ? job : job - S_HALF;
        const int word = jj >> 2, rowsel = (jj & 3) * 64 + lid;
        // scale word `word` of K-step ks for row r sits at
        //   r * sf_row + (SW * ks + word) * sf_word
        // (row-major (rows, K/32): sf_row = K/32, sf_word = 4; K-block planes
        // (K/128, rows, 4): sf_row = 4, sf_word = 4 * rows; SFB rows: L * N
        // dense with row g * N + n, N per expert discrete)
        s.s[u] = isA ? p.sfa + static_cast<int64_t>(tl.row0) * p.sf_row_a + static_cast<int64_t>(word) * p.sf_word_a
                     : tl.sg + static_cast<int64_t>(tl.n0) * p.sf_row_b + static_cast<int64_t>(word) * p.sf_word_b;
        s.so[u] = static_cast<uint32_t>(min(rowsel, isA ? alast : blast)) * static_cast<uint32_t>(isA ? p.sf_row_a : p.sf_row_b);
      }
    }
    return s;
  };

  // One LDS stage: the two A halves, B, scale words.
  struct Stage {
    uint8_t* al;
    uint8_t* ah;
    uint8_t* b;
    uint32_t* sa;
    uint32_t* sb;
  };
  const Stage st0{sAl0, sAh0, sB0, sSA0, sSB0};
  const Stage st1{sAl1, sAh1, sB1, sSA1, sSB1};
  // early set, first part: the low A half and the scale words
  // the per-wave LDS destinations are rebuilt from an opaque copy of the
  // wave id (two scalar operations) instead of being kept in scalar registers
  auto owave = [&]() __attribute__((always_inline)) {
    int w = wave;
    asm volatile("" : "+s"(w));
    return w;
  };
  auto issue_ea = [&](const Src& s, int ks, const Stage& d) __attribute__((always_inline)) {
    const int kb = ks * BK;
    const int wo = owave();
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(at(s.a + kb, s.oa[j]), d.al + (wo * 16 + j * 8) * BK);
    if constexpr (MX) {
#pragma unroll
      for (int u = 0; u < S_LOADS; ++u) {
        // LDS words: word w of row r at [w * rows + r], 64 rows per load
        const int job = wo * S_LOADS + u;
        const bool isA = job < S_HALF;
        const int jj = isA ? job : job - S_HALF;
        uint32_t* dst = (isA ? d.sa : d.sb) + (jj >> 2) * (isA ? BM : BN) + (jj & 3) * 64;
        dma4(at(s.s[u] + static_cast<int64_t>(SW * ks) * (isA ? p.sf_word_a : p.sf_word_b), s.so[u]), dst);
      }
    }
  };
  // early set, second part: B row load j (0..3)
  auto issue_eb = [&](const Src& s, int ks, const Stage& d, int j) __attribute__((always_inline)) {
    dma16(at(s.b + ks * BK, s.ob[j]), d.b + (owave() * 32 + j * 8) * BK);
  };
  // late set: high A half load j (0..1)
  auto issue_l = [&](const Src& s, int ks, const Stage& d, int j) __attribute__((always_inline)) {
    dma16(at(s.a + ks * BK, s.oa[2 + j]), d.ah + (owave() * 16 + j * 8) * BK);
  };
  // a whole stage, in the order early (first part, second part), late
  auto issue = [&](const Src& s, int ks, const Stage& d) __attribute__((always_inline)) {
    issue_ea(s, ks, d);
#pragma unroll
    for (int j = 0; j < N_EB; ++j) issue_eb(s, ks, d, j);
#pragma unroll
    for (int j = 0; j < N_LATE; ++j) issue_l(s, ks, d, j);
  };

  v16f acc[TM][TN];
  // The K loop runs in clusters: an M cluster reads operands from LDS into
  // registers and issues direct loads, a C cluster runs MFMAs only.  Step s
  // is M0 (B and the A tiles 0, 1 of the wave, all scale words), C0 (those
  // A tiles), M1 (A tiles 2, 3), C1 (those, with B still in registers).  The
  // two waves sharing a SIMD (w and w + 4) run one cluster apart, so one of
  // them issues MFMAs while the other reads LDS and issues loads.
  // A lane's 16-byte pieces of a 32-row tile for one step: chunks hi + 2c,
  // c = 0..3.  E4M3 window kk uses pieces 2kk, 2kk+1 (K [16hi, 16hi+16) and
  // [32+16hi, 48+16hi) of the window; its scale byte covers the 32-element
  // block hi of the window); E2M1 (32 elements) and BF16 (8 elements) window
  // kk use piece kk.
  typedef v4u Pieces[4];
  auto read_tile = [&](const uint8_t* base, int l32, int hi, Pieces& x) __attribute__((always_inline)) {
    const int sw = (l32 >> 1) & 7;      // swizzle of this lane's rows (tiles start at multiples of 32)
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = *reinterpret_cast<const v4u*>(base + (((hi + 2 * c) ^ sw) * 16));
  };
  auto settle = [&](Pieces& x) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(x[c]));
  };
  struct Ops0 {
    Pieces a[2], b[TN];
    uint32_t sa[TM][SW], sb[TN][SW];
  };
  struct Ops1 {
    Pieces a[2];
  };
  // M0: B, A tiles 0, 1 and the scale words (fin0 waits for them and
  // shifts the scale words so that byte 0 / 2 is this lane's block of an
  // even / odd window)
  auto read0 = [&](const Stage& st) __attribute__((always_inline)) {
    int lid = lane;
    asm volatile("" : "+v"(lid));
    const int l32 = lid & 31, hi = lid >> 5;
    Ops0 o;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) read_tile(st.b + (wn * WN + tn * 32 + l32) * BK, l32, hi, o.b[tn]);
#pragma unroll
    for (int t = 0; t < 2; ++t) read_tile(st.al + (wm * 64 + t * 32 + l32) * BK, l32, hi, o.a[t]);
    if constexpr (MX) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int w = 0; w < SW; ++w) o.sa[tm][w] = st.sa[w * BM + wm * WM + tm * 32 + l32];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int w = 0; w < SW; ++w) o.sb[tn][w] = st.sb[w * BN + wn * WN + tn * 32 + l32];
    }
    return o;
  };
  auto fin0 = [&](Ops0& o) __attribute__((always_inline)) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) settle(o.b[tn]);
#pragma unroll
    for (int t = 0; t < 2; ++t) settle(o.a[t]);
    if constexpr (MX) {
      int lid = lane;
      asm volatile("" : "+v"(lid));
      const int sh = 8 * (lid >> 5);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int w = 0; w < SW; ++w) {
          asm volatile("" : "+v"(o.sa[tm][w]));
          o.sa[tm][w] >>= sh;
        }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int w = 0; w < SW; ++w) {
          asm volatile("" : "+v"(o.sb[tn][w]));
          o.sb[tn][w] >>= sh;
        }
    }
  };
  // M1: A tiles 2, 3
  auto read1 = [&](const Stage& st) __attribute__((always_inline)) {
    int lid = lane;
    asm volatile("" : "+v"(lid));
    const int l32 = lid & 31, hi = lid >> 5;
    Ops1 o;
#pragma unroll
    for (int t = 0; t < 2; ++t) read_tile(st.ah + (wm * 64 + t * 32 + l32) * BK, l32, hi, o.a[t]);
    return o;
  };
  auto fin1 = [&](Ops1& o) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) settle(o.a[t]);
  };
  // C cluster: MFMA tiles tm0, tm0 + 1 (A pieces a[0], a[1]) x all tn, all
  // windows of the step
  // `hook(i)` runs right after the cluster's MFMA number i (0 .. NMMA-1)
  constexpr int NWIN = F8 ? 2 : 4;
  constexpr int NMMA = NWIN * 2 * TN;
  // zc: std::integral_constant<bool, Z>; with Z the first window starts from
  // a zero accumulator (the MFMA's inline constant 0), as a tile's first step
  // does instead of clearing the accumulators
  auto mma = [&](int tm0, const Pieces* a, const Ops0& o0, auto&& hook, auto zc) __attribute__((always_inline)) {
    constexpr bool ZERO = decltype(zc)::value;
    static_for<0, NWIN>([&](auto kc) {
      constexpr int kk = decltype(kc)::value;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int mi = (kk * 2 + t) * TN + tn;
          v16f& c = acc[tm0 + t][tn];
          const v16f cin = ZERO && kk == 0 ? v16f{} : c;
          if constexpr (F8) {
            const v4u a0 = a[t][2 * kk], a1 = a[t][2 * kk + 1], b0 = o0.b[tn][2 * kk], b1 = o0.b[tn][2 * kk + 1];
            const v8i fa{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const v8i fb{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, cin, FMT8, FMT8, kk * 2, (int)o0.sb[tn][0],
                                                                kk * 2, (int)o0.sa[tm0 + t][0]);
          } else if constexpr (AB == AB_E2M1) {
            const v4u a0 = a[t][kk], b0 = o0.b[tn][kk];
            const v8i fa{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
            const v8i fb{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, cin, 4, 4, (kk & 1) * 2, (int)o0.sb[tn][kk >> 1],
                                                                (kk & 1) * 2, (int)o0.sa[tm0 + t][kk >> 1]);
          } else {
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, o0.b[tn][kk]),
                                                        __builtin_bit_cast(v8bf, a[t][kk]), cin, 0, 0, 0);
          }
          hook(mi);
        }
    });
  };

  // ---- epilogue of one tile (accumulators -> outputs) ----
  float nc = 1.0f;
  if constexpr (OUT == OUT_E4M3) nc = p.norm_const[0];
  // this wave's epilogue scratch: 8 KB of stage 1 (free once every wave has
  // finished the tile's last K-step)
  float* scratch = reinterpret_cast<float*>(wave < 2   ? sAl1 + wave * kScratch
                                            : wave < 4 ? sAh1 + (wave - 2) * kScratch
                                                       : sB1 + (wave - 4) * kScratch);
  float* sT = scratch;
  float* sS = scratch + 32 * kTPitch;
  // C_in staging of the backward epilogues: two blocks of 32 rows x 64 bytes;
  // block 0 and rows [0, 16) of block 1 in the 3 KB behind the wave's
  // transpose scratch, rows [16, 32) of block 1 in sCin
  static_assert(32 * kTPitch * 4 + 32 * 4 + 3072 <= kScratch, "C_in staging fits the wave's scratch");
  uint8_t* const stgA = reinterpret_cast<uint8_t*>(sS + 32);
  uint8_t* const stgB = sCin[wave];
  // destination of direct load k (rows [16 k, 16 k + 16)) of block b
  auto stg_dst = [&](int b, int k) __attribute__((always_inline)) {
    return b == 0 ? stgA + 1024 * k : k == 0 ? stgA + 2048 : stgB;
  };
  // row r of block b
  auto stg_row = [&](int b, int r) __attribute__((always_inline)) {
    return b == 0 ? stgA + 64 * r : r < 16 ? stgA + 2048 + 64 * r : stgB + 64 * (r - 16);
  };

  // Per-tile epilogue factors: alpha_g (a scalar load issued before the
  // tile's last K-step) and prob of the wave's 128 rows, copied to LDS by two
  // direct loads issued just before the next tile's first stage, so that no
  // register holds them across the last K-step.
  struct EpiIn {
    float alpha;
  };
  auto epi_in = [&](const Tile& tl) __attribute__((always_inline)) {
    EpiIn e;
    e.alpha = p.alpha[tl.g];
    return e;
  };
  auto load_prob = [&](const Tile& tl) __attribute__((always_inline)) {
    const int mb = min(tl.row0 + wm * WM, vm - WM);      // rows of idle waves: any valid ones
    dma4(p.prob + mb + lane, sPr[wave]);
    dma4(p.prob + mb + 64 + lane, sPr[wave] + 64);
  };

  auto epilogue = [&](const Tile& tl, const EpiIn& ein) __attribute__((always_inline)) {
    if (wm * WM >= tl.rows) return;     // rows of a 128-row tile (or an empty one) handled by wm = 0
    // lane-dependent addresses are rebuilt here from an opaque copy of the
    // lane id rather than kept live (and spilled) across the K loop
    int lid = lane;
    asm volatile("" : "+v"(lid));
    const int l32 = lid & 31, hi = lid >> 5;
    const int g = tl.g;
    const float alpha = ein.alpha;
    const int mbase = tl.row0 + wm * WM;
    const int nbase = tl.n0 + wn * WN;
    const int64_t mb = mbase;
    // FP8 outputs: the wave's first row of D, D_col and SFD_row (uniform)
    uint8_t* const dW0 = OUT == OUT_E4M3 ? p.d + mb * p.n_out : nullptr;
    uint8_t* const dcW0 = OUT == OUT_E4M3 ? p.d_col + mb * p.n_out : nullptr;
    uint8_t* const sfW0 = OUT == OUT_E4M3 ? p.sfd_row + mb * (p.n_out >> 5) : nullptr;
    const uint32_t sfc_pitch = static_cast<uint32_t>(vm >> 5);     // bytes per SFD_col row
    float pr[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) pr[tm] = sPr[wave][tm * 32 + l32];

    if constexpr (ACT == ACT_DSWIGLU || ACT == ACT_DGEGLU) {
      // GLU backwards over pairs of 32-column blocks of the saved C_in, R =
      // alpha^2 acc ("Grouped GEMM + dGLU (SM100)", BF16 contract equations
      // and the block-scaled contract's Step 2).
      // dSwiGLU: X = beta * C_in, blocks [input_b | gate_b], s = sigmoid(gate):
      //   d_input = R prob swish(gate), d_gate = R prob input s (1 + gate (1 - s)),
      //   dprob += R input swish(gate)
      // dGeGLU: C_in as stored, blocks [gate_b | up_b], gate_c = min(gate, cmax),
      //   up_c = clamp(up, cmin, cmax), s = sigmoid(a gate_c):
      //   d_gate = R prob (up_c + off) s (1 + a gate_c (1 - s)) [gate <= cmax],
      //   d_up = R prob gate_c s [cmin <= up <= cmax], dprob += R gate_c s (up_c + off)
      // The outputs keep the pair order of the input blocks.
      const float a2 = alpha * alpha;
      float beta = 1.0f;
      if constexpr (ACT == ACT_DSWIGLU) beta = p.beta[g];
      const float nqf = OUT == OUT_E4M3 ? nc : 1.0f;     // FP8 dC carries norm_const
      const int ld2 = 2 * p.n;
      const uint16_t* const cinW = p.c_in + mb * ld2 + 2 * nbase;   // wave's first row, block pair 0
      uint8_t* const dbW = p.d + (mb * ld2 + 2 * nbase) * 2;          // BF16 dC, same layout
      // block-scaled operands with a BF16 output: amax per group of the first
      // and of the second blocks of the pairs (amax of shape (L, 2))
      constexpr bool AMAX2 = MX && OUT == OUT_BF16;
      float amax0 = 0.0f, amax1 = 0.0f;
      uint32_t colw0[TN], colw1[TN];          // E4M3: column scale bytes of 4 row blocks
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) colw0[tn] = colw1[tn] = 0;
      // C_in of sub-tile (tm, tn): packed bf16 of the pair's two blocks
      // (block b = ncol/32 of R pairs with C_in columns [64b, 64b + 64))
      auto has_cols = [&](int tn) __attribute__((always_inline)) { return nbase + tn * 32 < p.n; };
      // C_in is loaded one sub-tile ahead of its use, so that its latency
      // overlaps the previous sub-tile's arithmetic and stores (in
      // registers it would spill): by direct loads into the LDS staging,
      // the first block of the pair as block 0, the second as block 1
      auto stage_x = [&](int tm, int tn) __attribute__((always_inline)) {
        int lid2 = lane;
        asm volatile("" : "+v"(lid2));
        const uint16_t* const xb = cinW + 64 * tn;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          // lane i of load k: row 16 k + i / 4, 16-byte chunk i % 4
          const uint32_t off = (tm * 32 + 16 * k + (lid2 >> 2)) * static_cast<uint32_t>(ld2) * 2 + 16 * (lid2 & 3);
          dma16(at(xb, off), stg_dst(0, k));
          dma16(at(xb + 32, off), stg_dst(1, k));
        }
      };
      auto read_x = [&](v4u* q) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          q[i] = *reinterpret_cast<const v4u*>(stg_row(0, l32) + 32 * i + 16 * hi);
          q[2 + i] = *reinterpret_cast<const v4u*>(stg_row(1, l32) + 32 * i + 16 * hi);
        }
      };
      // (raw reads q[0, 2) of the first block, q[2, 4) of the second)
      v4u nq[4];
      if (has_cols(0)) stage_x(0, 0);
      // the outputs of a 32-row block go out in whole 128-byte row segments
      // (store_rows through the transpose scratch): BF16 dC per column pair,
      // FP8 dC (4 blocks of 32 columns) once both pairs are quantised
      float* const stg = sT;
      int lid3 = lane;
      asm volatile("" : "+v"(lid3));
      const uint32_t dpitch = static_cast<uint32_t>(p.n_out);                     // FP8 dC row, bytes
      const uint32_t dvalid = static_cast<uint32_t>(max(min(128, p.n_out - 2 * nbase), 0));
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const uint32_t ml = tm * 32 + l32;                 // row within the wave's 128
        float dp = 0.0f;
        v4u rq[2 * TN] = {}, kq[2 * TN] = {};             // FP8 dC row / column pieces of the 4 blocks
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          if (!has_cols(tn)) continue;
          const int ncol = nbase + tn * 32;
          // (loads of later sub-tiles are not hoisted above this point:
          // holding more of them would spill)
          v2u wi[4], wg[4];          // packed bf16 of the first and second blocks of the pair
          if constexpr (OUT == OUT_E4M3) asm volatile("" ::: "memory");
          // this sub-tile's staged C_in has landed (every direct load of this
          // wave complete) before the LDS reads
          wait_vmcnt<0>();
          read_x(nq);
          unpack_bf16(nq, wi);
          unpack_bf16(nq + 2, wg);
          // the reads above have returned before the next sub-tile's loads
          // overwrite the staging
          __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
          __builtin_amdgcn_sched_barrier(0);
          if (tn + 1 < TN && has_cols(tn + 1)) stage_x(tm, tn + 1);
          else if (tm + 1 < TM) stage_x(tm + 1, 0);
          // element v of a packed block (columns 8(v/4) + 4 hi + v%4)
          auto bf = [](const v2u* w, int v) __attribute__((always_inline)) {
            const uint32_t u = (v & 2) ? w[v >> 2].y : w[v >> 2].x;
            return __uint_as_float((v & 1) ? (u & 0xFFFF0000u) : (u << 16));
          };
          // dC of element v in the first (part 0) or second (part 1) block;
          // part 0 also accumulates the dprob term
          // The row's constant factors are taken out of the element terms:
          // dC = acc (alpha^2 prob [norm_const for FP8 dC]) (...) with the
          // dSwiGLU input's beta in the second block's factor, and the dprob
          // terms summed over acc, times alpha^2 [beta] once per row.
          const float k0 = (a2 * pr[tm]) * nqf;
          const float k1 = ACT == ACT_DSWIGLU ? k0 * beta : k0;
          // the sigmoid of an element: computed by its part-0 call, which
          // returns it in sgv, and passed to its part-1 call (sgv >= 0)
          auto dglu = [&](int v, int part, float& dpv, float& sgv) __attribute__((always_inline)) -> float {
            const float av = acc[tm][tn][v];
            if constexpr (ACT == ACT_DSWIGLU) {
              const float xr = bf(wi, v);              // input / beta
              const float gt = beta * bf(wg, v);
              const float sg = part == 0 ? sigmoid_f(gt) : sgv;
              sgv = sg;
              if (part == 0) {
                const float swish = gt * sg;
                dpv = fmaf(av, xr * swish, dpv);
                return (av * k0) * swish;
              }
              return (av * k1) * (xr * sg * fmaf(gt, 1.0f - sg, 1.0f));
            } else {
              const float gate = bf(wi, v), up = bf(wg, v);
              const float gc = fminf(gate, p.glu_clamp_max);
              const float uc = fminf(fmaxf(up, p.glu_clamp_min), p.glu_clamp_max);
              const float sg = part == 0 ? sigmoid_f(p.geglu_alpha * gc) : sgv;
              sgv = sg;
              const float uo = uc + p.linear_offset;
              if (part == 0) {
                dpv = fmaf(av, gc * sg * uo, dpv);
                return gate <= p.glu_clamp_max ? (av * k0) * (uo * sg * fmaf(p.geglu_alpha * gc, 1.0f - sg, 1.0f))
                                               : 0.0f;
              }
              // evaluated in every lane, then masked by a select: left to
              // itself the compiler branched around the sigmoid per element
              float du = (av * k0) * (gc * sg);
              asm volatile("" : "+v"(du));
              return (up >= p.glu_clamp_min && up <= p.glu_clamp_max) ? du : 0.0f;
            }
          };
          if constexpr (OUT == OUT_BF16) {
            float d0[16], d1[16], unused = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float sgv = 0.0f;
              d0[v] = dglu(v, 0, dp, sgv);
              d1[v] = dglu(v, 1, unused, sgv);
              // (dGeGLU: pinned in groups of eight, as in the FP8 branch below)
              if (ACT == ACT_DGEGLU && (v & 7) == 7)
                asm volatile("" : "+v"(d0[v - 7]), "+v"(d0[v - 6]), "+v"(d0[v - 5]), "+v"(d0[v - 4]), "+v"(d0[v - 3]),
                             "+v"(d0[v - 2]), "+v"(d0[v - 1]), "+v"(d0[v]), "+v"(d1[v - 7]), "+v"(d1[v - 6]),
                             "+v"(d1[v - 5]), "+v"(d1[v - 4]), "+v"(d1[v - 3]), "+v"(d1[v - 2]), "+v"(d1[v - 1]),
                             "+v"(d1[v]), "+v"(dp));
            }
            if constexpr (AMAX2) {
#pragma unroll
              for (int v = 0; v < 16; v += 2) {
                amax0 = max_abs2(amax0, d0[v], d0[v + 1]);
                amax1 = max_abs2(amax1, d1[v], d1[v + 1]);
              }
            }
            v4u q[4];
            bf16_pieces(d0, q);
            bf16_pieces(d1, q + 2);
            store_rows<128>(dbW + 128 * tn + tm * 32 * ld2 * 2, static_cast<uint32_t>(ld2) * 2, q, stg, lid3);
          } else {
            // FP8 dC: each 32-column output block quantised by rows and
            // columns like a forward D ("Grouped GEMM + dGLU (SM100)",
            // block-scaled Step 3).  One block at a time: the sigmoids of the
            // first block's elements are kept for the second (a transcendental
            // pair per element saved), the other shared terms recomputed, so
            // that a single block of values is live during a quantisation.
            const int oc = 2 * ncol;
            const uint32_t so = ml * static_cast<uint32_t>(p.n_out >> 5);
            // (dGeGLU: the elements in groups of eight, pinned after each
            // group, so that the scheduler does not keep sixteen sigmoid
            // chains in flight at once and spill; dSwiGLU does not need it)
            float d[16], sgk[16], unused = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              d[v] = dglu(v, 0, dp, sgk[v]);
              if (ACT == ACT_DGEGLU && (v & 7) == 7) asm volatile("" : "+v"(d[v - 7]), "+v"(d[v - 6]), "+v"(d[v - 5]), "+v"(d[v - 4]), "+v"(d[v - 3]), "+v"(d[v - 2]), "+v"(d[v - 1]), "+v"(d[v]), "+v"(dp));
            }
            colw0[tn] |= quant_codes(sT, sS, sfW0 + (oc >> 5), so, hi, l32, d, rq[2 * tn], kq[2 * tn]) << (8 * tm);
            // opaque copies: the second block's other terms are recomputed, not kept
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              asm volatile("" : "+v"(wi[j]));
              asm volatile("" : "+v"(wg[j]));
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              d[v] = dglu(v, 1, unused, sgk[v]);
              if (ACT == ACT_DGEGLU && (v & 7) == 7) asm volatile("" : "+v"(d[v - 7]), "+v"(d[v - 6]), "+v"(d[v - 5]), "+v"(d[v - 4]), "+v"(d[v - 3]), "+v"(d[v - 2]), "+v"(d[v - 1]), "+v"(d[v]));
            }
            colw1[tn] |= quant_codes(sT, sS, sfW0 + (oc >> 5) + 1, so, hi, l32, d, rq[2 * tn + 1], kq[2 * tn + 1])
                         << (8 * tm);
          }
        }
        if constexpr (OUT == OUT_E4M3) {
          store_rows<128>(dW0 + 2 * nbase + tm * 32 * dpitch, dpitch, rq, stg, lid3, dvalid);
          store_rows<128>(dcW0 + 2 * nbase + tm * 32 * dpitch, dpitch, kq, stg, lid3, dvalid);
        }
        dp = halves_sum(dp * (ACT == ACT_DSWIGLU ? a2 * beta : a2));
        if (hi == 0) atomicAdd(at(p.dprob + mb, 4 * ml), dp);
      }
      if constexpr (OUT == OUT_E4M3) {
        // column l32's scale bytes of the wave's 4 consecutive 32-row blocks
        const int mblk0 = mbase >> 5;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int ncol = nbase + tn * 32;
          if (ncol >= p.n || hi != 0) continue;
          uint8_t* const c0 = p.sfd_col + static_cast<int64_t>(2 * ncol) * (vm >> 5) + mblk0;
          *at(reinterpret_cast<uint32_t*>(c0), l32 * sfc_pitch) = colw0[tn];
          *at(reinterpret_cast<uint32_t*>(c0 + 32 * (vm >> 5)), l32 * sfc_pitch) = colw1[tn];
        }
      }
      if constexpr (AMAX2) {
        const float wi = wave_max(amax0), wg = wave_max(amax1);
        if (lane == 0) {
          atomicMax(&sAmax[0], __float_as_uint(wi));
          atomicMax(&sAmax[1], __float_as_uint(wg));
        }
      }
    } else if constexpr (ACT == ACT_DSRELU) {
      // sReLU backward (derived from "Grouped GEMM + sReLU (SM100)",
      // §Equations / §Tanh soft clamp): R = alpha^2 acc, C the saved forward
      // C; with t = min(tanh(relu(C)/s), 1), c = s t: dC = R prob 2 c sech^2(relu(C)/s)
      // (= 1 - t^2, evaluated without its cancellation near t = 1),
      // dprob += R c^2 (s = 0: c = relu(C), dC = R prob 2 c)
      const float a2 = alpha * alpha;
      const float sc = p.srelu_s;
      const float rs = sc > 0.0f ? 1.0f / sc : 0.0f;
      const float nq = OUT == OUT_E4M3 ? nc : 1.0f;     // FP8 dC carries norm_const
      float amax_l = 0.0f;
      uint32_t colw[TN];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) colw[tn] = 0;
      const uint16_t* const cinW = p.c_in + mb * p.n + nbase;
      // C_in of one row of sub-tiles (32 rows, TN blocks of 32 columns),
      // loaded one row ahead so that its latency overlaps the previous row's
      // work: by direct loads into the LDS staging, column block tn as
      // staging block tn
      static_assert(TN == 2, "one staging block per column block");
      auto stage_row = [&](int tm) __attribute__((always_inline)) {
        int lid2 = lane;
        asm volatile("" : "+v"(lid2));
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          if (nbase + tn * 32 >= p.n) continue;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            // lane i of load k: row 16 k + i / 4, 16-byte chunk i % 4
            const uint32_t off = (tm * 32 + 16 * k + (lid2 >> 2)) * static_cast<uint32_t>(p.n) * 2 + 16 * (lid2 & 3);
            dma16(at(cinW + 32 * tn, off), stg_dst(tn, k));
          }
        }
      };
      v2u cw[TN][4];
      stage_row(0);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const uint32_t ml = tm * 32 + l32;
        float dp = 0.0f;
        // dC pieces of the row's TN blocks: bf16 (2 a block) or E4M3 row and
        // column codes (1 a block)
        v4u dq[OUT == OUT_BF16 ? 2 * TN : TN] = {}, kq[TN] = {};
        // this row's staged C_in has landed before the LDS reads, and the
        // reads have returned before the next row's loads overwrite it
        wait_vmcnt<0>();
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          if (nbase + tn * 32 >= p.n) continue;
          v4u q[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) q[i] = *reinterpret_cast<const v4u*>(stg_row(tn, l32) + 32 * i + 16 * hi);
          unpack_bf16(q, cw[tn]);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        if (tm + 1 < TM) stage_row(tm + 1);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int ncol = nbase + tn * 32;
          if (ncol >= p.n) continue;
          float cv[16];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v2u w = cw[tn][j];
            cv[4 * j + 0] = __uint_as_float(w.x << 16);
            cv[4 * j + 1] = __uint_as_float(w.x & 0xFFFF0000u);
            cv[4 * j + 2] = __uint_as_float(w.y << 16);
            cv[4 * j + 3] = __uint_as_float(w.y & 0xFFFF0000u);
          }
          float d[16];
          // (the clamp test outside the element loop, as in the forward)
          // R = alpha^2 acc: dC = acc (alpha^2 prob 8 s [nc]) t (sech^2 / 4) and
          // dprob += alpha^2 s^2 sum acc t^2 (s = 0: dC = acc (alpha^2 prob 2 [nc]) c,
          // dprob += alpha^2 sum acc c^2); t <= 1 by construction
          float sq = 0.0f;
          if (sc > 0.0f) {
            const float k = (a2 * pr[tm]) * ((8.0f * sc) * nq);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float t, s4;
              tanh_sech2_nonneg(fmaxf(cv[v], 0.0f) * rs, t, s4);
              d[v] = (acc[tm][tn][v] * k) * (t * s4);
              sq = fmaf(acc[tm][tn][v], t * t, sq);
            }
            dp = fmaf(a2 * (sc * sc), sq, dp);
          } else {
            const float k = (a2 * pr[tm]) * (2.0f * nq);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float c = fmaxf(cv[v], 0.0f);
              d[v] = (acc[tm][tn][v] * k) * c;
              sq = fmaf(acc[tm][tn][v], c * c, sq);
            }
            dp = fmaf(a2, sq, dp);
          }
          if constexpr (OUT == OUT_BF16) {
            bf16_pieces(d, dq + 2 * tn);
            if constexpr (MX) {
#pragma unroll
              for (int v = 0; v < 16; v += 2) amax_l = max_abs2(amax_l, d[v], d[v + 1]);
            }
          } else {
            colw[tn] |= quant_codes(sT, sS, sfW0 + (ncol >> 5), ml * static_cast<uint32_t>(p.n_out >> 5), hi, l32, d,
                                    dq[tn], kq[tn])
                        << (8 * tm);
          }
        }
        // the row's dC in whole row segments of the wave's columns
        // (store_rows through the transpose scratch)
        {
          constexpr int DW = (OUT == OUT_BF16 ? 2 : 1) * 32 * TN;
          const uint32_t dpitch = static_cast<uint32_t>(p.n_out) * (OUT == OUT_BF16 ? 2 : 1);
          const uint32_t dvalid = static_cast<uint32_t>(max(min(DW, (OUT == OUT_BF16 ? 2 : 1) * (p.n_out - nbase)), 0));
          uint8_t* const dB = (OUT == OUT_BF16 ? reinterpret_cast<uint8_t*>(p.d) + (mb * p.n_out + nbase) * 2
                                               : dW0 + nbase) + tm * 32 * dpitch;
          int lid3 = lane;
          asm volatile("" : "+v"(lid3));
          store_rows<DW>(dB, dpitch, dq, sT, lid3, dvalid);
          if constexpr (OUT == OUT_E4M3)
            store_rows<DW>(dcW0 + nbase + tm * 32 * dpitch, dpitch, kq, sT, lid3, dvalid);
        }
        dp = halves_sum(dp);
        if (hi == 0) atomicAdd(at(p.dprob + mb, 4 * ml), dp);
      }
      if constexpr (OUT == OUT_E4M3) {
        const int mblk0 = mbase >> 5;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int ncol = nbase + tn * 32;
          if (ncol >= p.n || hi != 0) continue;
          *at(reinterpret_cast<uint32_t*>(p.sfd_col + static_cast<int64_t>(ncol) * (vm >> 5) + mblk0), l32 * sfc_pitch) =
              colw[tn];
        }
      }
      if constexpr (MX && OUT == OUT_BF16) {
        const float w = wave_max(amax_l);
        if (lane == 0) atomicMax(&sAmax[0], __float_as_uint(w));
      }
    } else {
      float amax_l = 0.0f;
      const int mblk0 = mbase >> 5;
      // output column tiles of this wave: SwiGLU turns a [X_b | G_b] pair of
      // 32-column MFMA tiles into one, GeGLU a [G_b | U_b] pair
      constexpr bool PAIR = ACT == ACT_SWIGLU || ACT == ACT_GEGLU;
      constexpr int TO = PAIR ? TN / 2 : TN;
      // Each 32-row block is stored once all its column tiles are done, in
      // whole row segments of the wave's columns (store_rows through the
      // transpose scratch, which is free between quantisations): C (bf16,
      // 128 bytes a row), D (bf16: 64 or 128 bytes, E4M3: 64 bytes without
      // pairs; E4M3 with pairs has 32 bytes a row and is stored directly).
      // GEMM columns [nbase, nbase + 64): the last wave of an N = 32 mod 64
      // problem has the first 32 only.
      if (nbase < p.n) {
        const int ocol0 = PAIR ? nbase >> 1 : nbase;              // first output column
        const uint32_t cpitch = static_cast<uint32_t>(p.n) * 2;    // bytes per C row
        const uint32_t dpitch = static_cast<uint32_t>(p.n_out) * (OUT == OUT_BF16 ? 2 : 1);
        constexpr int DW = (OUT == OUT_BF16 ? 2 : 1) * 32 * TO;      // D bytes per row of the wave
        const uint32_t cvalid = static_cast<uint32_t>(min(128, 2 * (p.n - nbase)));
        const uint32_t dvalid = static_cast<uint32_t>(min(DW, (OUT == OUT_BF16 ? 2 : 1) * (p.n_out - ocol0)));
        uint8_t* const cW = reinterpret_cast<uint8_t*>(p.c + mb * p.n + nbase);      // the wave's first C row
        uint8_t* const dW = OUT == OUT_BF16 ? reinterpret_cast<uint8_t*>(p.d + (mb * p.n_out + ocol0) * 2)
                                            : dW0 + ocol0;
        float* const stg = sT;
        int lid2 = lane;
        asm volatile("" : "+v"(lid2));
        uint32_t colw[TO];                                          // E8M0 bytes of 4 column blocks
#pragma unroll
        for (int to = 0; to < TO; ++to) colw[to] = 0;
        auto tile_ok = [&](int to) __attribute__((always_inline)) { return PAIR || nbase + 32 * to < p.n; };
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const uint32_t ml = tm * 32 + l32;
          if constexpr (ACT == ACT_SRELU) {
            // C = alpha acc, formed once for both the C store and the
            // activation (the accumulators are not read again)
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[tm][t][v] *= alpha;
          }
          const float ca = ACT == ACT_SRELU ? 1.0f : alpha;
          if (p.c) {
            // C = alpha acc of the wave's 64 GEMM columns
            v4u cq[4] = {};
#pragma unroll
            for (int t = 0; t < TN; ++t) {
              if (!tile_ok(PAIR ? 0 : t)) continue;
              float c[16];
#pragma unroll
              for (int v = 0; v < 16; ++v) c[v] = ca * acc[tm][t][v];
              bf16_pieces(c, cq + 2 * t);
            }
            store_rows<128>(cW + tm * 32 * cpitch, cpitch, cq, stg, lid2, cvalid);
          }
          v4u dq[OUT == OUT_BF16 ? 2 * TO : TO] = {};    // bf16 D pieces, or E4M3 row pieces
          v4u kq[TO] = {};                               // E4M3 D_col pieces
#pragma unroll
          for (int to = 0; to < TO; ++to) {
            if (!tile_ok(to)) continue;
            const int ocol = ocol0 + 32 * to;
            float d[16];
            if constexpr (ACT == ACT_SWIGLU) {
              // pairs [X_b | G_b] of 32 columns ("Grouped GEMM + SwiGLU (SM100)",
              // Step 2): D = prob * (alpha X) * silu(alpha G), times norm_const
              // for FP8 output, evaluated as (X G) (prob nc alpha^2) sigmoid(alpha G)
              const v16f& ax = acc[tm][2 * to];
              const v16f& ag = acc[tm][2 * to + 1];
              const float f = pr[tm] * nc * (alpha * alpha);
              const float nal = -alpha * kLog2e;
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(ag[v] * nal));
                d[v] = (ax[v] * ag[v]) * (f * s);
              }
            } else if constexpr (ACT == ACT_GEGLU) {
              // pairs [G_b | U_b] of 32 columns, gate first ("Grouped GEMM + GLU +
              // Hadamard", §Equations, GeGLU): both halves of C = alpha acc
              // clamped to [glu_clamp_min, glu_clamp_max], then
              // D = gamma prob (U + offset) G sigmoid(geglu_alpha G), times norm_const
              const v16f& ag = acc[tm][2 * to];
              const v16f& au = acc[tm][2 * to + 1];
              const float f = pr[tm] * nc * p.glu_gamma;
              const float nga = -p.geglu_alpha * kLog2e;
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const float g = fminf(fmaxf(alpha * ag[v], p.glu_clamp_min), p.glu_clamp_max);
                const float u = fminf(fmaxf(alpha * au[v], p.glu_clamp_min), p.glu_clamp_max);
                const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * nga));
                d[v] = ((u + p.linear_offset) * g) * (f * s);
              }
            } else {
              const float f = pr[tm] * nc;
              if constexpr (ACT == ACT_SRELU) {
                // D = prob * (s * min(tanh(relu(C)/s), 1))^2, or prob * relu(C)^2 for s = 0,
                // evaluated as (prob s^2) t^2 with t = tanh(relu(C)/s) <= 1
                // ("Grouped GEMM + sReLU (SM100)", §Equations, §Tanh soft clamp)
                // (the clamp test outside the element loop: inside it, the
                // compiler made one branch per element, which kept the sixteen
                // tanh chains from overlapping)
                const float s = p.srelu_s;
                if (s > 0.0f) {
                  const float rs = 1.0f / s;
                  const float fs2 = f * (s * s);
#pragma unroll
                  for (int v = 0; v < 16; ++v) {
                    const float t = tanh_nonneg(fmaxf(acc[tm][to][v], 0.0f) * rs);
                    d[v] = fs2 * (t * t);
                  }
                } else {
#pragma unroll
                  for (int v = 0; v < 16; ++v) {
                    const float r = fmaxf(acc[tm][to][v], 0.0f);
                    d[v] = f * (r * r);
                  }
                }
              } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) d[v] = f * (alpha * acc[tm][to][v]);
              }
            }
            if constexpr (OUT == OUT_BF16) {
              bf16_pieces(d, dq + 2 * to);
#pragma unroll
              for (int v = 0; v < 16; v += 2) amax_l = max_abs2(amax_l, d[v], d[v + 1]);
            } else {
              colw[to] |= quant_codes(sT, sS, sfW0 + (ocol >> 5), ml * static_cast<uint32_t>(p.n_out >> 5), hi, l32, d,
                                      dq[to], kq[to])
                          << (8 * tm);
            }
          }
          uint8_t* const dB = dW + tm * 32 * dpitch;     // this 32-row block's first D row
          if constexpr (OUT == OUT_E4M3 && PAIR) {
            *at(reinterpret_cast<v4u*>(dW0 + ocol0), ml * dpitch + 16 * hi) = dq[0];
            *at(reinterpret_cast<v4u*>(dcW0 + ocol0), ml * dpitch + 16 * hi) = kq[0];
          } else {
            store_rows<DW>(dB, dpitch, dq, stg, lid2, dvalid);
            if constexpr (OUT == OUT_E4M3) store_rows<DW>(dcW0 + ocol0 + tm * 32 * dpitch, dpitch, kq, stg, lid2, dvalid);
          }
        }
        if constexpr (OUT == OUT_E4M3) {
          // column l32's scale bytes of the wave's 4 consecutive 32-row blocks
#pragma unroll
          for (int to = 0; to < TO; ++to) {
            const int ocol = ocol0 + 32 * to;
            if (tile_ok(to) && hi == 0)
              *at(reinterpret_cast<uint32_t*>(p.sfd_col + static_cast<int64_t>(ocol) * (vm >> 5) + mblk0),
                  l32 * sfc_pitch) = colw[to];
          }
        }
      }
      if constexpr (OUT == OUT_BF16) {
        const float w = wave_max(amax_l);
        if (lane == 0) atomicMax(&sAmax[0], __float_as_uint(w));
      }
    }
  };

  // Per-group amax: each wave folds its value for the tile into sAmax (an
  // LDS atomic max on the float bits, which order like the values: |D| >= 0).
  // After the barrier that starts the workgroup's next tile (or the one
  // after its last), lane 0 of wave 0 sends the tile's value to the group's
  // amax with one global atomic and clears the slots: one global atomic per
  // tile instead of one per wave, on addresses that every workgroup holding
  // a tile of the group updates (measured: FC2 with Zipf routing spent 16 %
  // of its time in these atomics at one per wave).
  constexpr int NAMAX = OUT != OUT_BF16 ? 0
                        : (ACT == ACT_DSWIGLU || ACT == ACT_DGEGLU) ? (MX ? 2 : 0)
                        : ACT == ACT_DSRELU ? (MX ? 1 : 0)
                                            : 1;
  auto flush_amax = [&](int gf) __attribute__((always_inline)) {
    if constexpr (NAMAX > 0) {
      if (gf >= 0 && wave == 0 && lane < NAMAX) {
        const uint32_t v = sAmax[lane];
        sAmax[lane] = 0;
        if (v) atomicMax(reinterpret_cast<unsigned int*>(p.amax) + NAMAX * gf + lane, v);
      }
    }
  };
  // the LDS atomics of this wave's epilogue performed before a barrier
  auto wait_lds = []() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0xC07F); };

  // ---- persistent tile loop ----
  // Two LDS stages.  Every cluster ends at a workgroup barrier; waves 4-7
  // pass one extra barrier at the start of a tile and waves 0-3 one at its
  // end, so between two barriers one wave of each SIMD is in a C cluster and
  // the other in an M cluster.  A stage's early set (read in M0) is free once
  // both wave groups have passed M0, its late set once both have passed M1.
  //
  // Even step counts >= 4: stage s+2's early set is issued in M1(s) into the
  // buffer of stage s, its late set in M0(s+1); M1(s) waits for stage s+1's
  // early set and M0(s+1) for its late set, so every load has about four
  // clusters to arrive and the barrier after the wait publishes it before
  // any wave reads it.  A tile's last two steps load the next tile's first
  // stage into buffer 0 (the current tile's again when there is none), so
  // every tile starts in buffer 0; the tile's first M0 loads stage 1 whole
  // into buffer 1, which the previous epilogue used as scratch.
  // Other step counts: stage s+1 is loaded whole in M0(s) and waited for in
  // M1(s); the next tile's first stage is loaded during the epilogue.
  // The K loop is unrolled by two (no exits inside) so every buffer is named
  // statically.
  const int nks = p.k_steps;
  int t = __builtin_amdgcn_readfirstlane(slot);
  if (t >= total) return;
  int done_g = -1;     // group of the tile whose amax waits in sAmax
  Tile cur = tile_of(t);
  Src src = make_src(cur);
  issue(src, 0, st0);

  auto sync = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // pin the accumulators after each MFMA cluster (the MFMAs are pure
  // operations that the compiler would otherwise sink past the barriers,
  // out of their cluster and into the code after the K loop)
  // (rows [0, tm_end): a tile's first step pins after its first cluster only
  // the rows that cluster wrote, so the previous tile's values of the other
  // rows are not kept alive through the epilogue)
  auto pin_acc = [&](int tm_end = TM) __attribute__((always_inline)) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        if (tm < tm_end) asm volatile("" : "+v"(acc[tm][tn]));
  };
  using NoWait = std::integral_constant<int, -1>;
  using WaitAll = std::integral_constant<int, 0>;
  // steady state: M0(s) waits for stage s's late set, M1(s) for stage s+1's
  // early set (see the issue order in the loop below)
  using WaitM0 = std::integral_constant<int, N_EARLY>;
  using WaitM1 = std::integral_constant<int, N_LATE + N_EA>;
  auto no_loads = []() __attribute__((always_inline)) {};
  auto no_hook = [](int) __attribute__((always_inline)) {};
  // hook issuing N loads spread evenly over a C cluster's MFMAs
  auto spread = [&](auto nc, auto&& f) __attribute__((always_inline)) {
    constexpr int N = decltype(nc)::value;
    return [f](int i) __attribute__((always_inline)) {
      constexpr int gap = NMMA / N;
      if (i % gap == 0 && i / gap < N) f(i / gap);
    };
  };
  // one K-step out of stage `st`: m0 / m1 issue loads in the M clusters
  // after the LDS reads, c0 / c1 are hooks run between the MFMAs of the C
  // clusters; the M clusters then wait until at most W0 / W1 of this wave's
  // loads are outstanding (no wait for -1)
  auto step_impl = [&](auto zc, const Stage& st, auto&& m0, auto&& c0, auto&& m1, auto&& c1, auto w0c, auto w1c)
      __attribute__((always_inline)) {
    constexpr int W0 = decltype(w0c)::value, W1 = decltype(w1c)::value;
    Ops0 o0 = read0(st);
    m0();
    fin0(o0);
    if constexpr (W0 >= 0) wait_vmcnt<W0>();
    sync();
    mma(0, o0.a, o0, c0, zc);
    pin_acc(decltype(zc)::value ? 2 : TM);
    sync();
    Ops1 o1 = read1(st);
    m1();
    fin1(o1);
    if constexpr (W1 >= 0) wait_vmcnt<W1>();
    sync();
    mma(2, o1.a, o0, c1, zc);
    pin_acc();
    sync();
  };
  // a K-step accumulating onto the tile's sums, and a tile's first K-step,
  // which starts them from zero
  auto step = [&](auto&&... args) __attribute__((always_inline)) {
    step_impl(std::false_type{}, static_cast<decltype(args)&&>(args)...);
  };
  auto step_z = [&](auto&&... args) __attribute__((always_inline)) {
    step_impl(std::true_type{}, static_cast<decltype(args)&&>(args)...);
  };

  // Stage s+2 is loaded during step s: its early first part in M1(s), its
  // B rows in C1(s), its late set in C0(s+1).  Hooks and waits of a
  // steady-state pair of steps (s even in buffer 0, s+1 in buffer 1):
  using I2 = std::integral_constant<int, N_LATE>;
  using I4 = std::integral_constant<int, N_EB>;
  auto lhook = [&](int ks, Stage d) __attribute__((always_inline)) {
    return spread(I2{}, [&, ks, d](int j) __attribute__((always_inline)) { issue_l(src, ks, d, j); });
  };
  auto ehook = [&](int ks, Stage d) __attribute__((always_inline)) {
    return spread(I4{}, [&, ks, d](int j) __attribute__((always_inline)) { issue_eb(src, ks, d, j); });
  };
  // steps 0 and 1 of a tile (stage 0 resident): stage 1 whole in M0(0)
  auto first_pair = [&]() __attribute__((always_inline)) {
    step_z(st0, [&]() __attribute__((always_inline)) { issue(src, 1, st1); }, no_hook,
         [&]() __attribute__((always_inline)) { issue_ea(src, 2, st0); }, ehook(2, st0), NoWait{}, WaitM1{});
    step(st1, no_loads, lhook(2, st0), [&]() __attribute__((always_inline)) { issue_ea(src, 3, st1); }, ehook(3, st1),
         WaitM0{}, WaitM1{});
  };
  // steps ks (buffer 0) and ks+1 (buffer 1), loading stages up to ks+3
  auto mid_pair = [&](int ks) __attribute__((always_inline)) {
    step(st0, no_loads, lhook(ks + 1, st1), [&]() __attribute__((always_inline)) { issue_ea(src, ks + 2, st0); },
         ehook(ks + 2, st0), WaitM0{}, WaitM1{});
    step(st1, no_loads, lhook(ks + 2, st0), [&]() __attribute__((always_inline)) { issue_ea(src, ks + 3, st1); },
         ehook(ks + 3, st1), WaitM0{}, WaitM1{});
  };

  // MODE 0: even step counts >= 4, the next tile's first stage loaded
  // during the last two steps; MODE 1: odd step counts >= 5, MODE 3: three
  // steps and MODE 2: one or two steps, the next tile's first stage loaded
  // during the epilogue.  (No mode branches on the step count between
  // different step bodies: such branches make the register allocator spill.)
  auto run = [&](auto mode_c) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    while (true) {
      int t_next = t + nwg;
      // The last pass is usually partial: its tiles are split evenly over the
      // XCDs, each XCD's share contiguous, rather than filling the first
      // slots (which would leave some XCDs idle and crowd the others' L2).
      // Grids of a multiple of 8 workgroups (nwg / 8 on each XCD) only.
      if (nwg >= 8 && (nwg & 7) == 0) {
        const int base = t_next - slot;                 // first tile of the next pass
        if (base < total && total - base < nwg) {
          const int rem = total - base, xcd = wg & 7, jx = wg >> 3;
          const int lo = rem * xcd / 8, hi8 = rem * (xcd + 1) / 8;
          t_next = lo + jx < hi8 ? base + lo + jx : total;
        }
      }
      const bool has_next = t_next < total;
      const Tile nxt = tile_of(has_next ? t_next : t);
      // stage 0 (and whatever the previous epilogue left in flight) complete
      // and visible, the previous epilogue's scratch free
      wait_vmcnt<0>();
      if constexpr (NAMAX > 0) wait_lds();
      sync();
      flush_amax(done_g);
      if (wm) sync();
      if constexpr (MODE == 0) {
        first_pair();
        for (int ks = 2; ks < nks - 2; ks += 2) mid_pair(ks);
        const EpiIn ein = epi_in(cur);
        step(st0, no_loads, lhook(nks - 1, st1),
             [&]() __attribute__((always_inline)) {
               src = make_src(nxt);
               issue_ea(src, 0, st0);
             },
             ehook(0, st0), WaitM0{}, WaitM1{});
        step(st1, no_loads,
             spread(I2{}, [&](int j) __attribute__((always_inline)) {
               if (j == 0) load_prob(cur);
               issue_l(src, 0, st0, j);
             }),
             no_loads, no_hook, WaitM0{}, NoWait{});
        if (!wm) sync();
        wait_vmcnt<N_LATE>();      // prob (issued before the next tile's late set)
        epilogue(cur, ein);
      } else {
        if constexpr (MODE == 1 || MODE == 3) {
          // steps 0 .. nks-4 in pairs, then nks-3 (buffer 0), nks-2 (buffer 1)
          // and nks-1 (buffer 0), which load nothing beyond stage nks-1
          // (MODE 1: odd nks >= 5; MODE 3: nks == 3, whose step 0 loads
          // stage 1 whole)
          if constexpr (MODE == 1) {
            first_pair();
            for (int ks = 2; ks < nks - 3; ks += 2) mid_pair(ks);
            step(st0, no_loads, lhook(nks - 2, st1),
                 [&]() __attribute__((always_inline)) { issue_ea(src, nks - 1, st0); }, ehook(nks - 1, st0), WaitM0{},
                 WaitM1{});
          } else {
            step_z(st0, [&]() __attribute__((always_inline)) { issue(src, 1, st1); }, no_hook,
                   [&]() __attribute__((always_inline)) { issue_ea(src, 2, st0); }, ehook(2, st0), NoWait{}, WaitM1{});
          }
          step(st1, no_loads, lhook(nks - 1, st0), no_loads, no_hook, WaitM0{},
               std::integral_constant<int, N_LATE>{});
          step(st0, no_loads, no_hook, no_loads, no_hook, WaitAll{}, NoWait{});
        } else {
          if (nks == 2) {
            step_z(st0, [&]() __attribute__((always_inline)) { issue(src, 1, st1); }, no_hook, no_loads, no_hook,
                   NoWait{}, WaitAll{});
            step(st1, no_loads, no_hook, no_loads, no_hook, NoWait{}, NoWait{});
          } else {
            step_z(st0, no_loads, no_hook, no_loads, no_hook, NoWait{}, NoWait{});
          }
        }
        const EpiIn ein = epi_in(cur);
        if (!wm) sync();
        src = make_src(nxt);
        load_prob(cur);
        issue(src, 0, st0);
        wait_vmcnt<N_EARLY + N_LATE>();   // prob (issued before the next tile's first stage)
        epilogue(cur, ein);
      }
      done_g = cur.g;
      if (!has_next) break;
      t = t_next;
      cur = nxt;
      // the new tile's per-lane source offsets are rebuilt here (from a fresh
      // opaque lane id) instead of being kept live through the epilogue
      src = make_src(cur);
    }
  };
  if ((nks & 1) == 0 && nks >= 4) run(std::integral_constant<int, 0>{});
  else if (nks >= 5) run(std::integral_constant<int, 1>{});
  else if (nks == 3) run(std::integral_constant<int, 3>{});
  else run(std::integral_constant<int, 2>{});
  // no direct-to-LDS write may still be in flight when the workgroup ends
  wait_vmcnt<0>();
  if constexpr (NAMAX > 0) {
    wait_lds();
    sync();
    flush_amax(done_g);
  }
}

template <int AB, int ACT, int OUT>
hipError_t launch_one(const KernelArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_kernel<AB, ACT, OUT>), dim3(static_cast<unsigned>(a.grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// Every instance of one operand family.  Backward activations with BF16
// operands write a BF16 dC only.
template <int AB>
hipError_t launch_family(int act, int out, const KernelArgs& a, hipStream_t s) {
  const bool e4 = out == OUT_E4M3;
  switch (act) {
    case ACT_NONE: return e4 ? launch_one<AB, ACT_NONE, OUT_E4M3>(a, s) : launch_one<AB, ACT_NONE, OUT_BF16>(a, s);
    case ACT_SWIGLU: return e4 ? launch_one<AB, ACT_SWIGLU, OUT_E4M3>(a, s) : launch_one<AB, ACT_SWIGLU, OUT_BF16>(a, s);
    case ACT_SRELU: return e4 ? launch_one<AB, ACT_SRELU, OUT_E4M3>(a, s) : launch_one<AB, ACT_SRELU, OUT_BF16>(a, s);
    case ACT_DSWIGLU:
      if constexpr (AB == AB_BF16) return e4 ? hipErrorInvalidValue : launch_one<AB, ACT_DSWIGLU, OUT_BF16>(a, s);
      else return e4 ? launch_one<AB, ACT_DSWIGLU, OUT_E4M3>(a, s) : launch_one<AB, ACT_DSWIGLU, OUT_BF16>(a, s);
    case ACT_DSRELU:
      if constexpr (AB == AB_BF16) return e4 ? hipErrorInvalidValue : launch_one<AB, ACT_DSRELU, OUT_BF16>(a, s);
      else return e4 ? launch_one<AB, ACT_DSRELU, OUT_E4M3>(a, s) : launch_one<AB, ACT_DSRELU, OUT_BF16>(a, s);
    case ACT_GEGLU: return e4 ? launch_one<AB, ACT_GEGLU, OUT_E4M3>(a, s) : launch_one<AB, ACT_GEGLU, OUT_BF16>(a, s);
    case ACT_DGEGLU:
      if constexpr (AB == AB_BF16) return e4 ? hipErrorInvalidValue : launch_one<AB, ACT_DGEGLU, OUT_BF16>(a, s);
      else return e4 ? launch_one<AB, ACT_DGEGLU, OUT_E4M3>(a, s) : launch_one<AB, ACT_DGEGLU, OUT_BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace moegg
