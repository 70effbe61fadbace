// HIP kernels of libmoegg for gfx950 (CDNA4): contiguous grouped
// block-scaled GEMM with fused epilogue.
//
// Method ("Grouped GEMM + Quant (SM100)", "Grouped GEMM + SwiGLU (SM100)",
// "Grouped GEMM + sReLU (SM100)", "Grouped GEMM + dGLU (SM100)", §Equations):
// rows m of A in [padded_offsets[g-1], padded_offsets[g]) are multiplied by
// expert g's weight B[g] (N x K, K-major) with per-32-element E8M0 block
// scales on both operands, scaled by alpha_g (alpha_g^2 for the dSwiGLU
// backward), then the activation / gating / output-formatting epilogue.
//
// Mapping onto CDNA4:
//  * one workgroup = 4 wave64s = a 128-row x 256-column output tile; a tile
//    never straddles two experts because groups are padded to a multiple of
//    128 rows, so the expert index is one per workgroup (binary search of
//    padded_offsets, wave-uniform).
//  * the contraction runs on the block-scaled matrix cores:
//    v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 or E2M1 operands, one E8M0 byte
//    per lane and operand selects the scale of that lane's 32 K-elements) or
//    v_mfma_f32_32x32x16_bf16.  The weight tile is the instruction's first
//    operand and the token tile the second, so an accumulator lane holds one
//    token row and 16 output columns (4 runs of 4 contiguous columns): row
//    reductions are lane-local, stores are 8-byte (bf16) / 4-byte (e4m3) runs.
//  * K advances in steps of 128 bytes per row (128 E4M3, 256 E2M1 or 64 BF16
//    elements); A/B step tiles are staged global -> registers -> LDS with a
//    double buffer (row stride 144 B, conflict-free 16-byte LDS reads), one
//    barrier per step.  Scale bytes go straight to registers.
//  * the epilogue runs on the fp32 accumulators in registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moegg_internal.h"

namespace moegg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));   // native vectors (HIP's uint4
typedef uint32_t v2u __attribute__((ext_vector_type(2)));   // struct defeats SROA)

constexpr int kBK = 128;          // bytes of K per row and pipeline stage (one cache line)
constexpr int kBandM = 8;         // m-tiles per raster band (L2 reuse of B)

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

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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

// Four fp32 -> four E4M3 codes (RNE by the conversion unit, saturated to
// +-448 beforehand), packed little-endian: a is the lowest byte.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)); saturates to 0 / 1 at the extremes.
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// tanh(x) for x >= 0: odd Taylor series below 1/8 (error < 2e-10), else
// (1 - e^-2x) / (1 + e^-2x).  Result <= 1.
__device__ __forceinline__ float tanh_nonneg(float x) {
  const float x2 = x * x;
  const float series = x * (1.0f + x2 * (-1.0f / 3.0f + x2 * (2.0f / 15.0f + x2 * (-17.0f / 315.0f))));
  const float e = __builtin_amdgcn_exp2f(-2.0f * kLog2e * x);
  const float big = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
  return x < 0.125f ? series : big;
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

// Column offset (within a 32-column MFMA tile) of accumulator element v of
// this lane: rows of the 32x32 result are spread as 8*(v/4) + 4*(lane/32) + v%4.
__device__ __forceinline__ int nofs(int v, int hi) { return 8 * (v >> 2) + 4 * hi + (v & 3); }

// Store 16 values of one row (one 32-column tile) as bf16: 4 runs of 4.
__device__ __forceinline__ void store_bf16_tile(uint8_t* base, int64_t m, int ld, int col, int hi,
                                                const float* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v2u w;
    w.x = bf16_rne(v[4 * j + 0]) | (bf16_rne(v[4 * j + 1]) << 16);
    w.y = bf16_rne(v[4 * j + 2]) | (bf16_rne(v[4 * j + 3]) << 16);
    *reinterpret_cast<v2u*>(base + (m * ld + col + 8 * j + 4 * hi) * 2) = w;
  }
}

// FP8 row + column quantisation of one 32-column output tile ("Grouped GEMM +
// Quant (SM100)", §Equations Step 3 and §Diagram Row/Col Quantize).  A row
// block is this lane's 16 values plus those of lane ^ 32; a column block is
// one accumulator element over the 32 lanes of this half-wave.
__device__ __forceinline__ void quant_store_tile(const KernelArgs& p, int m, int mblk, int ocol, int hi,
                                                 int l32, float nc, const float* d) {
  float ra = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) ra = fmaxf(ra, fabsf(d[v]));
  ra = halves_max(ra);
  const uint32_t br = e8m0_ceil((nc * ra) * kRcp448);
  const float sr = e8m0_inverse(br);
  const int64_t rowoff = static_cast<int64_t>(m) * p.n_out + ocol + 4 * hi;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = e4m3x4((d[4 * j] * nc) * sr, (d[4 * j + 1] * nc) * sr, (d[4 * j + 2] * nc) * sr,
                              (d[4 * j + 3] * nc) * sr);
    *reinterpret_cast<uint32_t*>(p.d + rowoff + 8 * j) = w;
  }
  if (hi == 0) p.sfd_row[static_cast<int64_t>(m) * (p.n_out >> 5) + (ocol >> 5)] = static_cast<uint8_t>(br);

  // column scales; lane l32 < 16 of each half keeps the byte of its element l32
  const int idx = l32 & 15;
  uint32_t bsel = 0;
  float sc[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float cm = half_max(fabsf(d[v]));
    const uint32_t b = e8m0_ceil((nc * cm) * kRcp448);
    sc[v] = e8m0_inverse(b);
    bsel = idx == v ? b : bsel;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = e4m3x4((d[4 * j] * nc) * sc[4 * j], (d[4 * j + 1] * nc) * sc[4 * j + 1],
                              (d[4 * j + 2] * nc) * sc[4 * j + 2], (d[4 * j + 3] * nc) * sc[4 * j + 3]);
    *reinterpret_cast<uint32_t*>(p.d_col + rowoff + 8 * j) = w;
  }
  if (l32 < 16)
    p.sfd_col[static_cast<int64_t>(ocol + nofs(idx, hi)) * (p.valid_m >> 5) + mblk] = static_cast<uint8_t>(bsel);
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

template <int AB, int ACT, int OUT>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(KernelArgs p) {
  constexpr int BM = kBM, BN = kBN, BK = kBK;
  constexpr int NW = kThreads / 64;  // 8 waves: 2 (m) x 4 (n), two per SIMD
  constexpr int WM = BM / 2;         // rows per wave (64)
  constexpr int WN = BN / 4;         // GEMM columns per wave (64)
  constexpr int TM = WM / 32;        // 32-row MFMA tiles per wave
  constexpr int TN = WN / 32;        // 32-column MFMA tiles per wave
  constexpr bool MX = AB != AB_BF16;
  constexpr int SW = AB == AB_E2M1 ? 2 : 1;          // scale words per row per step
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  // scale words per stage, word w of row r at [w * rows + r]; the A area has
  // spare room so that every wave issues the same number of loads
  constexpr int SA_WORDS = MX ? 4 * BM : 1, SB_WORDS = MX ? SW * BN : 1;

  // Three-stage LDS ring (about 150 KB: one workgroup per CU), one distinct
  // array per stage and operand: the compiler can then tell the stages apart
  // and adds no conservative waits for the direct-to-LDS loads (the explicit
  // waits below order them).  Rows are BK = 128 bytes, a whole cache line, so
  // every load instruction moves whole lines; the 16-byte chunk c of row r
  // sits at chunk slot c ^ ((r >> 1) & 7).  The LDS has 64 four-byte banks
  // (256 bytes), so two consecutive 128-byte rows fill one bank window and a
  // 16-lane group of 16-byte reads (16 consecutive rows, one chunk each) hits
  // 16 distinct bank quads.
  __shared__ __attribute__((aligned(16))) uint8_t sA0[A_BYTES], sA1[A_BYTES], sA2[A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[B_BYTES], sB1[B_BYTES], sB2[B_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t sSA0[SA_WORDS], sSA1[SA_WORDS], sSA2[SA_WORDS];
  __shared__ __attribute__((aligned(16))) uint32_t sSB0[SB_WORDS], sSB1[SB_WORDS], sSB2[SB_WORDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroup -> tile.  Workgroups are dispatched round-robin over the 8
  // XCDs (each with its own L2), so XCD x gets the contiguous logical range
  // [x*q + min(x, r), ...) of the nwg tiles; inside it tiles run in bands of
  // kBandM m-tiles, m fastest, so the tiles resident on one XCD form a
  // compact patch that shares each K-slice of A and B through L2.
  const int nwg = static_cast<int>(gridDim.x);
  const int wg = static_cast<int>(blockIdx.x);
  const int xcd = wg & 7, slot = wg >> 3, q = nwg >> 3, r = nwg & 7;
  const int logical = xcd * q + min(xcd, r) + slot;
  const int band = logical / (kBandM * p.n_tiles);
  const int in_band = logical - band * kBandM * p.n_tiles;
  const int band_rows = min(kBandM, p.m_tiles - band * kBandM);
  const int nt = in_band / band_rows;
  const int mt = band * kBandM + (in_band - nt * band_rows);
  const int row0 = mt * BM;
  const int n0 = nt * BN;

  // expert of this row tile: the number of padded_offsets entries <= row0
  int lo = 0, up = p.num_groups;
  while (lo < up) {
    const int mid = (lo + up) >> 1;
    if (p.po[mid] > row0) up = mid; else lo = mid + 1;
  }
  const int g = lo < p.num_groups ? lo : p.num_groups - 1;   // inconsistent offsets never index out of range

  // ---- direct global -> LDS staging ----
  // One wave instruction fills 8 rows (1 KB).  Wave w fills A rows
  // [16w, 16w+16) (2 instructions) and B rows [32w, 32w+32) (4
  // instructions): lane i writes row r = 8j + i/8, chunk slot i%8, i.e.
  // logical chunk (i%8) ^ ((r >> 1) & 7) of that row.  Scale dwords ride along, one per lane:
  // E4M3 (one dword per row and step): waves 0-1 load A rows, waves 2-5 B
  // rows, waves 6-7 a spare copy of A; E2M1 (two dwords per row and step):
  // two loads per wave covering both words of A and B.
  constexpr int A_INS = BM / 8 / NW, B_INS = BN / 8 / NW;
  const int lrow = lane >> 3;
  const uint8_t* gA[A_INS];
  const uint8_t* gB[B_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int r = wave * (8 * A_INS) + j * 8 + lrow;             // row in the tile
    gA[j] = p.a + static_cast<int64_t>(row0 + r) * p.row_bytes + (((lane & 7) ^ ((r >> 1) & 7)) * 16);
  }
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    const int r = wave * (8 * B_INS) + j * 8 + lrow;
    gB[j] = p.b + (static_cast<int64_t>(g) * p.n + min(n0 + r, p.n - 1)) * p.row_bytes +
            (((lane & 7) ^ ((r >> 1) & 7)) * 16);
  }
  // scale loads: for load slot u of this wave, the source row pointer and the
  // LDS word offset (rows of A: 128, of B: 256; 64 rows per load)
  constexpr int S_LOADS = AB == AB_E4M3 ? 1 : AB == AB_E2M1 ? 2 : 0;
  const uint8_t* gS[S_LOADS > 0 ? S_LOADS : 1];
  int sdst[S_LOADS > 0 ? S_LOADS : 1];
  bool sisA[S_LOADS > 0 ? S_LOADS : 1];
  if constexpr (MX) {
#pragma unroll
    for (int u = 0; u < S_LOADS; ++u) {
      // job = (wave * S_LOADS + u): E4M3 jobs 0-1 A rows, 2-5 B rows, 6-7 spare
      // A; E2M1 jobs 0-3 A (word, half), 4-11 B (word, quarter), 12-15 spare A
      const int job = wave * S_LOADS + u;
      int word, rowsel, isA;
      if (AB == AB_E4M3) {
        isA = job < 2 || job >= 6;
        word = 0;
        rowsel = job < 2 ? job * 64 : job >= 6 ? (job - 6) * 64 : (job - 2) * 64;
        sdst[u] = job < 2 ? job * 64 : job >= 6 ? 2 * BM + (job - 6) * 64 : (job - 2) * 64;
      } else {
        isA = job < 4 || job >= 12;
        const int aj = job < 4 ? job : job - 12, bj = job - 4;
        word = isA ? aj >> 1 : bj >> 2;
        rowsel = isA ? (aj & 1) * 64 : (bj & 3) * 64;
        sdst[u] = isA ? (job < 4 ? word * BM + rowsel : 2 * BM + word * BM + rowsel) : word * BN + rowsel;
      }
      sisA[u] = isA;
      gS[u] = isA ? p.sfa + static_cast<int64_t>(row0 + rowsel + lane) * p.ksf + word * 4
                  : p.sfb + (static_cast<int64_t>(g) * p.n + min(n0 + rowsel + lane, p.n - 1)) * p.ksf + word * 4;
    }
  }
  // vector-memory instructions per wave per stage
  constexpr int VM_PER_STAGE = A_INS + B_INS + S_LOADS;

  auto issue = [&](int ks, uint8_t* dA, uint8_t* dB, uint32_t* dSA, uint32_t* dSB) {
    const int kb = ks * BK;
#pragma unroll
    for (int j = 0; j < A_INS; ++j) dma16(gA[j] + kb, dA + (wave * (8 * A_INS) + j * 8) * BK);
#pragma unroll
    for (int j = 0; j < B_INS; ++j) dma16(gB[j] + kb, dB + (wave * (8 * B_INS) + j * 8) * BK);
    if constexpr (MX) {
#pragma unroll
      for (int u = 0; u < S_LOADS; ++u)
        dma4(gS[u] + ks * 4 * SW, (sisA[u] ? dSA : dSB) + sdst[u]);
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tm][tn][v] = 0.0f;

  const int sw = (l32 >> 1) & 7;              // swizzle of this lane's rows (tiles start at multiples of 32)
  const int a_rd = (wm * WM + l32) * BK;
  const int b_rd = (wn * WN + l32) * BK;
  // One K-step (BK bytes of every row) out of one LDS stage.
  auto compute = [&](const uint8_t* stA, const uint8_t* stB, const uint32_t* stSA, const uint32_t* stSB) {
    const uint8_t* sa = stA + a_rd;
    const uint8_t* sb = stB + b_rd;
    // scale words: byte 0 / 2 of the shifted word are this lane's K-blocks
    // for the first / second 64-element window of a word's four blocks
    uint32_t sca[TM][SW], scb[TN][SW];
    if constexpr (MX) {
      const int sh = 8 * hi;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int w = 0; w < SW; ++w) sca[tm][w] = stSA[w * BM + wm * WM + tm * 32 + l32] >> sh;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int w = 0; w < SW; ++w) scb[tn][w] = stSB[w * BN + wn * WN + tn * 32 + l32] >> sh;
    }
    if constexpr (AB == AB_E4M3) {
      static_for<0, 2>([&](auto kki) {
        constexpr int kk = decltype(kki)::value;
        // 8-bit operands: a lane of half h holds K [16h, 16h+16) and
        // [32+16h, 48+16h) of the 64-wide window (chunks h + 4kk and
        // h + 4kk + 2 of the row), while its scale byte covers the 32-element
        // block h of the window; FP4 operands hold [32h, 32h+32) instead.
        const int o0 = ((hi + 4 * kk) ^ sw) * 16, o1 = ((hi + 4 * kk + 2) ^ sw) * 16;
        v8i fa[TM], fb[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const v4u x0 = *reinterpret_cast<const v4u*>(sa + tm * 32 * BK + o0);
          const v4u x1 = *reinterpret_cast<const v4u*>(sa + tm * 32 * BK + o1);
          fa[tm] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const v4u x0 = *reinterpret_cast<const v4u*>(sb + tn * 32 * BK + o0);
          const v4u x1 = *reinterpret_cast<const v4u*>(sb + tn * 32 * BK + o1);
          fb[tn] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[tn], fa[tm], acc[tm][tn], 0, 0, kk * 2, (int)scb[tn][0], kk * 2, (int)sca[tm][0]);
      });
    } else if constexpr (AB == AB_E2M1) {
      static_for<0, 4>([&](auto kki) {
        constexpr int kk = decltype(kki)::value;
        const int o0 = ((hi + 2 * kk) ^ sw) * 16;
        v8i fa[TM], fb[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const v4u x0 = *reinterpret_cast<const v4u*>(sa + tm * 32 * BK + o0);
          fa[tm] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const v4u x0 = *reinterpret_cast<const v4u*>(sb + tn * 32 * BK + o0);
          fb[tn] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[tn], fa[tm], acc[tm][tn], 4, 4, (kk & 1) * 2, (int)scb[tn][kk >> 1], (kk & 1) * 2,
                (int)sca[tm][kk >> 1]);
      });
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int o0 = ((hi + 2 * kk) ^ sw) * 16;
        v8bf fa[TM], fb[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          fa[tm] = *reinterpret_cast<const v8bf*>(sa + tm * 32 * BK + o0);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          fb[tn] = *reinterpret_cast<const v8bf*>(sb + tn * 32 * BK + o0);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tn], fa[tm], acc[tm][tn], 0, 0, 0);
      }
    }
  };

  // ---- main loop: three LDS stages, loads two steps ahead ----
  // At the top of step ks the wave's outstanding loads are those of stages
  // ks and ks+1; waiting until only one stage's worth remains and then
  // meeting at the barrier makes stage ks visible to every wave, and every
  // wave has finished step ks-1, whose buffer then receives stage ks+2.
  // The loop is unrolled by three (no exits inside) so every buffer is named
  // statically; loads past the last stage repeat it (never computed) so the
  // count of outstanding loads per stage stays the same.  The last 0-2 steps
  // run after the loop.
  const int nks = p.k_steps;
  const int last = nks - 1;
  issue(0, sA0, sB0, sSA0, sSB0);
  issue(min(1, last), sA1, sB1, sSA1, sSB1);
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    wait_vmcnt<VM_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    issue(min(ks + 2, last), sA2, sB2, sSA2, sSB2);
    compute(sA0, sB0, sSA0, sSB0);
    wait_vmcnt<VM_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    issue(min(ks + 3, last), sA0, sB0, sSA0, sSB0);
    compute(sA1, sB1, sSA1, sSB1);
    wait_vmcnt<VM_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    issue(min(ks + 4, last), sA1, sB1, sSA1, sSB1);
    compute(sA2, sB2, sSA2, sSB2);
  }
  if (ks < nks) {                         // one or two steps left: stages in buffers 0 and 1
    wait_vmcnt<VM_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    compute(sA0, sB0, sSA0, sSB0);
    if (ks + 1 < nks) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      compute(sA1, sB1, sSA1, sSB1);
    }
  }
  // no direct-to-LDS write may still be in flight when the workgroup ends
  wait_vmcnt<0>();

  // ---- epilogue ----
  const float alpha = p.alpha[g];
  const int mbase = row0 + wm * WM;
  const int nbase = n0 + wn * WN;
  float amax_l = 0.0f;
  float nc = 1.0f;
  if constexpr (OUT == OUT_E4M3) nc = p.norm_const[0];

  if constexpr (ACT == ACT_DSWIGLU) {
    // R = alpha^2 acc; X = beta * C_in with blocks [input_b | gate_b]
    // ("Grouped GEMM + dGLU (SM100)", BF16 contract equations)
    const float a2 = alpha * alpha;
    const float beta = p.beta[g];
    const int ld2 = 2 * p.n;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int m = mbase + tm * 32 + l32;
      const float pr = p.prob[m];
      float dp = 0.0f;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int ncol = nbase + tn * 32;
        if (ncol >= p.n) continue;
        const int64_t xoff = static_cast<int64_t>(m) * ld2 + 2 * ncol;   // block b = ncol/32 starts at 64b
        float xin[16], xg[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v2u wi = *reinterpret_cast<const v2u*>(p.c_in + xoff + 8 * j + 4 * hi);
          const v2u wg = *reinterpret_cast<const v2u*>(p.c_in + xoff + 32 + 8 * j + 4 * hi);
          xin[4 * j + 0] = __uint_as_float(wi.x << 16);
          xin[4 * j + 1] = __uint_as_float(wi.x & 0xFFFF0000u);
          xin[4 * j + 2] = __uint_as_float(wi.y << 16);
          xin[4 * j + 3] = __uint_as_float(wi.y & 0xFFFF0000u);
          xg[4 * j + 0] = __uint_as_float(wg.x << 16);
          xg[4 * j + 1] = __uint_as_float(wg.x & 0xFFFF0000u);
          xg[4 * j + 2] = __uint_as_float(wg.y << 16);
          xg[4 * j + 3] = __uint_as_float(wg.y & 0xFFFF0000u);
        }
        float din[16], dgt[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float r = a2 * acc[tm][tn][v];
          const float x = beta * xin[v];
          const float gt = beta * xg[v];
          const float s = sigmoid_f(gt);
          const float swish = gt * s;
          din[v] = r * pr * swish;
          dgt[v] = r * pr * x * s * (1.0f + gt * (1.0f - s));
          dp += r * x * swish;
        }
        uint8_t* dbase = p.d;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v2u w;
          w.x = bf16_rne(din[4 * j]) | (bf16_rne(din[4 * j + 1]) << 16);
          w.y = bf16_rne(din[4 * j + 2]) | (bf16_rne(din[4 * j + 3]) << 16);
          *reinterpret_cast<v2u*>(dbase + (xoff + 8 * j + 4 * hi) * 2) = w;
          w.x = bf16_rne(dgt[4 * j]) | (bf16_rne(dgt[4 * j + 1]) << 16);
          w.y = bf16_rne(dgt[4 * j + 2]) | (bf16_rne(dgt[4 * j + 3]) << 16);
          *reinterpret_cast<v2u*>(dbase + (xoff + 32 + 8 * j + 4 * hi) * 2) = w;
        }
      }
      dp = halves_sum(dp);
      if (hi == 0) atomicAdd(p.dprob + m, dp);
    }
    return;
  } else {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int m = mbase + tm * 32 + l32;
      const int mblk = (mbase + tm * 32) >> 5;
      const float pr = p.prob[m];
      if constexpr (ACT == ACT_SWIGLU) {
        // pairs [X_b | G_b] of 32 columns ("Grouped GEMM + SwiGLU (SM100)", Step 2)
#pragma unroll
        for (int tp = 0; tp < TN / 2; ++tp) {
          const int xcol = nbase + tp * 64;
          if (xcol >= p.n) continue;
          float cx[16], cg[16], d[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            cx[v] = alpha * acc[tm][2 * tp][v];
            cg[v] = alpha * acc[tm][2 * tp + 1][v];
          }
          if (p.c) {
            store_bf16_tile(reinterpret_cast<uint8_t*>(p.c), m, p.n, xcol, hi, cx);
            store_bf16_tile(reinterpret_cast<uint8_t*>(p.c), m, p.n, xcol + 32, hi, cg);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) d[v] = pr * cx[v] * (cg[v] * sigmoid_f(cg[v]));
          const int ocol = xcol >> 1;
          if constexpr (OUT == OUT_BF16) {
            store_bf16_tile(p.d, m, p.n_out, ocol, hi, d);
#pragma unroll
            for (int v = 0; v < 16; ++v) amax_l = fmaxf(amax_l, fabsf(d[v]));
          } else {
            quant_store_tile(p, m, mblk, ocol, hi, l32, nc, d);
          }
        }
      } else {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int ncol = nbase + tn * 32;
          if (ncol >= p.n) continue;
          float c[16], d[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) c[v] = alpha * acc[tm][tn][v];
          if (p.c) store_bf16_tile(reinterpret_cast<uint8_t*>(p.c), m, p.n, ncol, hi, c);
          if constexpr (ACT == ACT_SRELU) {
            // D = prob * (s * min(tanh(relu(C)/s), 1))^2, or prob * relu(C)^2 for s = 0
            // ("Grouped GEMM + sReLU (SM100)", §Equations, §Tanh soft clamp)
            const float s = p.srelu_s;
            const float rs = s > 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float r = fmaxf(c[v], 0.0f);
              if (s > 0.0f) r = s * fminf(tanh_nonneg(r * rs), 1.0f);
              d[v] = pr * (r * r);
            }
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) d[v] = pr * c[v];
          }
          if constexpr (OUT == OUT_BF16) {
            store_bf16_tile(p.d, m, p.n_out, ncol, hi, d);
#pragma unroll
            for (int v = 0; v < 16; ++v) amax_l = fmaxf(amax_l, fabsf(d[v]));
          } else {
            quant_store_tile(p, m, mblk, ncol, hi, l32, nc, d);
          }
        }
      }
    }
    if constexpr (OUT == OUT_BF16) {
      const float w = wave_max(amax_l);
      if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(p.amax + g), __float_as_uint(w));
    }
  }
}

__global__ void fill_zero_kernel(float* ptr, int count) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < count) ptr[i] = 0.0f;
}

template <int AB, int ACT, int OUT>
hipError_t launch_one(const KernelArgs& a, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(a.m_tiles) * a.n_tiles;
  hipLaunchKernelGGL((grouped_gemm_kernel<AB, ACT, OUT>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int AB>
hipError_t launch_ab(int act, int out, const KernelArgs& a, hipStream_t s) {
  switch (act) {
    case ACT_NONE: return out == OUT_E4M3 ? launch_one<AB, ACT_NONE, OUT_E4M3>(a, s) : launch_one<AB, ACT_NONE, OUT_BF16>(a, s);
    case ACT_SWIGLU: return out == OUT_E4M3 ? launch_one<AB, ACT_SWIGLU, OUT_E4M3>(a, s) : launch_one<AB, ACT_SWIGLU, OUT_BF16>(a, s);
    case ACT_SRELU: return out == OUT_E4M3 ? launch_one<AB, ACT_SRELU, OUT_E4M3>(a, s) : launch_one<AB, ACT_SRELU, OUT_BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_grouped_gemm(int ab, int act, int out, const KernelArgs& a, hipStream_t s) {
  if (act == ACT_DSWIGLU) {
    if (ab != AB_BF16 || out != OUT_BF16) return hipErrorInvalidValue;
    return launch_one<AB_BF16, ACT_DSWIGLU, OUT_BF16>(a, s);
  }
  switch (ab) {
    case AB_E4M3: return launch_ab<AB_E4M3>(act, out, a, s);
    case AB_E2M1: return launch_ab<AB_E2M1>(act, out, a, s);
    case AB_BF16: return launch_ab<AB_BF16>(act, out, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill_zero(float* ptr, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((count + 255) / 256), dim3(256), 0, s, ptr, count);
  return hipGetLastError();
}

}  // namespace moegg
