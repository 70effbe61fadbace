// Internal interface between the C-ABI front (moegg_api.cpp) and the HIP
// kernels (grouped_gemm.h, instantiated by inst_*.hip; dispatch and the
// amax fill in moegg_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moegg {

// Operand family of A/B.
enum AbKind : int { AB_E4M3 = 0, AB_E2M1 = 1, AB_BF16 = 2, AB_E5M2 = 3 };
// Epilogue activation.
enum ActKind : int {
  ACT_NONE = 0, ACT_SWIGLU = 1, ACT_SRELU = 2, ACT_DSWIGLU = 3, ACT_DSRELU = 4, ACT_GEGLU = 5, ACT_DGEGLU = 6
};
// Output formatting of D.
enum OutKind : int { OUT_BF16 = 0, OUT_E4M3 = 1 };

// Block tile: BM token rows x BN GEMM columns, 512 threads (8 wave64s).
// Experts are cut into 256-row tiles plus at most one 128-row tile, so the
// row alignment of every expert (m_aligned) must be a multiple of kRowBlock.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kRowBlock = 128;
constexpr int kThreads = 512;

// Everything a kernel needs, passed by value (kernel argument segment).
struct KernelArgs {
  const uint8_t* a;        // (valid_m, row_bytes)
  const uint8_t* b;        // (L, n, row_bytes)
  const uint8_t* sfa;      // E8M0: (valid_m, K/32) row-major or (K/128, valid_m, 4) planes
  const uint8_t* sfb;      // (L*n, K/32) or (K/128, L*n, 4)
  const uint8_t* const* b_ptrs;     // discrete weights: (L) per-expert (n, row_bytes), or null
  const uint8_t* const* sfb_ptrs;   // discrete weights: (L) per-expert (n, K/32) or (K/128, n, 4), or null
  // scale word w (4 bytes: 128 K elements) of row r at r * sf_row + w * sf_word
  int64_t sf_word_a, sf_word_b;
  int32_t sf_row_a, sf_row_b;
  const int32_t* po;       // (L)
  const float* alpha;      // (L)
  const float* prob;       // (valid_m)
  const float* beta;       // (L) dSwiGLU
  const float* norm_const; // (1) E4M3 D
  const uint16_t* c_in;    // (valid_m, 2n) dSwiGLU, (valid_m, n) dsReLU
  uint16_t* c;             // (valid_m, n) optional
  uint8_t* d;              // (valid_m, n_out) bf16 or e4m3
  uint8_t* d_col;          // (valid_m, n_out) e4m3
  uint8_t* sfd_row;        // (valid_m, n_out/32)
  uint8_t* sfd_col;        // (n_out, valid_m/32)
  float* amax;             // (L)
  float* dprob;            // (valid_m)
  int64_t valid_m;
  int32_t num_groups;
  int32_t n;
  int32_t k;
  int32_t n_out;
  int32_t row_bytes;       // bytes per row of A and B
  int32_t ksf;             // scale bytes per row (K/32, a multiple of 4 per scale word of a step)
  int32_t n_tiles;         // ceil(n / kBN)
  int32_t k_steps;         // row bytes / 128 (one 128-byte step per row)
  int32_t grid;            // persistent workgroups launched (>= 1)
  float srelu_s;
  float glu_gamma;         // GeGLU forward output scale
  float geglu_alpha;       // GeGLU / dGeGLU sigmoid input scale
  float linear_offset;     // GeGLU / dGeGLU offset of the up branch
  float glu_clamp_min;     // GeGLU: both halves; dGeGLU: up only
  float glu_clamp_max;     // GeGLU: both halves; dGeGLU: gate and up
};

// Instances of one operand family (inst_*.hip).
hipError_t launch_e4m3(int act, int out, const KernelArgs& args, hipStream_t stream);
hipError_t launch_e2m1(int act, int out, const KernelArgs& args, hipStream_t stream);
hipError_t launch_bf16(int act, int out, const KernelArgs& args, hipStream_t stream);
hipError_t launch_e5m2(int act, int out, const KernelArgs& args, hipStream_t stream);

// Launch the grouped GEMM kernel instance for (ab, act, out).  Returns the
// HIP error of the launch (hipSuccess if enqueued).
hipError_t launch_grouped_gemm(int ab, int act, int out, const KernelArgs& args, hipStream_t stream);

// Row-major (rows, words) 32-bit scale words -> (words, rows) planes.
hipError_t launch_sf_kplanes(const uint8_t* src, uint8_t* dst, int64_t rows, int words, hipStream_t stream);

// Zero `count` floats with a fill kernel (usable under stream capture).
hipError_t launch_fill_zero(float* ptr, int count, hipStream_t stream);

}  // namespace moegg
