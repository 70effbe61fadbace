/*
 * moegg.h -- C ABI of libmoegg: the contiguous grouped block-scaled GEMM used
 * by MoE expert layers, with its fused epilogue, for AMD Instinct MI355X
 * (gfx950).
 *
 * What one call computes (cuDNN frontend pages "Grouped GEMM + Quant (SM100)",
 * "Grouped GEMM + SwiGLU (SM100)", "Grouped GEMM + sReLU (SM100)" and
 * "Grouped GEMM + dGLU (SM100)", §Equations of each):
 *
 *   rows m of A in [padded_offsets[g-1], padded_offsets[g]) belong to expert g
 *   acc[m,n] = sum_k dequant(A[m,k], SFA) * dequant(B[g,n,k], SFB)
 *   C = alpha_g * acc                       (forward activations)
 *   R = alpha_g^2 * acc                     (backward activations)
 *   then the activation / gating epilogue selected by `act`, and the output
 *   formatting selected by `d_dtype`:
 *     BF16  D (round to nearest even) + per-group amax = max |D| (fp32, before
 *           rounding) over the group's rows and all output columns;
 *     E4M3  D and D_col, the same logical output quantised over 32-column row
 *           blocks (SFD_row) and 32-row column blocks (SFD_col):
 *           SFD = smallest power of two >= norm_const * amax_blk / 448 (E8M0
 *           byte, 0 for an all-zero block), D_q = E4M3_rne(D * norm_const / SFD).
 *
 * Layouts ("logical" layouts defined by this library; every tensor is dense,
 * row-major, with no padding between rows):
 *   A       (valid_m, K)   E4M3 or E5M2 codes, or (valid_m, K/2) packed E2M1 pairs
 *                          (the even K element in the low nibble), or BF16
 *   B       (L, N, K)      same encoding as A, K contiguous ("K-major")
 *   SFA     (valid_m, K/32) E8M0 bytes, row-major: byte kb of row r (the
 *           scale of A[r, 32 kb .. 32 kb + 31]) at r * K/32 + kb (MX formats
 *           only; "Grouped GEMM + Quant (SM100)", §Shapes, SFA)
 *   SFB     (L, N, K/32) E8M0 bytes, row-major: expert g's row n at
 *           (g * N + n) * K/32 ("Grouped GEMM + Quant (SM100)", §Shapes, SFB)
 *   With sf_layout = MOEGG_SF_KPLANES the same bytes come instead as K-block
 *   planes of 32-bit words, (K/128, rows, 4): byte kb of row r at
 *   4 * ((kb / 4) * rows + r) + kb % 4 (rows = valid_m for SFA, L * N for a
 *   dense SFB, N for one expert's discrete SFB).  A plane holds the scales of
 *   128 consecutive K elements of every row, so those of a row tile for one
 *   K-step are contiguous and the kernel fetches them in whole cache lines
 *   (the pages' own kernels likewise take scale factors in a tiled layout of
 *   their own, §Shapes and Divisibility).  moegg_sf_to_kplanes converts.
 *   Discrete weights (the pages' b_ptrs / sfb_ptrs mode, "Grouped GEMM +
 *   sReLU (SM100)", §Discrete-weight wrapper): instead of B and SFB the
 *   caller passes device arrays of L device pointers; b_ptrs[g] points to
 *   expert g's (N, K) weights in B's encoding and sfb_ptrs[g] (MX only) to
 *   its (N, K/32) row-major scales (or (K/128, N, 4) planes with
 *   MOEGG_SF_KPLANES).  Each pointer must be 16-byte aligned
 *   (the kernel ignores its low 4 bits); entries of experts with no rows are
 *   never read.
 *   padded_offsets (L) int32, cumulative group ends; padded_offsets[L-1] ==
 *                          valid_m; every entry a multiple of m_aligned and
 *                          nondecreasing (empty groups repeat the previous end)
 *   alpha, beta (L) fp32; prob (valid_m) fp32; norm_const (1) fp32
 *   C       (valid_m, N) BF16                      [optional forward output]
 *   D, D_col (valid_m, N_out) BF16 or E4M3 codes   N_out = N/2 for SwiGLU and
 *                                                  GeGLU, 2N for dSwiGLU and
 *                                                  dGeGLU, else N
 *                                                  (dC for the backward
 *                                                  activations)
 *   SFD_row (valid_m, N_out/32) E8M0; SFD_col (N_out, valid_m/32) E8M0
 *   amax    (L) fp32, written by the call (zero-filled first); for dSwiGLU /
 *           dGeGLU with MX operands and a BF16 dC, (L, 2): the max |dC| of
 *           the first and of the second blocks of the pairs over the group's
 *           rows (the block-scaled dGLU contract's amax of shape (L, 2, 1);
 *           which quantity each entry holds is this library's reading)
 *   C_in    saved forward pre-activation, BF16: (valid_m, 2N) [dSwiGLU, dGeGLU]
 *           or (valid_m, N) [dsReLU]
 *   dprob   (valid_m) fp32, caller-zeroed, accumulated with atomics [dSwiGLU, dsReLU,
 *           dGeGLU]
 *
 * Ownership: every pointer is a caller-owned device pointer (except the
 * problem/args structs, which are host memory read during the call only).
 * The library keeps no pointer after a call returns and allocates no device
 * memory.  Buffers must stay alive and unchanged until the stream has run
 * the work.  Calls are asynchronous on `stream` (a hipStream_t; NULL = the
 * null stream).
 *
 * Errors: every shape, dtype, alignment and presence rule is checked on the
 * host before any HIP call; a failing call returns a status and enqueues
 * nothing.  padded_offsets values are device data and are not read on the
 * host (moegg_check_offsets is the opt-in, synchronising validator).
 * moegg_last_error() returns a thread-local text describing the last failure.
 */
#ifndef MOEGG_H_
#define MOEGG_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEGG_ABI_VERSION 5

typedef enum moegg_status {
  MOEGG_OK = 0,
  MOEGG_ERROR_INVALID_VALUE = 1, /* bad shape, dtype combination, NULL where required */
  MOEGG_ERROR_MISALIGNED = 2,    /* pointer not 16-byte aligned */
  MOEGG_ERROR_NOT_SUPPORTED = 3, /* valid per the pages, not supported by this library (e.g. K % 128 != 0) */
  MOEGG_ERROR_LAUNCH = 4         /* a HIP runtime call failed */
} moegg_status;

typedef enum moegg_dtype {
  MOEGG_DT_NONE = 0,
  MOEGG_DT_E4M3 = 1,   /* OCP E4M3FN: A/B operands (MXFP8) or D/D_col outputs */
  MOEGG_DT_E2M1X2 = 2, /* packed OCP E2M1 pairs: A/B operands (MXFP4) */
  MOEGG_DT_BF16 = 3,   /* A/B operands (dense BF16 backend) or C / D outputs */
  MOEGG_DT_E5M2 = 4    /* OCP E5M2: A/B operands (MXFP8, "Grouped GEMM + Quant", §Data Types) */
} moegg_dtype;

typedef enum moegg_sf_layout {
  MOEGG_SF_ROW_MAJOR = 0, /* SFA (valid_m, K/32), SFB (L, N, K/32): the default */
  MOEGG_SF_KPLANES = 1    /* SFA (K/128, valid_m, 4), SFB (K/128, L*N, 4) 32-bit word planes */
} moegg_sf_layout;

typedef enum moegg_act {
  MOEGG_ACT_NONE = 0,    /* D = prob * C            ("Grouped GEMM + Quant", Step 2)        */
  MOEGG_ACT_SWIGLU = 1,  /* D = prob * X_b * swish(G_b), pairs [X_b|G_b] of 32 columns
                            ("Grouped GEMM + SwiGLU", Step 2)                               */
  MOEGG_ACT_SRELU = 2,   /* D = prob * relu(C)^2, optional tanh soft clamp s
                            ("Grouped GEMM + sReLU", §Equations / §Tanh soft clamp)          */
  MOEGG_ACT_DSWIGLU = 3, /* dC = [d_input|d_gate] from R and beta*C_in, dprob += row sums
                            ("Grouped GEMM + dGLU", BF16 contract and block-scaled contract,
                            dSwiGLU): BF16 operands -> BF16 dC; MX operands -> BF16 dC + amax
                            (L, 2), or E4M3 dC as D/D_col with SFD_row/SFD_col             */
  MOEGG_ACT_DSRELU = 4,  /* sReLU backward: R = alpha_g^2 acc, C_in the saved forward C
                            (N wide, no beta), dC = R prob f'(C), dprob += sum R f(C),
                            f(C) = (s tanh(relu(C)/s))^2 or relu(C)^2 for s = 0 (derived
                            from "Grouped GEMM + sReLU", §Equations / §Tanh soft clamp; its
                            backward page is not among the sources).  Output formats as
                            dSwiGLU, amax (L) for a BF16 dC with MX operands              */
  MOEGG_ACT_GEGLU = 5,   /* D = gamma prob (U_b + offset) G_b sigmoid(a G_b), pairs [G_b|U_b]
                            of 32 columns, gate first, both clamped to [clamp_min, clamp_max]
                            ("Grouped GEMM + GLU + Hadamard", §Equations, GeGLU; the page's
                            constants are a = 1.702, offset = 1)                          */
  MOEGG_ACT_DGEGLU = 6   /* dGeGLU backward: C_in pairs [gate_b|up_b], dC = [dgate_b|dup_b],
                            gate clamped above at clamp_max, up to [clamp_min, clamp_max],
                            dprob += row sums ("Grouped GEMM + dGLU", dGeGLU equations; the
                            page's defaults a = 1.702, offset = 1, clamps -7 / 7).  Output
                            formats as dSwiGLU (amax (L, 2) = [dgate, dup] blocks)        */
} moegg_act;

/* Problem description (host struct). */
typedef struct moegg_problem {
  int32_t num_groups;   /* L, 1..1024 ("Shapes and Divisibility": expert count <= 1024) */
  int32_t m_aligned;    /* group row alignment; multiple of 128 here                     */
  int64_t valid_m;      /* rows of A == padded_offsets[L-1]; multiple of m_aligned,
                           < 2^31 here                                                    */
  int32_t n;            /* GEMM N (rows of each expert's B); multiple of 32, <= 2^20 here
                           (64 for SwiGLU / GeGLU)                                        */
  int32_t k;            /* reduction length K; multiple of 128 bytes per row here (128
                           E4M3 / E5M2, 256 E2M1, 64 BF16 elements), <= 2^20             */
  int32_t ab_dtype;     /* moegg_dtype of A and B: E4M3 | E5M2 | E2M1X2 | BF16            */
  int32_t c_dtype;      /* NONE (C not written) | BF16                                    */
  int32_t d_dtype;      /* BF16 (needs amax) | E4M3 (needs SFD_row, SFD_col, norm_const)  */
  int32_t act;          /* moegg_act                                                      */
  float srelu_tanh_s;   /* sReLU soft clamp s; 0 = plain relu^2                           */
  /* GeGLU / dGeGLU constants (read for those activations only; no implicit
   * defaults: the pages' values are gamma 1, geglu_alpha 1.702, linear_offset 1,
   * dGeGLU clamps -7 / 7; +-INFINITY disables a clamp) */
  float glu_gamma;      /* GeGLU output scale                                             */
  float geglu_alpha;    /* sigmoid input scale                                            */
  float linear_offset;  /* offset added to the (clamped) up branch                       */
  float glu_clamp_min;  /* lower clamp (GeGLU: both halves; dGeGLU: up)                   */
  float glu_clamp_max;  /* upper clamp (both halves, both directions)                     */
  int32_t sf_layout;    /* moegg_sf_layout of SFA / SFB (MX operands; 0 = row-major)       */
} moegg_problem;

/* Tensor pointers (device memory, caller-owned).  NULL where not used. */
typedef struct moegg_args {
  const void* a;
  const void* b;
  const uint8_t* sfa;            /* MX operands only; (valid_m, K/32) E8M0 (or planes, sf_layout) */
  const uint8_t* sfb;            /* MX operands only; (L, N, K/32) E8M0 (or planes, sf_layout) */
  const int32_t* padded_offsets;
  const float* alpha;
  const float* prob;             /* required ("prob ... Required", Quant page) */
  const float* beta;             /* dSwiGLU only (L) */
  const float* norm_const;       /* required iff d_dtype == E4M3 */
  const void* c_in;              /* backward: saved forward C, BF16 (valid_m, 2N) or (valid_m, N) dsReLU */
  void* c;                       /* optional C output (c_dtype BF16) */
  void* d;                       /* D (or dC for the backward activations) */
  void* d_col;                   /* E4M3 only */
  uint8_t* sfd_row;              /* E4M3 only */
  uint8_t* sfd_col;              /* E4M3 only */
  float* amax;                   /* BF16 D: (L), or (L, 2) for dSwiGLU / dGeGLU with MX operands */
  float* dprob;                  /* backward activations, caller-zeroed */
  const void* const* b_ptrs;     /* discrete weights instead of b: (L) device array, 8-byte aligned */
  const uint8_t* const* sfb_ptrs;/* discrete weights, MX only, instead of sfb: (L) device array */
} moegg_args;

/* Validate problem + pointers on the host.  No HIP call.  MOEGG_OK if
 * moegg_run would launch (or, for valid_m == 0, only zero-fill amax).
 * The rules are the pages' ("Grouped GEMM + Quant (SM100)", §Support Surface
 * and Constraints: §Layouts and Strides (16-byte alignment), §Data Types and
 * §Additional Type Constraints (A and B of one dtype, the SFD trio together),
 * §Scale Factor Output Requirements (amax with a BF16 D), §Shapes and
 * Divisibility (L <= 1024, groups aligned to m_aligned, valid_m =
 * padded_offsets[L-1]); "Grouped GEMM + dGLU (SM100)", §Support Surface and
 * Constraints for the backward tensors), plus this library's own limits,
 * reported as MOEGG_ERROR_NOT_SUPPORTED (K a multiple of 128 bytes per row,
 * N a multiple of 32, m_aligned a multiple of 128). */
moegg_status moegg_check(const moegg_problem* problem, const moegg_args* args);

/* Validate (as moegg_check), then enqueue the whole path on `stream`
 * (hipStream_t): the amax zero-fill (when amax is used) and the grouped GEMM
 * with its epilogue ("Grouped GEMM + Quant (SM100)", §Equations, Steps 1-3, and
 * the other pages' §Equations).  valid_m == 0: returns MOEGG_OK after
 * enqueuing only the amax zero-fill. */
moegg_status moegg_run(const moegg_problem* problem, const moegg_args* args, void* stream);

/* Opt-in validator of device padded_offsets (synchronises `stream`) against
 * the pages' offset rules ("Grouped GEMM + Quant (SM100)", §Shapes: the
 * cumulative sum of aligned group sizes with valid_m its last entry; §Shapes
 * and Divisibility: every group aligned to m_aligned): entries nondecreasing,
 * multiples of m_aligned, last == valid_m.  MOEGG_OK or
 * MOEGG_ERROR_INVALID_VALUE (MOEGG_ERROR_LAUNCH if the copy fails). */
moegg_status moegg_check_offsets(const moegg_problem* problem, const int32_t* padded_offsets,
                                 void* stream);

/* Lay out E8M0 scale bytes given row-major as (rows, K/32) (SFA with rows =
 * valid_m, a dense SFB with rows = L * N, one expert's SFB with rows = N)
 * as the K-block word planes (K/128, rows, 4) that MOEGG_SF_KPLANES reads:
 * dst[4 * ((kb / 4) * rows + r) + kb % 4] = src[r * K/32 + kb].  The layout is
 * this library's; the scale values follow "Grouped GEMM + Quant (SM100)",
 * §Shapes (SFA, SFB: one E8M0 byte per 32 K elements).  Enqueued on `stream`
 * with no allocation and no synchronisation (capturable).  k must be a
 * positive multiple of 128, rows >= 0 (0: nothing enqueued); src and dst are
 * caller-owned device buffers of rows * K/32 bytes, 16-byte aligned, not
 * overlapping.  Returns MOEGG_OK, MOEGG_ERROR_INVALID_VALUE,
 * MOEGG_ERROR_MISALIGNED or MOEGG_ERROR_LAUNCH. */
moegg_status moegg_sf_to_kplanes(const uint8_t* src, uint8_t* dst, int64_t rows, int32_t k, void* stream);

/* Output width N_out for a problem (N/2 SwiGLU / GeGLU, 2N dSwiGLU / dGeGLU, else N);
 * -1 if invalid act. */
int64_t moegg_n_out(const moegg_problem* problem);

const char* moegg_status_string(moegg_status status);
const char* moegg_last_error(void);   /* thread-local detail of the last failure */
int moegg_abi_version(void);

/* Testing hook; no passage defines it and it changes no result.  Caps the
 * persistent workgroups that later moegg_run calls launch, from any thread
 * (0 or a negative value: no cap, the default of one workgroup per compute
 * unit).  With a small cap every workgroup walks many output tiles, so that a
 * problem small enough for a CPU reference still passes through every
 * tile-to-tile hand-off of the kernel.  Returns the previous cap. */
int moegg_set_grid_limit(int max_workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MOEGG_H_ */
