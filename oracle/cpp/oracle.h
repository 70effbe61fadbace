/*
 * Plain float64 C++ oracle of the contiguous grouped block-scaled GEMM with
 * its fused epilogue.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load or call it.  It is
 * written from the equations of the cuDNN frontend pages "Grouped GEMM + Quant
 * (SM100)" (§Equations Steps 1-3, §Data Types), "Grouped GEMM + SwiGLU
 * (SM100)" (§Equations), "Grouped GEMM + sReLU (SM100)" (§Equations, §Tanh
 * soft clamp), "Grouped GEMM + dGLU (SM100)" (BF16 and block-scaled
 * contracts) and "Grouped GEMM + GLU + Hadamard" (§Equations, GeGLU), and
 * shares no code, header, table or constant with the HIP library or with the
 * numpy oracle next to it.  Each step is the plain definition: decode every
 * code, scale it by its block's power of two, multiply-accumulate in float64
 * in K order, apply the per-group alpha and the activation in float64, then
 * round or quantise the outputs (quantisation decisions in float32).
 *
 * Readings where the pages leave a step open are the same as the numpy
 * oracle's (listed in its module docstring); each function below names its
 * passage.
 *
 * All pointers are host memory owned by the caller.  Functions returning int
 * give 0 on success and 1 on a rejected argument (ox_last_error() says why).
 */
#ifndef MOEGG_ORACLE_CPP_H_
#define MOEGG_ORACLE_CPP_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats ("Grouped GEMM + Quant (SM100)", §Data Types) */
enum { OX_E4M3 = 0, OX_E5M2 = 1, OX_E2M1 = 2, OX_BF16 = 3, OX_E8M0 = 4 };

/* epilogues */
enum { OX_NONE = 0, OX_SWIGLU = 1, OX_SRELU = 2, OX_DSWIGLU = 3, OX_DSRELU = 4, OX_GEGLU = 5, OX_DGEGLU = 6 };

typedef struct {
  int32_t num_groups;   /* L */
  int64_t valid_m;      /* rows of A */
  int32_t n, k;         /* GEMM columns (rows of each expert's B), reduction length */
  int32_t ab;           /* OX_E4M3 | OX_E5M2 | OX_E2M1 (two per byte, low nibble = even K) | OX_BF16 */
  int32_t act;          /* OX_NONE .. OX_DGEGLU */
  int32_t d_fp8;        /* 1: D (or block-scaled dC) as E4M3 codes with E8M0 row / column scales */
  int32_t c_out;        /* 1: the forward C = alpha acc as BF16 as well */
  double srelu_s;       /* sReLU tanh clamp s (0: plain relu^2) */
  double glu_gamma, geglu_alpha, linear_offset, clamp_min, clamp_max;   /* GeGLU / dGeGLU */
  float norm_const;     /* FP8 outputs: D * norm_const / scale */
} ox_problem;

typedef struct {
  const void* a;                 /* (valid_m, row bytes): E4M3/E5M2 bytes, packed E2M1, or BF16 bits */
  const uint8_t* sfa;            /* (valid_m, k/32) E8M0, NULL for BF16 */
  const void* b;                 /* (L, n, row bytes) */
  const uint8_t* sfb;            /* (L, n, k/32) */
  const int32_t* padded_offsets; /* (L) cumulative row ends */
  const float* alpha;            /* (L) */
  const float* beta;             /* (L) dSwiGLU only */
  const float* prob;             /* (valid_m) */
  const uint16_t* c_in;          /* saved forward C, BF16: (valid_m, 2n) dSwiGLU / dGeGLU, (valid_m, n) dsReLU */
} ox_inputs;

/* Per-row outputs hold the requested rows, in the order requested.  n_out is
 * n (none, sReLU, dsReLU), n/2 (SwiGLU, GeGLU) or 2n (dSwiGLU, dGeGLU).  A
 * NULL pointer skips that output. */
typedef struct {
  int32_t* group;        /* (nrows) expert of each row */
  double* cr;            /* (nrows, n) C = alpha acc (forward) or R = alpha^2 acc (backward) */
  double* d;             /* (nrows, n_out) D, or dC, before any rounding */
  double* dprob;         /* (nrows) backward: sum over the row of R times the forward's f */
  uint16_t* c_bits;      /* (nrows, n) BF16 of C (forward, c_out) */
  uint16_t* d_bits;      /* (nrows, n_out) BF16 of D or dC */
  uint8_t* d_code;       /* (nrows, n_out) E4M3 codes of the row blocks (d_fp8) */
  uint8_t* sfd_row;      /* (nrows, n_out/32) */
  uint8_t* d_col_code;   /* (nrows, n_out) E4M3 codes of the column blocks: rows must form */
  uint8_t* sfd_col;      /* (n_out, nrows/32)   whole 32-row blocks starting at multiples of 32 */
  double* amax;          /* (L), or (L, 2) for block-scaled dSwiGLU / dGeGLU with a BF16 dC */
} ox_outputs;

/* The whole path for the rows `rows[0..nrows)` (each inside some group). */
int ox_run(const ox_problem* p, const ox_inputs* in, const int64_t* rows, int64_t nrows, ox_outputs* out);

/* Threads ox_run uses (OpenMP). */
int ox_threads(void);

const char* ox_last_error(void);

/* ---- the steps on their own, for the pins ---- */

/* codes -> float64 values; OX_E2M1 takes one nibble per byte */
void ox_decode(int fmt, const uint8_t* codes, int64_t count, double* out);
void ox_decode_bf16(const uint16_t* bits, int64_t count, double* out);
/* nearest E4M3 (ties to even mantissa, saturating at 448) and nearest BF16 */
void ox_encode_e4m3(const double* v, int64_t count, uint8_t* out);
void ox_encode_bf16(const double* v, int64_t count, uint16_t* out);
/* E8M0 byte of one block: smallest 2^e >= (nc amax) / 448 in float32, 0 for a zero block */
uint8_t ox_e8m0_scale(float amax, float nc);
/* The activation of `p->act` on float64 inputs of `rows` rows: cr is C (forward,
 * width n) or R (backward, width n); saved is the backward's saved tensor in
 * float64, already scaled by beta for dSwiGLU (width 2n, or n for dsReLU);
 * writes d (width n_out) and, for the backward, dprob. */
int ox_activation(const ox_problem* p, int64_t rows, const double* cr, const double* prob, const double* saved,
                  double* d, double* dprob);
/* FP8 quantisation of a (rows, cols) float64 array: axis 0 = row blocks (32
 * columns; sf (rows, cols/32)), axis 1 = column blocks (32 rows; sf (cols, rows/32)). */
int ox_quantize(int axis, const double* d, int64_t rows, int64_t cols, float nc, uint8_t* codes, uint8_t* sf);

#ifdef __cplusplus
}
#endif

#endif  /* MOEGG_ORACLE_CPP_H_ */
