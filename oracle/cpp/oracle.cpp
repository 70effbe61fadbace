// Plain float64 C++ oracle: definitions (see oracle.h).
//
// TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
//
// Built with -ffp-contract=off and without fast-math, so that every float32
// decision below is one IEEE float32 operation and every float64 step one
// float64 operation, in the order written.
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

thread_local char g_error[256] = "";

int reject(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return 1;
}

// ---------------------------------------------------------------------------
// element formats ("Grouped GEMM + Quant (SM100)", §Data Types: float8_e4m3fn,
// float8_e5m2, float4_e2m1fn_x2 elements, float8_e8m0fnu scales; BF16 as the
// upper half of a binary32)
// ---------------------------------------------------------------------------

// E4M3: sign, exponent field e (bias 7), mantissa m/8; e = 0 is subnormal
// (m/8 * 2^-6); S.1111.111 is NaN; no infinity.
double decode_e4m3(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -mag : mag;
}

// E5M2: exponent bias 15, mantissa m/4; e = 0 subnormal (m/4 * 2^-14); e = 31
// is infinity (m = 0) or NaN.
double decode_e5m2(uint8_t c) {
  const int e = (c >> 2) & 31, m = c & 3;
  double mag;
  if (e == 31) mag = m == 0 ? INFINITY : NAN;
  else mag = e == 0 ? std::ldexp(m / 4.0, -14) : std::ldexp(1.0 + m / 4.0, e - 15);
  return (c & 0x80) ? -mag : mag;
}

// E2M1 (one nibble): exponent bias 1, mantissa m/2; e = 0 gives m/2.
double decode_e2m1(uint8_t nib) {
  const int e = (nib >> 1) & 3, m = nib & 1;
  const double mag = e == 0 ? m / 2.0 : std::ldexp(1.0 + m / 2.0, e - 1);
  return (nib & 8) ? -mag : mag;
}

// E8M0: 2^(c - 127); 0xFF is NaN.
double decode_e8m0(uint8_t c) { return c == 0xFF ? NAN : std::ldexp(1.0, static_cast<int>(c) - 127); }

double decode_bf16(uint16_t bits) {
  const uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

// Nearest E4M3 value to v, ties to the even mantissa, magnitudes above 448
// saturating to 448; NaN gives the NaN code.
uint8_t encode_e4m3(double v) {
  if (std::isnan(v)) return 0x7F;
  const double mag = std::min(std::fabs(v), 448.0);
  int code;
  if (mag < std::ldexp(1.0, -6)) {
    // subnormal range: multiples of 2^-9; 8 * 2^-9 = 2^-6 is code 8 itself
    code = static_cast<int>(std::nearbyint(std::ldexp(mag, 9)));
  } else {
    int ex;
    std::frexp(mag, &ex);                 // 2^(ex-1) <= mag < 2^ex
    const int e = ex - 1;
    int q = static_cast<int>(std::nearbyint(std::ldexp(mag, 3 - e)));   // 8 .. 16: 1.m in eighths
    int field = e + 7;
    if (q == 16) {
      q = 8;
      ++field;
    }
    code = (field << 3) | (q - 8);
  }
  if (v < 0 && code != 0) code |= 0x80;
  return static_cast<uint8_t>(code);
}

// Nearest BF16 (8 significant bits, subnormal quantum 2^-133), ties to even,
// rounded once from the float64 value.
uint16_t encode_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  int ex = 0;
  std::frexp(v, &ex);
  const int qe = std::max(ex - 8, -133);
  const double r = std::ldexp(std::nearbyint(std::ldexp(v, -qe)), qe);
  const float f = static_cast<float>(r);    // exact, or +-inf past the range
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------------------
// FP8 output quantisation ("Grouped GEMM + Quant (SM100)", §Equations Step 3):
// SFD = norm_const * amax * rcp_max with rcp_max = 1/448, stored as E8M0 (the
// smallest power of two not below it), D_q = D * norm_const / SFD.  Decisions
// in float32.
// ---------------------------------------------------------------------------

const float kRcpMaxE4M3 = 1.0f / 448.0f;

uint8_t e8m0_scale(float amax, float nc) {
  const float sf = (nc * amax) * kRcpMaxE4M3;
  if (!(sf > 0.0f)) return 0;
  int ex;
  const float frac = std::frexp(sf, &ex);   // sf = frac 2^ex, frac in [0.5, 1)
  const int e = frac == 0.5f ? ex - 1 : ex; // ceil(log2 sf)
  return static_cast<uint8_t>(std::min(std::max(e + 127, 0), 254));
}

uint8_t quantize_value(double d, uint8_t byte, float nc) {
  const float prod = static_cast<float>(d) * nc;
  const float scaled = std::ldexp(prod, 127 - static_cast<int>(byte));
  return encode_e4m3(scaled);
}

// Row blocks of 32 columns.
void quantize_rows(const double* d, int64_t rows, int64_t cols, float nc, uint8_t* codes, uint8_t* sf) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < cols / 32; ++b) {
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(static_cast<float>(d[r * cols + 32 * b + i])));
      const uint8_t byte = e8m0_scale(amax, nc);
      sf[r * (cols / 32) + b] = byte;
      for (int i = 0; i < 32; ++i) codes[r * cols + 32 * b + i] = quantize_value(d[r * cols + 32 * b + i], byte, nc);
    }
}

// Column blocks of 32 consecutive rows; sf is (cols, rows/32).
void quantize_cols(const double* d, int64_t rows, int64_t cols, float nc, uint8_t* codes, uint8_t* sf) {
  for (int64_t b = 0; b < rows / 32; ++b)
    for (int64_t c = 0; c < cols; ++c) {
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(static_cast<float>(d[(32 * b + i) * cols + c])));
      const uint8_t byte = e8m0_scale(amax, nc);
      sf[c * (rows / 32) + b] = byte;
      for (int i = 0; i < 32; ++i) codes[(32 * b + i) * cols + c] = quantize_value(d[(32 * b + i) * cols + c], byte, nc);
    }
}

// ---------------------------------------------------------------------------
// activations, float64
// ---------------------------------------------------------------------------

double sigmoid(double t) { return 1.0 / (1.0 + std::exp(-t)); }

int64_t n_out_of(const ox_problem& p) {
  switch (p.act) {
    case OX_SWIGLU:
    case OX_GEGLU: return p.n / 2;
    case OX_DSWIGLU:
    case OX_DGEGLU: return 2 * static_cast<int64_t>(p.n);
    default: return p.n;
  }
}

bool backward(int act) { return act == OX_DSWIGLU || act == OX_DSRELU || act == OX_DGEGLU; }

// One row.  c: C (forward) or R (backward), width n; x: the saved tensor of
// the backward; pr: the row's prob.
void activation_row(const ox_problem& p, const double* c, double pr, const double* x, double* d, double* dprob) {
  const int n = p.n;
  switch (p.act) {
    case OX_NONE:
      // "Grouped GEMM + Quant (SM100)", §Equations Step 2: D = prob * C
      for (int j = 0; j < n; ++j) d[j] = pr * c[j];
      break;
    case OX_SWIGLU:
      // "Grouped GEMM + SwiGLU (SM100)", §Equations Step 2: pair b of 32-column
      // blocks is [X_b | G_b]; D_b = prob * X_b * G_b * sigmoid(G_b)
      for (int b = 0; b < n / 64; ++b)
        for (int i = 0; i < 32; ++i) {
          const double xv = c[64 * b + i], g = c[64 * b + 32 + i];
          d[32 * b + i] = pr * xv * (g * sigmoid(g));
        }
      break;
    case OX_SRELU:
      // "Grouped GEMM + sReLU (SM100)", §Equations and §Tanh soft clamp:
      // r = relu(C); with s > 0, r = s * min(tanh(r / s), 1); D = prob * r^2
      for (int j = 0; j < n; ++j) {
        double r = std::max(c[j], 0.0);
        if (p.srelu_s > 0) r = p.srelu_s * std::min(std::tanh(r / p.srelu_s), 1.0);
        d[j] = pr * (r * r);
      }
      break;
    case OX_GEGLU:
      // "Grouped GEMM + GLU + Hadamard", §Equations, GeGLU: pair b is
      // [G_b | U_b], both clamped to [clamp_min, clamp_max];
      // D_b = gamma * prob * (U_b + offset) * G_b * sigmoid(alpha G_b)
      for (int b = 0; b < n / 64; ++b)
        for (int i = 0; i < 32; ++i) {
          const double g = std::min(std::max(c[64 * b + i], p.clamp_min), p.clamp_max);
          const double u = std::min(std::max(c[64 * b + 32 + i], p.clamp_min), p.clamp_max);
          d[32 * b + i] = p.glu_gamma * pr * (u + p.linear_offset) * g * sigmoid(p.geglu_alpha * g);
        }
      break;
    case OX_DSWIGLU: {
      // "Grouped GEMM + dGLU (SM100)", dSwiGLU equations: column j of R pairs
      // with input x = X[64b + i] and gate g = X[64b + 32 + i] (b = j / 32,
      // i = j % 32); s = sigmoid(g):
      //   dC[64b + i]      = R prob g s
      //   dC[64b + 32 + i] = R prob x s (1 + g (1 - s))
      //   dprob           += R x g s
      double acc = 0.0;
      for (int j = 0; j < n; ++j) {
        const int b = j / 32, i = j % 32;
        const double xv = x[64 * b + i], g = x[64 * b + 32 + i], s = sigmoid(g);
        d[64 * b + i] = c[j] * pr * (g * s);
        d[64 * b + 32 + i] = c[j] * pr * xv * s * (1.0 + g * (1.0 - s));
        acc += c[j] * xv * g * s;
      }
      *dprob = acc;
      break;
    }
    case OX_DGEGLU: {
      // "Grouped GEMM + dGLU (SM100)", dGeGLU equations: saved pair [gate | up];
      // gate clamped from above, up on both sides, masks from the unclamped
      // values (kept at equality); s = sigmoid(alpha gate_c):
      //   dgate = R prob (up_c + offset) s (1 + alpha gate_c (1 - s)) [gate <= max]
      //   dup   = R prob gate_c s [min <= up <= max]
      //   dprob += R gate_c s (up_c + offset)
      double acc = 0.0;
      for (int j = 0; j < n; ++j) {
        const int b = j / 32, i = j % 32;
        const double gate = x[64 * b + i], up = x[64 * b + 32 + i];
        const double gc = std::min(gate, p.clamp_max);
        const double uc = std::min(std::max(up, p.clamp_min), p.clamp_max);
        const double s = sigmoid(p.geglu_alpha * gc);
        d[64 * b + i] = gate <= p.clamp_max
                            ? c[j] * pr * (uc + p.linear_offset) * s * (1.0 + p.geglu_alpha * gc * (1.0 - s))
                            : 0.0;
        d[64 * b + 32 + i] = (p.clamp_min <= up && up <= p.clamp_max) ? c[j] * pr * gc * s : 0.0;
        acc += c[j] * gc * s * (uc + p.linear_offset);
      }
      *dprob = acc;
      break;
    }
    case OX_DSRELU: {
      // derivative of the sReLU forward ("Grouped GEMM + sReLU (SM100)",
      // §Equations / §Tanh soft clamp): f(C) = c^2 with c = s t,
      // t = min(tanh(relu(C)/s), 1), f'(C) = 2 c (1 - t^2) = 2 c sech^2(relu(C)/s)
      // (s = 0: c = relu(C), f' = 2 c); dC = R prob f'(C), dprob += R f(C)
      double acc = 0.0;
      for (int j = 0; j < n; ++j) {
        const double r = std::max(x[j], 0.0);
        double cv, fp;
        if (p.srelu_s > 0) {
          const double t = std::min(std::tanh(r / p.srelu_s), 1.0);
          const double ch = std::cosh(r / p.srelu_s);
          cv = p.srelu_s * t;
          fp = 2.0 * cv / (ch * ch);              // 1 - t^2 = sech^2, free of its cancellation near t = 1
        } else {
          cv = r;
          fp = 2.0 * r;
        }
        d[j] = c[j] * pr * fp;
        acc += c[j] * (cv * cv);
      }
      *dprob = acc;
      break;
    }
  }
}

int check_problem(const ox_problem& p) {
  if (p.num_groups < 1 || p.n <= 0 || p.k <= 0 || p.valid_m < 0) return reject("bad shape");
  if (p.k % 32) return reject("k not a multiple of 32");
  if (p.ab < OX_E4M3 || p.ab > OX_BF16) return reject("bad operand format");
  if (p.act < OX_NONE || p.act > OX_DGEGLU) return reject("bad activation");
  if ((p.act == OX_SWIGLU || p.act == OX_GEGLU) && p.n % 64) return reject("paired activation needs n % 64 == 0");
  if ((p.act == OX_DSWIGLU || p.act == OX_DGEGLU) && p.n % 32) return reject("paired backward needs n % 32 == 0");
  if (p.d_fp8 && n_out_of(p) % 32) return reject("FP8 output needs n_out % 32 == 0");
  return 0;
}

// float64 values of one operand row (row bytes per the format), each element
// times its block's power of two ("Grouped GEMM + Quant (SM100)", §Equations
// Step 1: dequantize with the scale of its 32-element K block).
void dequantize_row(int ab, const uint8_t* codes, const uint8_t* sf, int k, double* out) {
  for (int kk = 0; kk < k; ++kk) {
    double v;
    switch (ab) {
      case OX_E4M3: v = decode_e4m3(codes[kk]); break;
      case OX_E5M2: v = decode_e5m2(codes[kk]); break;
      case OX_E2M1: v = decode_e2m1(kk % 2 == 0 ? (codes[kk / 2] & 0xF) : (codes[kk / 2] >> 4)); break;
      default: {
        uint16_t bits;
        std::memcpy(&bits, codes + 2 * kk, 2);
        v = decode_bf16(bits);
      }
    }
    out[kk] = ab == OX_BF16 ? v : v * decode_e8m0(sf[kk / 32]);
  }
}

int64_t row_bytes(const ox_problem& p) {
  return p.ab == OX_E2M1 ? p.k / 2 : p.ab == OX_BF16 ? 2 * static_cast<int64_t>(p.k) : p.k;
}

}  // namespace

extern "C" {

const char* ox_last_error(void) { return g_error; }

int ox_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void ox_decode(int fmt, const uint8_t* codes, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i) {
    switch (fmt) {
      case OX_E4M3: out[i] = decode_e4m3(codes[i]); break;
      case OX_E5M2: out[i] = decode_e5m2(codes[i]); break;
      case OX_E2M1: out[i] = decode_e2m1(codes[i] & 0xF); break;
      case OX_E8M0: out[i] = decode_e8m0(codes[i]); break;
      default: out[i] = NAN;
    }
  }
}

void ox_decode_bf16(const uint16_t* bits, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = decode_bf16(bits[i]);
}

void ox_encode_e4m3(const double* v, int64_t count, uint8_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = encode_e4m3(v[i]);
}

void ox_encode_bf16(const double* v, int64_t count, uint16_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = encode_bf16(v[i]);
}

uint8_t ox_e8m0_scale(float amax, float nc) { return e8m0_scale(amax, nc); }

int ox_activation(const ox_problem* p, int64_t rows, const double* cr, const double* prob, const double* saved,
                  double* d, double* dprob) {
  if (!p || check_problem(*p)) return 1;
  if (!cr || !prob || !d || (backward(p->act) && (!saved || !dprob))) return reject("NULL argument");
  const int64_t n = p->n, no = n_out_of(*p);
  const int64_t sw = p->act == OX_DSRELU ? n : 2 * n;
  for (int64_t r = 0; r < rows; ++r)
    activation_row(*p, cr + r * n, prob[r], backward(p->act) ? saved + r * sw : nullptr, d + r * no,
                   backward(p->act) ? dprob + r : nullptr);
  return 0;
}

int ox_quantize(int axis, const double* d, int64_t rows, int64_t cols, float nc, uint8_t* codes, uint8_t* sf) {
  if (!d || !codes || !sf) return reject("NULL argument");
  if (axis == 0) {
    if (cols % 32) return reject("row blocks need cols % 32 == 0");
    quantize_rows(d, rows, cols, nc, codes, sf);
  } else {
    if (rows % 32) return reject("column blocks need rows % 32 == 0");
    quantize_cols(d, rows, cols, nc, codes, sf);
  }
  return 0;
}

int ox_run(const ox_problem* pp, const ox_inputs* in, const int64_t* rows, int64_t nrows, ox_outputs* out) {
  if (!pp || !in || !out || (nrows > 0 && !rows)) return reject("NULL argument");
  const ox_problem& p = *pp;
  if (check_problem(p)) return 1;
  if (!in->a || !in->b || !in->padded_offsets || !in->alpha || !in->prob ||
      (p.ab != OX_BF16 && (!in->sfa || !in->sfb)) || (backward(p.act) && !in->c_in) ||
      (p.act == OX_DSWIGLU && !in->beta))
    return reject("missing input");
  const int L = p.num_groups, n = p.n, k = p.k;
  const int64_t no = n_out_of(p), rb = row_bytes(p);
  const bool bwd = backward(p.act), mx = p.ab != OX_BF16;

  // row -> expert: expert g owns rows [po[g-1], po[g]) ("Grouped GEMM + Quant
  // (SM100)", §Equations Step 1); empty experts own none
  std::vector<int32_t> grp(nrows);
  for (int64_t i = 0; i < nrows; ++i) {
    int g = 0;
    while (g < L && rows[i] >= in->padded_offsets[g]) ++g;
    if (g == L || rows[i] < 0 || rows[i] >= p.valid_m) return reject("row %lld outside every group", (long long)rows[i]);
    grp[i] = g;
  }

  // steps 1-3: per row, acc[j] = sum over k (ascending) of a[k] b_g[j][k] in
  // float64, then C = alpha_g acc or, for the backward, R = alpha_g^2 acc
  // ("Grouped GEMM + dGLU (SM100)", equation of R)
  std::vector<double> cr(static_cast<size_t>(nrows) * n);
  const uint8_t* A = static_cast<const uint8_t*>(in->a);
  const uint8_t* B = static_cast<const uint8_t*>(in->b);
  for (int g = 0; g < L; ++g) {
    std::vector<int64_t> mine;
    for (int64_t i = 0; i < nrows; ++i)
      if (grp[i] == g) mine.push_back(i);
    if (mine.empty()) continue;
    std::vector<double> bg(static_cast<size_t>(n) * k);
#pragma omp parallel for schedule(static)
    for (int j = 0; j < n; ++j)
      dequantize_row(p.ab, B + (static_cast<int64_t>(g) * n + j) * rb,
                     mx ? in->sfb + (static_cast<int64_t>(g) * n + j) * (k / 32) : nullptr, k, &bg[static_cast<size_t>(j) * k]);
    const double alpha = in->alpha[g];
    const double scale = bwd ? alpha * alpha : alpha;
#pragma omp parallel
    {
      std::vector<double> arow(k);
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = 0; t < static_cast<int64_t>(mine.size()); ++t) {
        const int64_t i = mine[t], r = rows[i];
        dequantize_row(p.ab, A + r * rb, mx ? in->sfa + r * (k / 32) : nullptr, k, arow.data());
        for (int j = 0; j < n; ++j) {
          const double* bj = &bg[static_cast<size_t>(j) * k];
          double acc = 0.0;
          for (int kk = 0; kk < k; ++kk) acc += arow[kk] * bj[kk];
          cr[static_cast<size_t>(i) * n + j] = scale * acc;
        }
      }
    }
  }

  // step 4: the activation, float64
  std::vector<double> d(static_cast<size_t>(nrows) * no), dprob(bwd ? nrows : 0);
  const int64_t sw = p.act == OX_DSRELU ? n : 2 * static_cast<int64_t>(n);
#pragma omp parallel
  {
    std::vector<double> x(bwd ? sw : 0);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
      if (bwd) {
        // saved C at its stored BF16 precision; dSwiGLU scales it by beta_g
        const double beta = p.act == OX_DSWIGLU ? static_cast<double>(in->beta[grp[i]]) : 1.0;
        for (int64_t j = 0; j < sw; ++j) x[j] = beta * decode_bf16(in->c_in[rows[i] * sw + j]);
      }
      activation_row(p, &cr[static_cast<size_t>(i) * n], in->prob[rows[i]], x.data(), &d[static_cast<size_t>(i) * no],
                     bwd ? &dprob[i] : nullptr);
    }
  }

  // step 5: outputs
  for (int64_t i = 0; i < nrows; ++i)
    if (out->group) out->group[i] = grp[i];
  if (out->cr) std::memcpy(out->cr, cr.data(), cr.size() * sizeof(double));
  if (out->d) std::memcpy(out->d, d.data(), d.size() * sizeof(double));
  if (bwd && out->dprob) std::memcpy(out->dprob, dprob.data(), dprob.size() * sizeof(double));
  if (!bwd && p.c_out && out->c_bits)
    for (size_t e = 0; e < cr.size(); ++e) out->c_bits[e] = encode_bf16(cr[e]);
  if (out->d_bits)
    for (size_t e = 0; e < d.size(); ++e) out->d_bits[e] = encode_bf16(d[e]);
  if (bwd && !mx) return 0;                          // BF16 backward: dC (BF16) and dprob only

  if (!p.d_fp8) {
    if (!out->amax) return 0;
    const bool pairs = bwd && p.act != OX_DSRELU;    // (L, 2): [first, second] block of each pair
    const int w = pairs ? 2 : 1;
    for (int e = 0; e < L * w; ++e) out->amax[e] = 0.0;
    for (int64_t i = 0; i < nrows; ++i)
      for (int64_t j = 0; j < no; ++j) {
        double& slot = out->amax[grp[i] * w + (pairs ? (j / 32) % 2 : 0)];
        slot = std::max(slot, std::fabs(d[static_cast<size_t>(i) * no + j]));
      }
    return 0;
  }
  if (out->d_code && out->sfd_row) quantize_rows(d.data(), nrows, no, p.norm_const, out->d_code, out->sfd_row);
  bool whole = nrows > 0 && nrows % 32 == 0;
  for (int64_t i = 0; whole && i < nrows; ++i) whole = rows[i] == rows[i - i % 32] + i % 32 && rows[i - i % 32] % 32 == 0;
  if (whole && out->d_col_code && out->sfd_col)
    quantize_cols(d.data(), nrows, no, p.norm_const, out->d_col_code, out->sfd_col);
  return 0;
}

}  // extern "C"
