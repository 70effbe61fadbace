// C-ABI front of libmoegg: host-side validation and dispatch.
//
// Every rule below is checked before any HIP call, so a rejected call
// enqueues nothing (the pages reject invalid configurations "before
// allocation or compilation": "Grouped GEMM + dGLU (SM100)", §Backend dispatch).
#include "moegg.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moegg_internal.h"

namespace {

thread_local char g_last_error[512] = "";

// Cap on the persistent workgroups of a launch (0 = none), set by
// moegg_set_grid_limit.
std::atomic<int> g_grid_limit{0};

moegg_status fail(moegg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

// Compute units of the current device (cached per device id; calls from
// several host threads may fill the cache concurrently), 0 on error.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t n_out_of(const moegg_problem& p) {
  switch (p.act) {
    case MOEGG_ACT_NONE:
    case MOEGG_ACT_SRELU: return p.n;
    case MOEGG_ACT_SWIGLU: return p.n / 2;
    case MOEGG_ACT_DSWIGLU: return 2 * static_cast<int64_t>(p.n);
    case MOEGG_ACT_DSRELU: return p.n;
    case MOEGG_ACT_GEGLU: return p.n / 2;
    case MOEGG_ACT_DGEGLU: return 2 * static_cast<int64_t>(p.n);
    default: return -1;
  }
}

moegg_status check_impl(const moegg_problem* pp, const moegg_args* ap) {
  if (!pp || !ap) return fail(MOEGG_ERROR_INVALID_VALUE, "problem and args must be non-NULL");
  const moegg_problem& p = *pp;
  const moegg_args& a = *ap;

  // --- shapes -----------------------------------------------------------
  if (p.num_groups < 1 || p.num_groups > 1024)
    return fail(MOEGG_ERROR_INVALID_VALUE, "num_groups=%d outside 1..1024", p.num_groups);
  if (p.n <= 0 || p.k <= 0) return fail(MOEGG_ERROR_INVALID_VALUE, "n=%d k=%d must be positive", p.n, p.k);
  if (p.valid_m < 0) return fail(MOEGG_ERROR_INVALID_VALUE, "valid_m=%lld negative", (long long)p.valid_m);
  if (p.m_aligned <= 0 || p.m_aligned % 32 != 0)
    return fail(MOEGG_ERROR_INVALID_VALUE, "m_aligned=%d must be a positive multiple of 32", p.m_aligned);
  if (p.m_aligned % moegg::kRowBlock != 0)
    return fail(MOEGG_ERROR_NOT_SUPPORTED, "m_aligned=%d: libmoegg needs a multiple of %d", p.m_aligned,
                moegg::kRowBlock);
  if (p.valid_m % p.m_aligned != 0)
    return fail(MOEGG_ERROR_INVALID_VALUE, "valid_m=%lld not a multiple of m_aligned=%d", (long long)p.valid_m, p.m_aligned);
  if (p.valid_m > (int64_t)INT32_MAX)
    return fail(MOEGG_ERROR_NOT_SUPPORTED, "valid_m=%lld above 2^31-1", (long long)p.valid_m);
  if (p.k % 32 != 0) return fail(MOEGG_ERROR_INVALID_VALUE, "k=%d not a multiple of 32 (sf_vec_size 32)", p.k);

  // --- dtypes / activation ------------------------------------------------
  const bool mx = p.ab_dtype == MOEGG_DT_E4M3 || p.ab_dtype == MOEGG_DT_E5M2 || p.ab_dtype == MOEGG_DT_E2M1X2;
  if (!mx && p.ab_dtype != MOEGG_DT_BF16)
    return fail(MOEGG_ERROR_INVALID_VALUE, "ab_dtype=%d must be E4M3, E5M2, E2M1X2 or BF16", p.ab_dtype);
  if (p.act < MOEGG_ACT_NONE || p.act > MOEGG_ACT_DGEGLU)
    return fail(MOEGG_ERROR_INVALID_VALUE, "act=%d unknown", p.act);
  if (p.d_dtype != MOEGG_DT_BF16 && p.d_dtype != MOEGG_DT_E4M3)
    return fail(MOEGG_ERROR_INVALID_VALUE, "d_dtype=%d must be BF16 or E4M3", p.d_dtype);
  if (p.c_dtype != MOEGG_DT_NONE && p.c_dtype != MOEGG_DT_BF16)
    return fail(MOEGG_ERROR_INVALID_VALUE, "c_dtype=%d must be NONE or BF16", p.c_dtype);
  if (p.sf_layout != MOEGG_SF_ROW_MAJOR && p.sf_layout != MOEGG_SF_KPLANES)
    return fail(MOEGG_ERROR_INVALID_VALUE, "sf_layout=%d must be ROW_MAJOR or KPLANES", p.sf_layout);
  if (!(p.srelu_tanh_s >= 0.0f) || !std::isfinite(p.srelu_tanh_s))
    return fail(MOEGG_ERROR_INVALID_VALUE, "srelu_tanh_s must be finite and >= 0");
  if ((p.act == MOEGG_ACT_SWIGLU || p.act == MOEGG_ACT_GEGLU) && p.n % 64 != 0)
    return fail(MOEGG_ERROR_INVALID_VALUE, "SwiGLU / GeGLU need n %% 64 == 0 (32-column pairs), n=%d", p.n);
  if (p.act == MOEGG_ACT_GEGLU || p.act == MOEGG_ACT_DGEGLU) {
    if (!std::isfinite(p.glu_gamma) || !std::isfinite(p.geglu_alpha) || !std::isfinite(p.linear_offset))
      return fail(MOEGG_ERROR_INVALID_VALUE, "glu_gamma, geglu_alpha and linear_offset must be finite");
    if (!(p.glu_clamp_min <= p.glu_clamp_max))
      return fail(MOEGG_ERROR_INVALID_VALUE, "glu_clamp_min must not exceed glu_clamp_max (NaN rejected)");
  }
  const bool bwd = p.act == MOEGG_ACT_DSWIGLU || p.act == MOEGG_ACT_DSRELU || p.act == MOEGG_ACT_DGEGLU;
  if (bwd) {
    if (p.n % 32 != 0) return fail(MOEGG_ERROR_INVALID_VALUE, "backward activations need n %% 32 == 0, n=%d", p.n);
    if (!mx && p.d_dtype != MOEGG_DT_BF16)
      return fail(MOEGG_ERROR_NOT_SUPPORTED, "backward activations with BF16 operands write a BF16 dC only");
    if (p.c_dtype != MOEGG_DT_NONE) return fail(MOEGG_ERROR_INVALID_VALUE, "backward activations write no C");
  }
  if (p.n % 32 != 0) return fail(MOEGG_ERROR_NOT_SUPPORTED, "n=%d: libmoegg needs n %% 32 == 0", p.n);
  const int kstep = p.ab_dtype == MOEGG_DT_E2M1X2 ? 256 : p.ab_dtype == MOEGG_DT_BF16 ? 64 : 128;   // 128-byte steps
  if (p.k % kstep != 0)
    return fail(MOEGG_ERROR_NOT_SUPPORTED, "k=%d: libmoegg needs k %% %d == 0 for this operand type", p.k, kstep);
  if (p.k > (1 << 20)) return fail(MOEGG_ERROR_NOT_SUPPORTED, "k=%d too large", p.k);
  if (p.n > (1 << 20)) return fail(MOEGG_ERROR_NOT_SUPPORTED, "n=%d above 2^20", p.n);
  const int64_t n_out = n_out_of(p);
  if (p.d_dtype == MOEGG_DT_E4M3 && n_out % 32 != 0)
    return fail(MOEGG_ERROR_INVALID_VALUE, "E4M3 D needs N_out %% 32 == 0 (row blocks), N_out=%lld", (long long)n_out);

  // --- presence ---------------------------------------------------------------
  if (!a.a || !a.padded_offsets || !a.alpha || !a.d)
    return fail(MOEGG_ERROR_INVALID_VALUE, "a, padded_offsets, alpha and d are required");
  if ((a.b != nullptr) == (a.b_ptrs != nullptr))
    return fail(MOEGG_ERROR_INVALID_VALUE, "exactly one of b (dense weights) and b_ptrs (discrete) is required");
  if (!a.prob) return fail(MOEGG_ERROR_INVALID_VALUE, "prob is required (pass ones for no gating)");
  if (a.b) {
    if (a.sfb_ptrs) return fail(MOEGG_ERROR_INVALID_VALUE, "sfb_ptrs is for discrete weights (b_ptrs) only");
    if (mx && (!a.sfa || !a.sfb)) return fail(MOEGG_ERROR_INVALID_VALUE, "MX operands need sfa and sfb");
    if (!mx && (a.sfa || a.sfb)) return fail(MOEGG_ERROR_INVALID_VALUE, "BF16 operands take no sfa/sfb");
  } else {
    if (a.sfb) return fail(MOEGG_ERROR_INVALID_VALUE, "discrete weights take sfb_ptrs, not sfb");
    if (mx && (!a.sfa || !a.sfb_ptrs)) return fail(MOEGG_ERROR_INVALID_VALUE, "MX operands need sfa and sfb_ptrs");
    if (!mx && (a.sfa || a.sfb_ptrs)) return fail(MOEGG_ERROR_INVALID_VALUE, "BF16 operands take no sfa/sfb_ptrs");
  }
  if (p.c_dtype == MOEGG_DT_BF16 && !a.c) return fail(MOEGG_ERROR_INVALID_VALUE, "c_dtype BF16 needs c");
  if (p.c_dtype == MOEGG_DT_NONE && a.c) return fail(MOEGG_ERROR_INVALID_VALUE, "c given but c_dtype NONE");
  const int nq = (a.sfd_row != nullptr) + (a.sfd_col != nullptr) + (a.norm_const != nullptr);
  if (p.d_dtype == MOEGG_DT_E4M3) {
    if (nq != 3 || !a.d_col)
      return fail(MOEGG_ERROR_INVALID_VALUE, "E4M3 D needs d_col, sfd_row, sfd_col and norm_const together");
    if (a.amax) return fail(MOEGG_ERROR_INVALID_VALUE, "amax is for BF16 D only");
  } else {
    if (nq != 0 || a.d_col)
      return fail(MOEGG_ERROR_INVALID_VALUE, "d_col/sfd_row/sfd_col/norm_const are for E4M3 D only");
    if ((!bwd || mx) && !a.amax)
      return fail(MOEGG_ERROR_INVALID_VALUE, "BF16 D needs amax");
  }
  if (bwd) {
    if (!a.c_in || !a.dprob) return fail(MOEGG_ERROR_INVALID_VALUE, "backward activations need c_in and dprob");
    if (p.act == MOEGG_ACT_DSWIGLU && !a.beta) return fail(MOEGG_ERROR_INVALID_VALUE, "dSwiGLU needs beta");
    if (p.act != MOEGG_ACT_DSWIGLU && a.beta)
      return fail(MOEGG_ERROR_INVALID_VALUE, "beta is for dSwiGLU only (dsReLU / dGeGLU read C_in as stored)");
    if (!mx && a.amax) return fail(MOEGG_ERROR_INVALID_VALUE, "backward activations with BF16 operands write no amax");
  } else if (a.beta || a.c_in || a.dprob) {
    return fail(MOEGG_ERROR_INVALID_VALUE, "beta/c_in/dprob are for the backward activations only");
  }

  // --- alignment (16 B on the contiguous dimension, as the pages require) ------
  const void* big[] = {a.a, a.b, a.c, a.d, a.d_col, a.c_in, a.sfa, a.sfb, a.sfd_row, a.sfd_col};
  for (const void* q : big)
    if (q && !aligned(q, 16)) return fail(MOEGG_ERROR_MISALIGNED, "tensor pointer %p not 16-byte aligned", q);
  const void* small[] = {a.padded_offsets, a.alpha, a.prob, a.beta, a.norm_const, a.amax, a.dprob};
  for (const void* q : small)
    if (q && !aligned(q, 4)) return fail(MOEGG_ERROR_MISALIGNED, "vector pointer %p not 4-byte aligned", q);
  const void* ptr_arrays[] = {a.b_ptrs, a.sfb_ptrs};
  for (const void* q : ptr_arrays)
    if (q && !aligned(q, 8)) return fail(MOEGG_ERROR_MISALIGNED, "pointer array %p not 8-byte aligned", q);
  return MOEGG_OK;
}

}  // namespace

extern "C" {

moegg_status moegg_check(const moegg_problem* problem, const moegg_args* args) {
  moegg_status st = check_impl(problem, args);
  if (st == MOEGG_OK) g_last_error[0] = '\0';
  return st;
}

moegg_status moegg_run(const moegg_problem* problem, const moegg_args* args, void* stream_) {
  moegg_status st = check_impl(problem, args);
  if (st != MOEGG_OK) return st;
  g_last_error[0] = '\0';
  const moegg_problem& p = *problem;
  const moegg_args& a = *args;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);

  if (a.amax) {
    // (L) per group, or (L, 2) for dSwiGLU / dGeGLU: [first blocks, second blocks] of the pairs
    const int count = p.act == MOEGG_ACT_DSWIGLU || p.act == MOEGG_ACT_DGEGLU ? 2 * p.num_groups : p.num_groups;
    hipError_t e = moegg::launch_fill_zero(a.amax, count, stream);
    if (e != hipSuccess) return fail(MOEGG_ERROR_LAUNCH, "amax fill: %s", hipGetErrorString(e));
  }
  if (p.valid_m == 0) return MOEGG_OK;

  moegg::KernelArgs k{};
  k.a = static_cast<const uint8_t*>(a.a);
  k.b = static_cast<const uint8_t*>(a.b);
  k.sfa = a.sfa;
  k.sfb = a.sfb;
  k.b_ptrs = reinterpret_cast<const uint8_t* const*>(a.b_ptrs);
  k.sfb_ptrs = a.sfb_ptrs;
  k.po = a.padded_offsets;
  k.alpha = a.alpha;
  k.prob = a.prob;
  k.beta = a.beta;
  k.norm_const = a.norm_const;
  k.c_in = static_cast<const uint16_t*>(a.c_in);
  k.c = static_cast<uint16_t*>(a.c);
  k.d = static_cast<uint8_t*>(a.d);
  k.d_col = static_cast<uint8_t*>(a.d_col);
  k.sfd_row = a.sfd_row;
  k.sfd_col = a.sfd_col;
  k.amax = a.amax;
  k.dprob = a.dprob;
  k.valid_m = p.valid_m;
  k.num_groups = p.num_groups;
  k.n = p.n;
  k.k = p.k;
  k.n_out = static_cast<int32_t>(n_out_of(p));
  const int ab = p.ab_dtype == MOEGG_DT_E4M3   ? moegg::AB_E4M3
                 : p.ab_dtype == MOEGG_DT_E5M2 ? moegg::AB_E5M2
                 : p.ab_dtype == MOEGG_DT_E2M1X2 ? moegg::AB_E2M1 : moegg::AB_BF16;
  k.row_bytes = ab == moegg::AB_E2M1 ? p.k / 2 : ab == moegg::AB_BF16 ? 2 * p.k : p.k;
  k.glu_gamma = p.glu_gamma;
  k.geglu_alpha = p.geglu_alpha;
  k.linear_offset = p.linear_offset;
  k.glu_clamp_min = p.glu_clamp_min;
  k.glu_clamp_max = p.glu_clamp_max;
  k.ksf = p.k / 32;
  if (p.sf_layout == MOEGG_SF_KPLANES) {
    k.sf_row_a = k.sf_row_b = 4;
    k.sf_word_a = 4 * p.valid_m;
    k.sf_word_b = 4 * (a.b_ptrs ? static_cast<int64_t>(p.n) : static_cast<int64_t>(p.num_groups) * p.n);
  } else {
    k.sf_row_a = k.sf_row_b = k.ksf;
    k.sf_word_a = k.sf_word_b = 4;
  }
  k.k_steps = k.row_bytes / 128;
  k.n_tiles = (p.n + moegg::kBN - 1) / moegg::kBN;
  // persistent grid: one workgroup per CU, never more than there are tiles
  // (at most (valid_m / 128 + L) / 2 row tiles, each n_tiles wide)
  const int64_t max_tiles = ((p.valid_m / moegg::kRowBlock + p.num_groups + 1) / 2) * k.n_tiles;
  if (max_tiles >= (int64_t{1} << 31))
    return fail(MOEGG_ERROR_NOT_SUPPORTED, "valid_m=%lld x n=%d: more than 2^31 output tiles",
                (long long)p.valid_m, p.n);
  const int cus = device_cus();
  if (cus <= 0) return fail(MOEGG_ERROR_LAUNCH, "cannot query the device's compute units");
  int64_t grid = max_tiles < cus ? max_tiles : cus;
  const int limit = g_grid_limit.load(std::memory_order_relaxed);
  if (limit > 0 && grid > limit) grid = limit;
  k.grid = static_cast<int32_t>(grid);
  k.srelu_s = p.srelu_tanh_s;
  const int out = p.d_dtype == MOEGG_DT_E4M3 ? moegg::OUT_E4M3 : moegg::OUT_BF16;
  hipError_t e = moegg::launch_grouped_gemm(ab, p.act, out, k, stream);
  if (e != hipSuccess) return fail(MOEGG_ERROR_LAUNCH, "kernel launch: %s", hipGetErrorString(e));
  return MOEGG_OK;
}

moegg_status moegg_check_offsets(const moegg_problem* problem, const int32_t* po, void* stream_) {
  if (!problem || !po) return fail(MOEGG_ERROR_INVALID_VALUE, "problem and padded_offsets must be non-NULL");
  const moegg_problem& p = *problem;
  if (p.num_groups < 1 || p.num_groups > 1024 || p.m_aligned <= 0)
    return fail(MOEGG_ERROR_INVALID_VALUE, "bad num_groups/m_aligned");
  std::vector<int32_t> h(p.num_groups);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  hipError_t e = hipMemcpyAsync(h.data(), po, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(MOEGG_ERROR_LAUNCH, "offset copy: %s", hipGetErrorString(e));
  int64_t prev = 0;
  for (int g = 0; g < p.num_groups; ++g) {
    if (h[g] < prev) return fail(MOEGG_ERROR_INVALID_VALUE, "padded_offsets[%d]=%d decreases", g, h[g]);
    if (h[g] % p.m_aligned != 0)
      return fail(MOEGG_ERROR_INVALID_VALUE, "padded_offsets[%d]=%d not a multiple of %d", g, h[g], p.m_aligned);
    prev = h[g];
  }
  if (prev != p.valid_m)
    return fail(MOEGG_ERROR_INVALID_VALUE, "padded_offsets[L-1]=%lld != valid_m=%lld", (long long)prev, (long long)p.valid_m);
  g_last_error[0] = '\0';
  return MOEGG_OK;
}

moegg_status moegg_sf_to_kplanes(const uint8_t* src, uint8_t* dst, int64_t rows, int32_t k, void* stream_) {
  if (rows < 0 || k <= 0 || k % 128 != 0)
    return fail(MOEGG_ERROR_INVALID_VALUE, "rows=%lld k=%d: rows >= 0 and k a positive multiple of 128 needed",
                (long long)rows, k);
  if (k / 128 > 65535) return fail(MOEGG_ERROR_INVALID_VALUE, "k=%d too large", k);
  if (rows == 0) {
    g_last_error[0] = '\0';
    return MOEGG_OK;
  }
  if (!src || !dst) return fail(MOEGG_ERROR_INVALID_VALUE, "src and dst must be non-NULL");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(MOEGG_ERROR_MISALIGNED, "src/dst not 16-byte aligned");
  const uintptr_t bytes = static_cast<uintptr_t>(rows) * (k / 32);
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(MOEGG_ERROR_INVALID_VALUE, "src and dst overlap");
  hipError_t e = moegg::launch_sf_kplanes(src, dst, rows, k / 128, reinterpret_cast<hipStream_t>(stream_));
  if (e != hipSuccess) return fail(MOEGG_ERROR_LAUNCH, "scale layout kernel: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return MOEGG_OK;
}

int64_t moegg_n_out(const moegg_problem* problem) { return problem ? n_out_of(*problem) : -1; }

const char* moegg_status_string(moegg_status s) {
  switch (s) {
    case MOEGG_OK: return "MOEGG_OK";
    case MOEGG_ERROR_INVALID_VALUE: return "MOEGG_ERROR_INVALID_VALUE";
    case MOEGG_ERROR_MISALIGNED: return "MOEGG_ERROR_MISALIGNED";
    case MOEGG_ERROR_NOT_SUPPORTED: return "MOEGG_ERROR_NOT_SUPPORTED";
    case MOEGG_ERROR_LAUNCH: return "MOEGG_ERROR_LAUNCH";
  }
  return "MOEGG_UNKNOWN_STATUS";
}

const char* moegg_last_error(void) { return g_last_error; }

int moegg_abi_version(void) { return MOEGG_ABI_VERSION; }

int moegg_set_grid_limit(int max_workgroups) {
  return g_grid_limit.exchange(max_workgroups > 0 ? max_workgroups : 0, std::memory_order_relaxed);
}

}  // extern "C"
