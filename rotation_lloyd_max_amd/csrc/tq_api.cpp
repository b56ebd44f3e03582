// Host side of libtq: the C entry points declared in include/tq.h.
//
// Every call validates its arguments before launching anything, reports failures through a
// negative status and a thread-local message, and never throws or aborts across the C
// interface. The Lloyd-Max codebooks are computed here once, in double precision, by
// Lloyd's iteration on the N(0,1) density (turboquant-mlx "How it works", "Quantizing a
// weight, with no data", third bullet: one fixed codebook per bit width, a mathematical
// constant; "The ternary tier (1.58 bits)": levels {-c, 0, +c}).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tq.h"
#include "internal.hpp"

namespace tq {
namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TQ_OK;
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- Lloyd-Max codebooks ---------------------------------------------------------------
double normal_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}
// P(X > x)
double normal_sf(double x) {
  if (x == INFINITY) return 0.0;
  if (x == -INFINITY) return 1.0;
  return 0.5 * std::erfc(x / std::sqrt(2.0));
}
// P(a < X <= b), evaluated on the side of 0 where it does not cancel
double cell_mass(double a, double b) {
  if (a >= 0.0) return normal_sf(a) - normal_sf(b);
  if (b <= 0.0) return normal_sf(-b) - normal_sf(-a);
  return 1.0 - normal_sf(-a) - normal_sf(b);
}

void lloyd(int L, double* c, double* t) {
  for (int k = 0; k < L; ++k) c[k] = -2.0 + 4.0 * (k + 0.5) / L;
  double nc[16];
  for (int it = 0; it < 200000; ++it) {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    for (int k = 0; k < L; ++k) {
      const double a = k == 0 ? -INFINITY : t[k - 1];
      const double b = k == L - 1 ? INFINITY : t[k];
      nc[k] = (normal_pdf(a) - normal_pdf(b)) / cell_mass(a, b);
    }
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      const double v = 0.5 * (nc[k] - nc[L - 1 - k]);  // keep the exact symmetry
      delta = std::fmax(delta, std::fabs(v - c[k]));
      c[k] = v;
    }
    if (delta < 1e-15) break;
  }
  for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
}

// The 256-level codebook (8-bit KV-cache keys): the same fixed point, but plain Lloyd
// iteration contracts at about 0.99985 per step there and the fixed point amplifies the
// map's rounding errors about 10^4 times, so it is computed in 80-bit long double: Lloyd
// steps from the same start, then Newton's method on lloyd(c) - c = 0 with the tridiagonal
// Jacobian of the map (d mean / d b = pdf(b) (b - mean) / P, d mean / d a = pdf(a)
// (mean - a) / P, each threshold the midpoint of its neighbours).
typedef long double ldbl;
ldbl pdf_l(ldbl x) { return std::exp(-0.5L * x * x) / std::sqrt(2.0L * 3.14159265358979323846264338327950288L); }
ldbl sf_l(ldbl x) { return 0.5L * std::erfc(x / std::sqrt(2.0L)); }
ldbl mass_l(ldbl a, ldbl b, bool a_inf, bool b_inf) {
  const ldbl Qa = a_inf ? 1.0L : sf_l(a), Qb = b_inf ? 0.0L : sf_l(b);
  if (!a_inf && a >= 0) return Qa - Qb;
  if (!b_inf && b <= 0) return (b_inf ? 1.0L : sf_l(-b)) - (a_inf ? 0.0L : sf_l(-a));
  return 1.0L - (a_inf ? 0.0L : sf_l(-a)) - Qb;
}

void lloyd_big(int L, double* c_out, double* t_out) {
  std::vector<ldbl> c(L), nc(L), t(L - 1), g(L), sub(L), dia(L), sup(L), cp(L), dp(L), d(L);
  for (int k = 0; k < L; ++k) c[k] = -2.0L + 4.0L * (k + 0.5L) / L;
  auto step = [&](bool jac) {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5L * (c[k] + c[k + 1]);
    for (int k = 0; k < L; ++k) {
      const bool ai = k == 0, bi = k == L - 1;
      const ldbl a = ai ? 0.0L : t[k - 1], b = bi ? 0.0L : t[k];
      const ldbl pa = ai ? 0.0L : pdf_l(a), pb = bi ? 0.0L : pdf_l(b);
      const ldbl P = mass_l(a, b, ai, bi);
      const ldbl m = (pa - pb) / P;
      nc[k] = m;
      if (jac) {
        const ldbl da = ai ? 0.0L : pa * (m - a) / P;
        const ldbl db = bi ? 0.0L : pb * (b - m) / P;
        sub[k] = da / 2;
        dia[k] = (da + db) / 2 - 1;
        sup[k] = db / 2;
      }
    }
  };
  for (int it = 0; it < 2000; ++it) {
    step(false);
    for (int k = 0; k < L; ++k) c[k] = 0.5L * (nc[k] - nc[L - 1 - k]);
  }
  for (int it = 0; it < 40; ++it) {
    step(true);
    for (int k = 0; k < L; ++k) g[k] = nc[k] - c[k];
    cp[0] = sup[0] / dia[0];
    dp[0] = -g[0] / dia[0];
    for (int k = 1; k < L; ++k) {
      const ldbl den = dia[k] - sub[k] * cp[k - 1];
      cp[k] = sup[k] / den;
      dp[k] = (-g[k] - sub[k] * dp[k - 1]) / den;
    }
    d[L - 1] = dp[L - 1];
    for (int k = L - 2; k >= 0; --k) d[k] = dp[k] - cp[k] * d[k + 1];
    ldbl dmax = 0;
    for (int k = 0; k < L; ++k) {
      c[k] += d[k];
      dmax = std::fmax(dmax, std::fabs(d[k]));
    }
    for (int k = 0; k < L; ++k) nc[k] = 0.5L * (c[k] - c[L - 1 - k]);
    for (int k = 0; k < L; ++k) c[k] = nc[k];
    if (dmax < 1e-17L) break;
  }
  for (int k = 0; k < L; ++k) c_out[k] = static_cast<double>(c[k]);
  for (int k = 0; k + 1 < L; ++k) t_out[k] = static_cast<double>(0.5L * (c[k] + c[k + 1]));
}

CodebookArgs g_books[4];
BigCodebook g_big;
std::once_flag g_books_once;

void init_books() {
  const int levels[4] = {3, 4, 8, 16};
  for (int i = 0; i < 4; ++i) {
    CodebookArgs& b = g_books[i];
    std::memset(&b, 0, sizeof b);
    const int L = levels[i];
    double c[16], t[15];
    lloyd(L, c, t);
    b.levels = L;
    for (int k = 0; k < L; ++k) {
      b.c[k] = static_cast<float>(c[k]);
      const _Float16 h = static_cast<_Float16>(c[k]);
      std::memcpy(&b.h[k], &h, 2);
    }
    for (int k = 0; k + 1 < L; ++k) b.t[k] = static_cast<float>(t[k]);
  }
  {
    std::vector<double> c(256), t(255);
    lloyd_big(256, c.data(), t.data());
    for (int k = 0; k < 256; ++k) {
      g_big.c[k] = static_cast<float>(c[k]);
      const _Float16 h = static_cast<_Float16>(c[k]);
      std::memcpy(&g_big.h[k], &h, 2);
    }
    for (int k = 0; k < 255; ++k) g_big.t[k] = static_cast<float>(t[k]);
  }
}

int64_t words_per_row(int64_t K, int levels) {
  switch (levels) {
    case 3: return (K + 19) / 20;
    case 4: return (2 * K + 31) / 32;
    case 8: return (3 * K + 31) / 32;
    case 16: return (4 * K + 31) / 32;
    case 256: return (8 * K + 31) / 32;
    default: return 0;
  }
}

bool valid_dtype(int d) { return d == TQ_F32 || d == TQ_BF16 || d == TQ_F16; }
size_t dtype_size(int d) { return d == TQ_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// allow256: the 8-bit codebook (KV-cache rows), for power-of-two K up to 4096 only;
// any_k: no Hadamard transform is applied (pre-rotated inputs, dense rotations,
// dequantization), so K need only be a multiple of 32 in [64, 8192]
int check_shape(int64_t K, int levels, int group, int* m, int* P, bool allow256 = false,
                bool any_k = false) {
  if (levels == 256 && allow256) {
    if (K < 64 || K > 4096 || (K & (K - 1)) != 0)
      return fail(TQ_ERR_UNSUPPORTED, "256 levels need K a power of two in [64, 4096] (got %lld)",
                  static_cast<long long>(K));
  } else if (levels != 3 && levels != 4 && levels != 8 && levels != 16) {
    return fail(TQ_ERR_UNSUPPORTED, "n_levels must be 3, 4, 8 or 16%s (got %d)",
                allow256 ? " (or 256)" : "", levels);
  }
  if (group != 16 && group != 32 && group != 64 && group != 128)
    return fail(TQ_ERR_UNSUPPORTED, "group must be 16, 32, 64 or 128 (got %d)", group);
  if (K < 64 || K > 8192 || K % 32 != 0)
    return fail(TQ_ERR_UNSUPPORTED, "K must be a multiple of 32 in [64, 8192] (got %lld)",
                static_cast<long long>(K));
  if (!split_dim(K, m, P)) {
    if (!any_k)
      return fail(TQ_ERR_UNSUPPORTED,
                  "K=%lld is not m*2^k with m in {1, 12, 20, 28} (a dense rotation and "
                  "TQ_X_ROTATED inputs take any multiple of 32)",
                  static_cast<long long>(K));
    *m = 1;
    *P = static_cast<int>(K);
  }
  if (K % group != 0)
    return fail(TQ_ERR_UNSUPPORTED, "group %d does not divide K=%lld", group,
                static_cast<long long>(K));
  return TQ_OK;
}

// rotated: the call applies no rotation of its own (TQ_X_ROTATED inputs, dequantization), so
// K may be any multiple of 32 in [64, 8192] and the sign bits are not needed
int check_weight(const tq_qweight* w, WeightArgs* out, bool allow256 = false,
                 bool rotated = false) {
  if (!w) return fail(TQ_ERR_ARG, "weight descriptor is NULL");
  int m = 1, P = 1;
  const int rc = check_shape(w->K, w->n_levels, w->group, &m, &P, allow256, rotated);
  if (rc != TQ_OK) return rc;
  if (w->N < 0 || w->N > (1 << 24)) return fail(TQ_ERR_ARG, "N out of range");
  if (w->E < 1 || w->E > 8192) return fail(TQ_ERR_ARG, "E must be in [1, 8192]");
  if (w->N > 0) {
    if (!w->codes || !w->scales || (!w->signs && !rotated))
      return fail(TQ_ERR_ARG, "codes, scales and signs must be non-NULL");
    if (!aligned(w->codes, 16)) return fail(TQ_ERR_ALIGN, "codes must be 16-byte aligned");
    if (!aligned(w->scales, 2) || (w->signs && !aligned(w->signs, 4)))
      return fail(TQ_ERR_ALIGN, "scales/signs misaligned");
  }
  out->codes = w->codes;
  out->scales = w->scales;
  out->signs = w->signs;
  out->levels = w->n_levels;
  out->group = w->group;
  out->K = static_cast<int>(w->K);
  out->N = static_cast<int>(w->N);
  out->E = static_cast<int>(w->E);
  out->wpr = static_cast<int>(words_per_row(w->K, w->n_levels));
  out->m = m;
  out->P = P;
  return TQ_OK;
}

// x is read with 16-byte loads (rows of K elements, K a multiple of 32, stay aligned).
int check_io(const void* x, int xdt, const void* y, int ydt, bool need) {
  if (!valid_dtype(xdt) || !valid_dtype(ydt)) return fail(TQ_ERR_ARG, "bad dtype");
  if (!need) return TQ_OK;
  if (!x || !y) return fail(TQ_ERR_ARG, "x and y must be non-NULL");
  if (!aligned(x, 16)) return fail(TQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, dtype_size(ydt))) return fail(TQ_ERR_ALIGN, "y misaligned for its dtype");
  return TQ_OK;
}

}  // namespace

const BigCodebook* codebook256() {
  std::call_once(g_books_once, init_books);
  return &g_big;
}

const CodebookArgs* codebook_for(int levels) {
  std::call_once(g_books_once, init_books);
  switch (levels) {
    case 3: return &g_books[0];
    case 4: return &g_books[1];
    case 8: return &g_books[2];
    case 16: return &g_books[3];
    default: return nullptr;
  }
}

bool split_dim(int64_t K, int* m, int* P) {
  const int ms[4] = {1, 12, 20, 28};
  for (int i = 0; i < 4; ++i) {
    if (K % ms[i] != 0) continue;
    const int64_t p = K / ms[i];
    if (p >= 1 && (p & (p - 1)) == 0) {
      *m = ms[i];
      *P = static_cast<int>(p);
      return true;
    }
  }
  return false;
}

}  // namespace tq

using namespace tq;

extern "C" {

int64_t tq_words_per_row(int64_t K, int32_t n_levels) {
  if (K <= 0) return 0;
  return words_per_row(K, n_levels);
}

int tq_codebook(int32_t n_levels, float* centroids, float* thresholds) {
  if (n_levels == 256) {
    if (!centroids) return fail(TQ_ERR_ARG, "centroids is NULL");
    const BigCodebook* g = codebook256();
    std::memcpy(centroids, g->c, sizeof(float) * 256);
    if (thresholds) std::memcpy(thresholds, g->t, sizeof(float) * 255);
    return TQ_OK;
  }
  const CodebookArgs* b = codebook_for(n_levels);
  if (!b) return fail(TQ_ERR_UNSUPPORTED, "n_levels must be 3, 4, 8 or 16 (got %d)", n_levels);
  if (!centroids) return fail(TQ_ERR_ARG, "centroids is NULL");
  std::memcpy(centroids, b->c, sizeof(float) * n_levels);
  if (thresholds) std::memcpy(thresholds, b->t, sizeof(float) * (n_levels - 1));
  return TQ_OK;
}

int tq_signs(uint64_t seed, int64_t K, uint32_t* bits, void* stream) {
  if (K <= 0 || K > (1 << 24)) return fail(TQ_ERR_ARG, "K out of range");
  if (!bits) return fail(TQ_ERR_ARG, "bits is NULL");
  if (!aligned(bits, 4)) return fail(TQ_ERR_ALIGN, "bits must be 4-byte aligned");
  return hip_status(launch_signs(seed, static_cast<int>(K), bits, static_cast<hipStream_t>(stream)),
                    "tq_signs");
}

int tq_encode(const void* W, tq_dtype w_dtype, int64_t rows, int64_t K, int32_t n_levels,
              int32_t group, uint64_t seed, uint32_t* codes, uint16_t* scales, void* stream) {
  int m = 1, P = 1;
  const int rc = check_shape(K, n_levels, group, &m, &P, /*allow256=*/true);
  if (rc != TQ_OK) return rc;
  if (!valid_dtype(w_dtype)) return fail(TQ_ERR_ARG, "bad weight dtype");
  if (rows < 0) return fail(TQ_ERR_ARG, "rows must be >= 0");
  if (rows == 0) return TQ_OK;
  if (!W || !codes || !scales) return fail(TQ_ERR_ARG, "W, codes and scales must be non-NULL");
  if (!aligned(W, dtype_size(w_dtype)) || !aligned(codes, 4) || !aligned(scales, 2))
    return fail(TQ_ERR_ALIGN, "W, codes or scales misaligned");
  if (n_levels == 256 && !aligned(W, 16))
    return fail(TQ_ERR_ALIGN, "256-level encode reads W with 16-byte loads: W must be 16-byte aligned");
  return hip_status(launch_encode(W, w_dtype, rows, static_cast<int>(K), m, P, n_levels, group,
                                  seed, codes, scales, static_cast<hipStream_t>(stream)),
                    "tq_encode");
}

int tq_encode_stream(const void* W_host, tq_dtype w_dtype, int64_t rows, int64_t K,
                     int32_t n_levels, int32_t group, uint64_t seed, uint32_t* codes,
                     uint16_t* scales, void* staging, size_t staging_bytes, void* stream,
                     void* copy_stream) {
  int m = 1, P = 1;
  const int rc = check_shape(K, n_levels, group, &m, &P, /*allow256=*/true);
  if (rc != TQ_OK) return rc;
  if (!valid_dtype(w_dtype)) return fail(TQ_ERR_ARG, "bad weight dtype");
  if (rows < 0) return fail(TQ_ERR_ARG, "rows must be >= 0");
  if (rows == 0) return TQ_OK;
  if (!W_host || !codes || !scales || !staging)
    return fail(TQ_ERR_ARG, "W_host, codes, scales and staging must be non-NULL");
  if (!aligned(W_host, dtype_size(w_dtype)) || !aligned(codes, 4) || !aligned(scales, 2))
    return fail(TQ_ERR_ALIGN, "W_host, codes or scales misaligned");
  if (!aligned(staging, 256)) return fail(TQ_ERR_ALIGN, "staging must be 256-byte aligned");
  // each half of the staging buffer holds `chunk` whole rows and starts 256-byte aligned
  const size_t row_bytes = static_cast<size_t>(K) * dtype_size(w_dtype);
  const size_t half = (staging_bytes / 2) & ~static_cast<size_t>(255);
  const int64_t chunk = static_cast<int64_t>(half / row_bytes);
  if (chunk < 1)
    return fail(TQ_ERR_ARG, "staging of %zu bytes holds fewer than two rows of %zu bytes",
                staging_bytes, row_bytes);
  const int64_t wpr = words_per_row(K, n_levels);
  const int64_t ngk = K / group;
  const hipStream_t cs = static_cast<hipStream_t>(stream);
  const hipStream_t xs = copy_stream ? static_cast<hipStream_t>(copy_stream) : cs;
  // filled[b]: half b holds its chunk (copy done); freed[b]: its encode is done; entry:
  // everything enqueued on `stream` before this call (which may still read `staging`)
  hipEvent_t filled[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr}, entry = nullptr;
  hipError_t e = hipSuccess;
  for (int b = 0; b < 2 && e == hipSuccess; ++b) {
    e = hipEventCreateWithFlags(&filled[b], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&freed[b], hipEventDisableTiming);
  }
  if (e == hipSuccess && xs != cs) {
    e = hipEventCreateWithFlags(&entry, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(entry, cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(xs, entry, 0);
  }
  const char* src = static_cast<const char*>(W_host);
  char* stage = static_cast<char*>(staging);
  for (int64_t i = 0, r0 = 0; e == hipSuccess && r0 < rows; ++i, r0 += chunk) {
    const int b = static_cast<int>(i & 1);
    const int64_t n = rows - r0 < chunk ? rows - r0 : chunk;
    char* buf = stage + b * half;
    // the half is reused once the encode of the chunk it held two steps ago is done
    if (i >= 2) e = hipStreamWaitEvent(xs, freed[b], 0);
    if (e == hipSuccess)
      e = hipMemcpyAsync(buf, src + static_cast<size_t>(r0) * row_bytes,
                         static_cast<size_t>(n) * row_bytes, hipMemcpyHostToDevice, xs);
    if (e == hipSuccess) e = hipEventRecord(filled[b], xs);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, filled[b], 0);
    if (e == hipSuccess)
      e = launch_encode(buf, w_dtype, n, static_cast<int>(K), m, P, n_levels, group, seed,
                        codes + r0 * wpr, scales + r0 * ngk, cs);
    if (e == hipSuccess) e = hipEventRecord(freed[b], cs);
  }
  for (int b = 0; b < 2; ++b) {
    if (filled[b]) (void)hipEventDestroy(filled[b]);
    if (freed[b]) (void)hipEventDestroy(freed[b]);
  }
  if (entry) (void)hipEventDestroy(entry);
  return hip_status(e, "tq_encode_stream");
}

int tq_fwht(const void* x, tq_dtype x_dtype, int64_t rows, int64_t K, uint64_t seed, void* out,
            tq_dtype out_dtype, void* stream) {
  int m = 1, P = 1;
  if (K < 64 || K > 8192 || K % 32 != 0 || !split_dim(K, &m, &P))
    return fail(TQ_ERR_UNSUPPORTED, "K must be m*2^k (m in {1,12,20,28}), a multiple of 32 in [64, 8192]");
  if (rows < 0) return fail(TQ_ERR_ARG, "rows must be >= 0");
  const int rc = check_io(x, x_dtype, out, out_dtype, rows > 0);
  if (rc != TQ_OK) return rc;
  if (rows == 0) return TQ_OK;
  return hip_status(launch_fwht(x, x_dtype, rows, static_cast<int>(K), m, P, nullptr, seed, out,
                                out_dtype, static_cast<hipStream_t>(stream)),
                    "tq_fwht");
}

size_t tq_workspace_bytes(int32_t op, const tq_qweight* w, int64_t count, int64_t T) {
  WeightArgs a{};
  if (check_weight(w, &a, false, /*rotated=*/true) != TQ_OK || count < 0 || T < 0) return SIZE_MAX;
  switch (op) {
    case TQ_OP_QMV:
    case TQ_OP_GATHER_QMV: return 0;
    case TQ_OP_MULTI_GATHER_QMV: return multi_gather_workspace(a, count);
    case TQ_OP_GATHER_QMM: return gather_qmm_workspace(a, count, T);
    case TQ_OP_ENCODE_DENSE: return static_cast<size_t>(count) * a.K * 8;
    default: fail(TQ_ERR_ARG, "unknown op %d", op); return SIZE_MAX;
  }
}

int tq_qmv(const tq_qweight* w, const void* x, tq_dtype x_dtype, void* y, tq_dtype y_dtype,
           uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  WeightArgs a{};
  int rc = check_weight(w, &a, false, (flags & TQ_X_ROTATED) != 0);
  if (rc != TQ_OK) return rc;
  if (a.E != 1) return fail(TQ_ERR_ARG, "tq_qmv needs E = 1 (use tq_gather_qmv for experts)");
  rc = check_io(x, x_dtype, y, y_dtype, a.N > 0);
  if (rc != TQ_OK) return rc;
  return hip_status(launch_qmv(a, nullptr, 1, x, x_dtype, (flags & TQ_X_ROTATED) != 0, y, y_dtype,
                               static_cast<hipStream_t>(stream)),
                    "tq_qmv");
}

int tq_gather_qmv(const tq_qweight* w, const int32_t* ids, int32_t n, const void* x,
                  tq_dtype x_dtype, void* y, tq_dtype y_dtype, uint32_t flags, void* ws,
                  size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  WeightArgs a{};
  int rc = check_weight(w, &a, false, (flags & TQ_X_ROTATED) != 0);
  if (rc != TQ_OK) return rc;
  if (n < 0) return fail(TQ_ERR_ARG, "n must be >= 0");
  if (n > 0 && !ids) return fail(TQ_ERR_ARG, "ids is NULL");
  if (n > 0 && !aligned(ids, 4)) return fail(TQ_ERR_ALIGN, "ids misaligned");
  rc = check_io(x, x_dtype, y, y_dtype, n > 0 && a.N > 0);
  if (rc != TQ_OK) return rc;
  return hip_status(launch_qmv(a, ids, n, x, x_dtype, (flags & TQ_X_ROTATED) != 0, y, y_dtype,
                               static_cast<hipStream_t>(stream)),
                    "tq_gather_qmv");
}

int tq_gather_qmv_pair(const tq_qweight* w1, const tq_qweight* w2, const int32_t* ids, int32_t n,
                       const void* x, tq_dtype x_dtype, void* y, tq_dtype y_dtype, uint32_t flags,
                       void* stream) {
  const bool rotated = (flags & TQ_X_ROTATED) != 0;
  WeightArgs a{}, b{};
  int rc = check_weight(w1, &a, false, rotated);
  if (rc != TQ_OK) return rc;
  rc = check_weight(w2, &b, false, rotated);
  if (rc != TQ_OK) return rc;
  if (a.levels != b.levels || a.group != b.group || a.K != b.K || a.N != b.N || a.E != b.E)
    return fail(TQ_ERR_ARG, "tq_gather_qmv_pair: the two weights differ in format or shape");
  if (!rotated && w1->signs != w2->signs)
    return fail(TQ_ERR_ARG, "tq_gather_qmv_pair: the two weights must share one signs array");
  if (n < 0 || n > 65535) return fail(TQ_ERR_ARG, "n must be in [0, 65535]");
  if (n > 0 && !ids) return fail(TQ_ERR_ARG, "ids is NULL");
  if (n > 0 && !aligned(ids, 4)) return fail(TQ_ERR_ALIGN, "ids misaligned");
  rc = check_io(x, x_dtype, y, y_dtype, n > 0 && a.N > 0);
  if (rc != TQ_OK) return rc;
  return hip_status(launch_qmv(a, ids, n, x, x_dtype, rotated, y, y_dtype,
                               static_cast<hipStream_t>(stream), &b),
                    "tq_gather_qmv_pair");
}

int tq_multi_gather_qmv(const tq_qweight* w, const int32_t* ids, int64_t P, const void* x,
                        tq_dtype x_dtype, void* y, tq_dtype y_dtype, uint32_t flags, void* ws,
                        size_t ws_bytes, void* stream) {
  WeightArgs a{};
  int rc = check_weight(w, &a, false, (flags & TQ_X_ROTATED) != 0);
  if (rc != TQ_OK) return rc;
  if (P < 0 || P > (1 << 30)) return fail(TQ_ERR_ARG, "P out of range");
  if (P > 0 && !ids) return fail(TQ_ERR_ARG, "ids is NULL");
  if (P > 0 && !aligned(ids, 4)) return fail(TQ_ERR_ALIGN, "ids misaligned");
  rc = check_io(x, x_dtype, y, y_dtype, P > 0 && a.N > 0);
  if (rc != TQ_OK) return rc;
  if (P == 0 || a.N == 0) return TQ_OK;
  const size_t need = multi_gather_workspace(a, P);
  if (!ws || ws_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned(ws, 16)) return fail(TQ_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(launch_multi_gather(a, ids, P, x, x_dtype, (flags & TQ_X_ROTATED) != 0, y,
                                        y_dtype, ws, static_cast<hipStream_t>(stream)),
                    "tq_multi_gather_qmv");
}

int tq_multi_gather_qmv_pair(const tq_qweight* w1, const tq_qweight* w2, const int32_t* ids,
                             int64_t P, const void* x, tq_dtype x_dtype, void* y,
                             tq_dtype y_dtype, uint32_t flags, void* ws, size_t ws_bytes,
                             void* stream) {
  const bool rotated = (flags & TQ_X_ROTATED) != 0;
  WeightArgs a{}, b{};
  int rc = check_weight(w1, &a, false, rotated);
  if (rc != TQ_OK) return rc;
  rc = check_weight(w2, &b, false, rotated);
  if (rc != TQ_OK) return rc;
  if (a.levels != b.levels || a.group != b.group || a.K != b.K || a.N != b.N || a.E != b.E)
    return fail(TQ_ERR_ARG, "tq_multi_gather_qmv_pair: the two weights differ in format or shape");
  if (!rotated && w1->signs != w2->signs)
    return fail(TQ_ERR_ARG, "tq_multi_gather_qmv_pair: the two weights must share one signs array");
  if (P < 0 || P > (1 << 29)) return fail(TQ_ERR_ARG, "P out of range");
  if (P > 0 && !ids) return fail(TQ_ERR_ARG, "ids is NULL");
  if (P > 0 && !aligned(ids, 4)) return fail(TQ_ERR_ALIGN, "ids misaligned");
  rc = check_io(x, x_dtype, y, y_dtype, P > 0 && a.N > 0);
  if (rc != TQ_OK) return rc;
  if (P == 0 || a.N == 0) return TQ_OK;
  const size_t need = multi_gather_workspace(a, P);
  if (!ws || ws_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned(ws, 16)) return fail(TQ_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(launch_multi_gather(a, ids, P, x, x_dtype, rotated, y, y_dtype, ws,
                                        static_cast<hipStream_t>(stream), &b),
                    "tq_multi_gather_qmv_pair");
}

int tq_multi_gather_qmv_static(const tq_qweight* w, const int32_t* ids, int64_t P,
                               const void* x, tq_dtype x_dtype, void* y, tq_dtype y_dtype,
                               uint32_t flags, void* stream) {
  WeightArgs a{};
  int rc = check_weight(w, &a, false, (flags & TQ_X_ROTATED) != 0);
  if (rc != TQ_OK) return rc;
  if (P < 0 || P > (1 << 30)) return fail(TQ_ERR_ARG, "P out of range");
  if (P > 0 && !ids) return fail(TQ_ERR_ARG, "ids is NULL");
  if (P > 0 && !aligned(ids, 4)) return fail(TQ_ERR_ALIGN, "ids misaligned");
  rc = check_io(x, x_dtype, y, y_dtype, P > 0 && a.N > 0);
  if (rc != TQ_OK) return rc;
  if (P == 0 || a.N == 0) return TQ_OK;
  const size_t need = multi_gather_workspace(a, P);
  if (need > kStaticScratchBytes)
    return fail(TQ_ERR_WORKSPACE,
                "tq_multi_gather_qmv_static: %lld pairs of K=%d need %zu bytes of workspace, "
                "above the fixed %zu (use tq_multi_gather_qmv with a workspace)",
                static_cast<long long>(P), a.K, need, kStaticScratchBytes);
  void* ws = nullptr;
  rc = hip_status(static_scratch(&ws), "tq_multi_gather_qmv_static");
  if (rc != TQ_OK) return rc;
  return hip_status(launch_multi_gather(a, ids, P, x, x_dtype, (flags & TQ_X_ROTATED) != 0, y,
                                        y_dtype, ws, static_cast<hipStream_t>(stream)),
                    "tq_multi_gather_qmv_static");
}

int tq_rotate_dense(const void* x, tq_dtype x_dtype, int64_t rows, int64_t K, const float* R,
                    void* out, tq_dtype out_dtype, void* stream) {
  if (K < 64 || K > 8192 || K % 32 != 0)
    return fail(TQ_ERR_UNSUPPORTED, "K must be a multiple of 32 in [64, 8192] (got %lld)",
                static_cast<long long>(K));
  if (rows < 0) return fail(TQ_ERR_ARG, "rows must be >= 0");
  if (!valid_dtype(x_dtype) || !valid_dtype(out_dtype)) return fail(TQ_ERR_ARG, "bad dtype");
  if (rows == 0) return TQ_OK;
  if (!x || !R || !out) return fail(TQ_ERR_ARG, "x, R and out must be non-NULL");
  if (!aligned(x, dtype_size(x_dtype)) || !aligned(R, 4) || !aligned(out, dtype_size(out_dtype)))
    return fail(TQ_ERR_ALIGN, "x, R or out misaligned");
  if ((rows + 63) / 64 > 65535) return fail(TQ_ERR_ARG, "rows must be below 64 * 65536");
  return hip_status(launch_dense_rot(x, x_dtype, rows, static_cast<int>(K), R, out, out_dtype,
                                     static_cast<hipStream_t>(stream)),
                    "tq_rotate_dense");
}

int tq_encode_dense(const void* W, tq_dtype w_dtype, int64_t rows, int64_t K, const float* R,
                    int32_t n_levels, int32_t group, uint32_t* codes, uint16_t* scales,
                    void* ws, size_t ws_bytes, void* stream) {
  int m = 1, P = 1;
  const int rc = check_shape(K, n_levels, group, &m, &P, false, /*any_k=*/true);
  if (rc != TQ_OK) return rc;
  if (!valid_dtype(w_dtype)) return fail(TQ_ERR_ARG, "bad weight dtype");
  if (rows < 0) return fail(TQ_ERR_ARG, "rows must be >= 0");
  if (rows == 0) return TQ_OK;
  if (!W || !R || !codes || !scales) return fail(TQ_ERR_ARG, "W, R, codes and scales must be non-NULL");
  if (!aligned(W, dtype_size(w_dtype)) || !aligned(R, 4) || !aligned(codes, 4) ||
      !aligned(scales, 2))
    return fail(TQ_ERR_ALIGN, "W, R, codes or scales misaligned");
  const size_t row_bytes = static_cast<size_t>(K) * 8;
  if (!ws || ws_bytes < row_bytes)
    return fail(TQ_ERR_WORKSPACE, "workspace of at least %zu bytes (one fp64 row) needed", row_bytes);
  if (!aligned(ws, 8)) return fail(TQ_ERR_ALIGN, "workspace must be 8-byte aligned");
  int64_t chunk = static_cast<int64_t>(ws_bytes / row_bytes);
  if (chunk > 64 * 65535) chunk = 64 * 65535;
  const int64_t wpr = words_per_row(K, n_levels), ngk = K / group;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const char* src = static_cast<const char*>(W);
  hipError_t e = hipSuccess;
  for (int64_t r0 = 0; r0 < rows && e == hipSuccess; r0 += chunk) {
    const int64_t n = rows - r0 < chunk ? rows - r0 : chunk;
    e = launch_dense_rot(src + static_cast<size_t>(r0) * K * dtype_size(w_dtype), w_dtype, n,
                         static_cast<int>(K), R, ws, 3, st);
    if (e == hipSuccess)
      e = launch_encode_rotated(static_cast<const double*>(ws), n, static_cast<int>(K), n_levels,
                                group, codes + r0 * wpr, scales + r0 * ngk, st);
  }
  return hip_status(e, "tq_encode_dense");
}

int tq_kv_fetch(const tq_qweight* w, void* out, tq_dtype out_dtype, void* stream) {
  WeightArgs a{};
  int rc = check_weight(w, &a, /*allow256=*/true);
  if (rc != TQ_OK) return rc;
  if (!kv_fetch_supported(a.K, a.levels))
    return fail(TQ_ERR_UNSUPPORTED,
                "tq_kv_fetch needs a bit format (4, 8, 16 or 256 levels) and K a power of two "
                "in [64, 2048] (got %d levels, K=%d)", a.levels, a.K);
  if (!valid_dtype(out_dtype)) return fail(TQ_ERR_ARG, "bad dtype");
  const int64_t rows = static_cast<int64_t>(a.E) * a.N;
  if (rows == 0) return TQ_OK;
  if (!out) return fail(TQ_ERR_ARG, "out is NULL");
  if (!aligned(out, 16)) return fail(TQ_ERR_ALIGN, "out must be 16-byte aligned");
  return hip_status(launch_kv_fetch(a, rows, out, out_dtype, static_cast<hipStream_t>(stream)),
                    "tq_kv_fetch");
}

int tq_dequant(const tq_qweight* w, const int32_t* ids, int64_t n, void* out,
               tq_dtype out_dtype, void* stream) {
  WeightArgs a{};
  int rc = check_weight(w, &a, false, /*rotated=*/true);
  if (rc != TQ_OK) return rc;
  if (!valid_dtype(out_dtype)) return fail(TQ_ERR_ARG, "bad dtype");
  if (n < 0 || n > 65535) return fail(TQ_ERR_ARG, "n must be in [0, 65535]");
  if (!ids && n > a.E) return fail(TQ_ERR_ARG, "without ids n must be at most E");
  if (n == 0 || a.N == 0) return TQ_OK;
  if (ids && !aligned(ids, 4)) return fail(TQ_ERR_ALIGN, "ids misaligned");
  if (!out) return fail(TQ_ERR_ARG, "out is NULL");
  if (!aligned(out, 16)) return fail(TQ_ERR_ALIGN, "out must be 16-byte aligned");
  return hip_status(launch_dequant(a, ids, static_cast<int>(n), out, out_dtype,
                                   static_cast<hipStream_t>(stream)),
                    "tq_dequant");
}

int tq_gather_qmm(const tq_qweight* w, const void* x, tq_dtype x_dtype, int64_t T,
                  const int32_t* row_token, const int32_t* expert_offsets, int64_t M, void* y,
                  tq_dtype y_dtype, uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  WeightArgs a{};
  int rc = check_weight(w, &a, false, (flags & TQ_X_ROTATED) != 0);
  if (rc != TQ_OK) return rc;
  if (T < 0 || M < 0 || M > (1ll << 31) - 1 || T > (1ll << 31) - 1)
    return fail(TQ_ERR_ARG, "T and M must be in [0, 2^31)");
  rc = check_io(x, x_dtype, y, y_dtype, M > 0 && a.N > 0);
  if (rc != TQ_OK) return rc;
  if (M == 0 || a.N == 0) return TQ_OK;
  if (T == 0) return fail(TQ_ERR_ARG, "T must be > 0 when M > 0");
  if (!row_token || !expert_offsets) return fail(TQ_ERR_ARG, "row_token and expert_offsets needed");
  if (!aligned(row_token, 4) || !aligned(expert_offsets, 4))
    return fail(TQ_ERR_ALIGN, "row_token/expert_offsets misaligned");
  const bool rotated = (flags & TQ_X_ROTATED) != 0;
  if (rotated && x_dtype == TQ_BF16 && !aligned(x, 16))
    return fail(TQ_ERR_ALIGN, "rotated bf16 x must be 16-byte aligned");
  const size_t need = gather_qmm_workspace(a, M, T);
  if (!ws || ws_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned(ws, 256)) return fail(TQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  return hip_status(launch_gather_qmm(a, x, x_dtype, T, row_token, expert_offsets, M, rotated, y,
                                      y_dtype, ws, static_cast<hipStream_t>(stream)),
                    "tq_gather_qmm");
}

int tq_gather_qmm_pair(const tq_qweight* w1, const tq_qweight* w2, const void* x,
                       tq_dtype x_dtype, int64_t T, const int32_t* row_token,
                       const int32_t* expert_offsets, int64_t M, void* y, tq_dtype y_dtype,
                       uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  const bool rotated = (flags & TQ_X_ROTATED) != 0;
  WeightArgs a{}, b{};
  int rc = check_weight(w1, &a, false, rotated);
  if (rc != TQ_OK) return rc;
  rc = check_weight(w2, &b, false, rotated);
  if (rc != TQ_OK) return rc;
  if (a.levels != b.levels || a.group != b.group || a.K != b.K || a.N != b.N || a.E != b.E)
    return fail(TQ_ERR_ARG, "tq_gather_qmm_pair: the two weights differ in format or shape");
  if (!rotated && w1->signs != w2->signs)
    return fail(TQ_ERR_ARG, "tq_gather_qmm_pair: the two weights must share one signs array");
  if (T < 0 || M < 0 || M > (1ll << 30) - 1 || T > (1ll << 31) - 1)
    return fail(TQ_ERR_ARG, "T must be in [0, 2^31) and M in [0, 2^30)");
  rc = check_io(x, x_dtype, y, y_dtype, M > 0 && a.N > 0);
  if (rc != TQ_OK) return rc;
  if (M == 0 || a.N == 0) return TQ_OK;
  if (T == 0) return fail(TQ_ERR_ARG, "T must be > 0 when M > 0");
  if (!row_token || !expert_offsets) return fail(TQ_ERR_ARG, "row_token and expert_offsets needed");
  if (!aligned(row_token, 4) || !aligned(expert_offsets, 4))
    return fail(TQ_ERR_ALIGN, "row_token/expert_offsets misaligned");
  if (rotated && x_dtype == TQ_BF16 && !aligned(x, 16))
    return fail(TQ_ERR_ALIGN, "rotated bf16 x must be 16-byte aligned");
  const size_t need = gather_qmm_workspace(a, M, T);
  if (!ws || ws_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned(ws, 256)) return fail(TQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  return hip_status(launch_gather_qmm(a, x, x_dtype, T, row_token, expert_offsets, M, rotated, y,
                                      y_dtype, ws, static_cast<hipStream_t>(stream), &b),
                    "tq_gather_qmm_pair");
}

// ---- expert cache ------------------------------------------------------------------------
// Host state (caller-owned memory): a header, then slot_expert[slots] (int32, -1 = empty),
// slot_tick[slots] (uint64, the call that last used the slot), expert_slot[E] (int32, -1 =
// not resident).
namespace {
constexpr uint64_t kCacheMagic = 0x7471657863616368ull;  // "tqexcach"
struct CacheHeader {
  uint64_t magic;
  int64_t E;
  uint64_t tick;
  int64_t hits, misses;
  int32_t slots, pad;
};
size_t align8(size_t n) { return (n + 7) & ~static_cast<size_t>(7); }
size_t cache_bytes(int64_t slots, int64_t E) {
  return sizeof(CacheHeader) + align8(static_cast<size_t>(slots) * 4) +
         static_cast<size_t>(slots) * 8 + align8(static_cast<size_t>(E) * 4);
}
struct CacheView {
  CacheHeader* h;
  int32_t* slot_expert;
  uint64_t* slot_tick;
  int32_t* expert_slot;
};
CacheView cache_view(void* state) {
  CacheView v{};
  v.h = static_cast<CacheHeader*>(state);
  char* p = static_cast<char*>(state) + sizeof(CacheHeader);
  v.slot_expert = reinterpret_cast<int32_t*>(p);
  p += align8(static_cast<size_t>(v.h->slots) * 4);
  v.slot_tick = reinterpret_cast<uint64_t*>(p);
  p += static_cast<size_t>(v.h->slots) * 8;
  v.expert_slot = reinterpret_cast<int32_t*>(p);
  return v;
}
}  // namespace

size_t tq_expert_cache_bytes(int32_t slots, int64_t E) {
  if (slots < 1 || slots > 8192 || E < 1 || E > 8192) return SIZE_MAX;
  return cache_bytes(slots, E);
}

int tq_expert_cache_init(void* state, size_t state_bytes, int32_t slots, int64_t E) {
  if (slots < 1 || slots > 8192 || E < 1 || E > 8192)
    return fail(TQ_ERR_ARG, "slots and E must be in [1, 8192]");
  if (!state) return fail(TQ_ERR_ARG, "state is NULL");
  if (!aligned(state, 8)) return fail(TQ_ERR_ALIGN, "state must be 8-byte aligned");
  if (state_bytes < cache_bytes(slots, E))
    return fail(TQ_ERR_ARG, "state of %zu bytes needed (got %zu)", cache_bytes(slots, E),
                state_bytes);
  CacheHeader* h = static_cast<CacheHeader*>(state);
  std::memset(h, 0, sizeof *h);
  h->magic = kCacheMagic;
  h->E = E;
  h->slots = slots;
  CacheView v = cache_view(state);
  for (int32_t s = 0; s < slots; ++s) {
    v.slot_expert[s] = -1;
    v.slot_tick[s] = 0;
  }
  for (int64_t e = 0; e < E; ++e) v.expert_slot[e] = -1;
  return TQ_OK;
}

int tq_expert_cache_fetch(void* state, const tq_qweight* host, const tq_qweight* pool,
                          const int32_t* ids_host, int32_t n, int32_t* slot_ids_dev,
                          int32_t* slot_ids_host, int32_t* copied, void* stream,
                          void* copy_stream) {
  if (!state || !aligned(state, 8) || static_cast<CacheHeader*>(state)->magic != kCacheMagic)
    return fail(TQ_ERR_ARG, "state was not set up by tq_expert_cache_init");
  CacheView v = cache_view(state);
  WeightArgs hw{}, pw{};
  int rc = check_weight(host, &hw);
  if (rc != TQ_OK) return rc;
  rc = check_weight(pool, &pw);
  if (rc != TQ_OK) return rc;
  if (hw.levels != pw.levels || hw.group != pw.group || hw.K != pw.K || hw.N != pw.N)
    return fail(TQ_ERR_ARG, "host weight and slot pool differ in levels, group, K or N");
  if (hw.E != v.h->E || pw.E != v.h->slots)
    return fail(TQ_ERR_ARG, "host weight must have the cache's E experts and the pool its slots");
  if (n < 0 || n > kMaxSlotIds) return fail(TQ_ERR_ARG, "n must be in [0, %d]", kMaxSlotIds);
  if (n > 0 && (!ids_host || !slot_ids_dev)) return fail(TQ_ERR_ARG, "ids_host and slot_ids_dev needed");
  if (n > 0 && !aligned(slot_ids_dev, 4)) return fail(TQ_ERR_ALIGN, "slot_ids_dev misaligned");
  for (int32_t k = 0; k < n; ++k)
    if (ids_host[k] < 0 || ids_host[k] >= hw.E)
      return fail(TQ_ERR_ARG, "ids_host[%d] = %d is outside [0, %d)", k, ids_host[k], hw.E);
  // distinct experts of this call must fit the pool
  {
    int32_t distinct = 0;
    for (int32_t k = 0; k < n; ++k) {
      bool seen = false;
      for (int32_t j = 0; j < k && !seen; ++j) seen = ids_host[j] == ids_host[k];
      distinct += seen ? 0 : 1;
    }
    if (distinct > pw.E)
      return fail(TQ_ERR_ARG, "%d distinct experts do not fit %d slots", distinct, pw.E);
  }
  // residency: hits first (so that no expert this call needs is evicted), then misses take
  // the least recently used slots that this call does not use
  const uint64_t tick = ++v.h->tick;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t s = v.expert_slot[ids_host[k]];
    if (s >= 0) v.slot_tick[s] = tick;
  }
  int32_t load_e[kMaxSlotIds], load_s[kMaxSlotIds];
  int32_t nload = 0;
  SlotIds out{};
  out.n = n;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t e = ids_host[k];
    int32_t s = v.expert_slot[e];
    if (s < 0) {
      int32_t best = -1;
      for (int32_t c = 0; c < pw.E; ++c) {
        if (v.slot_tick[c] == tick) continue;
        if (best < 0 || v.slot_tick[c] < v.slot_tick[best]) best = c;
      }
      s = best;  // exists: distinct experts <= slots
      if (v.slot_expert[s] >= 0) v.expert_slot[v.slot_expert[s]] = -1;
      v.slot_expert[s] = e;
      v.expert_slot[e] = s;
      v.slot_tick[s] = tick;
      load_e[nload] = e;
      load_s[nload] = s;
      ++nload;
      ++v.h->misses;
    } else {
      ++v.h->hits;
    }
    out.v[k] = s;
    if (slot_ids_host) slot_ids_host[k] = s;
  }
  if (copied) *copied = nload;
  const hipStream_t cs = static_cast<hipStream_t>(stream);
  const hipStream_t xs = copy_stream ? static_cast<hipStream_t>(copy_stream) : cs;
  hipError_t e = hipSuccess;
  if (nload > 0) {
    const size_t cb = static_cast<size_t>(hw.N) * hw.wpr * 4;
    const size_t sb = static_cast<size_t>(hw.N) * (hw.K / hw.group) * 2;
    hipEvent_t entry = nullptr, done = nullptr;
    // a slot being refilled may still be read by work already on `stream`
    if (xs != cs) {
      e = hipEventCreateWithFlags(&entry, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventRecord(entry, cs);
      if (e == hipSuccess) e = hipStreamWaitEvent(xs, entry, 0);
    }
    for (int32_t i = 0; i < nload && e == hipSuccess; ++i) {
      const char* hc = reinterpret_cast<const char*>(hw.codes) + cb * load_e[i];
      const char* hs = reinterpret_cast<const char*>(hw.scales) + sb * load_e[i];
      char* dc = reinterpret_cast<char*>(const_cast<uint32_t*>(pw.codes)) + cb * load_s[i];
      char* ds = reinterpret_cast<char*>(const_cast<uint16_t*>(pw.scales)) + sb * load_s[i];
      e = hipMemcpyAsync(dc, hc, cb, hipMemcpyHostToDevice, xs);
      if (e == hipSuccess) e = hipMemcpyAsync(ds, hs, sb, hipMemcpyHostToDevice, xs);
    }
    if (xs != cs && e == hipSuccess) {
      e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventRecord(done, xs);
      if (e == hipSuccess) e = hipStreamWaitEvent(cs, done, 0);
    }
    if (entry) (void)hipEventDestroy(entry);
    if (done) (void)hipEventDestroy(done);
  }
  if (e == hipSuccess) e = launch_put_ids(out, slot_ids_dev, cs);
  return hip_status(e, "tq_expert_cache_fetch");
}

int tq_expert_cache_stats(const void* state, int64_t* hits, int64_t* misses) {
  if (!state || !aligned(state, 8) || static_cast<const CacheHeader*>(state)->magic != kCacheMagic)
    return fail(TQ_ERR_ARG, "state was not set up by tq_expert_cache_init");
  const CacheHeader* h = static_cast<const CacheHeader*>(state);
  if (hits) *hits = h->hits;
  if (misses) *misses = h->misses;
  return TQ_OK;
}

const char* tq_last_error(void) { return g_err.c_str(); }

}  // extern "C"
