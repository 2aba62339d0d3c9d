// capi.hip -- the C ABI of libqlora (declared in include/qlora.h): host-side
// validation, workspace layout and kernel orchestration on the caller's
// stream.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "qlora.h"

#pragma clang fp contract(off)

namespace qlora {

// ------------------------------------------------------------ NF4 table --
//
// Inverse of the standard normal CDF: Wichura's algorithm AS 241 (PPND16,
// Applied Statistics 37 (1988) 477-484), accurate to about 1e-16 relative.
static double ppnd16(double p) {
  const double q = p - 0.5;
  if (std::fabs(q) <= 0.425) {
    const double r = 0.180625 - q * q;
    const double num =
        (((((((2509.0809287301226727 * r + 33430.575583588128105) * r + 67265.770927008700853) * r +
             45921.953931549871457) * r + 13731.693765509461125) * r + 1971.5909503065514427) * r +
          133.14166789178437745) * r + 3.387132872796366608);
    const double den =
        (((((((5226.495278852545925 * r + 28729.085735721942674) * r + 39307.89580009271061) * r +
             21213.794301586595867) * r + 5394.1960214247511077) * r + 687.1870074920579083) * r +
          42.313330701600911252) * r + 1.0);
    return q * num / den;
  }
  double r = q < 0 ? p : 1.0 - p;
  r = std::sqrt(-std::log(r));
  double val;
  if (r <= 5.0) {
    r -= 1.6;
    const double num =
        (((((((7.7454501427834140764e-4 * r + 0.0227238449892691845833) * r + 0.24178072517745061177) * r +
             1.27045825245236838258) * r + 3.64784832476320460504) * r + 5.7694972214606914055) * r +
          4.6303378461565452959) * r + 1.42343711074968357734);
    const double den =
        (((((((1.05075007164441684324e-9 * r + 5.475938084995344946e-4) * r + 0.0151986665636164571966) * r +
             0.14810397642748007459) * r + 0.68976733498510000455) * r + 1.6763848301838038494) * r +
          2.05319162663775882187) * r + 1.0);
    val = num / den;
  } else {
    r -= 5.0;
    const double num =
        (((((((2.01033439929228813265e-7 * r + 2.71155556874348757815e-5) * r + 0.0012426609473880784386) * r +
             0.026532189526576123093) * r + 0.29656057182850489123) * r + 1.7848265399172913358) * r +
          5.4637849111641143699) * r + 6.6579046435011037772);
    const double den =
        (((((((2.04426310338993978564e-15 * r + 1.4215117583164458887e-7) * r + 1.8463183175100546818e-5) * r +
             7.868691311456132591e-4) * r + 0.0148753612908506148525) * r + 0.13692988092273580531) * r +
          0.59983220655588793769) * r + 1.0);
    val = num / den;
  }
  return q < 0 ? -val : val;
}

// The 16 levels: standard-normal quantiles at equally spaced probabilities,
// 2^(k-1) = 8 on the negative side and 2^(k-1)+1 = 9 on the positive side
// (both containing zero, one zero dropped), normalised by the outermost
// quantile (page "LoRA and QLoRA fine-tuning: mechanics, ...", paragraph
// "4-bit NormalFloat").  The probability grid runs from 1/2 to delta, the
// mean of the top-bin centre probabilities of 16-bin and 15-bin equal-mass
// grids (the pages leave the outermost probability open).
static Nf4Table build_table() {
  const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
  const double z = ppnd16(delta);
  double v[16];
  int n = 0;
  for (int j = 7; j >= 1; --j) v[n++] = -ppnd16(0.5 + j * (delta - 0.5) / 7.0) / z;
  for (int j = 0; j <= 8; ++j) v[n++] = ppnd16(0.5 + j * (delta - 0.5) / 8.0) / z;
  Nf4Table t;
  for (int i = 0; i < 16; ++i) t.q[i] = (float)v[i];
  for (int i = 0; i < 15; ++i) t.mid[i] = (float)(((double)t.q[i] + (double)t.q[i + 1]) / 2.0);
  t.mid[15] = 0.0f;
  return t;
}

const Nf4Table& nf4_table() {
  static const Nf4Table t = build_table();  // thread-safe one-time init
  return t;
}

// ----------------------------------------------------------- validation --

constexpr int64_t kMaxElems = (int64_t)1 << 31;

static bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static int check_dk(int64_t d, int64_t k) {
  if (d < 16 || k < 64 || (k % 64) != 0 || (d % 16) != 0) return QLORA_ERR_SHAPE;
  if (d >= kMaxElems || k >= kMaxElems || d * k >= kMaxElems) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

static int check_mdk(int64_t M, int64_t d, int64_t k) {
  int s = check_dk(d, k);
  if (s) return s;
  if (M < 0 || M >= kMaxElems || M * k >= kMaxElems || M * d >= kMaxElems) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

static int check_nf4(const qlora_nf4_t* w) {
  if (w == nullptr || w->codes == nullptr || w->absmax_q == nullptr || w->absmax_scale == nullptr ||
      w->absmax_mean == nullptr)
    return QLORA_ERR_NULL;
  return QLORA_OK;
}

static int check_nf4_align(const qlora_nf4_t* w) {
  // codes are read 16 bytes at a time; the other buffers element-wise
  if (!aligned16(w->codes) || ((uintptr_t)w->absmax_scale & 3u) || ((uintptr_t)w->absmax_mean & 3u))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

static size_t nf4_codes_bytes(const qlora_nf4_t* w) { return (size_t)(w->d * w->k / 2); }

// Overlap of an output region with any of the four NF4 buffers (nsec
// means when the rows form sections).
static bool overlaps_nf4(const void* p, size_t n, const qlora_nf4_t* w, int nsec = 1) {
  const int64_t nb = w->d * w->k / 64;
  return overlaps(p, n, w->codes, nf4_codes_bytes(w)) || overlaps(p, n, w->absmax_q, (size_t)nb) ||
         overlaps(p, n, w->absmax_scale, (size_t)((nb + 255) / 256) * 4) ||
         overlaps(p, n, w->absmax_mean, 4 * (size_t)nsec);
}

// Row sections: nsec equal blocks of rows, each a whole number of 256-row
// tiles (so no tile, block or second-level group straddles two sections),
// each with r <= kMaxRank adapter ranks, a multiple of 16.
static int check_sections(const qlora_nf4_t* w, int32_t nsec, int32_t r) {
  if (nsec < 1 || nsec > kMaxSections || w->d % nsec != 0) return QLORA_ERR_SHAPE;
  if (nsec == 1) return QLORA_OK;
  if ((w->d / nsec) % 256 != 0) return QLORA_ERR_SHAPE;
  if (r % 16 != 0) return QLORA_ERR_RANK;
  return QLORA_OK;
}

static int check_rank_alpha(int32_t r, float alpha) {
  if (r < 0 || r > kMaxRank) return QLORA_ERR_RANK;
  if (r > 0 && !std::isfinite(alpha)) return QLORA_ERR_ALPHA;
  return QLORA_OK;
}

static float lora_scale(int32_t r, float alpha) { return r > 0 ? alpha / (float)r : 0.0f; }

static Nf4Dev dev_view(const qlora_nf4_t* w, int nsec = 1) {
  return Nf4Dev{w->codes, w->absmax_q, w->absmax_scale, w->absmax_mean, (int)w->d, (int)w->k,
                (int)(w->d / nsec)};
}

// Workspace carving: the size queries run the same layout with no base.
struct Carve {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t bytes) {
    off = (size_t)align_up((int64_t)off, 256);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

struct FwdWs {
  uint16_t* T = nullptr;
  float* proj = nullptr;
  float* dec = nullptr;
  uint16_t* Xd = nullptr;  // LoRA dropout: the dropped adapter input
  size_t bytes = 0;
};

static FwdWs carve_forward(void* ws, int M, int d, int k, int r, bool drop = false) {
  Carve c{reinterpret_cast<char*>(ws)};
  FwdWs o;
  if (drop && r > 0) o.Xd = c.take<uint16_t>((size_t)M * k * 2);
  const int rp = r > 0 ? padded_rank(r) : 0;
  if (forward_uses_decode(M, d, k)) {
    o.dec = c.take<float>(forward_gemm_ws_bytes(M, d, k, r, drop && r > 0));
  } else {
    if (r > 0) {
      o.T = c.take<uint16_t>((size_t)M * rp * 2);
      o.proj = c.take<float>(lora_proj_ws_bytes(M, k, r, 1, false));
    }
    const size_t split = forward_gemm_ws_bytes(M, d, k, r);  // split-K partials of the token-rich GEMM
    if (split > 0) o.dec = c.take<float>(split);
  }
  o.bytes = c.off;
  return o;
}

struct BwdWs {
  uint16_t *Bt = nullptr, *At = nullptr, *U = nullptr, *Ut = nullptr, *Tt = nullptr, *Tscr = nullptr;
  uint16_t* Xd = nullptr;  // LoRA dropout: the dropped adapter input
  float* proj = nullptr;
  float* dxpart = nullptr;  // split-K partials of dX
  size_t bytes = 0;
};

static size_t max2(size_t a, size_t b) { return a > b ? a : b; }

static BwdWs carve_backward(void* ws, int M, int d, int k, int r, bool drop = false) {
  Carve c{reinterpret_cast<char*>(ws)};
  BwdWs o;
  if (r > 0) {
    if (drop) o.Xd = c.take<uint16_t>((size_t)M * k * 2);
    const int rp = padded_rank(r), ldt = tsave_ld(M);
    o.Bt = c.take<uint16_t>((size_t)rp * d * 2);
    o.At = c.take<uint16_t>((size_t)k * rp * 2);
    o.U = c.take<uint16_t>((size_t)M * rp * 2);
    o.Ut = c.take<uint16_t>((size_t)r * ldt * 2);
    o.Tt = c.take<uint16_t>((size_t)r * ldt * 2);
    o.Tscr = c.take<uint16_t>((size_t)M * rp * 2);
    // U = dY B: the ranks may form up to kMaxSections sections (not known
    // here: the largest need of any valid split); T = X A^T
    size_t pu = 0;
    for (int ns = 1; ns <= kMaxSections; ++ns) pu = max2(pu, lora_proj_ws_bytes(M, d, r, ns, r % 8 == 0));
    o.proj = c.take<float>(max2(pu, lora_proj_ws_bytes(M, k, r, 1, false)));
  }
  const size_t dxp = dx_ws_bytes(M, d, k);
  if (dxp > 0) o.dxpart = c.take<float>(dxp);
  o.bytes = c.off;
  return o;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

// ------------------------------------------------------ static scratch --
//
// The workspace of qlora_backward_noalloc: one array per GPU the library
// runs on, reserved when the library's device code is loaded on that GPU
// and held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address is asked of the
// runtime once per device, with that device current, and kept in
// g_scratch_dev; kernels, copies and fills only ever see that address.
static __device__ __align__(256) char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];

// Device address of this process's scratch array on the GPU that `stream`
// belongs to (the current GPU for the null stream).
static int scratch_for_stream(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return QLORA_ERR_HIP;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return QLORA_ERR_HIP;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return QLORA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return QLORA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return QLORA_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return QLORA_OK;
}

}  // namespace qlora

using namespace qlora;

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "invalid shape (need d%16==0, k%64==0, sizes < 2^31 elements)";
    case QLORA_ERR_RANK: return "rank r must be in [0, 64]";
    case QLORA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_ALPHA: return "alpha is not finite";
    case QLORA_ERR_ALIAS: return "an output overlaps an input";
    case QLORA_ERR_HIP: return "HIP runtime or kernel launch failure";
    default: return "unknown status";
  }
}

int qlora_version(void) { return (0 << 16) | 1; }

int qlora_nf4_levels(float* out) {
  if (out == nullptr) return QLORA_ERR_NULL;
  std::memcpy(out, nf4_table().q, 16 * sizeof(float));
  return QLORA_OK;
}

int qlora_nf4_sizes(int64_t d, int64_t k, size_t* codes_bytes, size_t* absmax_q_bytes,
                    size_t* absmax_scale_bytes, size_t* absmax_mean_bytes) {
  if (int s = check_dk(d, k)) return s;
  const int64_t nb = d * k / 64;
  if (codes_bytes) *codes_bytes = (size_t)(d * k / 2);
  if (absmax_q_bytes) *absmax_q_bytes = (size_t)nb;
  if (absmax_scale_bytes) *absmax_scale_bytes = (size_t)((nb + 255) / 256) * 4;
  if (absmax_mean_bytes) *absmax_mean_bytes = 4;
  return QLORA_OK;
}

size_t qlora_quantize_workspace_bytes(int64_t d, int64_t k) {
  if (check_dk(d, k)) return 0;
  return quantize_ws_bytes(d, k);
}

int nf4_quantize(const float* W0, int64_t d, int64_t k, const qlora_nf4_t* out, void* ws,
                 size_t ws_bytes, void* stream) {
  if (W0 == nullptr) return QLORA_ERR_NULL;
  if (int s = check_nf4(out)) return s;
  if (int s = check_dk(d, k)) return s;
  if (out->d != d || out->k != k) return QLORA_ERR_SHAPE;
  if (!aligned16(W0) || !aligned16(out->codes) || !aligned16(ws) || check_nf4_align(out))
    return QLORA_ERR_ALIGN;
  const size_t need = quantize_ws_bytes(d, k);
  if (ws == nullptr || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  const size_t wbytes = (size_t)(d * k) * 4;
  if (overlaps_nf4(W0, wbytes, out) || overlaps_nf4(ws, need, out) || overlaps(ws, need, W0, wbytes))
    return QLORA_ERR_ALIAS;
  {
    // the four outputs must not overlap each other
    const int64_t nb = d * k / 64;
    const void* p[4] = {out->codes, out->absmax_q, out->absmax_scale, out->absmax_mean};
    const size_t n[4] = {(size_t)(d * k / 2), (size_t)nb, (size_t)((nb + 255) / 256) * 4, 4};
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (overlaps(p[i], n[i], p[j], n[j])) return QLORA_ERR_ALIAS;
  }
  return hip_status(launch_quantize(W0, d, k, nf4_table(), out->codes, out->absmax_q,
                                    out->absmax_scale, out->absmax_mean, ws,
                                    reinterpret_cast<hipStream_t>(stream)));
}

size_t qlora_tsave_bytes(int64_t M, int32_t r) {
  if (M < 0 || M >= kMaxElems || r < 0 || r > kMaxSections * kMaxRank) return 0;
  return (size_t)r * tsave_ld((int)M) * 2;
}

size_t qlora_forward_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r) {
  if (check_mdk(M, d, k) || r < 0 || r > kMaxSections * kMaxRank || M == 0) return 0;
  return carve_forward(nullptr, (int)M, (int)d, (int)k, r).bytes;
}

// LoRA dropout (keep != nullptr): keep is M x k bytes, p in [0, 1), and
// the adapter path reads Xd = bf16(x / (1 - p)) where keep != 0, else 0.
static int check_dropout(const uint8_t* keep, float p) {
  if (keep == nullptr) return QLORA_ERR_NULL;
  if (!(p >= 0.0f && p < 1.0f)) return QLORA_ERR_ALPHA;
  if (((uintptr_t)keep & 15u) != 0) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}
static float dropout_scale(float p) { return 1.0f / (1.0f - p); }

static int forward_impl(const uint16_t* X, int64_t M, const qlora_nf4_t* W0, int32_t nsec, const uint16_t* A,
                        const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* T_save, void* ws,
                        size_t ws_bytes, void* stream, const uint8_t* keep = nullptr, float p = 0.0f,
                        uint16_t* Xd_save = nullptr) {
  if (int s = check_nf4(W0)) return s;
  if (X == nullptr || Y == nullptr) return QLORA_ERR_NULL;
  if (r > 0 && (A == nullptr || B == nullptr)) return QLORA_ERR_NULL;
  const int64_t d = W0->d, k = W0->k;
  if (int s = check_mdk(M, d, k)) return s;
  if (int s = check_rank_alpha(r, alpha)) return s;
  if (int s = check_sections(W0, nsec, r)) return s;
  if (M == 0) return QLORA_OK;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(ws) || check_nf4_align(W0)) return QLORA_ERR_ALIGN;
  if (r > 0 && (!aligned16(A) || !aligned16(B) || !aligned16(T_save))) return QLORA_ERR_ALIGN;
  const int rt = nsec * r;  // ranks of T over all sections
  const bool drop = keep != nullptr && r > 0;
  const FwdWs need = carve_forward(nullptr, (int)M, (int)d, (int)k, rt, drop);
  if (need.bytes > 0 && (ws == nullptr || ws_bytes < need.bytes)) return QLORA_ERR_WORKSPACE;
  const size_t xb = (size_t)(M * k) * 2, yb = (size_t)(M * d) * 2;
  const size_t ab = (size_t)rt * k * 2, bb = (size_t)d * r * 2;
  const size_t tb = (r > 0 && T_save) ? qlora_tsave_bytes(M, rt) : 0;
  if (overlaps(Y, yb, X, xb) || overlaps_nf4(Y, yb, W0, nsec) || overlaps(Y, yb, ws, need.bytes))
    return QLORA_ERR_ALIAS;
  if (r > 0) {
    if (overlaps(Y, yb, A, ab) || overlaps(Y, yb, B, bb) || overlaps(Y, yb, T_save, tb) ||
        overlaps(T_save, tb, X, xb) || overlaps(T_save, tb, A, ab) || overlaps(T_save, tb, B, bb) ||
        overlaps_nf4(T_save, tb, W0, nsec) || overlaps(T_save, tb, ws, need.bytes) ||
        overlaps(ws, need.bytes, A, ab) || overlaps(ws, need.bytes, B, bb))
      return QLORA_ERR_ALIAS;
  }
  if (overlaps(ws, need.bytes, X, xb) || overlaps_nf4(ws, need.bytes, W0, nsec)) return QLORA_ERR_ALIAS;
  if (drop && (overlaps(Y, yb, keep, (size_t)(M * k)) || overlaps(T_save, tb, keep, (size_t)(M * k)) ||
               overlaps(ws, need.bytes, keep, (size_t)(M * k))))
    return QLORA_ERR_ALIAS;
  if (drop && Xd_save != nullptr) {
    if (!aligned16(Xd_save)) return QLORA_ERR_ALIGN;
    const void* other[8] = {X, Y, A, B, T_save, ws, keep, nullptr};
    const size_t on[8] = {xb, yb, ab, bb, tb, need.bytes, (size_t)(M * k), 0};
    for (int i = 0; i < 7; ++i)
      if (overlaps(Xd_save, xb, other[i], on[i])) return QLORA_ERR_ALIAS;
    if (overlaps_nf4(Xd_save, xb, W0, nsec)) return QLORA_ERR_ALIAS;
  }

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const FwdWs w = carve_forward(ws, (int)M, (int)d, (int)k, rt, drop);
  const Nf4Dev wd = dev_view(W0, nsec);
  const float s = lora_scale(r, alpha);
  const Nf4Table& tab = nf4_table();
  const int ldt = tsave_ld((int)M);
  hipError_t e = hipSuccess;
  const uint16_t* Xa = X;  // the adapter path's input
  if (drop) {
    uint16_t* xd = Xd_save != nullptr ? Xd_save : w.Xd;
    e = launch_drop_input(X, keep, M * k, dropout_scale(p), xd, st);
    Xa = xd;
  }
  if (e != hipSuccess) return hip_status(e);
  if (forward_uses_decode((int)M, (int)d, (int)k)) {
    e = launch_forward_decode(X, (int)M, wd, nsec, A, B, r, s, Y, r > 0 ? T_save : nullptr, ldt, w.dec, tab, st,
                              nullptr, Xa);
  } else {
    if (r > 0)
      e = launch_lora_proj(Xa, (int)M, (int)k, A, false, rt, 1, w.T, T_save, ldt, w.proj, nullptr, 0, 0.0f, nullptr,
                           st);
    if (e == hipSuccess) e = launch_forward(X, (int)M, wd, nsec, w.T, B, r, s, Y, tab, st, w.dec);
  }
  return hip_status(e);
}

int qlora_forward(const uint16_t* X, int64_t M, const qlora_nf4_t* W0, const uint16_t* A,
                  const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* T_save, void* ws,
                  size_t ws_bytes, void* stream) {
  return forward_impl(X, M, W0, 1, A, B, r, alpha, Y, T_save, ws, ws_bytes, stream);
}

size_t qlora_forward_dropout_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r) {
  if (check_mdk(M, d, k) || r < 0 || r > kMaxRank || M == 0) return 0;
  return carve_forward(nullptr, (int)M, (int)d, (int)k, r, true).bytes;
}

int qlora_forward_dropout(const uint16_t* X, int64_t M, const qlora_nf4_t* W0, const uint16_t* A,
                          const uint16_t* B, int32_t r, float alpha, const uint8_t* keep, float p, uint16_t* Y,
                          uint16_t* T_save, uint16_t* Xd_save, void* ws, size_t ws_bytes, void* stream) {
  if (r > 0 && M > 0) {
    if (int s = check_dropout(keep, p)) return s;
  }
  return forward_impl(X, M, W0, 1, A, B, r, alpha, Y, T_save, ws, ws_bytes, stream, r > 0 ? keep : nullptr, p,
                      Xd_save);
}

int qlora_forward_sections(const uint16_t* X, int64_t M, const qlora_nf4_t* W0, int32_t nsec,
                           const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                           uint16_t* T_save, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(X, M, W0, nsec, A, B, r, alpha, Y, T_save, ws, ws_bytes, stream);
}

// Per-token adapters: tokens go through the decode path in chunks of at
// most multi_chunk(k) (the decode kernels' token limit), every chunk
// computing T for all nad adapters' ranks.
static constexpr int kMaxAdapters = 64;
static int multi_chunk(int64_t d, int64_t k) { return forward_uses_decode(128, (int)d, (int)k) ? 128 : 64; }

size_t qlora_forward_multi_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t nad, int32_t r) {
  if (check_mdk(M, d, k) || M == 0 || nad < 1 || nad > kMaxAdapters || r < 0 || r > kMaxRank) return 0;
  const int64_t ch = multi_chunk(d, k);
  const int mc = (int)(M < ch ? M : ch);
  return forward_gemm_ws_bytes(mc, (int)d, (int)k, nad * r, true);
}

int qlora_forward_multi(const uint16_t* X, int64_t M, const qlora_nf4_t* W0, int32_t nad, const uint16_t* A,
                        const uint16_t* B, const int32_t* idx, int32_t r, float alpha, uint16_t* Y, void* ws,
                        size_t ws_bytes, void* stream) {
  if (int s = check_nf4(W0)) return s;
  if (X == nullptr || Y == nullptr) return QLORA_ERR_NULL;
  if (r > 0 && (A == nullptr || B == nullptr || idx == nullptr)) return QLORA_ERR_NULL;
  const int64_t d = W0->d, k = W0->k;
  if (int s = check_mdk(M, d, k)) return s;
  if (int s = check_rank_alpha(r, alpha)) return s;
  if (nad < 1 || nad > kMaxAdapters) return QLORA_ERR_RANK;
  if (M == 0) return QLORA_OK;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(ws) || check_nf4_align(W0)) return QLORA_ERR_ALIGN;
  if (r > 0 && (!aligned16(A) || !aligned16(B) || ((uintptr_t)idx & 3u))) return QLORA_ERR_ALIGN;
  const size_t need = qlora_forward_multi_workspace_bytes(M, d, k, nad, r);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  const size_t xb = (size_t)(M * k) * 2, yb = (size_t)(M * d) * 2;
  const size_t ab = (size_t)nad * r * k * 2, bb = (size_t)nad * d * r * 2, ib = (size_t)M * 4;
  if (overlaps(Y, yb, X, xb) || overlaps_nf4(Y, yb, W0) || overlaps(Y, yb, ws, need)) return QLORA_ERR_ALIAS;
  if (r > 0 && (overlaps(Y, yb, A, ab) || overlaps(Y, yb, B, bb) || overlaps(Y, yb, idx, ib) ||
                overlaps(ws, need, A, ab) || overlaps(ws, need, B, bb) || overlaps(ws, need, idx, ib)))
    return QLORA_ERR_ALIAS;
  if (overlaps(ws, need, X, xb) || overlaps_nf4(ws, need, W0)) return QLORA_ERR_ALIAS;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Nf4Dev wd = dev_view(W0);
  const float s = lora_scale(r, alpha);
  const Nf4Table& tab = nf4_table();
  hipError_t e = hipSuccess;
  const int64_t ch = multi_chunk(d, k);
  for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += ch) {
    const int mc = (int)(M - m0 < ch ? M - m0 : ch);
    e = launch_forward_decode(X + m0 * k, mc, wd, r > 0 ? nad : 1, A, B, r, s, Y + m0 * d, nullptr, 0,
                              reinterpret_cast<float*>(ws), tab, st, r > 0 ? idx + m0 : nullptr);
  }
  return hip_status(e);
}

size_t qlora_backward_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r) {
  if (check_mdk(M, d, k) || r < 0 || r > kMaxSections * kMaxRank || M == 0) return 0;
  return carve_backward(nullptr, (int)M, (int)d, (int)k, r).bytes;
}

// noalloc: the workspace is the library's static scratch array of the
// stream's GPU, looked up after every argument has been validated (ws and
// ws_bytes are then ignored).
static int backward_impl(const uint16_t* dY, const uint16_t* X, int64_t M, const qlora_nf4_t* W0, int32_t nsec,
                         const uint16_t* A, const uint16_t* B, int32_t r, float alpha, const uint16_t* T_saved,
                         uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws, size_t ws_bytes, void* stream,
                         const uint8_t* keep = nullptr, float p = 0.0f, const uint16_t* Xd_saved = nullptr,
                         bool noalloc = false) {
  if (noalloc) {
    ws = nullptr;
    ws_bytes = 0;
  }
  if (int s = check_nf4(W0)) return s;
  if (dY == nullptr || X == nullptr) return QLORA_ERR_NULL;
  if (r > 0 && (A == nullptr || B == nullptr || dA == nullptr || dB == nullptr)) return QLORA_ERR_NULL;
  const int64_t d = W0->d, k = W0->k;
  if (int s = check_mdk(M, d, k)) return s;
  if (int s = check_rank_alpha(r, alpha)) return s;
  if (int s = check_sections(W0, nsec, r)) return s;
  if (M == 0) return QLORA_OK;
  if (!aligned16(dY) || !aligned16(X) || !aligned16(dX) || !aligned16(ws) || check_nf4_align(W0))
    return QLORA_ERR_ALIGN;
  if (r > 0 && (!aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB) ||
                !aligned16(T_saved)))
    return QLORA_ERR_ALIGN;
  const int rt = nsec * r;  // ranks of T and U over all sections
  const bool drop = keep != nullptr && r > 0;
  const BwdWs need = carve_backward(nullptr, (int)M, (int)d, (int)k, rt, drop);
  if (noalloc) {
    if (need.bytes > QLORA_NOALLOC_SCRATCH_BYTES) return QLORA_ERR_WORKSPACE;
  } else if (need.bytes > 0 && (ws == nullptr || ws_bytes < need.bytes)) {
    return QLORA_ERR_WORKSPACE;
  }

  const size_t xb = (size_t)(M * k) * 2, yb = (size_t)(M * d) * 2;
  const size_t ab = (size_t)rt * k * 2, bb = (size_t)d * r * 2;
  const size_t tb = (r > 0 && T_saved) ? qlora_tsave_bytes(M, rt) : 0;
  const void* in_p[6] = {dY, X, A, B, T_saved, ws};
  const size_t in_n[6] = {yb, xb, r > 0 ? ab : 0, r > 0 ? bb : 0, tb, need.bytes};
  void* out_p[3] = {dX, r > 0 ? dA : nullptr, r > 0 ? dB : nullptr};
  const size_t out_n[3] = {dX ? xb : 0, ab, bb};
  for (int i = 0; i < 3; ++i) {
    if (overlaps_nf4(out_p[i], out_n[i], W0, nsec)) return QLORA_ERR_ALIAS;
    for (int j = 0; j < 6; ++j)
      if (overlaps(out_p[i], out_n[i], in_p[j], in_n[j])) return QLORA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(out_p[i], out_n[i], out_p[j], out_n[j])) return QLORA_ERR_ALIAS;
  }
  for (int j = 0; j < 5; ++j)
    if (overlaps(ws, need.bytes, in_p[j], in_n[j])) return QLORA_ERR_ALIAS;
  if (overlaps_nf4(ws, need.bytes, W0, nsec)) return QLORA_ERR_ALIAS;
  if (drop) {
    for (int i = 0; i < 3; ++i)
      if (overlaps(out_p[i], out_n[i], keep, (size_t)(M * k)) || overlaps(out_p[i], out_n[i], Xd_saved, xb))
        return QLORA_ERR_ALIAS;
    if (overlaps(ws, need.bytes, keep, (size_t)(M * k)) || overlaps(ws, need.bytes, Xd_saved, xb))
      return QLORA_ERR_ALIAS;
    if (!aligned16(Xd_saved)) return QLORA_ERR_ALIGN;
  }

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (noalloc && need.bytes > 0) {
    if (int sc = scratch_for_stream(st, &ws)) return sc;
  }
  const BwdWs w = carve_backward(ws, (int)M, (int)d, (int)k, rt, drop);
  const Nf4Dev wd = dev_view(W0, nsec);
  const float s = lora_scale(r, alpha);
  const Nf4Table& tab = nf4_table();
  const int ldt = tsave_ld((int)M);
  hipError_t e = hipSuccess;
  if (r > 0) {
    // U = dY B (row-major for the dX epilogue, transposed for dA); the same
    // launch writes bf16(s A)^T for the dX epilogue.  B is read as stored
    // when r is a multiple of 8, else from a transposed copy.  With
    // sections, U's ranks of section p sum over that section's columns of
    // dY only.
    if (r % 8 == 0) {
      e = launch_lora_proj(dY, (int)M, (int)d, B, true, rt, nsec, w.U, w.Ut, ldt, w.proj, A, (int)k, s, w.At, st);
    } else {
      e = launch_prep_adapters(A, B, (int)d, (int)k, r, s, nullptr, w.Bt, nullptr, st);
      if (e == hipSuccess)
        e = launch_lora_proj(dY, (int)M, (int)d, w.Bt, false, r, 1, w.U, w.Ut, ldt, w.proj, A, (int)k, s, w.At, st);
    }
  }
  // LoRA dropout: the adapter path's input is Xd (T and dA read it) and
  // dX's LoRA term is masked and scaled like the input it came from.
  const uint16_t* Xa = X;
  if (drop && Xd_saved != nullptr) {
    Xa = Xd_saved;  // the forward's dropped input, same X, mask and p
  } else if (drop && e == hipSuccess) {
    e = launch_drop_input(X, keep, M * k, dropout_scale(p), w.Xd, st);
    Xa = w.Xd;
  }
  if (e == hipSuccess && dX != nullptr)
    e = launch_dx(dY, (int)M, wd, w.U, w.At, rt, s, dX, tab, st, drop ? keep : nullptr, drop ? dropout_scale(p) : 1.0f,
                  w.dxpart);
  if (r > 0) {
    const uint16_t* Tt = T_saved;
    if (Tt == nullptr && e == hipSuccess) {
      e = launch_lora_proj(Xa, (int)M, (int)k, A, false, rt, 1, w.Tscr, w.Tt, ldt, w.proj, nullptr, 0, 0.0f, nullptr,
                           st);
      Tt = w.Tt;
    }
    if (e == hipSuccess)
      e = launch_token_reduce2(w.Ut, Xa, (int)k, dA, false, Tt, dY, (int)d, dB, true, ldt, (int)M, rt, nsec, s, st);
  }
  return hip_status(e);
}

int qlora_backward(const uint16_t* dY, const uint16_t* X, int64_t M, const qlora_nf4_t* W0,
                   const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                   const uint16_t* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws,
                   size_t ws_bytes, void* stream) {
  return backward_impl(dY, X, M, W0, 1, A, B, r, alpha, T_saved, dX, dA, dB, ws, ws_bytes, stream);
}

size_t qlora_backward_dropout_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r) {
  if (check_mdk(M, d, k) || r < 0 || r > kMaxRank || M == 0) return 0;
  return carve_backward(nullptr, (int)M, (int)d, (int)k, r, true).bytes;
}

int qlora_backward_dropout(const uint16_t* dY, const uint16_t* X, int64_t M, const qlora_nf4_t* W0,
                           const uint16_t* A, const uint16_t* B, int32_t r, float alpha, const uint8_t* keep,
                           float p, const uint16_t* T_saved, const uint16_t* Xd_saved, uint16_t* dX, uint16_t* dA,
                           uint16_t* dB, void* ws, size_t ws_bytes, void* stream) {
  if (r > 0 && M > 0) {
    if (int s = check_dropout(keep, p)) return s;
  }
  return backward_impl(dY, X, M, W0, 1, A, B, r, alpha, T_saved, dX, dA, dB, ws, ws_bytes, stream,
                       r > 0 ? keep : nullptr, p, Xd_saved);
}

int qlora_backward_noalloc(const uint16_t* dY, const uint16_t* X, int64_t M, const qlora_nf4_t* W0,
                           const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                           const uint16_t* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                           void* stream) {
  return backward_impl(dY, X, M, W0, 1, A, B, r, alpha, T_saved, dX, dA, dB, nullptr, 0, stream, nullptr, 0.0f,
                       nullptr, true);
}

int qlora_backward_sections(const uint16_t* dY, const uint16_t* X, int64_t M, const qlora_nf4_t* W0,
                            int32_t nsec, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                            const uint16_t* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws,
                            size_t ws_bytes, void* stream) {
  return backward_impl(dY, X, M, W0, nsec, A, B, r, alpha, T_saved, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_adam_step(uint16_t* P, float* W, const uint16_t* G, float* m, float* v, int64_t n, float lr,
                    float beta1, float beta2, float eps, float weight_decay, int64_t step, void* stream) {
  if (n < 0 || n >= kMaxElems) return QLORA_ERR_SHAPE;
  if (n == 0) return QLORA_OK;
  if (P == nullptr || W == nullptr || G == nullptr || m == nullptr || v == nullptr) return QLORA_ERR_NULL;
  if (!std::isfinite(lr) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) ||
      !(eps > 0.0f) || !std::isfinite(eps) || !(weight_decay >= 0.0f) || !std::isfinite(weight_decay) || step < 1)
    return QLORA_ERR_ALPHA;
  if (!aligned16(P) || !aligned16(W) || !aligned16(G) || !aligned16(m) || !aligned16(v)) return QLORA_ERR_ALIGN;
  const void* pp[5] = {P, W, G, m, v};
  const size_t pn[5] = {(size_t)n * 2, (size_t)n * 4, (size_t)n * 2, (size_t)n * 4, (size_t)n * 4};
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(pp[i], pn[i], pp[j], pn[j])) return QLORA_ERR_ALIAS;
  return hip_status(launch_adam(W, G, m, v, P, n, lr, beta1, beta2, eps, weight_decay, step,
                                reinterpret_cast<hipStream_t>(stream)));
}

static int merge_common(const qlora_nf4_t* W0, const uint16_t* Win, int64_t d, int64_t k,
                        const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* Wout,
                        bool subtract, void* stream) {
  if (int s = check_rank_alpha(r, alpha)) return s;
  const size_t wb = (size_t)(d * k) * 2, ab = (size_t)r * k * 2, bb = (size_t)d * r * 2;
  if (!aligned16(Wout) || !aligned16(Win)) return QLORA_ERR_ALIGN;
  if (r > 0 && (!aligned16(A) || !aligned16(B))) return QLORA_ERR_ALIGN;
  if (W0 && check_nf4_align(W0)) return QLORA_ERR_ALIGN;
  if (r > 0 && (overlaps(Wout, wb, A, ab) || overlaps(Wout, wb, B, bb))) return QLORA_ERR_ALIAS;
  if (W0 && overlaps_nf4(Wout, wb, W0)) return QLORA_ERR_ALIAS;
  if (Win && Win != Wout && overlaps(Wout, wb, Win, wb)) return QLORA_ERR_ALIAS;
  const float s = lora_scale(r, alpha);
  Nf4Dev wd{};
  if (W0) wd = dev_view(W0);
  return hip_status(launch_merge(wd, Win, (int)d, (int)k, A, B, r, subtract ? -s : s, Wout, nf4_table(),
                                 reinterpret_cast<hipStream_t>(stream)));
}

int lora_merge(const qlora_nf4_t* W0, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
               uint16_t* W, void* stream) {
  if (int s = check_nf4(W0)) return s;
  if (W == nullptr) return QLORA_ERR_NULL;
  if (r > 0 && (A == nullptr || B == nullptr)) return QLORA_ERR_NULL;
  if (int s = check_dk(W0->d, W0->k)) return s;
  return merge_common(W0, nullptr, W0->d, W0->k, A, B, r, alpha, W, false, stream);
}

int lora_unmerge(const uint16_t* W, int64_t d, int64_t k, const uint16_t* A, const uint16_t* B,
                 int32_t r, float alpha, uint16_t* W0_out, void* stream) {
  if (W == nullptr || W0_out == nullptr) return QLORA_ERR_NULL;
  if (r > 0 && (A == nullptr || B == nullptr)) return QLORA_ERR_NULL;
  if (int s = check_dk(d, k)) return s;
  return merge_common(nullptr, W, d, k, A, B, r, alpha, W0_out, true, stream);
}

}  // extern "C"
