// launch.hpp -- host-side launchers of the gfx950 kernels (internal to
// libqlora; the public interface is include/qlora.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include "common.hpp"

namespace qlora {

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Per-kernel timing (qlora_timing_enable): while it is on, a launch takes
// two HIP events that the dispatch itself stamps with the kernel's start and
// end (hipExtLaunchKernel), so a bracket holds the kernel alone and no marker
// packets enter the stream; while it is off, an ordinary launch.
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t st);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;
  bool active() const { return active_; }
  hipEvent_t start() const { return a_; }
  hipEvent_t stop() const { return b_; }

 private:
  bool active_;
  const char* name_;
  hipEvent_t a_, b_;
};

template <typename F, typename... Args>
inline void launch_kernel(const char* name, F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                          Args... args) {
  TimedLaunch tl(name, st);
  if (tl.active()) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, tl.start(), tl.stop(), 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  }
}

// QLORA_LAUNCH(name, stream, kernel, grid, block, shmem, stream, args...)
#define QLORA_LAUNCH(name, st, ...) ::qlora::launch_kernel((name), __VA_ARGS__)

// Device view of one NF4 weight.  Its d rows may form sections of dsec
// rows (dsec == d: one section), section p with its own mean mean[p].
struct Nf4Dev {
  const uint8_t* codes;
  const uint8_t* c2;
  const float* c1;
  const float* mean;
  int d;
  int k;
  int dsec;
};

// Padded rank used by the MFMA tiles: r rounded up to a multiple of 16.
inline int padded_rank(int r) { return (r + 15) / 16 * 16; }

const Nf4Table& nf4_table();  // built once per process (host)

// quant.hip
hipError_t launch_quantize(const float* W, int64_t d, int64_t k, const Nf4Table& t, uint8_t* codes,
                           uint8_t* c2, float* c1, float* mean, void* ws, hipStream_t st);
size_t quantize_ws_bytes(int64_t d, int64_t k);

// merge.hip: W = bf16(base + sign * s * B A); base is w~ (Win == nullptr)
// or the bf16 matrix Win.
hipError_t launch_merge(const Nf4Dev& w, const uint16_t* Win, int d, int k, const uint16_t* A,
                        const uint16_t* B, int r, float s_signed, uint16_t* Wout, const Nf4Table& t,
                        hipStream_t st);

// lora.hip: adapter preparation, skinny projections and token reductions.
hipError_t launch_prep_adapters(const uint16_t* A, const uint16_t* B, int d, int k, int r, float s,
                                uint16_t* Bp, uint16_t* Bt, uint16_t* At, hipStream_t st);
// P (M x rp) = V (M x K) L^T; L is r x K, or K x r when l_transposed (then
// r must be a multiple of 8); Pt (r x ldt) optional.  When At is given, the
// same launch also writes At = bf16(s_at A)^T (k_at x rp) from A (r x k_at).
// nsec > 1 (transposed L only): L is K x (r / nsec) and output ranks
// p*r/nsec .. of section p sum over its K rows p*K/nsec .. only.  Up to
// kMaxSections * kMaxRank ranks (more than kMaxRank only with sections, or
// with L not transposed).
hipError_t launch_lora_proj(const uint16_t* V, int M, int K, const uint16_t* L, bool l_transposed, int r,
                            int nsec, uint16_t* P, uint16_t* Pt, int ldt, float* partial,
                            const uint16_t* A_for_at, int k_at, float s_at, uint16_t* At, hipStream_t st);
// Bytes of `partial` for launch_lora_proj with the same arguments (0 when
// they are invalid or need none).
size_t lora_proj_ws_bytes(int M, int K, int r, int nsec, bool l_transposed);
// LoRA dropout of the adapter input: Xd = bf16(x * scale) where keep[i] != 0,
// else 0 (n elements, a multiple of 8).
hipError_t launch_drop_input(const uint16_t* X, const uint8_t* keep, int64_t n, float scale, uint16_t* Xd,
                             hipStream_t st);
// out = s Z^T V over tokens; Zt is r x ldz, V is M x N; out is r x N or,
// transposed, N x r.
// dA = s U^T X and dB = s dY^T T (written transposed) in one launch: two
// reductions out = s Z^T V over the M tokens (Z^T: r x ldz, tokens
// contiguous).  A null V1 launches job 0 alone.  Job 1's columns form nsec1
// sections, each reduced against its own r / nsec1 ranks of Zt1.  More than
// kMaxRank ranks (up to kMaxSections * kMaxRank) need job 1, out0 not
// transposed and out1 transposed: one launch per group of whole sections.
hipError_t launch_token_reduce2(const uint16_t* Zt0, const uint16_t* V0, int N0, uint16_t* out0, bool tr0,
                                const uint16_t* Zt1, const uint16_t* V1, int N1, uint16_t* out1, bool tr1,
                                int ldz, int M, int r, int nsec1, float s, hipStream_t st);

// gemm_fwd.hip
bool forward_uses_decode(int M, int d, int k);
// Sections (w.dsec < w.d): nsec = d / dsec row sections; T holds r ranks
// per section (row stride nsec * padded r) and A stacks nsec r x k blocks;
// B is d x r, its row n serving section n / dsec.
// part: split-K partials (forward_gemm_ws_bytes of the token-rich path;
// may be null when that size is 0).
hipError_t launch_forward(const uint16_t* X, int M, const Nf4Dev& w, int nsec, const uint16_t* T,
                          const uint16_t* B, int r, float s, uint16_t* Y, const Nf4Table& t,
                          hipStream_t st, float* part = nullptr);
// idx (device, M entries): per-token adapters; then nsec is the adapter
// count, A stacks the adapters' r x k blocks, B their d x r blocks, and
// the weight has one section.
// Xa (optional): the adapter path's input (the dropped input under LoRA
// dropout) in place of X for T.
hipError_t launch_forward_decode(const uint16_t* X, int M, const Nf4Dev& w, int nsec, const uint16_t* A,
                                 const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* Tsave,
                                 int ldt, float* part, const Nf4Table& t, hipStream_t st,
                                 const int* idx = nullptr, const uint16_t* Xa = nullptr);
// split_only: per-token adapters or LoRA dropout (those always take the
// split-K decode kernels).
size_t forward_gemm_ws_bytes(int M, int d, int k, int r, bool split_only = false);

// gemm_dx.hip
// keep (optional, M x k bytes): LoRA dropout; the LoRA term of dX[m, c] is
// multiplied by dscale where keep[m, c] != 0 and dropped elsewhere.
// part: split-K partials, dx_ws_bytes(M, d, k) bytes (may be null when 0).
hipError_t launch_dx(const uint16_t* dY, int M, const Nf4Dev& w, const uint16_t* U,
                     const uint16_t* At, int r, float s, uint16_t* dX, const Nf4Table& t,
                     hipStream_t st, const uint8_t* keep = nullptr, float dscale = 1.0f,
                     float* part = nullptr);
size_t dx_ws_bytes(int M, int d, int k);

// optim.hip: Adam step on n adapter parameters: fp32 master W, fp32 moments
// m and v updated in place, bf16 copy P written; bias corrections of step
// `step` (>= 1); wd is decoupled weight decay (0: plain Adam).
hipError_t launch_adam(float* W, const uint16_t* G, float* m, float* v, uint16_t* P, int64_t n, float lr,
                       float b1, float b2, float eps, float wd, int64_t step, hipStream_t st);

// Tile height forced through the environment (QLORA_TILE=128 or 256) for
// tests of each variant on small shapes; 0 = choose by shape.
inline int tile_override() {
  const char* e = getenv("QLORA_TILE");
  if (e == nullptr) return 0;
  const int v = atoi(e);
  return (v == 128 || v == 256) ? v : 0;
}

// Row stride (elements) of the transposed rank-r activations (T^T, U^T).
inline int tsave_ld(int M) { return (int)align_up(M, 64); }

}  // namespace qlora
