// optim.hip -- the adapter's optimiser step: Adam on A and B with an fp32
// master copy (page "Fine-Tuning on a Budget", "Why full fine-tuning costs
// so much": each trained parameter carries a 16-bit weight, a 32-bit master
// copy, Adam's two 32-bit moments and a gradient; page "LoRA and QLoRA
// fine-tuning: mechanics, ...": only the adapter has optimiser state, and
// QLoRA keeps that state in paged memory).
//
// One elementwise pass, HBM-bound: per parameter it reads the bf16 gradient
// and the fp32 master, m and v, and writes the fp32 master, m, v and the
// bf16 copy the forward reads (24 bytes).  A thread takes eight parameters
// (16-byte and 32-byte accesses); the last n % 8 go one by one.  The state
// may live in any memory the GPU can address (device memory, or pinned or
// managed memory for paged state).
#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

struct AdamArgs {
  float lr, b1, b2, eps, wd, bc1, bc2;  // bc1 = 1 - b1^t, bc2 = 1 - b2^t
};

__device__ __forceinline__ float adam_one(float g, float& w, float& m, float& v, const AdamArgs& a) {
  m = __fadd_rn(__fmul_rn(a.b1, m), __fmul_rn(1.0f - a.b1, g));
  v = __fadd_rn(__fmul_rn(a.b2, v), __fmul_rn(1.0f - a.b2, __fmul_rn(g, g)));
  const float mh = __fdiv_rn(m, a.bc1);
  const float vh = __fdiv_rn(v, a.bc2);
  const float upd = __fadd_rn(__fdiv_rn(mh, __fadd_rn(__fsqrt_rn(vh), a.eps)), __fmul_rn(a.wd, w));
  w = __fsub_rn(w, __fmul_rn(a.lr, upd));
  return w;
}

__global__ __launch_bounds__(256) void k_adam(float* __restrict__ W, const uint16_t* __restrict__ G,
                                              float* __restrict__ Mm, float* __restrict__ Vv,
                                              uint16_t* __restrict__ P, int64_t n, AdamArgs a) {
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const u32x4 g = *reinterpret_cast<const u32x4*>(G + 8 * i);
    f32x4 w[2], m[2], v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w[h] = *reinterpret_cast<const f32x4*>(W + 8 * i + 4 * h);
      m[h] = *reinterpret_cast<const f32x4*>(Mm + 8 * i + 4 * h);
      v[h] = *reinterpret_cast<const f32x4*>(Vv + 8 * i + 4 * h);
    }
    u32x4 p;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int h = q / 2, e = 2 * (q % 2);
      float w0 = w[h][e], m0 = m[h][e], v0 = v[h][e];
      float w1 = w[h][e + 1], m1 = m[h][e + 1], v1 = v[h][e + 1];
      adam_one(bf16_lo(g[q]), w0, m0, v0, a);
      adam_one(bf16_hi(g[q]), w1, m1, v1, a);
      w[h][e] = w0; m[h][e] = m0; v[h][e] = v0;
      w[h][e + 1] = w1; m[h][e + 1] = m1; v[h][e + 1] = v1;
      p[q] = pack_bf16x2(w0, w1);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<f32x4*>(W + 8 * i + 4 * h) = w[h];
      *reinterpret_cast<f32x4*>(Mm + 8 * i + 4 * h) = m[h];
      *reinterpret_cast<f32x4*>(Vv + 8 * i + 4 * h) = v[h];
    }
    *reinterpret_cast<u32x4*>(P + 8 * i) = p;
  }
  // the tail, one parameter per thread of the first work-group
  if (blockIdx.x == 0) {
    const int64_t j = 8 * n8 + threadIdx.x;
    if (j < n) {
      float w = W[j], m = Mm[j], v = Vv[j];
      adam_one(bf16_to_f32(G[j]), w, m, v, a);
      W[j] = w;
      Mm[j] = m;
      Vv[j] = v;
      P[j] = (uint16_t)pack_bf16x2(w, 0.0f);
    }
  }
}

hipError_t launch_adam(float* W, const uint16_t* G, float* m, float* v, uint16_t* P, int64_t n, float lr,
                       float b1, float b2, float eps, float wd, int64_t step, hipStream_t st) {
  const AdamArgs a{lr, b1, b2, eps, wd, (float)(1.0 - std::pow((double)b1, (double)step)),
                   (float)(1.0 - std::pow((double)b2, (double)step))};
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  QLORA_LAUNCH("adam", st, k_adam, dim3((unsigned)blocks), dim3(256), 0, st, W, G, m, v, P, n, a);
  return hipGetLastError();
}

}  // namespace qlora
