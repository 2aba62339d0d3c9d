// gemm_dx.hip -- input gradient dX = dY w~ + s U A, U = dY B
// (page "LoRA and QLoRA fine-tuning: mechanics, and when not to fine-tune":
// the backward pass still dequantises W to BF16 to form the activation
// gradient that reaches the adapter; no gradient is formed for W0).
//
// Transposed-dequant GEMM on bf16 MFMA (32x32x16), fp32 accumulation.
// The contraction runs over d, the weight's row index, while each packed
// code word holds 8 consecutive columns of one row, so the weight tile must
// be transposed before it can feed MFMA.  Each K step (64 weight rows x BN
// columns) is decoded once per work-group into LDS in column-major order:
// wave q decodes column chunk q, lane i decodes weight row i (16 bytes =
// 32 codes, one block-constant table per lane) and writes its 32 bf16 values
// down 32 LDS rows at consecutive addresses across the wave (no bank
// conflicts).  dY tiles are double-buffered through LDS.  The LoRA term
// s U A is one more MFMA pass in the epilogue from U (M x rp) and the
// transposed, zero-padded A (k x rp).
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

constexpr int kDxBK = 64;
constexpr int kDxPitch = kDxBK + 8;

template <int BM, int BN>
__global__ __launch_bounds__(256) void k_dx(const uint16_t* __restrict__ dY, int M,
                                           const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ c2,
                                           const float* __restrict__ c1,
                                           const float* __restrict__ mean, int d, int k,
                                           const uint16_t* __restrict__ U,
                                           const uint16_t* __restrict__ At, int rp, float s,
                                           uint16_t* __restrict__ dX, Nf4Table tab) {
  constexpr int WM = BM / 2, WN = BN / 2;   // 2 x 2 waves
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int YCH = BM * 8 / 256;         // 16-byte dY chunks per thread
  constexpr int WCH = BN / 32 / 4;          // 32-column code chunks per wave
  __shared__ __attribute__((aligned(16))) uint16_t ys[2][BM * kDxPitch];
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][BN * kDxPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, c0 = blockIdx.x * BN;
  const int ksteps = (d + kDxBK - 1) / kDxBK;
  const int kblocks = k / 64;
  const float mu = mean[0];

  u32x4 yreg[YCH];
  auto load_y = [&](int ks) {
#pragma unroll
    for (int i = 0; i < YCH; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      const int m = m0 + row, dc = ks * kDxBK + ch * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < M && dc < d) v = *reinterpret_cast<const u32x4*>(dY + (size_t)m * d + dc);
      yreg[i] = v;
    }
  };
  auto store_y = [&](int buf) {
#pragma unroll
    for (int i = 0; i < YCH; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(&ys[buf][row * kDxPitch + ch * 8]) = yreg[i];
    }
  };
  // Weight row handled by this lane in each K step: d0 + lane.
  u32x4 wreg[WCH];
  float wah[WCH];
  auto load_w = [&](int ks) {
    const int dr = ks * kDxBK + lane;
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const int col = c0 + (wave + 4 * q) * 32;
      u32x4 v = {0u, 0u, 0u, 0u};
      float ah = 0.0f;
      if (dr < d && col < k) {
        const size_t blk = (size_t)dr * kblocks + (col >> 6);
        v = *reinterpret_cast<const u32x4*>(codes + (size_t)dr * (k >> 1) + (col >> 1));
        ah = block_scale(c2[blk], c1[blk >> 8], mu);
      }
      wreg[q] = v;
      wah[q] = ah;
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const Lut t = build_lut(tab, wah[q]);
      uint16_t* dst = &wt[buf][((wave + 4 * q) * 32) * kDxPitch + lane];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const u32x4 v = dequant8(wreg[q][wd], t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[(wd * 8 + 2 * e) * kDxPitch] = (uint16_t)(v[e] & 0xFFFFu);
          dst[(wd * 8 + 2 * e + 1) * kDxPitch] = (uint16_t)(v[e] >> 16);
        }
      }
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  load_y(0);
  load_w(0);
  store_y(0);
  store_w(0);
  __syncthreads();
  int buf = 0;
  for (int ks = 0; ks < ksteps; ++ks) {
    const bool more = ks + 1 < ksteps;
    if (more) {
      load_y(ks + 1);
      load_w(ks + 1);
    }
    const uint16_t* yb = ys[buf];
    const uint16_t* wb = wt[buf];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4 bf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bf[nb] = *reinterpret_cast<const u32x4*>(&wb[(wn * WN + nb * 32 + l32) * kDxPitch + st * 16 + half * 8]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&yb[(wm * WM + mb * 32 + l32) * kDxPitch + st * 16 + half * 8]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(a, bf[nb], acc[mb][nb]);
      }
    }
    if (more) {
      store_y(buf ^ 1);
      store_w(buf ^ 1);
    }
    __syncthreads();
    buf ^= 1;
  }

  // LoRA term: acc += s * (U_tile . At_tile^T), K = rp.
  if (rp > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + wm * WM + mb * 32 + l32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int c = c0 + wn * WN + nb * 32 + l32;
        f32x16 tmp;
#pragma unroll
        for (int i = 0; i < 16; ++i) tmp[i] = 0.0f;
        for (int jb = 0; jb < rp; jb += 16) {
          u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
          if (m < M) a = *reinterpret_cast<const u32x4*>(U + (size_t)m * rp + jb + half * 8);
          if (c < k) b = *reinterpret_cast<const u32x4*>(At + (size_t)c * rp + jb + half * 8);
          tmp = mfma32(a, b, tmp);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = fmaf(s, tmp[i], acc[mb][nb][i]);
      }
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = c0 + wn * WN + nb * 32 + l32;
      if (c >= k) continue;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wm * WM + mb * 32 + blk * 8 + half * 4 + i;
          if (m < M) dX[(size_t)m * k + c] = (uint16_t)pack_bf16x2(acc[mb][nb][blk * 4 + i], 0.0f);
        }
    }
}

hipError_t launch_dx(const uint16_t* dY, int M, const Nf4Dev& w, const uint16_t* U,
                     const uint16_t* At, int r, float s, uint16_t* dX, const Nf4Table& t,
                     hipStream_t st) {
  const int rp = r > 0 ? padded_rank(r) : 0;
  constexpr int BM = 128, BN = 128;
  dim3 grid((unsigned)((w.k + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  QLORA_LAUNCH("dx", st, (k_dx<BM, BN>), grid, dim3(256), 0, st, dY, M, w.codes, w.c2, w.c1, w.mean, w.d,
                     w.k, U, At, rp, s, dX, t);
  return hipGetLastError();
}

}  // namespace qlora
