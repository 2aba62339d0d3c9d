// gemm_dx.hip -- input gradient dX = dY w~ + s U A, U = dY B
// (page "LoRA and QLoRA fine-tuning: mechanics, and when not to fine-tune":
// the backward pass still dequantises W to BF16 to form the activation
// gradient that reaches the adapter; no gradient is formed for W0).
//
// Transposed-dequant GEMM on bf16 MFMA (32x32x16), fp32 accumulation;
// 256 x 256 work-group tiles of 2 x 2 waves (128 x 128 each, 256
// accumulators per lane), 128 x 128 when the grid would not cover the CUs.
// The contraction runs over d, the weight's row index, while each packed
// code word holds 8 consecutive columns of one row, so the weight tile must
// be transposed before it can feed MFMA.  Each K step (64 weight rows x BN
// columns) is decoded once per work-group into LDS in column-major order:
// wave q decodes column chunks q (and q + 4), lane i decodes weight row i
// (16 bytes = 32 codes, one block-constant table per lane) and writes its 32
// bf16 values down 32 LDS rows at consecutive addresses across the wave (no
// bank conflicts).  dY and weight tiles are double-buffered through
// XOR-swizzled LDS (128 KB for 256 x 256 tiles).  The LoRA term
// s U A is one more MFMA pass in the epilogue, accumulating into the same
// registers, from U (M x rp) and bf16(s A)^T, zero-padded (k x rp).
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

constexpr int kDxBK = 64;

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
  constexpr int YT = BM * kDxBK, WT = BN * kDxBK;  // tile sizes (elements)
  // [ys0 | ys1 | wt0 | wt1]; the epilogue reuses it to stage outputs
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * YT + 2 * WT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (k + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, c0 = tn * BN;
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
  auto store_y = [&](uint16_t* ys) {
#pragma unroll
    for (int i = 0; i < YCH; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(&ys[swz(row, ch)]) = yreg[i];
    }
  };
  // Weight row decoded by this lane in each K step: ks * 64 + lane.
  // Next K step's codes and raw block constants (decoded when stored to LDS,
  // so the loads stay in flight during the MFMAs).
  u32x4 wreg[WCH];
  uint32_t wc2[WCH];
  float wc1[WCH];
  bool wval[WCH];
  auto load_w = [&](int ks) {
    const int dr = ks * kDxBK + lane;
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const int col = c0 + (wave + 4 * q) * 32;
      u32x4 v = {0u, 0u, 0u, 0u};
      uint32_t q2 = 0u;
      float q1 = 0.0f;
      const bool ok = dr < d && col < k;
      if (ok) {
        const size_t blk = (size_t)dr * kblocks + (col >> 6);
        v = *reinterpret_cast<const u32x4*>(codes + (size_t)dr * (k >> 1) + (col >> 1));
        q2 = c2[blk];
        q1 = c1[blk >> 8];
      }
      wreg[q] = v;
      wc2[q] = q2;
      wc1[q] = q1;
      wval[q] = ok;
    }
  };
  // Transposed tile: element (column c, weight row dd) at swz(c, dd/8) + dd%8.
  auto store_w = [&](uint16_t* wt) {
    const int sub = (lane >> 3), lo = lane & 7;
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const Lut t = build_lut(tab, wval[q] ? block_scale(wc2[q], wc1[q], mu) : 0.0f);
      const int cbase = (wave + 4 * q) * 32;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const u32x4 v = dequant8(wreg[q][wd], t);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int ca = cbase + wd * 8 + 2 * p;
          wt[swz(ca, sub) + lo] = (uint16_t)(v[p] & 0xFFFFu);
          wt[swz(ca + 1, sub) + lo] = (uint16_t)(v[p] >> 16);
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

  load_w(0);
  load_y(0);
  store_y(smem);
  store_w(smem + 2 * YT);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const bool more = ks + 1 < ksteps;
    if (more) {
      load_w(ks + 1);
      load_y(ks + 1);
    }
    const uint16_t* yb = smem + (ks & 1) * YT;
    const uint16_t* wb = smem + 2 * YT + (ks & 1) * WT;
    // fragments double-buffered one substep ahead of their MFMAs
    u32x4 af[2][MB], bf[2][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      bf[0][nb] = *reinterpret_cast<const u32x4*>(&wb[swz(wn * WN + nb * 32 + l32, half)]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      af[0][mb] = *reinterpret_cast<const u32x4*>(&yb[swz(wm * WM + mb * 32 + l32, half)]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int cur = st & 1, nxt = cur ^ 1;
      if (st < 3) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          bf[nxt][nb] = *reinterpret_cast<const u32x4*>(&wb[swz(wn * WN + nb * 32 + l32, (st + 1) * 2 + half)]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[nxt][mb] = *reinterpret_cast<const u32x4*>(&yb[swz(wm * WM + mb * 32 + l32, (st + 1) * 2 + half)]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(af[cur][mb], bf[cur][nb], acc[mb][nb]);
    }
    if (more) {
      store_y(smem + ((ks + 1) & 1) * YT);
      store_w(smem + 2 * YT + ((ks + 1) & 1) * WT);
    }
    __syncthreads();
  }

  // LoRA term: acc += U_tile . (s A)_tile^T, K = rp (At holds bf16(s A)^T),
  // accumulated straight into the MFMA accumulators.
  if (rp > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + wm * WM + mb * 32 + l32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int c = c0 + wn * WN + nb * 32 + l32;
        for (int jb = 0; jb < rp; jb += 16) {
          u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
          if (m < M) a = *reinterpret_cast<const u32x4*>(U + (size_t)m * rp + jb + half * 8);
          if (c < k) b = *reinterpret_cast<const u32x4*>(At + (size_t)c * rp + jb + half * 8);
          acc[mb][nb] = mfma32(a, b, acc[mb][nb]);
        }
      }
    }
  }

  // Output through LDS: each wave stages WM x 64 bf16 (two 32-column blocks)
  // at a time and stores 16-byte row chunks.
  uint16_t* stage = smem + wave * (WM * 64);
#pragma unroll
  for (int pass = 0; pass < NB / 2; ++pass) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = mb * 32 + blk * 8 + half * 4 + i, col = q * 32 + l32;
            stage[swz(row, col >> 3) + (col & 7)] =
                (uint16_t)pack_bf16x2(acc[mb][pass * 2 + q][blk * 4 + i], 0.0f);
          }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < WM / 8; ++i) {
      const int c = i * 64 + lane, row = c >> 3, ch = c & 7;
      const int m = m0 + wm * WM + row, col = c0 + wn * WN + pass * 64 + ch * 8;
      if (m < M && col < k)
        *reinterpret_cast<u32x4*>(dX + (size_t)m * k + col) = *reinterpret_cast<const u32x4*>(&stage[swz(row, ch)]);
    }
    __syncthreads();
  }
}

hipError_t launch_dx(const uint16_t* dY, int M, const Nf4Dev& w, const uint16_t* U,
                     const uint16_t* At, int r, float s, uint16_t* dX, const Nf4Table& t,
                     hipStream_t st) {
  const int rp = r > 0 ? padded_rank(r) : 0;
  const int tiles256 = ((M + 255) / 256) * ((w.k + 255) / 256);
  const int forced = tile_override();
  if (forced == 256 || (forced == 0 && tiles256 >= 256)) {
    dim3 grid((unsigned)tiles256);
    QLORA_LAUNCH("dx", st, (k_dx<256, 256>), grid, dim3(256), 0, st, dY, M, w.codes, w.c2, w.c1, w.mean,
                 w.d, w.k, U, At, rp, s, dX, t);
  } else {
    dim3 grid((unsigned)(((M + 127) / 128) * ((w.k + 127) / 128)));
    QLORA_LAUNCH("dx", st, (k_dx<128, 128>), grid, dim3(256), 0, st, dY, M, w.codes, w.c2, w.c1, w.mean,
                 w.d, w.k, U, At, rp, s, dX, t);
  }
  return hipGetLastError();
}

}  // namespace qlora
