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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_dx(
    const uint16_t* __restrict__ dY, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ c2, const float* __restrict__ c1, const float* __restrict__ mean,
    int d, int k, const uint16_t* __restrict__ U, const uint16_t* __restrict__ At, int rp,
    float s, uint16_t* __restrict__ dX, Nf4Table tab) {
  constexpr int WM = BM / 2, WN = BN / 2;   // 2 x 2 waves
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int YCH = BM / 32;              // 1 KB dY loads per wave per K step
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

  // dY tile (BM x 64) -> LDS by direct global->LDS loads: wave w fills rows
  // [w*BM/4, (w+1)*BM/4), eight rows per instruction (see the forward
  // kernel).  Rows past M repeat row M-1; columns past d read row m's first
  // columns and meet zero weights (rows past d decode to zero).
  auto dma_y = [&](int ks, uint16_t* ys) {
    const int lr = lane >> 3, pc = lane & 7;
#pragma unroll
    for (int j = 0; j < YCH; ++j) {
      const int r0 = wave * (BM / 4) + j * 8;
      const int m = min(m0 + r0 + lr, M - 1);
      int dc = ks * kDxBK + ((pc ^ swz_f(r0 + lr)) << 3);
      if (dc >= d) dc = 0;
      const uint16_t* src = dY + (size_t)m * d + dc;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(ys + r0 * kDxBK), 16, 0, 0);
    }
  };
  // Codes of weight row ks*64 + lane for this wave's column chunks, with
  // their raw block constants (decoded when the tile is decoded).
  struct WTile {
    u32x4 v[WCH];
    uint32_t q2[WCH];
    float q1[WCH];
    bool ok[WCH];
  };
  auto load_w = [&](int ks, WTile& t) {
    const int dr = ks * kDxBK + lane;
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const int col = c0 + (wave + 4 * q) * 32;
      const bool ok = dr < d && col < k;
      const int drc = ok ? dr : 0, colc = ok ? col : 0;
      const size_t blk = (size_t)drc * kblocks + (colc >> 6);
      t.v[q] = *reinterpret_cast<const u32x4*>(codes + (size_t)drc * (k >> 1) + (colc >> 1));
      t.q2[q] = c2[blk];
      t.q1[q] = c1[blk >> 8];
      t.ok[q] = ok;
    }
  };
  // Decoded weights of one tile for this lane: chunk q, word wd -> 8 bf16.
  u32x4 dq[WCH][4];
  Lut lut[WCH];
  auto tables = [&](const WTile& t) {
#pragma unroll
    for (int q = 0; q < WCH; ++q) lut[q] = build_lut(tab, t.ok[q] ? block_scale(t.q2[q], t.q1[q], mu) : 0.0f);
  };
  // Transposed tile: element (column c, weight row dd) at swz(c, dd/8) + dd%8.
  auto store_dq = [&](uint16_t* wt) {
    const int sub = (lane >> 3), lo = lane & 7;
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const int cbase = (wave + 4 * q) * 32;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int ca = cbase + wd * 8 + 2 * p;
          wt[swz(ca, sub) + lo] = (uint16_t)(dq[q][wd][p] & 0xFFFFu);
          wt[swz(ca + 1, sub) + lo] = (uint16_t)(dq[q][wd][p] >> 16);
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

  // Pipeline: codes two K steps ahead, dY one ahead; the weights of step
  // ks+1 are decoded during the MFMAs of step ks and stored to LDS at its end.
  WTile wnext, wfar;
  load_w(0, wnext);
  dma_y(0, smem);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  tables(wnext);
#pragma unroll
  for (int q = 0; q < WCH; ++q)
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) dq[q][wd] = dequant8(wnext.v[q][wd], lut[q]);
  store_dq(smem + 2 * YT);
  if (ksteps > 1) {
    load_w(1, wnext);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const bool more = ks + 1 < ksteps;
    if (ks + 2 < ksteps) load_w(ks + 2, wfar);
    if (more) dma_y(ks + 1, smem + ((ks + 1) & 1) * YT);
    const uint16_t* yb = smem + (ks & 1) * YT;
    const uint16_t* wb = smem + 2 * YT + (ks & 1) * WT;
    if (more) tables(wnext);
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
      __builtin_amdgcn_sched_barrier(0);
      if (st < 3) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          bf[nxt][nb] = *reinterpret_cast<const u32x4*>(&wb[swz(wn * WN + nb * 32 + l32, (st + 1) * 2 + half)]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[nxt][mb] = *reinterpret_cast<const u32x4*>(&yb[swz(wm * WM + mb * 32 + l32, (st + 1) * 2 + half)]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // decode word st of every chunk of the next weight tile (VALU)
      if (more) {
#pragma unroll
        for (int q = 0; q < WCH; ++q) dq[q][st] = dequant8(wnext.v[q][st], lut[q]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(af[cur][mb], bf[cur][nb], acc[mb][nb]);
#pragma unroll
      for (int i = 0; i < MB * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) store_dq(smem + 2 * YT + ((ks + 1) & 1) * WT);
    // dY tile ks+1 and codes ks+2 have landed once every load is complete
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    wnext = wfar;
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
