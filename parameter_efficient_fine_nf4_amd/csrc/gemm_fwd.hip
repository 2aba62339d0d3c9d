// gemm_fwd.hip -- QLoRA forward Y = X w~^T + s T B^T, T = X A^T
// (page "LoRA and QLoRA fine-tuning: mechanics, and when not to fine-tune",
// forward equation of "What QLoRA freezes, and in how many bits": a
// dequantised base matmul plus a LoRA matmul, both in BF16).
//
// Two variants, chosen by token count:
//
// k_fwd_rich (M > 64): fused NF4-dequant GEMM on bf16 MFMA (32x32x16) with
//   fp32 accumulation.  Work-group tile BM x 256, four waves side by side
//   along N (each wave: all BM rows x 64 output features), K step 64 = one
//   NF4 block per weight row.  X tiles are double-buffered through LDS.
//   The packed codes go straight from global memory into registers; each
//   lane owns one weight row and half a block (16 bytes = 32 codes), turns
//   its block constant into a 16-entry bf16 table and decodes 8 codes per
//   MFMA operand with byte permutes.  Every weight element is decoded once
//   per work-group.  The LoRA up-projection s T B^T runs on MFMA in the
//   epilogue from the bf16 T (M x rp) and the zero-padded B (d x rp).
//
// k_fwd_decode (M <= 64): HBM-streaming split-K variant for few tokens.
//   Tile = 64 weight rows x a K range; MFMA 16x16x32 with the tokens as the
//   16-row operand.  Each weight element is decoded exactly once.  Extra
//   tiles treat the rows of A as bf16 "weights" to form partial T = X A^T.
//   fp32 partials go to the workspace; k_fwd_decode_finish sums them in a
//   fixed order, adds s T B^T and rounds to bf16.
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

// ------------------------------------------------------------ token-rich --

constexpr int kRichBN = 256;
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // LDS row pitch (bf16) for 64-wide K tiles

template <int BM>
__global__ __launch_bounds__(256) void k_fwd_rich(const uint16_t* __restrict__ X, int M,
                                                 const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ c2,
                                                 const float* __restrict__ c1,
                                                 const float* __restrict__ mean, int d, int k,
                                                 const uint16_t* __restrict__ T,
                                                 const uint16_t* __restrict__ Bp, int rp, float s,
                                                 uint16_t* __restrict__ Y, Nf4Table tab) {
  constexpr int MB = BM / 32;       // 32-row MFMA blocks per wave
  constexpr int XCH = BM * 8 / 256; // 16-byte X chunks per thread per K tile
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * kRichBN + wave * 64;
  const int kblocks = k / kBK;
  const float mu = mean[0];

  // Weight rows owned by this lane (one per 32-column MFMA block).
  int nrow[2];
  bool nval[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    nrow[nb] = n0 + nb * 32 + l32;
    nval[nb] = nrow[nb] < d;
  }

  u32x4 xreg[XCH];
  auto load_x = [&](int kb) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      const int m = m0 + row;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < M) v = *reinterpret_cast<const u32x4*>(X + (size_t)m * k + kb * kBK + ch * 8);
      xreg[i] = v;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(&xs[buf][row * kPitch + ch * 8]) = xreg[i];
    }
  };
  u32x4 wreg[2];
  float wah[2];
  auto load_w = [&](int kb) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      u32x4 v = {0u, 0u, 0u, 0u};
      float ah = 0.0f;
      if (nval[nb]) {
        const size_t blk = (size_t)nrow[nb] * kblocks + kb;
        v = *reinterpret_cast<const u32x4*>(codes + blk * 32 + half * 16);
        ah = block_scale(c2[blk], c1[blk >> 8], mu);
      }
      wreg[nb] = v;
      wah[nb] = ah;
    }
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.0f;

  load_x(0);
  load_w(0);
  store_x(0);
  __syncthreads();
  int buf = 0;
  for (int kb = 0; kb < kblocks; ++kb) {
    const u32x4 w0 = wreg[0], w1 = wreg[1];
    const Lut t0 = build_lut(tab, wah[0]);
    const Lut t1 = build_lut(tab, wah[1]);
    const bool more = kb + 1 < kblocks;
    if (more) {
      load_x(kb + 1);
      load_w(kb + 1);
    }
    const uint16_t* xb = xs[buf];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      // this lane's MFMA k indices: half*32 + st*8 + (0..7) of the block
      const u32x4 b0 = dequant8(w0[st], t0);
      const u32x4 b1 = dequant8(w1[st], t1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&xb[(mb * 32 + l32) * kPitch + half * 32 + st * 8]);
        acc[mb][0] = mfma32(a, b0, acc[mb][0]);
        acc[mb][1] = mfma32(a, b1, acc[mb][1]);
      }
    }
    if (more) store_x(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // LoRA up-projection: acc += s * (T_tile . Bp_tile^T), K = rp.
  if (rp > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 32 + l32;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x16 tmp;
#pragma unroll
        for (int i = 0; i < 16; ++i) tmp[i] = 0.0f;
        for (int jb = 0; jb < rp; jb += 16) {
          u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
          if (m < M) a = *reinterpret_cast<const u32x4*>(T + (size_t)m * rp + jb + half * 8);
          if (nval[nb]) b = *reinterpret_cast<const u32x4*>(Bp + (size_t)nrow[nb] * rp + jb + half * 8);
          tmp = mfma32(a, b, tmp);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = fmaf(s, tmp[i], acc[mb][nb][i]);
      }
    }
  }

  // Store: lane holds column l32 of each 32x32 block, rows 8*blk + 4*half + i.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (!nval[nb]) continue;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + mb * 32 + blk * 8 + half * 4 + i;
          if (m < M) Y[(size_t)m * d + nrow[nb]] = (uint16_t)pack_bf16x2(acc[mb][nb][blk * 4 + i], 0.0f);
        }
    }
}

// ---------------------------------------------------------------- decode --

constexpr int kDecRows = 64;   // weight rows per tile
constexpr int kDecStep = 128;  // K per wave step (4 lane quarters x 32)

template <int MBLK>
__global__ __launch_bounds__(256) void k_fwd_decode(const uint16_t* __restrict__ X, int M,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ c2,
                                                   const float* __restrict__ c1,
                                                   const float* __restrict__ mean, int d, int k,
                                                   const uint16_t* __restrict__ A, int r, int ntw,
                                                   int steps_per_split, float* __restrict__ part,
                                                   int ldp, Nf4Table tab) {
  __shared__ float red[4][MBLK][4][64][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int tile = blockIdx.x, split = blockIdx.y;
  const bool is_w = tile < ntw;
  const int row_base = is_w ? tile * kDecRows : (tile - ntw) * kDecRows;
  const int nsteps = (k + kDecStep - 1) / kDecStep;
  const int s_begin = split * steps_per_split;
  const int s_end = min(nsteps, s_begin + steps_per_split);
  const int kblocks = k / 64;
  const float mu = mean[0];

  f32x4 acc[MBLK][4];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = s_begin + wave; st < s_end; st += 4) {
    const int k0 = st * kDecStep + 32 * g;  // this lane's 32-wide K chunk
    const bool kval = k0 < k;
    u32x4 xa[MBLK][4];
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
      const int m = mb * 16 + l16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (kval && m < M) v = *reinterpret_cast<const u32x4*>(X + (size_t)m * k + k0 + q * 8);
        xa[mb][q] = v;
      }
    }
    if (is_w) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = row_base + nb * 16 + l16;
        u32x4 w = {0u, 0u, 0u, 0u};
        float ah = 0.0f;
        if (kval && n < d) {
          const size_t blk = (size_t)n * kblocks + (k0 >> 6);
          w = *reinterpret_cast<const u32x4*>(codes + (size_t)n * (k >> 1) + (k0 >> 1));
          ah = block_scale(c2[blk], c1[blk >> 8], mu);
        }
        const Lut t = build_lut(tab, ah);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 b = dequant8(w[q], t);
#pragma unroll
          for (int mb = 0; mb < MBLK; ++mb) acc[mb][nb] = mfma16(xa[mb][q], b, acc[mb][nb]);
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int j = row_base + nb * 16 + l16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x4 b = {0u, 0u, 0u, 0u};
          if (kval && j < r) b = *reinterpret_cast<const u32x4*>(A + (size_t)j * k + k0 + q * 8);
#pragma unroll
          for (int mb = 0; mb < MBLK; ++mb) acc[mb][nb] = mfma16(xa[mb][q], b, acc[mb][nb]);
        }
      }
    }
  }

  // Sum the four waves in a fixed order.
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][mb][nb][lane][i] = acc[mb][nb][i];
  __syncthreads();
  if (wave == 0) {
    const int col_base = is_w ? row_base : d + row_base;
    const int col_lim = is_w ? d : d + r;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = col_base + nb * 16 + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mb * 16 + 4 * g + i;
          const float v = ((red[0][mb][nb][lane][i] + red[1][mb][nb][lane][i]) + red[2][mb][nb][lane][i]) +
                          red[3][mb][nb][lane][i];
          if (m < M && col < col_lim) part[((size_t)split * M + m) * ldp + col] = v;
        }
      }
  }
}

// One work-group per (token, 256 output features): sum the split partials,
// form T (rounded to bf16, as in the token-rich path), add s T B^T, round.
__global__ __launch_bounds__(256) void k_fwd_decode_finish(const float* __restrict__ part, int nsplit,
                                                          int M, int d, int ldp,
                                                          const uint16_t* __restrict__ B, int r,
                                                          float s, uint16_t* __restrict__ Y,
                                                          uint16_t* __restrict__ Tsave, int ldt) {
  __shared__ float tsh[kMaxRank];
  const int m = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < r) {
    float t = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) t += part[((size_t)sp * M + m) * ldp + d + tid];
    const uint32_t tb = pack_bf16x2(t, 0.0f) & 0xFFFFu;
    tsh[tid] = bf16_to_f32((uint16_t)tb);
    if (Tsave != nullptr && blockIdx.x == 0) Tsave[(size_t)tid * ldt + m] = (uint16_t)tb;
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n >= d) return;
  float y = 0.0f;
  for (int sp = 0; sp < nsplit; ++sp) y += part[((size_t)sp * M + m) * ldp + n];
  if (r > 0) {
    float l = 0.0f;
    for (int j = 0; j < r; ++j) l = fmaf(tsh[j], bf16_to_f32(B[(size_t)n * r + j]), l);
    y = fmaf(s, l, y);
  }
  Y[(size_t)m * d + n] = (uint16_t)pack_bf16x2(y, 0.0f);
}

// ---------------------------------------------------------------- launch --

bool forward_uses_decode(int M, int d, int k) { return M <= 64; }

static void decode_split(int M, int d, int k, int r, int* ntiles, int* ntw, int* nsplit, int* sps) {
  const int tw = (d + kDecRows - 1) / kDecRows;
  const int ta = r > 0 ? (r + kDecRows - 1) / kDecRows : 0;
  const int nsteps = (k + kDecStep - 1) / kDecStep;
  int want = (512 + tw - 1) / tw;
  if (want < 1) want = 1;
  int maxs = (nsteps + 3) / 4;  // keep at least four steps (one per wave) per split
  if (maxs < 1) maxs = 1;
  int ns = want < maxs ? want : maxs;
  const int per = (nsteps + ns - 1) / ns;
  ns = (nsteps + per - 1) / per;
  *ntiles = tw + ta;
  *ntw = tw;
  *nsplit = ns;
  *sps = per;
}

size_t forward_gemm_ws_bytes(int M, int d, int k, int r) {
  if (!forward_uses_decode(M, d, k)) return 0;
  int ntiles, ntw, ns, sps;
  decode_split(M, d, k, r, &ntiles, &ntw, &ns, &sps);
  return (size_t)ns * M * (d + padded_rank(r)) * sizeof(float);
}

hipError_t launch_forward_decode(const uint16_t* X, int M, const Nf4Dev& w, const uint16_t* A,
                                 const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* Tsave,
                                 int ldt, float* part, const Nf4Table& t, hipStream_t st) {
  int ntiles, ntw, ns, sps;
  decode_split(M, w.d, w.k, r, &ntiles, &ntw, &ns, &sps);
  const int ldp = w.d + padded_rank(r);
  dim3 grid((unsigned)ntiles, (unsigned)ns);
  const int mblk = (M + 15) / 16;
#define QLORA_DEC(MB)                                                                            \
  QLORA_LAUNCH("fwd_decode", st, k_fwd_decode<MB>, grid, dim3(256), 0, st, X, M, w.codes, w.c2, w.c1, w.mean, \
                     w.d, w.k, A, r, ntw, sps, part, ldp, t)
  switch (mblk) {
    case 1: QLORA_DEC(1); break;
    case 2: QLORA_DEC(2); break;
    case 3: QLORA_DEC(3); break;
    default: QLORA_DEC(4); break;
  }
#undef QLORA_DEC
  QLORA_LAUNCH("fwd_decode_finish", st, k_fwd_decode_finish, dim3((unsigned)((w.d + 255) / 256), (unsigned)M), dim3(256),
                     0, st, part, ns, M, w.d, ldp, B, r, s, Y, Tsave, ldt);
  return hipGetLastError();
}

hipError_t launch_forward(const uint16_t* X, int M, const Nf4Dev& w, const uint16_t* T,
                          const uint16_t* Bp, int r, float s, uint16_t* Y, const Nf4Table& t,
                          hipStream_t st) {
  const int rp = r > 0 ? padded_rank(r) : 0;
  constexpr int BM = 128;
  dim3 grid((unsigned)((w.d + kRichBN - 1) / kRichBN), (unsigned)((M + BM - 1) / BM));
  QLORA_LAUNCH("fwd_rich", st, k_fwd_rich<BM>, grid, dim3(256), 0, st, X, M, w.codes, w.c2, w.c1, w.mean, w.d,
                     w.k, T, Bp, rp, s, Y, t);
  return hipGetLastError();
}

}  // namespace qlora
