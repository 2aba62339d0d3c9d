// gemm_fwd.hip -- QLoRA forward Y = X w~^T + s T B^T, T = X A^T
// (page "LoRA and QLoRA fine-tuning: mechanics, and when not to fine-tune",
// forward equation of "What QLoRA freezes, and in how many bits": the 4-bit
// base is expanded to bf16 and multiplied, the adapter product is added, and
// both multiplies run in bf16).
//
// Variants, chosen by token count and shape:
//
// k_fwd8 (M > 64, d and k multiples of 256): the eight-wave form of
//   k_fwd_rich, two waves per SIMD (described at the kernel).
//
// k_fwd_rich (M > 64, other shapes): fused NF4-dequant GEMM on bf16 MFMA (32x32x16) with
//   fp32 accumulation.  Work-group tile BM x 256 (BM = 256, or 128 when the
//   grid would not cover the CUs), four waves side by side along N (each
//   wave: all BM rows x 64 output features, BM*64/64 accumulators per lane),
//   K step 64 = one NF4 block per weight row.  Decoding costs about four
//   VALU operations per weight and each decoded weight feeds BM tokens, so
//   BM = 256 keeps the decode well under the MFMA time.  X tiles are
//   double-buffered through XOR-swizzled LDS; outputs leave through LDS as
//   16-byte row chunks.
//   The packed codes go straight from global memory into registers; each
//   lane owns one weight row and half a block (16 bytes = 32 codes), turns
//   its block constant into a 16-entry bf16 table and decodes 8 codes per
//   MFMA operand with byte permutes.  Every weight element is decoded once
//   per work-group.  The LoRA up-projection s T B^T runs on MFMA in the
//   epilogue, accumulating into the same registers, from the bf16 T (M x rp)
//   and bf16(s B), scaled and zero-padded in registers as it is loaded.
//
// k_fwd_decode (M <= 64): HBM-streaming split-K variant for few tokens.
//   Tile = 64 weight rows x a K range; MFMA 16x16x32 with the tokens as the
//   16-row operand.  Each weight element is decoded exactly once.  Extra
//   tiles treat the rows of A as bf16 "weights" to form partial T = X A^T.
//   fp32 partials go to the workspace; k_fwd_decode_finish sums them in a
//   fixed order, adds s T B^T and rounds to bf16.
#include <string.h>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

// ------------------------------------------------------------ token-rich --

constexpr int kRichBN = 256;
constexpr int kBK = 64;

template <int BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_fwd_rich(const uint16_t* __restrict__ X, int M,
                                                 const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ c2,
                                                 const float* __restrict__ c1,
                                                 const float* __restrict__ mean, int d, int k, int dsec,
                                                 const uint16_t* __restrict__ T,
                                                 const uint16_t* __restrict__ B, int r, int rp, int ldr, float s,
                                                 uint16_t* __restrict__ Y, Nf4Table tab) {
  constexpr int MB = BM / 32;        // 32-row MFMA blocks per wave
  constexpr int XCH = BM / 32;       // 1 KB X loads per wave per K tile
  // One ring slot holds everything a K tile needs: the X tile (BM x 64 bf16,
  // swizzled), then per wave the packed codes of its 64 weight rows (2 KB)
  // and the 32-bit words holding their c2 bytes (256 B) and c1 values
  // (256 B).  Three slots; the epilogue reuses the space for output staging.
  constexpr int kXBytes = BM * kBK * 2;
  constexpr int kCodeOff = kXBytes;
  constexpr int kC2Off = kCodeOff + 4 * 2048;
  constexpr int kC1Off = kC2Off + 4 * 256;
  constexpr int kSlot = kC1Off + 4 * 256;
  constexpr int kRing = 3 * kSlot;
  constexpr int kStage = 4 * 128 * 64 * 2;
  constexpr int kSmem = kRing > kStage ? kRing : kStage;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (d + kRichBN - 1) / kRichBN, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * kRichBN + wave * 64;
  const int kblocks = k / kBK;
  // Sections (row blocks of W with their own mean and adapter ranks) never
  // split a tile: the tile's section gives the mean and its columns of T.
  const int sec = tn * kRichBN / dsec;
  const float mu = mean[sec];
  float qh[8];  // this lane's half of the levels, for build_lut_pair
#pragma unroll
  for (int i = 0; i < 8; ++i) qh[i] = half ? tab.q[8 + i] : tab.q[i];

  // Weight rows of this lane's two B operands (nb = 0, 1): n0 + nb*32 + l32.
  // Rows past d read row 0 and are zeroed through their block constant.
  int nrow[2];
  bool nval[2];
  uint32_t cbase[2];  // (clamped row) * kblocks: block index of the row's K tile 0
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    nrow[nb] = n0 + nb * 32 + l32;
    nval[nb] = nrow[nb] < d;
    cbase[nb] = (uint32_t)(nval[nb] ? nrow[nb] : 0) * (uint32_t)kblocks;
  }

  // Direct global->LDS fetches (each instruction writes 64 lanes x size
  // bytes contiguously at a wave-uniform LDS address):
  //  X: wave w fills X rows [w*BM/4, (w+1)*BM/4), eight rows per 16-byte
  //     instruction; lane l lands in row r0 + l/8, physical chunk l%8, so it
  //     fetches the logical chunk (l%8) ^ swz_f(row).  Rows past M repeat
  //     row M-1 (their outputs are never stored).
  //  codes: instruction j, lane l fetches K-half l/32 (16 bytes) of weight
  //     row j*32 + l%32, so a lane later reads back exactly what it fetched.
  //  c2 / c1: lane l fetches the aligned word holding the c2 byte, and the
  //     c1 value, of weight row l of its wave.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t xoff[XCH];
#pragma unroll
  for (int j = 0; j < XCH; ++j) {
    const int lr = lane >> 3, pc = lane & 7;
    const int r0 = wave * (BM / 4) + j * 8;
    const int m = min(m0 + r0 + lr, M - 1);
    xoff[j] = (uint32_t)(((size_t)m * k + ((pc ^ swz_f(r0 + lr)) << 3)) * 2);
  }
  uint32_t coff[2];  // byte offset of this lane's codes of K tile 0, per fetch j
#pragma unroll
  for (int j = 0; j < 2; ++j) coff[j] = (uint32_t)(nval[j] ? nrow[j] : 0) * (uint32_t)(k >> 1) + half * 16;
  const uint32_t dbase = half ? cbase[1] : cbase[0];  // row n0 + lane
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc rx = make_rsrc(X, (uint64_t)M * k * 2);
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);
  // Fetch number i (0 <= i < kLoads) of tile kb into ring slot sl: X chunks
  // first, then the two code chunks, then the c2 and c1 words.  Issuing
  // them a few at a time between MFMAs keeps the address unit's queue short
  // enough that a wave never stalls on issue.
  auto dma_one = [&](int i, int kb, int sl) {
    char* slot = smem + sl * kSlot;
    if (i < XCH) {
      dma_lds16(rx, xoff[i] + (uint32_t)kb * (kBK * 2), slot + (wave_s * (BM / 4) + i * 8) * (kBK * 2));
    } else if (i < XCH + 2) {
      const int j = i - XCH;
      dma_lds16(rc, coff[j] + (uint32_t)kb * 32, slot + kCodeOff + wave_s * 2048 + j * 1024);
    } else {
      const uint32_t blk = dbase + (uint32_t)kb;
      if (i == XCH + 2)
        dma_lds4(r2, blk & ~3u, slot + kC2Off + wave_s * 256);
      else
        dma_lds4(r1, (blk >> 8) * 4, slot + kC1Off + wave_s * 256);
    }
  };
  auto dma_tile = [&](int kb, int sl) {
#pragma unroll
    for (int i = 0; i < XCH + 4; ++i) dma_one(i, kb, sl);
  };
  constexpr int kLoads = XCH + 4;  // fetch instructions per wave per K tile
  constexpr int kPerSub = (kLoads + 2) / 3;  // issued in each of substeps 0..2

  // This lane's codes and block tables of tile kb from ring slot sl.
  struct WTile {
    u32x4 v[2];
    uint32_t q2[2];
    float q1[2];
  };
  auto read_w = [&](int sl, WTile& W) {
    const char* slot = smem + sl * kSlot;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      W.v[nb] = *reinterpret_cast<const u32x4*>(slot + kCodeOff + wave_s * 2048 + nb * 1024 + lane * 16);
      W.q2[nb] = *reinterpret_cast<const uint32_t*>(slot + kC2Off + wave_s * 256 + (nb * 32 + l32) * 4);
      W.q1[nb] = *reinterpret_cast<const float*>(slot + kC1Off + wave_s * 256 + (nb * 32 + l32) * 4);
    }
  };
  auto tables = [&](const WTile& W, int kb, Lut& a, Lut& b) {
    float sc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t sh = ((cbase[nb] + (uint32_t)kb) & 3u) * 8u;
      const float v = block_scale((W.q2[nb] >> sh) & 0xFFu, W.q1[nb], mu);
      sc[nb] = nval[nb] ? v : 0.0f;
    }
    a = build_lut_pair(qh, sc[0]);
    b = build_lut_pair(qh, sc[1]);
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.0f;

  // Byte offset, inside an X tile, of this lane's A fragment of MFMA row
  // block mb and substep st: aoff[mb & 1][st] + (mb >> 1) * 8192.  The
  // swizzle of row mb*32 + l32 depends on mb only through its parity.
  uint32_t aoff[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int st = 0; st < 4; ++st) aoff[p][st] = (uint32_t)(2 * swz(p * 32 + l32, half * 4 + st));
  auto read_a = [&](const char* xs, int st, u32x4 (&dst)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      dst[mb] = *reinterpret_cast<const u32x4*>(xs + aoff[mb & 1][st] + (mb >> 1) * 8192);
  };

  // Software pipeline.  Tiles kb+1 and kb+2 are in flight while tile kb is
  // multiplied: substeps 0..2 of every K step issue the kLoads fetches of
  // tile kb+2 (a tile past the end re-fetches the last one, so the count
  // per step is fixed), interleaved with the MFMAs.  At the end of substep
  // 2 the wave waits until only those are outstanding -- its own share of
  // tile kb+1 is then in LDS, issued at least a full step earlier -- and
  // completes its reads of tile kb, then meets the other waves at a
  // barrier: tile kb+1 is complete in LDS and the slot of tile kb is free
  // for the next step's fetches.  Substep 3 reads this lane's codes and
  // block constants and the first A fragments of tile kb+1 and decodes its
  // first B operands, so the next step starts without waiting.  A
  // fragments are double-buffered (the reads for substep st+1 are issued
  // before the MFMAs of substep st) and the B operands of substep st+1 are
  // decoded (VALU) while the MFMAs of substep st run.
  dma_tile(0, 0);
  dma_tile(kblocks > 1 ? 1 : 0, 1);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");
  WTile W;
  read_w(0, W);
  u32x4 wcur0 = W.v[0], wcur1 = W.v[1];
  Lut t0, t1;
  tables(W, 0, t0, t1);
  u32x4 bc0 = dequant8(wcur0[0], t0), bc1 = dequant8(wcur1[0], t1);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  u32x4 afr[2][MB];
  read_a(smem, 0, afr[0]);

  int sl_cur = 0;
  for (int kb = 0; kb < kblocks; ++kb) {
    const int sl_next = sl_cur == 2 ? 0 : sl_cur + 1;
    const int sl_far = sl_next == 2 ? 0 : sl_next + 1;
    const int kf = kb + 2 < kblocks ? kb + 2 : kblocks - 1;
    const char* xs = smem + sl_cur * kSlot;
    const char* xn = smem + sl_next * kSlot;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      // The first MFMA of the substep goes before the next LDS reads: its
      // operand wait then covers only reads issued a substep ago (the
      // compiler waits for all outstanding LDS reads at that point).
      __builtin_amdgcn_sched_barrier(0);
      acc[0][0] = mfma32(afr[st & 1][0], bc0, acc[0][0]);
      __builtin_amdgcn_sched_barrier(0);
      if (st < 3) {
        read_a(xs, st + 1, afr[(st + 1) & 1]);
      } else {
        read_w(sl_next, W);
        read_a(xn, 0, afr[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // decode the next operands (VALU) while this substep's MFMAs run
      u32x4 bn0, bn1;
      if (st < 3) {
        bn0 = dequant8(wcur0[st + 1], t0);
        bn1 = dequant8(wcur1[st + 1], t1);
      } else {
        wcur0 = W.v[0];
        wcur1 = W.v[1];
        tables(W, kb + 1, t0, t1);
        bn0 = dequant8(wcur0[0], t0);
        bn1 = dequant8(wcur1[0], t1);
      }
      if (st < 3) {
#pragma unroll
        for (int i = st * kPerSub; i < (st + 1) * kPerSub && i < kLoads; ++i) dma_one(i, kf, sl_far);
      }
      // this lane's MFMA k indices: half*32 + st*8 + (0..7) of the block
      acc[0][1] = mfma32(afr[st & 1][0], bc1, acc[0][1]);
#pragma unroll
      for (int mb = 1; mb < MB; ++mb) {
        acc[mb][0] = mfma32(afr[st & 1][mb], bc0, acc[mb][0]);
        acc[mb][1] = mfma32(afr[st & 1][mb], bc1, acc[mb][1]);
      }
      constexpr int kDma = kPerSub;
#pragma unroll
      for (int i = 0; i < 2 * MB - 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        if (st < 3 && i < kDma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (st == 2) {
        // own share of tile kb+1 landed; own reads of tile kb complete;
        // then every wave's share of tile kb+1 is visible
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      bc0 = bn0;
      bc1 = bn1;
    }
    sl_cur = sl_next;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // LoRA up-projection: acc += T_tile . (s B)_tile^T, K = rp, accumulated
  // straight into the MFMA accumulators.  The B operand is bf16(s B) (one
  // fp32 product and one rounding per entry; exact when s is a power of
  // two), ranks past r zero.
  if (rp > 0) {
    // all operand loads first (B operands are the same for every row block)
    for (int jb = 0; jb < rp; jb += 16) {
      u32x4 bop[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        bop[nb] = u32x4{0u, 0u, 0u, 0u};
        if (nval[nb]) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int j = jb + half * 8 + 2 * p;
            const float b0 = j < r ? s * bf16_to_f32(B[(size_t)nrow[nb] * r + j]) : 0.0f;
            const float b1 = j + 1 < r ? s * bf16_to_f32(B[(size_t)nrow[nb] * r + j + 1]) : 0.0f;
            bop[nb][p] = pack_bf16x2(b0, b1);
          }
        }
      }
      u32x4 top[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + mb * 32 + l32;
        top[mb] = u32x4{0u, 0u, 0u, 0u};
        if (m < M) top[mb] = *reinterpret_cast<const u32x4*>(T + (size_t)m * ldr + sec * r + jb + half * 8);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(top[mb], bop[nb], acc[mb][nb]);
    }
  }

  // Output through LDS, 128 rows at a time: each wave stages its 128 x 64
  // bf16 sub-tile (16 KB, swizzled like the X tiles) and stores it as
  // 16-byte row chunks.
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem) + wave * (128 * 64);
#pragma unroll
  for (int pass = 0; pass < (MB + 3) / 4; ++pass) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mb = pass * 4 + q;
      if (mb >= MB) break;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = q * 32 + blk * 8 + half * 4 + i, col = nb * 32 + l32;
            stage[swz(row, col >> 3) + (col & 7)] = (uint16_t)pack_bf16x2(acc[mb][nb][blk * 4 + i], 0.0f);
          }
    }
    __syncthreads();
    const int rows = (MB - pass * 4) < 4 ? (MB - pass * 4) * 32 : 128;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = i * 64 + lane, row = c >> 3, ch = c & 7;
      const int m = m0 + pass * 128 + row, n = n0 + ch * 8;
      if (row < rows && m < M && n < d)
        *reinterpret_cast<u32x4*>(Y + (size_t)m * d + n) = *reinterpret_cast<const u32x4*>(&stage[swz(row, ch)]);
    }
    __syncthreads();
  }
}

// Eight-wave form of the token-rich kernel for the common shapes (d and k
// multiples of 256, M > 64): BM x 256 work-group tiles of eight waves side
// by side along N (each wave: all BM tokens x 32 output features), two waves
// per SIMD, so that one wave's decode and LDS reads overlap the other's
// MFMAs.  Each lane pair decodes one weight row's block straight into MFMA
// operands, as in k_fwd_rich; every weight is decoded once per work-group.
// A K step covers KS NF4 blocks (KS = 1 for 256-row tiles, 2 for 128-row
// tiles, so that every tile height does the same MFMA work between two
// barriers).  Per K step each wave fetches its share of the X tile in 1 KB
// pieces (KS sub-tiles of 64 K), the codes of its 32 weight rows (1 KB per
// block) and the c2 words (waves 0-3) or c1 words (waves 4-7) of 64 weight
// rows of the tile; with k a multiple of 256 a c2 word holds a row's blocks
// 4j..4j+3, so one word and one c1 scale serve a whole step.  X, code and c2
// offsets are a per-lane constant plus a scalar per-step offset; there are
// no bounds checks in the K loop (token rows past M repeat row M-1 and are
// never stored).
constexpr int kFwd8Waves = 8;

template <int BM, int KS>
__global__ __launch_bounds__(64 * kFwd8Waves) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_fwd8(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ c2, const float* __restrict__ c1, const float* __restrict__ mean, int d,
    int k, int dsec, const uint16_t* __restrict__ T, const uint16_t* __restrict__ B, int r, int rp, int ldr, float s,
    uint16_t* __restrict__ Y, Nf4Table tab, int nbase, int ntn, int sps, float* __restrict__ part) {
  constexpr int BN = kRichBN, MB = BM / 32;
  constexpr int NS = 4 * KS;                                 // MFMA substeps per K step
  constexpr int XF1 = BM / 64;                               // 1 KB X fetches per wave per sub-tile
  constexpr int XF = XF1 * KS;
  constexpr int kSub = BM * kBK * 2;                         // one 64-K sub-tile of X
  constexpr int kXBytes = KS * kSub;
  constexpr int kCodeOff = kXBytes;                          // 8 waves x KS x 1 KB of codes
  constexpr int kC2Off = kCodeOff + kFwd8Waves * KS * 1024;  // 256 c2 words, then 256 c1 words
  constexpr int kSlot = kC2Off + 2048;
  constexpr int kRing = 3 * kSlot;
  constexpr int kStage = kFwd8Waves * 128 * 32 * 2;         // up to 128 rows x 32 columns per wave
  constexpr int kSmem = kRing > kStage ? kRing : kStage;
  constexpr int kLoads = XF + KS + 1;                        // fetches per wave per K step
  static_assert(kSmem <= 160 * 1024, "LDS");
  static_assert(kLoads <= 2 * (NS - 1), "fetches fit the substeps before the barrier");
  __shared__ __attribute__((aligned(16))) char smem[kSmem];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, ntn, tm, tn);
  const int m0 = tm * BM, n0 = nbase + tn * BN;  // this launch covers output features nbase .. nbase + ntn*BN
  const int kblocks = k / kBK;
  // Split K (sps > 0): work-group column blockIdx.y takes K steps kbase ..
  // kbase + sps - 1 and writes fp32 partials (split 0 also carries the LoRA
  // term); k_sum_splits adds the splits in order and rounds.
  const int split = blockIdx.y;
  const int kbase = sps > 0 ? split * sps : 0;
  const int ksteps = sps > 0 ? min(sps, kblocks / KS - kbase) : kblocks / KS;
  const int sec = n0 / dsec;  // section of the tile (its mean and its columns of T)
  const float mu = mean[sec];
  float qh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qh[i] = half ? tab.q[8 + i] : tab.q[i];

  const BufRsrc rx = make_rsrc(X, (uint64_t)M * k * 2);
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);

  // X sub-tile kk: wave w fills its rows [w*BM/8, (w+1)*BM/8), eight rows
  // per fetch, lane l -> row r0 + l/8, physical chunk l%8 (logical chunk
  // (l%8) ^ swz_f(row)).
  uint32_t xoff[XF1];
#pragma unroll
  for (int j = 0; j < XF1; ++j) {
    const int row = wave * (BM / 8) + j * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ swz_f(row);
    xoff[j] = ((uint32_t)min(m0 + row, M - 1) * (uint32_t)k + (uint32_t)(lc * 8)) * 2u;
  }
  // This lane's weight row (tile row wrow = output feature n0 + wrow) and K
  // half of each block.
  const int wrow = wave * 32 + l32;
  const uint32_t coff = (uint32_t)(n0 + wrow) * (uint32_t)(k >> 1) + (uint32_t)half * 16u;
  // block constants of tile row erow (waves 0-3: c2 words, 4-7: c1 words)
  const int erow = (wave & 3) * 64 + lane;
  const uint32_t eblk = (uint32_t)(n0 + erow) * (uint32_t)kblocks;

  // Fetch i of K step ks into slot sl: 0 block constants, 1..XF X (sub-tile
  // (i-1)/XF1), XF+1.. codes of block i-XF-1.
  auto dma_one = [&](int i, int ks, int sl) {
    char* slot = smem + sl * kSlot;
    const uint32_t kb = (uint32_t)(kbase + ks) * KS;  // first block of the step
    if (i == 0) {
      if (wave_s < 4)
        dma_lds4s(r2, eblk, kb & ~3u, slot + kC2Off + (wave_s & 3) * 256);
      else
        dma_lds4(r1, ((eblk + kb) >> 8) * 4u, slot + kC2Off + 1024 + (wave_s & 3) * 256);
    } else if (i <= XF) {
      const int kk = (i - 1) / XF1, j = (i - 1) % XF1;
      dma_lds16s(rx, xoff[j], (kb + (uint32_t)kk) * (kBK * 2),
                 slot + kk * kSub + (wave_s * (BM / 8) + j * 8) * (kBK * 2));
    } else {
      const int kk = i - XF - 1;
      dma_lds16s(rc, coff, (kb + (uint32_t)kk) * 32u, slot + kCodeOff + (wave_s * KS + kk) * 1024);
    }
  };

  struct WTile {
    u32x4 v[KS];
    uint32_t q2;
    float q1;
  };
  auto read_w = [&](int sl, WTile& W) {
    const char* slot = smem + sl * kSlot;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      W.v[kk] = *reinterpret_cast<const u32x4*>(slot + kCodeOff + (wave_s * KS + kk) * 1024 + lane * 16);
    W.q2 = *reinterpret_cast<const uint32_t*>(slot + kC2Off + wrow * 4);
    W.q1 = *reinterpret_cast<const float*>(slot + kC2Off + 1024 + wrow * 4);
  };
  auto table = [&](const WTile& W, int blk) {  // blk counts from this split's first block
    return build_lut_pair(qh, block_scale((W.q2 >> (((blk + kbase * KS) & 3) * 8)) & 0xFFu, W.q1, mu));
  };

  // A fragment of row block mb, substep st (block st/4, K chunk half*4 +
  // st%4) of row mb*32 + l32 (the swizzle depends on mb only through its
  // parity).
  uint32_t aoff[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int st = 0; st < 4; ++st) aoff[p][st] = (uint32_t)(2 * swz(p * 32 + l32, half * 4 + st));
  auto read_a = [&](const char* xs, int st, u32x4 (&dst)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      dst[mb] = *reinterpret_cast<const u32x4*>(xs + (st >> 2) * kSub + aoff[mb & 1][st & 3] + (mb >> 1) * 8192);
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;

  // Pipeline as in k_fwd_rich: steps ks+1 and ks+2 in flight while step ks
  // is multiplied; substeps 0..NS-2 issue step ks+2's fetches; at substep
  // NS-2 the wave waits for its share of step ks+1 and meets the others at
  // a barrier; substep NS-1 reads step ks+1's codes, constants and first A
  // fragments.
#pragma unroll
  for (int i = 0; i < kLoads; ++i) dma_one(i, 0, 0);
#pragma unroll
  for (int i = 0; i < kLoads; ++i) dma_one(i, ksteps > 1 ? 1 : 0, 1);
  // LoRA up-projection first, while the first tiles land: acc = T_tile .
  // bf16(s B)_tile^T (B rounded to bf16 after scaling, as in k_fwd_rich).
  // Token rows past M and ranks past r load zeros.  With split K only the
  // first split carries it.
  if (rp > 0 && split == 0) {
    const BufRsrc rt = make_rsrc(T, (uint64_t)M * ldr * 2);
    const BufRsrc rb = make_rsrc(B, (uint64_t)d * r * 2);
    const int n = n0 + wrow;
    for (int jb = 0; jb < rp; jb += 16) {
      const int j0 = jb + half * 8;
      u32x4 top[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + mb * 32 + l32;
        const u32x4 v = ld_buf16(rt, ((uint32_t)min(m, M - 1) * (uint32_t)ldr + (uint32_t)(sec * r + j0)) * 2u);
        top[mb] = m < M ? v : u32x4{0u, 0u, 0u, 0u};
      }
      u32x4 bop;
      if ((r & 7) == 0) {
        const u32x4 v = ld_buf16(rb, ((uint32_t)n * (uint32_t)r + (uint32_t)min(j0, r - 8)) * 2u);
#pragma unroll
        for (int p = 0; p < 4; ++p)
          bop[p] = j0 < r ? pack_bf16x2(s * bf16_to_f32((uint16_t)(v[p] & 0xFFFFu)), s * bf16_to_f32((uint16_t)(v[p] >> 16)))
                          : 0u;
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int j = j0 + 2 * p;
          const float b0 = j < r ? s * bf16_to_f32(B[(size_t)n * r + j]) : 0.0f;
          const float b1 = j + 1 < r ? s * bf16_to_f32(B[(size_t)n * r + j + 1]) : 0.0f;
          bop[p] = pack_bf16x2(b0, b1);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32(top[mb], bop, acc[mb]);
    }
  }
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  WTile W;
  read_w(0, W);
  u32x4 wcur[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) wcur[kk] = W.v[kk];
  Lut tb[KS];
  tb[0] = table(W, 0);
  u32x4 bc = dequant8(wcur[0][0], tb[0]);
  u32x4 afr[2][MB];
  read_a(smem, 0, afr[0]);

  int sl_cur = 0;
  for (int ks = 0; ks < ksteps; ++ks) {
    const int sl_next = sl_cur == 2 ? 0 : sl_cur + 1;
    const int sl_far = sl_next == 2 ? 0 : sl_next + 1;
    const int kf = ks + 2 < ksteps ? ks + 2 : ksteps - 1;
    const char* xs = smem + sl_cur * kSlot;
    const char* xn = smem + sl_next * kSlot;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      acc[0] = mfma32(afr[st & 1][0], bc, acc[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (st < NS - 1) {
        read_a(xs, st + 1, afr[(st + 1) & 1]);
      } else {
        read_w(sl_next, W);
        read_a(xn, 0, afr[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
      u32x4 bn;
      if (st < NS - 1) {
        // the second block's table is formed early, at substep 1
        if (KS > 1 && st == 1) tb[1] = table(W, ks * KS + 1);
        bn = dequant8(wcur[(st + 1) >> 2][(st + 1) & 3], tb[(st + 1) >> 2]);
      } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) wcur[kk] = W.v[kk];
        tb[0] = table(W, (ks + 1) * KS);
        bn = dequant8(wcur[0][0], tb[0]);
      }
      if (st < NS - 1) {
        constexpr int kPer = (kLoads + NS - 2) / (NS - 1);  // fetches per substep
#pragma unroll
        for (int i = kPer * st; i < kPer * st + kPer && i < kLoads; ++i) dma_one(i, kf, sl_far);
      }
#pragma unroll
      for (int mb = 1; mb < MB; ++mb) acc[mb] = mfma32(afr[st & 1][mb], bc, acc[mb]);
#pragma unroll
      for (int i = 0; i < MB - 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        if (st < NS - 1 && i < 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (st == NS - 2) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      bc = bn;
    }
    sl_cur = sl_next;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  if (part != nullptr) {
    // fp32 partial of this split: lane (half, l32) of 32 x 32 block (mb)
    // holds rows 8*(e/4) + 4*half + e%4, column l32; 32 lanes store 128
    // contiguous bytes of a row
    float* pp = part + (size_t)split * M * d;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + mb * 32 + 8 * (e / 4) + 4 * half + e % 4;
        if (m < M) pp[(size_t)m * d + n0 + wave * 32 + l32] = acc[mb][e];
      }
    return;
  }
  // Output through LDS, 128 rows at a time: each wave stages its (up to) 128 x 32
  // sub-tile (rows of 64 B: four 16-byte chunks, chunk c of row r at
  // c ^ (r / 2 % 4)) and stores 16-byte row chunks.
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem) + wave * (128 * 32);
  auto sidx = [](int row, int ch) { return row * 32 + ((ch ^ ((row >> 1) & 3)) << 3); };
#pragma unroll
  for (int pass = 0; pass < BM / 128; ++pass) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = q * 32 + blk * 8 + half * 4 + i;
          stage[sidx(row, l32 >> 3) + (l32 & 7)] = (uint16_t)pack_bf16x2(acc[pass * 4 + q][blk * 4 + i], 0.0f);
        }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * 64 + lane, row = c >> 2, ch = c & 3;
      const int m = m0 + pass * 128 + row;
      if (m < M)
        *reinterpret_cast<u32x4*>(Y + (size_t)m * d + n0 + wave * 32 + ch * 8) =
            *reinterpret_cast<const u32x4*>(&stage[sidx(row, ch)]);
    }
    __syncthreads();
  }
}

// Sum of the split-K partials in split order, rounded once: Y = bf16(sum_s
// part[s]) over n = M*d outputs, four per thread.
__global__ __launch_bounds__(256) void k_sum_splits(const float* __restrict__ part, int ns, int64_t n,
                                                    uint16_t* __restrict__ Y) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 a = *reinterpret_cast<const f32x4*>(part + 4 * i);
    for (int sp = 1; sp < ns; ++sp) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(part + (size_t)sp * n + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += b[e];
    }
    *reinterpret_cast<u32x2*>(Y + 4 * i) = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  }
}

// ---------------------------------------------------------------- decode --

constexpr int kDecStep = 128;  // K per wave step (two NF4 blocks)

// One tile = 16*NB weight rows (NB 16-row MFMA column blocks) x a K range of
// 4*SPW steps of 128; wave w takes steps w, w+4, ...  Lane l supplies MFMA
// K group l/16; the four groups cover K offsets 0, 64, 32, 96 of the step, so
// lanes l and l+32 read the two halves of one 64-weight block and build its
// table together.  Every load of the wave is issued before any arithmetic
// (buffer loads from clamped addresses, no branches): the kernel streams the
// codes once and then spends its time decoding.
template <int MBLK, int SPW, int NB>
__global__ __launch_bounds__(256) void k_fwd_decode(const uint16_t* __restrict__ X, int M,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ c2,
                                                   const float* __restrict__ c1,
                                                   const float* __restrict__ mean, int d, int k, int dsec,
                                                   const uint16_t* __restrict__ A, int r, int ntw,
                                                   int steps_per_split, float* __restrict__ part,
                                                   int ldp, Nf4Table tab, const uint16_t* __restrict__ Xa) {
  __shared__ float red[4][MBLK][NB][64][4];
  constexpr int kRows = NB * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15, half = lane >> 5;
  const int kofs = 64 * (g & 1) + 32 * (g >> 1);
  const int tile = blockIdx.x, split = blockIdx.y;
  const int na = (int)gridDim.x - ntw;  // rank tiles first (their K loop is the longest)
  const bool is_w = tile >= na;
  const int row_base = is_w ? (tile - na) * kRows : tile * kRows;
  const int nsteps = (k + kDecStep - 1) / kDecStep;
  const int s_begin = split * steps_per_split;
  const int s_end = min(nsteps, s_begin + steps_per_split);
  const int kblocks = k / 64;
  const float mu = mean[is_w ? row_base / dsec : 0];
  float qh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qh[i] = half ? tab.q[8 + i] : tab.q[i];

  const BufRsrc rx = make_rsrc(is_w ? X : Xa, (uint64_t)M * k * 2);  // rank tiles read the adapter input
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);
  const BufRsrc ra = make_rsrc(A, (uint64_t)(r > 0 ? r : 1) * k * 2);

  // this lane's rows: weight row (or rank) row_base + nb*16 + l16, clamped;
  // byte offsets of their codes and block indices at K = 0.  Full 32-bit
  // products: row * k / 2 < d k / 2, token * k * 2 < 2 M k and m * ldp
  // (ldp = d + padded r, M <= 64) all stay below 2^32 for the shapes the
  // C ABI admits (d k, M k < 2^31), although d or k alone may exceed 2^24.
  int nrow[NB];
  bool nok[NB];
  uint32_t coff[NB], boff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = row_base + nb * 16 + l16;
    nok[nb] = is_w ? n < d : n < r;
    nrow[nb] = nok[nb] ? n : 0;
    const uint32_t nw = is_w ? (uint32_t)nrow[nb] : 0u;  // A tiles: harmless row-0 loads
    coff[nb] = nw * (uint32_t)(k >> 1);
    boff[nb] = nw * (uint32_t)kblocks;
  }
  uint32_t xoff[MBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb) xoff[mb] = (uint32_t)min(mb * 16 + l16, M - 1) * (uint32_t)k * 2u;
  const uint32_t xoob = (uint32_t)M * (uint32_t)k * 2u;  // X offsets here read zeros

  // This lane's K offset in step i of the wave, and whether it lies in the
  // matrix (past the end: X reads zeros, so nothing is added).
  int kcs[SPW];
  bool kok[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int st = s_begin + wave + 4 * i;
    const int k0 = st * kDecStep + kofs;
    kok[i] = st < s_end && k0 < k;
    kcs[i] = kok[i] ? k0 : 0;
  }
  auto load_x = [&](u32x4 (&xa)[SPW][MBLK][4]) {
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xa[i][mb][q] = ld_buf16(rx, kok[i] ? xoff[mb] + (uint32_t)(kcs[i] + 8 * q) * 2u : xoob);
  };

  f32x4 acc[MBLK][NB];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (is_w) {
    // Every load of the wave before any arithmetic: the codes and block
    // constants (the HBM stream) first, then X (cached).  Rows past d decode
    // row 0's codes into columns that are never stored.
    u32x4 wv[SPW][NB];
    uint32_t q2[SPW][NB];
    float q1[SPW][NB];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t blk = boff[nb] + (uint32_t)(kcs[i] >> 6);
        wv[i][nb] = ld_buf16(rc, coff[nb] + (uint32_t)(kcs[i] >> 1));
        q2[i][nb] = ld_buf4(r2, blk & ~3u) >> ((blk & 3u) * 8u);
        q1[i][nb] = __uint_as_float(ld_buf4(r1, (blk >> 8) * 4));
      }
    u32x4 xa[SPW][MBLK][4];
    load_x(xa);
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const Lut t = build_lut_pair(qh, block_scale(q2[i][nb] & 0xFFu, q1[i][nb], mu));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 b = dequant8(wv[i][nb][q], t);
#pragma unroll
          for (int mb = 0; mb < MBLK; ++mb) acc[mb][nb] = mfma16(xa[i][mb][q], b, acc[mb][nb]);
        }
      }
  } else {
    // Rows of A as bf16 "weights" (T = X A^T): only the column blocks that
    // hold ranks below r; each step's loads are issued together.
    const int nbv = min(NB, (r - row_base + 15) / 16);
    const uint32_t aoob = (uint32_t)r * (uint32_t)k * 2u;  // A offsets here read zeros
    u32x4 xa[SPW][MBLK][4];
    load_x(xa);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      u32x4 av[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (nb < nbv) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            av[nb][q] = ld_buf16(ra, nok[nb] ? ((uint32_t)nrow[nb] * (uint32_t)k + (uint32_t)(kcs[i] + 8 * q)) * 2u
                                             : aoob);
        }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (nb < nbv) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) acc[mb][nb] = mfma16(xa[i][mb][q], av[nb][q], acc[mb][nb]);
        }
    }
  }

  // Sum the four waves in a fixed order, ((w0 + w1) + w2) + w3; wave w
  // adds and stores column block nb = w.
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4*>(&red[wave][mb][nb][lane][0]) = acc[mb][nb];
  __syncthreads();
  if (wave < NB) {
    const int nb = wave;
    const int col_base = is_w ? row_base : d + row_base;
    const int col_lim = is_w ? d : d + r;
    const int col = col_base + nb * 16 + l16;
    float* __restrict__ pw = part + (size_t)split * M * ldp + col;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
      f32x4 v = *reinterpret_cast<const f32x4*>(&red[0][mb][nb][lane][0]);
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(&red[w][mb][nb][lane][0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += o[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = mb * 16 + 4 * g + e;
        if (m < M && col < col_lim) pw[(uint32_t)m * (uint32_t)ldp] = v[e];
      }
    }
  }
}

// Token-poor forward for k a multiple of 256 (the usual case).  A work-group
// owns kDcRows = 64 weight rows and a K range of whole 256-wide chunks; its
// four waves take 16 rows each over the same K, so the chunk's X slab is
// fetched once per work-group and shared.  Each chunk (X slab, the rows'
// codes, their c2 words and c1 scales) is fetched global->LDS with 1 KB
// coalesced fetches into one of two slots, the next chunk in flight while
// this one is decoded.  Lane (n, g) of a wave owns weight row n of the wave
// and the chunk's 64-weight block g: it builds that block's table alone and
// decodes its 64 codes into eight MFMA B operands (16x16x32; MFMA u takes K
// offsets 64g + 8u .. 64g + 8u + 7 in lane group g, X read with the same
// mapping), so every weight is decoded once and no table is shared between
// lanes.  The 16-byte pieces of the X slab and of the codes are placed (XOR
// swizzle chosen per fetch lane) so that the LDS reads are free of bank
// conflicts.  Waves own disjoint rows: the partial of the K range goes
// straight to the workspace, and k_fwd_decode_finish sums the splits.
// The first work-groups of the grid form partial T = X A^T from global
// loads, 16 ranks each (all adapters' ranks when tokens pick adapters).
//
// (Measured on the decode shapes: issuing the loads is not the limit; the
// kernel is bound by per-wave latency chains and the decode arithmetic.  A
// single-launch form whose last-arriving work-group per tile summed the
// partials was slower: its counters and coherent partial traffic cost more
// than the second launch.)
constexpr int kDcK = 256;     // K per chunk
constexpr int kDcWaves = 4;   // waves per work-group (16 weight rows each)
constexpr int kDcRows = 16 * kDcWaves;

template <int MT>
struct DcSlot {
  static constexpr int kX = 0;                        // MT*16 token rows of 512 B
  static constexpr int kCodes = MT * 16 * 512;         // kDcRows rows of 128 B
  static constexpr int kC2 = kCodes + kDcRows * 128;   // c2 words (blocks 4c..4c+3) per row
  static constexpr int kC1 = kC2 + kDcRows * 4;        // c1 scale per row
  static constexpr int kBytes = kC1 + kDcRows * 4;
};

template <int MT>
__global__ __launch_bounds__(64 * kDcWaves) void k_fwd_dec(const uint16_t* __restrict__ X, int M,
                                                const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ c2,
                                                const float* __restrict__ c1,
                                                const float* __restrict__ mean, int d, int k, int dsec,
                                                const uint16_t* __restrict__ A, int r, int ntw, int cps,
                                                float* __restrict__ part, int ldp, Nf4Table tab,
                                                const uint16_t* __restrict__ Xa) {
  using S = DcSlot<MT>;
  __shared__ __attribute__((aligned(16))) char smem[2 * S::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int n = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x, split = blockIdx.y;
  // The rank tiles (partial T) come first in the grid: their serial K
  // loop is the longest per work-group, so they start before the weight
  // tiles rather than after them.
  const int na = (int)gridDim.x - ntw;
  const bool is_w = tile >= na;
  const int row0 = (tile - na) * kDcRows;  // weight tiles
  const int c0 = split * cps;
  const int nc = min(cps, k / kDcK - c0);
  const int kblocks = k / 64;
  const BufRsrc rx = make_rsrc(X, (uint64_t)M * k * 2);
  const uint32_t xoob = (uint32_t)M * (uint32_t)k * 2u;  // X offsets here read zeros

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (!is_w) {
    // Rank tile: partial T for the 16 ranks 16*tile + n (B operands straight
    // from A, A operands straight from X).  The four waves split the K
    // range (half chunk h, 32 K per lane group, to wave h % 4), each with
    // the next half chunk's loads in flight, and are summed in LDS in a
    // fixed order; a work-group thus moves 16 ranks' share of A however
    // many ranks there are.
    const BufRsrc ra = make_rsrc(A, (uint64_t)r * k * 2);
    const BufRsrc rxa = make_rsrc(Xa, (uint64_t)M * k * 2);  // the adapter path's input
    const uint32_t aoob = (uint32_t)r * (uint32_t)k * 2u;
    const int rank = 16 * tile + n;
    auto load = [&](int h, u32x4 (&av)[4], u32x4 (&xv)[4][MT]) {
      const int kb = (c0 + h / 2) * kDcK + 64 * g + 32 * (h & 1);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = ld_buf16(ra, rank < r ? ((uint32_t)rank * (uint32_t)k + (uint32_t)(kb + 8 * u)) * 2u : aoob);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + n;
          xv[u][mt] = ld_buf16(rxa, m < M ? ((uint32_t)m * (uint32_t)k + (uint32_t)(kb + 8 * u)) * 2u : xoob);
        }
      }
    };
    auto mma = [&](const u32x4 (&av)[4], const u32x4 (&xv)[4][MT]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(xv[u][mt], av[u], acc[mt]);
    };
    const int nh = 2 * nc;
    if constexpr (MT <= 4) {
      u32x4 a0[4], x0[4][MT], a1[4], x1[4][MT];
      if (wave_s < nh) load(wave_s, a0, x0);
      for (int h = wave_s; h < nh; h += 2 * kDcWaves) {
        if (h + kDcWaves < nh) load(h + kDcWaves, a1, x1);
        mma(a0, x0);
        if (h + kDcWaves < nh) {
          if (h + 2 * kDcWaves < nh) load(h + 2 * kDcWaves, a0, x0);
          mma(a1, x1);
        }
      }
    } else {  // more token blocks: one set of operands in registers
      u32x4 a0[4], x0[4][MT];
      for (int h = wave_s; h < nh; h += kDcWaves) {
        load(h, a0, x0);
        mma(a0, x0);
      }
    }
    float* red = reinterpret_cast<float*>(smem);  // (kDcWaves - 1) x MT x 64 lanes x 4
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4*>(red + (((wave - 1) * MT + mt) * 64 + lane) * 4) = acc[mt];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 v = acc[mt];
#pragma unroll
        for (int w = 0; w < kDcWaves - 1; ++w) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(red + ((w * MT + mt) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += o[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * mt + 4 * g + e;
          if (m < M && rank < r) part[((size_t)split * M + m) * ldp + d + rank] = v[e];
        }
      }
    }
    return;
  }

  const float mu = mean[row0 / dsec];  // the 64 rows of a tile lie in one section
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);

  // Fetch lanes.  X: fetch j (wave w issues j = w + 8i) fills token rows
  // 2j, 2j+1; lane l -> token 2j + l/32, physical piece l%32 holding logical
  // piece (l%32) ^ (token%16).  Codes: fetch j (wave w issues 2w, 2w+1)
  // fills rows 8j..8j+7; lane l -> row 8j + l/8, piece (l%8) ^ (row/2%8).
  // c2 words of 64 rows per fetch: waves 0 .. CF-1; c1 scales: waves
  // CF .. 2CF-1.
  constexpr int XF = 8 * MT / kDcWaves;  // X fetches per wave and chunk
  constexpr int CF = kDcRows / 64;       // constant fetches of each kind
  static_assert(XF * kDcWaves == 8 * MT && 2 * CF <= kDcWaves, "fetch split");
  const uint32_t coob = (uint32_t)d * (uint32_t)(k >> 1);  // code offsets here read zeros
  uint32_t xo[XF], co[2];
#pragma unroll
  for (int i = 0; i < XF; ++i) {
    const int t = 2 * (wave + kDcWaves * i) + (lane >> 5);
    const int lp = (lane & 31) ^ (t & 15);
    xo[i] = t < M ? ((uint32_t)t * (uint32_t)k + (uint32_t)(lp * 8)) * 2u : xoob;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (2 * wave + i) + (lane >> 3);
    const int lp = (lane & 7) ^ ((row >> 1) & 7);
    co[i] = row0 + row < d ? (uint32_t)(row0 + row) * (uint32_t)(k >> 1) + (uint32_t)(lp * 16) : coob;
  }
  const int erow = 64 * (wave % CF) + lane;
  const bool rok = row0 + erow < d;
  const uint32_t eblk = (uint32_t)(rok ? row0 + erow : 0) * (uint32_t)kblocks;

  auto fetch = [&](int c, int sl) {
    char* slot = smem + sl * S::kBytes;
    const uint32_t kb = (uint32_t)(c0 + c) * kDcK;
#pragma unroll
    for (int i = 0; i < XF; ++i)
      dma_lds16(rx, xo[i] == xoob ? xoob : xo[i] + kb * 2u, slot + S::kX + (wave_s + kDcWaves * i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma_lds16(rc, co[i] == coob ? coob : co[i] + kb / 2u, slot + S::kCodes + (2 * wave_s + i) * 1024);
    if (wave_s < CF) dma_lds4(r2, eblk + kb / 64u, slot + S::kC2 + 256 * wave_s);
    else if (wave_s < 2 * CF) dma_lds4(r1, ((eblk + kb / 64u) >> 8) * 4u, slot + S::kC1 + 256 * (wave_s - CF));
  };

  fetch(0, 0);
  if (nc > 1) fetch(1, 1);
  const int row = 16 * wave + n;
  const int sg = (row >> 1) & 7;
  for (int c = 0; c < nc; ++c) {
    // this wave's fetches of chunk c have landed once only chunk c+1's
    // (XF + 2, plus one constant fetch for waves below 2 CF) are in flight
    if (c + 1 < nc) {
      if (wave_s < 2 * CF)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(XF + 3) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(XF + 2) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* slot = smem + (c & 1) * S::kBytes;
    const uint32_t q2 = *reinterpret_cast<const uint32_t*>(slot + S::kC2 + row * 4);
    const float q1 = *reinterpret_cast<const float*>(slot + S::kC1 + row * 4);
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(slot + S::kCodes + row * 128 + (((2 * g) ^ sg) << 4));
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(slot + S::kCodes + row * 128 + (((2 * g + 1) ^ sg) << 4));
    const Lut t = build_lut(tab, block_scale((q2 >> (8 * g)) & 0xFFu, q1, mu));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const u32x4 b = dequant8(u < 4 ? w0[u] : w1[u - 4], t);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(slot + S::kX + (16 * mt + n) * 512 + (((8 * g + u) ^ n) << 4));
        acc[mt] = mfma16(a, b, acc[mt]);
      }
    }
    if (c + 2 < nc) {
      __syncthreads();
      fetch(c + 2, c & 1);
    }
  }
  const int col = row0 + row;
  if (col < d) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * g + e;
        if (m < M) part[((size_t)split * M + m) * ldp + col] = acc[mt][e];
      }
  }
}

// Single-launch token-poor forward: up to 16 tokens, k a multiple of 256,
// at most 16 adapter ranks per section, one adapter for every token and no
// LoRA dropout (those keep the split-K kernels above).  A work-group owns
// 16*NB weight rows over the whole K, so no partial sum leaves it: its
// eight waves take the 128-wide K steps in turn (step h to wave h % 8), each
// wave with two LDS slots of its own, and their accumulators are summed in
// LDS in a fixed order at the end.
//  - X and A: a step's slab of X (16 token rows x 256 B) and of A (16 rank
//    rows x 256 B) is fetched global->LDS by the wave that uses it, 1 KB
//    per fetch (four whole 256-byte row pieces), so a work-group reads X
//    and A once each, in whole lines; rows past M (tokens) or r (ranks)
//    read zeros.  The 16-byte piece p of row t sits at p ^ (t % 16), which
//    keeps the MFMA reads free of bank conflicts.
//  - MFMA u (u = 0..3) of a step contracts over K offsets 32g + 8u .. + 7 in
//    lane group g, for the weight rows (B operand: lane (n, g) decodes word
//    4g + u of row n's step, its four words one 16-byte load) and for the
//    ranks of T = X A^T alike, so one X fragment feeds both.  Lane groups
//    2p and 2p+1 share one 64-weight block: each builds half of its table
//    and v_permlane16_swap hands over the other half.
// T is rounded to bf16 once (as in the token-rich path), s T B^T goes into
// the row blocks' sums with one more MFMA (B operand bf16(s B), zero past
// r), and Y is rounded once.  The first work-group of each section saves T.
// Every pass of the K loop issues the same loads (a wave with an odd number
// of steps ends with a phantom one that adds zeros), so each wait is a
// static count covering exactly the step about to be used.
constexpr int kD1Waves = 8;
constexpr int kD1K = 128;             // K per step
constexpr int kD1Slab = 16 * 2 * kD1K;  // 16 rows of one step (X or A)

// Table of one block built by the lanes of two neighbouring 16-lane rows
// (same block): the even row forms the products of levels 0..7, the odd row
// those of levels 8..15, and v_permlane16_swap gives every lane both.
__device__ __forceinline__ Lut build_lut_rows(const Nf4Table& t, float ah, bool odd) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = odd ? t.q[8 + 2 * i] : t.q[2 * i];
    const float q1 = odd ? t.q[9 + 2 * i] : t.q[2 * i + 1];
    w[i] = pack_bf16x2(__fmul_rn(q0, ah), __fmul_rn(q1, ah));
  }
  const uint32_t pl0 = perm(w[1], w[0], 0x06040200u), pl1 = perm(w[3], w[2], 0x06040200u);
  const uint32_t ph0 = perm(w[1], w[0], 0x07050301u), ph1 = perm(w[3], w[2], 0x07050301u);
  Lut r;
#if defined(__HIP_DEVICE_COMPILE__)  // device-only builtin; the host pass never runs this
  // result [0]: the even row's value, [1]: the odd row's
  const auto s0 = __builtin_amdgcn_permlane16_swap(pl0, pl0, false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(pl1, pl1, false, false);
  const auto s2 = __builtin_amdgcn_permlane16_swap(ph0, ph0, false, false);
  const auto s3 = __builtin_amdgcn_permlane16_swap(ph1, ph1, false, false);
  r.L0 = s0[0]; r.L2 = s0[1];
  r.L1 = s1[0]; r.L3 = s1[1];
  r.H0 = s2[0]; r.H2 = s2[1];
  r.H1 = s3[0]; r.H3 = s3[1];
#else
  r.L0 = r.L2 = pl0; r.L1 = r.L3 = pl1; r.H0 = r.H2 = ph0; r.H1 = r.H3 = ph1;
#endif
  return r;
}

// The up-projection's B rows for the single-launch kernels' epilogue:
// lane (n, g < 2) of wave nb < NB holds B[col][8g .. 8g+7] of its output
// row col = row0 + 16 nb + n (clamped to d - 1), zero past r.
template <int NB>
__device__ __forceinline__ u32x4 d1_b_rows(const uint16_t* __restrict__ B, int r, int d, int row0, int wave_s,
                                           int n, int g) {
  u32x4 bw = u32x4{0u, 0u, 0u, 0u};
  if (wave_s < NB && g < 2 && 8 * g < r) {
    const int rowc = min(row0 + wave_s * 16 + n, d - 1);
    const uint16_t* Bp = B + (size_t)rowc * r + 8 * g;
    if ((r & 7) == 0) {
      bw = *reinterpret_cast<const u32x4*>(Bp);
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = 8 * g + 2 * p < r ? Bp[2 * p] : 0u;
        const uint32_t hi = 8 * g + 2 * p + 1 < r ? Bp[2 * p + 1] : 0u;
        bw[p] = lo | (hi << 16);
      }
    }
  }
  return bw;
}

// Epilogue of the single-launch kernels, after the K loop (every fetch
// landed, a barrier passed): the waves' accumulators (NB row blocks, then
// T with adapters) are summed through `red` in a fixed order,
// ((w0 + w1) + w2) + ...; T is rounded to bf16 once, kept in tsh for the
// up-projection and saved transposed (rows sec*r + n) by the first
// work-group of the section; s T B^T goes in with one more MFMA (A operand
// T[n][8g .. 8g+7], ranks past 15 zero; B operand bf16(s B[col][8g ..]),
// zero past r) and Y is rounded once.
template <int NB, bool LORA>
__device__ __forceinline__ void d1_epilogue(const f32x4 (&acc)[NB + (LORA ? 1 : 0)], f32x4* red,
                                            uint16_t (*tsh)[16], const u32x4& bw, int wave, int lane, int n,
                                            int g, int row0, int sec, int dsec, int M, int d, int r, float s,
                                            uint16_t* __restrict__ Y, uint16_t* __restrict__ Tsave, int ldt) {
  constexpr int NA = LORA ? 1 : 0;
#pragma unroll
  for (int i = 0; i < NB + NA; ++i) red[(wave * (NB + NA) + i) * 64 + lane] = acc[i];
  __syncthreads();
  f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave < NB + NA) {
    v = red[wave * 64 + lane];
#pragma unroll
    for (int w = 1; w < kD1Waves; ++w) {
      const f32x4 o = red[(w * (NB + NA) + wave) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += o[e];
    }
    if (LORA && wave == NB) {
      // lane holds T[4g + e][n]
      const bool save = Tsave != nullptr && row0 % dsec == 0 && n < r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h = (uint16_t)pack_bf16x2(v[e], 0.0f);
        tsh[4 * g + e][n] = h;
        const int m = 4 * g + e;
        if (save && m < M) Tsave[(size_t)(sec * r + n) * ldt + m] = h;
      }
    }
  }
  if constexpr (LORA) __syncthreads();
  if (wave < NB) {
    const int col = row0 + wave * 16 + n;
    if constexpr (LORA) {
      const u32x4 ta = g < 2 ? *reinterpret_cast<const u32x4*>(&tsh[n][8 * g]) : u32x4{0u, 0u, 0u, 0u};
      u32x4 bb;
#pragma unroll
      for (int p = 0; p < 4; ++p) bb[p] = pack_bf16x2(s * bf16_lo(bw[p]), s * bf16_hi(bw[p]));
      v = mfma16(ta, bb, v);
    }
    if (col < d) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * g + e;
        if (m < M) Y[(size_t)m * d + col] = (uint16_t)pack_bf16x2(v[e], 0.0f);
      }
    }
  }
}

template <int NB, bool LORA>
__global__ __launch_bounds__(64 * kD1Waves) void k_fwd_dec1(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ c2,
    const float* __restrict__ c1, const float* __restrict__ mean, int d, int k, int dsec,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ Y,
    uint16_t* __restrict__ Tsave, int ldt, Nf4Table tab) {
  constexpr int NA = LORA ? 1 : 0;
  constexpr int kSlot = (1 + NA) * kD1Slab;  // X slab, then A slab
  // two slots per wave; after the K loop the same bytes hold the waves'
  // accumulators for the fixed-order sum
  __shared__ __attribute__((aligned(16))) char smem[kD1Waves * 2 * 2 * kD1Slab];
  __shared__ __attribute__((aligned(16))) uint16_t tsh[16][16];  // bf16 T, token x rank
  static_assert(kD1Waves * (NB + NA) * 64 * 16 <= kD1Waves * 2 * 2 * kD1Slab, "reduction fits the slots");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: scalar loop bounds
  const int n = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16 * NB;
  const int sec = row0 / dsec;  // all rows of a work-group lie in one section
  const float mu = mean[sec];
  const int kblocks = k / 64;
  const int nsteps = k / kD1K;

  const BufRsrc rx = make_rsrc(X, (uint64_t)M * k * 2);
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);
  const BufRsrc ra = make_rsrc(A, (uint64_t)(sec + 1) * (r > 0 ? r : 1) * k * 2);
  const uint32_t xoob = (uint32_t)M * (uint32_t)k * 2u;  // reads zeros
  const uint32_t aoob = (uint32_t)(sec + 1) * (uint32_t)(r > 0 ? r : 1) * (uint32_t)k * 2u;

  // The up-projection's B rows, loaded before anything else (so that the
  // first step's wait covers them) and used only after the K loop.  (With
  // r % 8 == 0 one 16-byte load, so nothing has to wait for it here.)
  u32x4 bw = u32x4{0u, 0u, 0u, 0u};
  if constexpr (LORA) bw = d1_b_rows<NB>(B, r, d, row0, wave_s, n, g);

  // Fetch lanes of a slab: fetch i fills rows 4i .. 4i+3, lane l row
  // 4i + l/16, physical piece l % 16 holding logical piece (l % 16) ^ row.
  uint32_t xo[4], ao[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * i + (lane >> 4);
    const uint32_t lp = (uint32_t)((lane & 15) ^ t);
    xo[i] = t < M ? ((uint32_t)t * (uint32_t)k + lp * 8u) * 2u : xoob;
    ao[i] = (LORA && t < r) ? ((uint32_t)(sec * r + t) * (uint32_t)k + lp * 8u) * 2u : aoob;
  }
  uint32_t coff[NB], boff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint32_t row = (uint32_t)min(row0 + nb * 16 + n, d - 1);  // rows past d: never stored
    coff[nb] = row * (uint32_t)(k >> 1) + (uint32_t)g * 16u;        // words 4g .. 4g+3 of the step
    boff[nb] = row * (uint32_t)kblocks + (uint32_t)(g >> 1);
  }

  struct Step {
    u32x4 w[NB];
    uint32_t q2[NB];
    float q1[NB];
  };
  char* myslots = smem + wave_s * 2 * kSlot;
  // The wave's i-th step.  Past its last one (i >= nmine) a step is a
  // phantom: its X and A slabs read zeros (so its MFMAs add zeros) and its
  // code words repeat the last step's, so that every pass of the loop below
  // issues the same loads and has no branch between a step's loads and its
  // arithmetic.
  const int nmine = wave_s < nsteps ? (nsteps - 1 - wave_s) / kD1Waves + 1 : 0;
  const int hlast = wave_s < nsteps ? wave_s + (nmine - 1) * kD1Waves : 0;
  auto load = [&](int i, int sl, Step& S) {
    const bool real = i < nmine;
    const uint32_t kb = (uint32_t)(real ? wave_s + i * kD1Waves : hlast) * kD1K;
    char* slot = myslots + sl * kSlot;
#pragma unroll
    for (int f = 0; f < 4; ++f) dma_lds16(rx, (!real || xo[f] == xoob) ? xoob : xo[f] + kb * 2u, slot + f * 1024);
    if constexpr (LORA) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
        dma_lds16(ra, (!real || ao[f] == aoob) ? aoob : ao[f] + kb * 2u, slot + kD1Slab + f * 1024);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      S.w[nb] = ld_buf16(rc, coff[nb] + kb / 2u);
      const uint32_t blk = boff[nb] + kb / 64u;
      S.q2[nb] = ld_buf1(r2, blk);
      S.q1[nb] = __uint_as_float(ld_buf4(r1, (blk >> 8) * 4u));
    }
  };
  constexpr int kLoads = 4 * (1 + NA) + 3 * NB;  // per step and lane

  f32x4 acc[NB + NA];
#pragma unroll
  for (int i = 0; i < NB + NA; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool odd = (g & 1) != 0;
  auto compute = [&](const Step& S, int sl) {
    const char* xs = myslots + sl * kSlot + n * 256;
    Lut t[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) t[nb] = build_lut_rows(tab, block_scale(S.q2[nb], S.q1[nb], mu), odd);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = ((4 * g + u) ^ n) << 4;
      const u32x4 xa = *reinterpret_cast<const u32x4*>(xs + pc);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16(xa, dequant8(S.w[nb][u], t[nb]), acc[nb]);
      if constexpr (LORA) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(xs + kD1Slab + pc);
        acc[NB] = mfma16(xa, av, acc[NB]);
      }
    }
  };

  // steps wave, wave + 8, ...: two register sets and two LDS slots in turn
  Step st0, st1;
  load(0, 0, st0);
  for (int i = 0; i < nmine; i += 2) {
    load(i + 1, 1, st1);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");  // step i has landed
    compute(st0, 0);
    // slot 0 is refilled only once this wave's reads of it have returned
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    load(i + 2, 0, st0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");  // step i + 1 has landed
    compute(st1, 1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  // every fetch (the last, unused ones included) has landed before the
  // slots are reused
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();

  d1_epilogue<NB, LORA>(acc, reinterpret_cast<f32x4*>(smem), tsh, bw, wave, lane, n, g, row0, sec, dsec, M, d, r, s, Y,
                        Tsave, ldt);
}

// k_fwd_dec1 with every load of the work-group in flight at once, for
// k <= 8 * S * 128 (S <= 4 steps per wave, k <= 4096).  The two-slot ring
// above issues a wave's third step only once its first has been used, so
// a call pays two or three memory round trips one after another; here the
// wave owns S consecutive K steps and issues all of their loads before any
// arithmetic, then waits for them one step at a time.
//  - X slabs go global->LDS as above, S slots per wave (128 KB at S = 4).
//  - A (with adapters) goes straight to registers, 16 rank rows x 64
//    contiguous bytes per load: MFMA u of the T product contracts over K
//    offsets 32u + 8g .. + 7 in lane group g (the usual operand layout),
//    and reads its X operand from the same slab at those offsets.  The
//    weight rows keep the layout above (K offsets 32g + 8u, one 16-byte
//    code load per step), so each step reads X fragments in both layouts.
//  - The block constants of a lane's S steps come from one 8-byte load of
//    c2 and two loads of c1 (its first and last block's groups).
// Step h of the K loop is owned by wave h / S; a wave whose steps pass the
// end of K reads zeros for X and A there, so those MFMAs add zeros.
// (Fewer round trips pay without adapters; with them the call's time
// follows the bytes each CU must fetch -- all of X and A, 256 KB at
// k = 4096 -- however they are loaded.  S is capped by the LDS: each step
// of each wave holds a 4 KB X slab, 128 KB over eight waves at S = 4.)
template <int NB, bool LORA, int S>
__global__ __launch_bounds__(64 * kD1Waves) void k_fwd_dec1s(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ c2,
    const float* __restrict__ c1, const float* __restrict__ mean, int d, int k, int dsec,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ Y,
    uint16_t* __restrict__ Tsave, int ldt, Nf4Table tab) {
  constexpr int NA = LORA ? 1 : 0;
  constexpr int kXs = kD1Waves * S * kD1Slab;
  constexpr int kRed = kD1Waves * (NB + NA) * 64 * 16;
  // S X slabs per wave; after the K loop the same bytes hold the waves'
  // accumulators for the fixed-order sum
  __shared__ __attribute__((aligned(16))) char smem[kXs > kRed ? kXs : kRed];
  __shared__ __attribute__((aligned(16))) uint16_t tsh[16][16];  // bf16 T, token x rank
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int n = lane & 15, g = lane >> 4, gg = g >> 1;
  const int row0 = blockIdx.x * 16 * NB;
  const int sec = row0 / dsec;
  const float mu = mean[sec];
  const int kblocks = k / 64;
  const int nsteps = k / kD1K;
  const int h0 = wave_s * S;  // this wave's first step

  const BufRsrc rx = make_rsrc(X, (uint64_t)M * k * 2);
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);
  const BufRsrc ra = make_rsrc(A, (uint64_t)(sec + 1) * (r > 0 ? r : 1) * k * 2);
  const uint32_t xoob = (uint32_t)M * (uint32_t)k * 2u;
  const uint32_t aoob = (uint32_t)(sec + 1) * (uint32_t)(r > 0 ? r : 1) * (uint32_t)k * 2u;

  // the up-projection's B rows, as in k_fwd_dec1
  u32x4 bw = u32x4{0u, 0u, 0u, 0u};
  if constexpr (LORA) bw = d1_b_rows<NB>(B, r, d, row0, wave_s, n, g);

  // X fetch lanes: fetch f of a slab fills rows 4f .. 4f+3, lane l row
  // 4f + l/16, physical piece l % 16 holding logical piece (l % 16) ^ row.
  uint32_t xo[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int t = 4 * f + (lane >> 4);
    const uint32_t lp = (uint32_t)((lane & 15) ^ t);
    xo[f] = t < M ? ((uint32_t)t * (uint32_t)k + lp * 8u) * 2u : xoob;
  }
  // A rows in registers: lane (n, g) holds rank n, bytes 64u + 16g of a step
  const bool arow = LORA && n < r;
  const uint32_t ao = arow ? (uint32_t)(sec * r + n) * (uint32_t)k * 2u + 16u * (uint32_t)g : aoob;
  uint32_t coff[NB], b0[NB];
  u32x2 q2w[NB];
  uint32_t q2o[NB];  // byte offset of step h0's block (lane group pair 0) in q2w
  float q1a[NB], q1b[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint32_t row = (uint32_t)min(row0 + nb * 16 + n, d - 1);  // rows past d: never stored
    coff[nb] = row * (uint32_t)(k >> 1) + (uint32_t)g * 16u;
    b0[nb] = row * (uint32_t)kblocks + 2u * (uint32_t)h0;  // block of step h0, lane group pair 0
    // kblocks % 4 == 0, so b0 % 4 == (2 h0) % 4: the 8 bytes at b0 & ~3
    // hold the constants of all S steps (2S <= 8 bytes from offset b0 % 4).
    // Where those 8 bytes would run past the end of c2 (nblk, a multiple
    // of 4), the load starts 4 bytes lower: the steps' bytes then all lie
    // in the last word, and the load stays wholly inside the buffer.
    uint32_t q2a = b0[nb] & ~3u;
    if (q2a + 8u > nblk) q2a -= 4u;
    q2o[nb] = b0[nb] - q2a;
    q2w[nb] = ld_buf8(r2, q2a);
    q1a[nb] = __uint_as_float(ld_buf4(r1, (b0[nb] >> 8) * 4u));
    q1b[nb] = __uint_as_float(ld_buf4(r1, ((b0[nb] + 2u * S - 1u) >> 8) * 4u));
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  constexpr int kLoads = 4 + 4 * NA + NB;  // per step and lane, in this order
  char* myslots = smem + wave_s * S * kD1Slab;
  u32x4 cw[S][NB];
  u32x4 av[S][4];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const bool real = h0 + i < nsteps;
    const uint32_t kb = (uint32_t)(real ? h0 + i : nsteps - 1) * kD1K;
    char* slot = myslots + i * kD1Slab;
#pragma unroll
    for (int f = 0; f < 4; ++f) dma_lds16(rx, (!real || xo[f] == xoob) ? xoob : xo[f] + kb * 2u, slot + f * 1024);
    if constexpr (LORA) {
#pragma unroll
      for (int u = 0; u < 4; ++u) av[i][u] = ld_buf16(ra, (!real || !arow) ? aoob : ao + kb * 2u + 64u * u);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) cw[i][nb] = ld_buf16(rc, coff[nb] + kb / 2u);
    // each step's loads stay together, in step order, and ahead of every
    // wait below (the waits count the loads issued after a step's fetches;
    // the scheduler would otherwise sink loads it sees as invariant)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4 acc[NB + NA];
#pragma unroll
  for (int i = 0; i < NB + NA; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool odd = (g & 1) != 0;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    // loads issued after step i's: (S - 1 - i) steps' worth
    if (i == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 1) * kLoads) : "memory");
    if (i == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S > 1 ? S - 2 : 0) * kLoads) : "memory");
    if (i == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S > 2 ? S - 3 : 0) * kLoads) : "memory");
    if (i == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S > 3 ? S - 4 : 0) * kLoads) : "memory");
    const char* xs = myslots + i * kD1Slab + n * 256;
    Lut t[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t o = q2o[nb] + 2u * i + (uint32_t)gg;  // byte of this step's block in q2w
      const uint64_t w64 = ((uint64_t)q2w[nb].y << 32) | q2w[nb].x;
      const uint32_t q2 = (uint32_t)(w64 >> (8u * (o & 7u))) & 0xFFu;  // (o <= 7 for every real step)
      const uint32_t blk = b0[nb] + 2u * i + (uint32_t)gg;
      const float q1 = (blk >> 8) == (b0[nb] >> 8) ? q1a[nb] : q1b[nb];
      t[nb] = build_lut_rows(tab, block_scale(q2, q1, mu), odd);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 xa = *reinterpret_cast<const u32x4*>(xs + (((4 * g + u) ^ n) << 4));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16(xa, dequant8(cw[i][nb][u], t[nb]), acc[nb]);
      if constexpr (LORA) {
        const u32x4 xt = *reinterpret_cast<const u32x4*>(xs + (((4 * u + g) ^ n) << 4));
        acc[NB] = mfma16(xt, av[i][u], acc[NB]);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();

  d1_epilogue<NB, LORA>(acc, reinterpret_cast<f32x4*>(smem), tsh, bw, wave, lane, n, g, row0, sec, dsec, M, d, r, s, Y,
                        Tsave, ldt);
}

// One work-group per (token, 256 output features): sum the split partials,
// form T (rounded to bf16, as in the token-rich path), add s T B^T, round.
// Sections: T has rt = nsec * r ranks; output feature n (section n / dsec)
// takes ranks (n / dsec) * r .. + r - 1.
// Per-token adapters (idx != nullptr): T has rt = nad * r ranks, those of
// every adapter; token m takes adapter a = idx[m] (ranks a*r .., B_a at
// B + a*d*r), or none when a is outside [0, nad).
// Every load the thread needs -- its first eight split partials of Y, those
// of its rank of T, and its output feature's row of B -- is issued before
// any of them is used, so the kernel waits for memory once (splits past
// the eighth, which only the k % 256 != 0 kernel produces at large k, are
// added after, eight at a time, in split order).
constexpr int kFinBatch = 8;

__global__ __launch_bounds__(256) void k_fwd_decode_finish(const float* __restrict__ part, int nsplit,
                                                          int M, int d, int ldp,
                                                          const uint16_t* __restrict__ B, int r, int rt,
                                                          int dsec, const int* __restrict__ idx, float s,
                                                          uint16_t* __restrict__ Y,
                                                          uint16_t* __restrict__ Tsave, int ldt) {
  __shared__ float tsh[kMaxSections * kMaxRank];  // all sections' ranks (one per thread)
  static_assert(kMaxSections * kMaxRank <= 256, "one rank of T per thread");
  const int m = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = blockIdx.x * 256 + tid;
  const int nc = n < d ? n : d - 1;
  int a = 0;
  bool lora = r > 0;
  if (idx != nullptr) {
    a = idx[m];
    lora = lora && a >= 0 && a < rt / r;
  }
  const int t0 = idx != nullptr ? a * r : 0;  // first rank of this token's T
  const int nt = idx != nullptr ? r : rt;     // ranks kept
  const bool tl = lora && tid < nt;
  const size_t stride = (size_t)M * ldp;
  const float* __restrict__ py = part + (size_t)m * ldp + nc;
  const float* __restrict__ pt = part + (size_t)m * ldp + d + t0 + (tl ? tid : 0);
  const uint16_t* __restrict__ Bn = B + (size_t)a * d * r + (size_t)nc * r;

  float yv[kFinBatch], tv[kFinBatch], bv[kMaxRank];
#pragma unroll
  for (int u = 0; u < kFinBatch; ++u) {
    yv[u] = u < nsplit ? py[u * stride] : 0.0f;
    tv[u] = (tl && u < nsplit) ? pt[u * stride] : 0.0f;
  }
  if (lora && (r & 7) == 0) {  // the row is 16-byte aligned: eight ranks per load
#pragma unroll
    for (int q = 0; q < kMaxRank / 8; ++q) {
      const u32x4 w = 8 * q < r ? *reinterpret_cast<const u32x4*>(Bn + 8 * q) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bv[8 * q + 2 * e] = bf16_lo(w[e]);
        bv[8 * q + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxRank; ++j) bv[j] = (lora && j < r) ? bf16_to_f32(Bn[j]) : 0.0f;
  }
  float y = 0.0f, t = 0.0f;
#pragma unroll
  for (int u = 0; u < kFinBatch; ++u) {
    y += yv[u];
    t += tv[u];
  }
  if (nsplit > kFinBatch) {
    y += sum_strided(py + kFinBatch * stride, stride, nsplit - kFinBatch);
    if (tl) t += sum_strided(pt + kFinBatch * stride, stride, nsplit - kFinBatch);
  }
  if (tl) {
    const uint32_t tb = pack_bf16x2(t, 0.0f) & 0xFFFFu;
    tsh[tid] = bf16_to_f32((uint16_t)tb);
    if (Tsave != nullptr && blockIdx.x == 0) Tsave[(size_t)tid * ldt + m] = (uint16_t)tb;
  }
  __syncthreads();
  if (n >= d) return;
  if (lora) {
    const float* ts = tsh + (idx != nullptr ? 0 : (n / dsec) * r);
    float l = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxRank; ++j)
      if (j < r) l = fmaf(ts[j], bv[j], l);
    y = fmaf(s, l, y);
  }
  Y[(size_t)m * d + n] = (uint16_t)pack_bf16x2(y, 0.0f);
}

// ---------------------------------------------------------------- launch --

// Split-K decode kernels up to 64 tokens, and up to 128 for the chunked one
// (k % 256 == 0): past 64 tokens a token-rich grid has one row of tiles
// (16 work-groups at d = 4096) whose K loops run serially (measured: 66 us
// at 65..512 tokens against 24 us at 64).
bool forward_uses_decode(int M, int d, int k) { return M <= 64 || (M <= 128 && k % kDcK == 0); }

// The single-launch kernel k_fwd_dec1 can serve up to 16 tokens when k is a
// multiple of 256 and a section has at most 16 adapter ranks (r_sec); it
// needs no workspace.  Measured on the decode shapes (M = 16, HIP graph of
// 64 calls over rotating weights, per call), against the split-K pair:
//   r = 16: 9.8-10.2 / 15.8-15.9 / 20.3 us at 4096^2 / 11008 x 4096 /
//           4096 x 11008, against 11.1-11.5 / 16.3-16.6 / 15.6 us;
//   r = 0:  7.2 / 13.0-13.2 / 14.6 us, against 10.1-10.2 / 16.1-16.4 / 14.8 us.
// Every work-group reads all of X (and A, with adapters): 128 KB each at
// k = 4096, which the pair avoids; with long K rows (k = 11008) and
// adapters that costs more than the pair's second launch.
// With every load in flight at once (k_fwd_dec1s, k <= 4096) the same
// calls take 9.96 / 14.95 us (r = 16) and 6.4 / 11.8 us (r = 0) against
// 9.9-10.1 / 15.2-15.5 and 7.1-7.4 / 12.9 us for the two-slot ring: the
// time tracks the bytes each CU fetches (X, A and the codes, about 35 GB/s
// per CU whichever way they are loaded), not the number of round trips.  So the single
// launch is taken without adapters, or with k <= 4096; QLORA_DECODE=single
// or =split forces either form where both apply (tests of both forms).
// split_only: per-token adapters or LoRA dropout, which always take the
// split-K kernels.
static int d1_row_blocks(int d, int dsec, bool sections) {
  int nb = 1;
  while (nb < 3 && (d + 16 * nb - 1) / (16 * nb) > 256 && (!sections || dsec % (16 * (nb + 1)) == 0)) ++nb;
  return nb;
}

static bool decode_single(int M, int k, int r_sec, bool split_only) {
  if (split_only || M > 16 || k % kDcK != 0 || r_sec > 16) return false;
  const char* e = getenv("QLORA_DECODE");
  if (e != nullptr && strcmp(e, "single") == 0) return true;
  if (e != nullptr && strcmp(e, "split") == 0) return false;
  return r_sec == 0 || k <= 4096;
}

// Tile height of the token-rich kernel: 256 rows when that still gives at
// least one work-group per CU, else 128.
static int rich_bm(int M, int d) {
  const int forced = tile_override();
  if (forced) return forced;
  const int tiles256 = ((M + 255) / 256) * ((d + kRichBN - 1) / kRichBN);
  return tiles256 >= 256 ? 256 : 128;
}

// Steps per wave (1, 2 or 4) and K splits: the fewest steps per wave that
// keep the grid at no more than 1536 work-groups.  The kernel is bound by
// the decode arithmetic, so more waves per SIMD (one step each) beat fewer
// waves that overlap their own loads (measured).
constexpr int kDecNB = 4;  // 16-row MFMA blocks per decode tile

static void decode_split(int M, int d, int k, int r, int* ntiles, int* ntw, int* nsplit, int* sps) {
  constexpr int kRows = 16 * kDecNB;
  const int tw = (d + kRows - 1) / kRows;
  const int ta = r > 0 ? (r + kRows - 1) / kRows : 0;
  const int nsteps = (k + kDecStep - 1) / kDecStep;
  int spw = 1;
  while (spw < 4 && (int64_t)(tw + ta) * ((nsteps + 4 * spw - 1) / (4 * spw)) > 1536) spw *= 2;
  *ntiles = tw + ta;
  *ntw = tw;
  *sps = 4 * spw;
  *nsplit = (nsteps + *sps - 1) / *sps;
}

// Chunked kernel (k a multiple of 256): chunks per split chosen for about
// 256 weight work-groups (one per CU, all resident at once).
static void dec_split(int d, int k, int r, int* ntiles, int* ntw, int* nsplit, int* cps) {
  const int tw = (d + kDcRows - 1) / kDcRows;
  const int ta = r > 0 ? (r + 15) / 16 : 0;  // rank tiles of 16 ranks
  const int chunks = k / kDcK;
  const int c = max(1, min(chunks, (int)(((int64_t)tw * chunks + 511) / 512)));
  *ntiles = tw + ta;
  *ntw = tw;
  *cps = c;
  *nsplit = (chunks + c - 1) / c;
}

// Split K for the token-rich forward when its 128-row tiles would leave
// most CUs idle (a few hundred tokens: 32 work-groups at 256 tokens and
// d = 4096, each running the whole K loop): up to four column groups of K
// steps, at least four steps each.
static int rich_split(int M, int d, int k) {
  if (tile_override() != 0 || M <= 128 || d % kRichBN != 0 || k % 256 != 0 || rich_bm(M, d) != 128) return 1;
  if ((uint64_t)M * k * 2 >= (1ull << 32)) return 1;
  const int tiles = ((M + 127) / 128) * (d / kRichBN);
  if (tiles > 128) return 1;  // (128 tiles: one per two CUs, split in two)
  const int ksteps = k / 128;  // k_fwd8<128, 2>: two blocks per step
  const int S = min(min(256 / tiles, 4), ksteps / 4);
  return max(S, 1);
}

size_t forward_gemm_ws_bytes(int M, int d, int k, int r, bool split_only) {
  if (forward_uses_decode(M, d, k) && decode_single(M, k, r, split_only)) return 0;
  if (!forward_uses_decode(M, d, k)) {
    const int S = rich_split(M, d, k);
    return S > 1 ? (size_t)S * M * d * sizeof(float) : 0;
  }
  int ntiles, ntw, ns, sps;
  if (k % kDcK == 0)
    dec_split(d, k, r, &ntiles, &ntw, &ns, &sps);
  else
    decode_split(M, d, k, r, &ntiles, &ntw, &ns, &sps);
  return (size_t)ns * M * (d + padded_rank(r)) * sizeof(float);
}

hipError_t launch_forward_decode(const uint16_t* X, int M, const Nf4Dev& w, int nsec, const uint16_t* A,
                                 const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* Tsave,
                                 int ldt, float* part, const Nf4Table& t, hipStream_t st, const int* idx,
                                 const uint16_t* Xa) {
  const bool xad = Xa != nullptr && Xa != X;  // the adapter path reads its own input
  if (Xa == nullptr) Xa = X;
  if (decode_single(M, w.k, r, idx != nullptr || xad)) {
    // 16, 32 or 48 rows per work-group: the fewest that keep the grid
    // within one work-group per CU (a work-group holds 128 KB of LDS)
    const int nb = d1_row_blocks(w.d, w.dsec, w.d != w.dsec);
    const dim3 grid((unsigned)((w.d + 16 * nb - 1) / (16 * nb)));
    // k <= 4096: every load in flight at once (k_fwd_dec1s), unless
    // QLORA_DEC1=ring asks for the two-slot ring
    const int spw = (w.k / kD1K + kD1Waves - 1) / kD1Waves;
    const char* ring = getenv("QLORA_DEC1");
    if (spw <= 4 && !(ring != nullptr && strcmp(ring, "ring") == 0)) {
#define QLORA_D1S(NB, LORA, S)                                                                               \
  QLORA_LAUNCH("fwd_decode", st, (k_fwd_dec1s<NB, LORA, S>), grid, dim3(64 * kD1Waves), 0, st, X, M, w.codes,  \
               w.c2, w.c1, w.mean, w.d, w.k, w.dsec, A, B, r, s, Y, Tsave, ldt, t)
#define QLORA_D1S_NB(LORA, S) \
  if (nb == 3) QLORA_D1S(3, LORA, S); else if (nb == 2) QLORA_D1S(2, LORA, S); else QLORA_D1S(1, LORA, S);
#define QLORA_D1S_S(LORA)                                                                                     \
  switch (spw) {                                                                                             \
    case 1: QLORA_D1S_NB(LORA, 1) break;                                                                     \
    case 2: QLORA_D1S_NB(LORA, 2) break;                                                                     \
    case 3: QLORA_D1S_NB(LORA, 3) break;                                                                     \
    default: QLORA_D1S_NB(LORA, 4) break;                                                                    \
  }
      if (r == 0) {
        QLORA_D1S_S(false)
      } else {
        QLORA_D1S_S(true)
      }
#undef QLORA_D1S_S
#undef QLORA_D1S_NB
#undef QLORA_D1S
      return hipGetLastError();
    }
#define QLORA_D1(NB, LORA)                                                                                   \
  QLORA_LAUNCH("fwd_decode", st, (k_fwd_dec1<NB, LORA>), grid, dim3(64 * kD1Waves), 0, st, X, M, w.codes, w.c2, \
               w.c1, w.mean, w.d, w.k, w.dsec, A, B, r, s, Y, Tsave, ldt, t)
    if (r == 0) {
      if (nb == 3) QLORA_D1(3, false); else if (nb == 2) QLORA_D1(2, false); else QLORA_D1(1, false);
    } else {
      if (nb == 3) QLORA_D1(3, true); else if (nb == 2) QLORA_D1(2, true); else QLORA_D1(1, true);
    }
#undef QLORA_D1
    return hipGetLastError();
  }
  int ntiles, ntw, ns, sps;
  const int rt = nsec * r;  // ranks of T: r per section (or per adapter, with idx)
  const int ldp = w.d + padded_rank(rt);
  const int mblk = (M + 15) / 16;
  if (w.k % kDcK == 0) {
    dec_split(w.d, w.k, rt, &ntiles, &ntw, &ns, &sps);
    dim3 grid((unsigned)ntiles, (unsigned)ns);
#define QLORA_DC(MT)                                                                                    \
  QLORA_LAUNCH("fwd_decode", st, k_fwd_dec<MT>, grid, dim3(64 * kDcWaves), 0, st, X, M, w.codes, w.c2, w.c1, w.mean, \
               w.d, w.k, w.dsec, A, rt, ntw, sps, part, ldp, t, Xa)
    switch (mblk) {
      case 1: QLORA_DC(1); break;
      case 2: QLORA_DC(2); break;
      case 3: QLORA_DC(3); break;
      case 4: QLORA_DC(4); break;
      case 5:
      case 6: QLORA_DC(6); break;
      default: QLORA_DC(8); break;
    }
#undef QLORA_DC
  } else {
  decode_split(M, w.d, w.k, rt, &ntiles, &ntw, &ns, &sps);
  dim3 grid((unsigned)ntiles, (unsigned)ns);
#define QLORA_DEC(MB, SPW)                                                                       \
  QLORA_LAUNCH("fwd_decode", st, (k_fwd_decode<MB, SPW, kDecNB>), grid, dim3(256), 0, st, X, M, w.codes, w.c2, w.c1, \
               w.mean, w.d, w.k, w.dsec, A, rt, ntw, sps, part, ldp, t, Xa)
#define QLORA_DEC_M(SPW)                \
  switch (mblk) {                       \
    case 1: QLORA_DEC(1, SPW); break;   \
    case 2: QLORA_DEC(2, SPW); break;   \
    case 3: QLORA_DEC(3, SPW); break;   \
    default: QLORA_DEC(4, SPW); break;  \
  }
  switch (sps / 4) {
    case 1: QLORA_DEC_M(1); break;
    case 2: QLORA_DEC_M(2); break;
    default: QLORA_DEC_M(4); break;
  }
#undef QLORA_DEC_M
#undef QLORA_DEC
  }
  QLORA_LAUNCH("fwd_decode_finish", st, k_fwd_decode_finish, dim3((unsigned)((w.d + 255) / 256), (unsigned)M), dim3(256),
                     0, st, part, ns, M, w.d, ldp, B, r, rt, w.dsec, idx, s, Y, Tsave, ldt);
  return hipGetLastError();
}

hipError_t launch_forward(const uint16_t* X, int M, const Nf4Dev& w, int nsec, const uint16_t* T,
                          const uint16_t* B, int r, float s, uint16_t* Y, const Nf4Table& t,
                          hipStream_t st, float* part) {
  const int rp = r > 0 ? padded_rank(r) : 0;
  const int ldr = nsec * rp;  // row stride of T: rp ranks per section (rp == r when nsec > 1)
  const int ntn = (w.d + kRichBN - 1) / kRichBN;
  const bool even = w.d % kRichBN == 0 && w.k % 256 == 0 && (uint64_t)M * w.k * 2 < (1ull << 32);
  const int S = rich_split(M, w.d, w.k);
  if (S > 1 && part != nullptr) {
    const int ksteps = w.k / 128;
    const int sps = (ksteps + S - 1) / S;
    const int ns = (ksteps + sps - 1) / sps;
    dim3 grid((unsigned)(ntn * ((M + 127) / 128)), (unsigned)ns);
    QLORA_LAUNCH("fwd_rich", st, (k_fwd8<128, 2>), grid, dim3(64 * kFwd8Waves), 0, st, X, M, w.codes, w.c2, w.c1,
                 w.mean, w.d, w.k, w.dsec, T, B, r, rp, ldr, s, Y, t, 0, ntn, sps, part);
    const int64_t n = (int64_t)M * w.d;
    const int64_t blocks = (n / 4 + 255) / 256;
    QLORA_LAUNCH("fwd_sum_splits", st, k_sum_splits, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                 st, part, ns, n, Y);
  } else if (even && tile_override() == 0) {
    // Whole rounds of 256-row tiles (one work-group per CU per round); with
    // one or two full rounds, the column tiles that would make a last,
    // partial round run instead as 128-row tiles in a second launch, when
    // those fit in one round (2048 tokens at d = 11008: 216 -> 200 us).
    int c256 = 0, c128 = ntn;
    if (rich_bm(M, w.d) == 256) {
      const int ntm = (M + 255) / 256, tiles = ntm * ntn;
      c256 = ntn;
      if (tiles % 256 != 0 && tiles < 3 * 256) {  // with more full rounds the tail overlaps them (measured)
        const int full = (tiles / 256) * 256 / ntm;
        if ((ntn - full) * ((M + 127) / 128) <= 256) c256 = full;
      }
      c128 = ntn - c256;
    }
    if (c256 > 0) {
      dim3 grid((unsigned)(c256 * ((M + 255) / 256)));
      QLORA_LAUNCH("fwd_rich", st, (k_fwd8<256, 1>), grid, dim3(64 * kFwd8Waves), 0, st, X, M, w.codes, w.c2, w.c1,
                   w.mean, w.d, w.k, w.dsec, T, B, r, rp, ldr, s, Y, t, 0, c256, 0, nullptr);
    }
    if (c128 > 0) {
      dim3 grid((unsigned)(c128 * ((M + 127) / 128)));
      QLORA_LAUNCH("fwd_rich", st, (k_fwd8<128, 2>), grid, dim3(64 * kFwd8Waves), 0, st, X, M, w.codes, w.c2, w.c1,
                   w.mean, w.d, w.k, w.dsec, T, B, r, rp, ldr, s, Y, t, c256 * kRichBN, c128, 0, nullptr);
    }
  } else if (rich_bm(M, w.d) == 256) {
    dim3 grid((unsigned)(ntn * ((M + 255) / 256)));
    QLORA_LAUNCH("fwd_rich", st, k_fwd_rich<256>, grid, dim3(256), 0, st, X, M, w.codes, w.c2, w.c1,
                 w.mean, w.d, w.k, w.dsec, T, B, r, rp, ldr, s, Y, t);
  } else {
    dim3 grid((unsigned)(ntn * ((M + 127) / 128)));
    QLORA_LAUNCH("fwd_rich", st, k_fwd_rich<128>, grid, dim3(256), 0, st, X, M, w.codes, w.c2, w.c1,
                 w.mean, w.d, w.k, w.dsec, T, B, r, rp, ldr, s, Y, t);
  }
  return hipGetLastError();
}

}  // namespace qlora
