// gemm_dx.hip -- input gradient dX = dY w~ + s U A, U = dY B
// (page "LoRA and QLoRA fine-tuning: mechanics, and when not to fine-tune",
// section "What QLoRA freezes, and in how many bits": dX needs the bf16
// expansion of the frozen 4-bit weight, while W0 itself gets no gradient).
//
// k_dx8 (d a multiple of 64, k a multiple of 256) is the eight-wave form,
// two waves per SIMD, described at the kernel; k_dx covers other shapes.
//
// Transposed-dequant GEMM on bf16 MFMA (32x32x16), fp32 accumulation;
// BM x BN work-group tiles (256 x 256, or 128 x 128 when the grid would not
// cover the CUs) of 2 x 2 waves, each wave BM/2 x BN/2 outputs.  The
// contraction runs over d, the weight's row index, while a packed code word
// holds 8 consecutive columns of one row.  Each K step (64 weight rows x BN
// columns) is decoded once per work-group: a lane pair (l, l + 32) takes one
// 64-column block of one weight row (a half each, sharing the block's table)
// and writes its bf16 values row-major into LDS with 16-byte stores; the MFMA
// B operands are then read with gfx950's transposing LDS read
// (ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte loads of lanes 4r + i / 4, r = 0..3), which turns four
// rows x 16 columns into 16 lanes x four rows.  dY tiles (2 slots), decoded
// weight tiles (2 slots) and packed codes with their block constants (3
// slots, fetched three K steps ahead) live in swizzled LDS; every fetch
// is a buffer-addressed global->LDS load.  The LoRA term s U A is one more
// MFMA pass in the epilogue, accumulating into the same registers, from U
// (M x rp) and bf16(s A)^T, zero-padded (k x rp).
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

constexpr int kDxBK = 64;

// LoRA dropout in dX: the LoRA term of element (m, c) is scaled by dscale
// where keep[m, c] != 0 and dropped elsewhere.  f32x16 accumulator element
// e of lane (half, l32) of a 32 x 32 MFMA block at (row0, col0) is row
// row0 + 8*(e/4) + 4*half + e%4, column col0 + l32.
__device__ __forceinline__ void drop_block(f32x16& t, const BufRsrc& rk, int row0, int col, int M, int k,
                                           int half, float dscale) {
  uint32_t kv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int m = row0 + 8 * (e / 4) + 4 * half + e % 4;
    kv[e] = ld_buf1(rk, m < M ? (uint32_t)m * (uint32_t)k + (uint32_t)col : (uint32_t)M * (uint32_t)k);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] *= kv[e] ? dscale : 0.0f;
}

// Mean of the section holding weight rows kc*64 .. kc*64 + 63 (sections of
// dsec rows, dsec a multiple of 64, at most kMaxSections of them), from the
// means held in registers.
__device__ __forceinline__ float section_mean(const float (&mus)[kMaxSections], int kc, int dsec) {
  const int sec = kc * kDxBK / dsec;
  float m = mus[0];
#pragma unroll
  for (int i = 1; i < kMaxSections; ++i) m = sec == i ? mus[i] : m;
  return m;
}

// Placement of the 16-byte piece c (8 columns) of decoded weight row r inside
// its row.  LDS serves a 16-byte store to eight lanes at a time over 128
// bytes of banks and a transposing 8-byte read to 32 lanes at a time over
// 256 bytes, so the two access patterns of the decoded tile need:
//   decode stores  piece c of 8 consecutive rows 8a..8a+7 in 8 distinct
//                  slots modulo 128 bytes;
//   B reads        pieces 4b..4b+3 of rows 4a..4a+3 (and of rows 8 further
//                  on) in 16 distinct slots modulo 256 bytes.
// Slot bits: [1:0] = (r % 4) ^ (c / 4), [2] = (r / 4) ^ c, [3] = (r / 8) ^
// (c / 2), all mod 2 per bit; c's bit 4 (which 256-byte half of a 512-byte
// row) is kept, so the map is a permutation of each row's pieces.
__device__ __forceinline__ int wslot(int r, int c) {
  return (c & ~15) | (((r & 3) ^ (c >> 2)) & 3) | ((((r >> 2) ^ c) & 1) << 2) | ((((r >> 3) ^ (c >> 1)) & 1) << 3);
}

template <int BM, int BN, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_dx(
    const uint16_t* __restrict__ dY, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ c2, const float* __restrict__ c1, const float* __restrict__ mean,
    int d, int k, int dsec, const uint16_t* __restrict__ U, const uint16_t* __restrict__ At, int rp,
    float s, uint16_t* __restrict__ dX, Nf4Table tab,
    const uint8_t* __restrict__ keep, float dscale) {
  constexpr int WM = BM / 2, WN = BN / 2;   // 2 x 2 waves
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int YCH = BM / 32;              // 1 KB dY fetches per wave per K step
  constexpr int NP = BN / 128;              // half-block rows decoded per lane per K step
  constexpr int ROWB = BN * 2;              // bytes per row of a decoded weight tile
  constexpr int kYBytes = BM * kDxBK * 2, kWBytes = kDxBK * BN * 2;
  constexpr int kCWave = NP * 1024 + 512;   // per wave: codes, then c2 and c1 words
  constexpr int kCSlot = 4 * kCWave;
  constexpr int kCOff = 2 * kYBytes;
  constexpr int kSmem = kCOff + 3 * kCSlot;
  constexpr int kStage = 4 * WM * 64 * 2;
  static_assert(kStage <= kSmem, "output staging must fit");
  static_assert(kSmem + 2 * kWBytes <= 160 * 1024, "LDS");
  // Fetch targets (dY and code rings) and decoded weights are separate LDS
  // objects: the compiler can then see that the transposing reads of the
  // decoded weights never alias an in-flight global->LDS fetch.
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ __attribute__((aligned(16))) char wsm[2 * kWBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (k + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, c0 = tn * BN;
  const int ksteps = (d + kDxBK - 1) / kDxBK;
  const int kblocks = k / 64;
  // The contraction runs over all weight rows, so a K step's mean is that
  // of its section.
  float mus[kMaxSections];
#pragma unroll
  for (int i = 0; i < kMaxSections; ++i) mus[i] = mean[min(i, d / dsec - 1)];
  float qh[8];  // this lane's half of the levels, for build_lut_pair
#pragma unroll
  for (int i = 0; i < 8; ++i) qh[i] = half ? tab.q[8 + i] : tab.q[i];

  const BufRsrc ry = make_rsrc(dY, (uint64_t)M * d * 2);
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);

  // dY tile (BM x 64) fetch: wave w fills rows [w*BM/4, (w+1)*BM/4), eight
  // rows per instruction, lane l -> row r0 + l/8, physical chunk l%8 (the
  // logical chunk (l%8) ^ swz_f(row)).  Rows past M repeat row M-1 (never
  // stored); columns past d read the same row's first columns, which meet
  // weight rows that decode to zero.
  int yrow[YCH], ycol[YCH];
#pragma unroll
  for (int j = 0; j < YCH; ++j) {
    const int lr = lane >> 3, pc = lane & 7;
    const int r0 = wave * (BM / 4) + j * 8;
    yrow[j] = min(m0 + r0 + lr, M - 1);
    ycol[j] = (pc ^ swz_f(r0 + lr)) << 3;
  }
  // Block rows decoded by this wave: G = wave*(BN/4) + j, j < BN/4, is
  // weight row (G % 64) of the step and 64-column block (G / 64) of the
  // tile.  Pass i of lane l handles j = i*32 + l%32, column half l/32.
  // The c2/c1 fetch lane l covers j = l % (BN/4).
  int brow[NP], bblk[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int G = wave * (BN / 4) + i * 32 + l32;
    brow[i] = G % 64;
    bblk[i] = G / 64;
  }
  const int Gc = wave * (BN / 4) + (lane % (BN / 4));
  const int crow = Gc % 64, cblk = Gc / 64;
  // byte offset of (weight row n, column c) in the codes; block index
  auto code_off = [&](int n, int c) { return (uint32_t)n * (uint32_t)(k >> 1) + (uint32_t)(c >> 1); };

  auto dma_one = [&](int i, int ks, int ysl, int kc, int csl) {
    // i < YCH: dY chunk of K step ks into dY slot ysl; then the NP code
    // fetches, c2 and c1 of K step kc into code slot csl
    if (i < YCH) {
      const char* slot = smem + ysl * kYBytes;
      const int dc = ks * kDxBK + ycol[i];
      const uint32_t off = ((uint32_t)yrow[i] * (uint32_t)d + (uint32_t)(dc < d ? dc : ycol[i])) * 2u;
      dma_lds16(ry, off, (void*)(slot + (wave_s * (BM / 4) + i * 8) * (kDxBK * 2)));
    } else {
      char* cs = smem + kCOff + csl * kCSlot + wave_s * kCWave;
      const int j = i - YCH;
      if (j < NP) {
        const int n = kc * kDxBK + brow[j], c = c0 + bblk[j] * 64 + half * 32;
        const bool ok = n < d && c < k;
        dma_lds16(rc, code_off(ok ? n : 0, ok ? c : 0), (void*)(cs + j * 1024));
      } else {
        const int n = kc * kDxBK + crow, c = c0 + cblk * 64;
        const bool ok = n < d && c < k;
        const uint32_t blk = (uint32_t)(ok ? n : 0) * (uint32_t)kblocks + (uint32_t)((ok ? c : 0) >> 6);
        if (j == NP)
          dma_lds4(r2, blk & ~3u, (void*)(cs + NP * 1024));
        else
          dma_lds4(r1, (blk >> 8) * 4, (void*)(cs + NP * 1024 + 256));
      }
    }
  };
  constexpr int kLoads = YCH + NP + 2;
  constexpr int kCodeLoads = NP + 2;

  // Codes and block tables of K step kc for this lane (from its own fetches).
  struct WTile {
    u32x4 v[NP];
    uint32_t q2[NP];
    float q1[NP];
  };
  auto read_w = [&](int csl, WTile& W) {
    const char* cs = smem + kCOff + csl * kCSlot + wave_s * kCWave;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      W.v[i] = *reinterpret_cast<const u32x4*>(cs + i * 1024 + lane * 16);
      W.q2[i] = *reinterpret_cast<const uint32_t*>(cs + NP * 1024 + (i * 32 + l32) * 4);
      W.q1[i] = *reinterpret_cast<const float*>(cs + NP * 1024 + 256 + (i * 32 + l32) * 4);
    }
  };
  Lut lut[NP];
  auto tables = [&](const WTile& W, int kc) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int n = kc * kDxBK + brow[i], c = c0 + bblk[i] * 64;
      const bool ok = n < d && c < k;
      const uint32_t blk = (uint32_t)(ok ? n : 0) * (uint32_t)kblocks + (uint32_t)((ok ? c : 0) >> 6);
      const float v = block_scale((W.q2[i] >> ((blk & 3u) * 8u)) & 0xFFu, W.q1[i], section_mean(mus, kc, dsec));
      lut[i] = build_lut_pair(qh, ok ? v : 0.0f);
    }
  };
  // Decode word wd of every pass into the decoded-weight slot ws (row-major,
  // 16-byte pieces placed by wslot).
  auto decode_word = [&](const WTile& W, int wd, char* ws) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const u32x4 v = dequant8(W.v[i][wd], lut[i]);
      const int r = brow[i], c = (bblk[i] * 64 + half * 32 + wd * 8) >> 3;
      *reinterpret_cast<u32x4*>(ws + r * ROWB + (wslot(r, c) << 4)) = v;
    }
  };

  // A fragment byte offsets (dY tile): row wm*WM + mb*32 + l32, chunk st*2 + half.
  uint32_t aoff[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int st = 0; st < 4; ++st) aoff[mb][st] = (uint32_t)(2 * swz(wm * WM + mb * 32 + l32, st * 2 + half));
  // B fragment byte offsets (decoded tile), per column block nb and row
  // quad q; substep st adds st*16 rows (wslot depends on r % 16 only).
  // 16-lane group g: columns (g & 1)*16 + 4*(l % 4) .. +3 of the block, rows
  // 8*(g >> 1) + (l%16)/4 + 4q.
  uint32_t boff[NB][2];
  {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = 8 * (g >> 1) + (sl >> 2) + 4 * q;
        const int col = wn * WN + nb * 32 + (g & 1) * 16 + 4 * (sl & 3);
        boff[nb][q] = (uint32_t)(r * ROWB + (wslot(r, col >> 3) << 4) + (col & 7) * 2);
      }
  }
  auto read_ab = [&](int ks, int st, u32x4 (&af)[MB], u32x4 (&bf)[NB]) {
    const char* ys = smem + (ks & 1) * kYBytes;
    const char* ws = wsm + (ks & 1) * kWBytes + st * 16 * ROWB;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u32x2 lo = lds_read_tr16(ws + boff[nb][0]);
      const u32x2 hi = lds_read_tr16(ws + boff[nb][1]);
      bf[nb] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const u32x4*>(ys + aoff[mb][st]);
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  // Pipeline.  K step ks multiplies dY tile ks by decoded tile ks while it
  // (a) fetches dY tile ks+1 and the codes of step ks+3 (clamped to the last
  // step, so every step issues kLoads fetches), spread between its MFMAs,
  // and (b) decodes step ks+1 from codes fetched two steps earlier into the
  // other decoded-weight slot.  At the end of the step each wave waits until
  // only its code fetches of this step are outstanding (its dY share of
  // ks+1 and its codes of ks+2 have landed) and its LDS traffic is done;
  // the barrier then publishes dY tile ks+1 and decoded tile ks+1 and frees
  // the slots of step ks.
  const auto clampk = [&](int x) { return x < ksteps ? x : ksteps - 1; };
#pragma unroll
  for (int i = YCH; i < kLoads; ++i) dma_one(i, 0, 0, 0, 0);           // codes of step 0
#pragma unroll
  for (int i = 0; i < YCH; ++i) dma_one(i, 0, 0, 0, 0);                // dY tile 0
#pragma unroll
  for (int i = YCH; i < kLoads; ++i) dma_one(i, 0, 0, clampk(1), 1);   // codes of step 1
#pragma unroll
  for (int i = YCH; i < kLoads; ++i) dma_one(i, 0, 0, clampk(2), 2);   // codes of step 2
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kCodeLoads) : "memory");
  WTile W;
  read_w(0, W);
  tables(W, 0);
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) decode_word(W, wd, wsm);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCodeLoads) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  constexpr int kPerSub = (kLoads + 2) / 3;
  int csl_next = 1;  // code slot of step ks+1 (ring of three)
  for (int ks = 0; ks < ksteps; ++ks) {
    const int ky = clampk(ks + 1), kc = clampk(ks + 3), kd = clampk(ks + 1);
    const int ysl = (ks + 1) & 1;
    const int csl_far = csl_next == 0 ? 2 : csl_next - 1;  // slot of step ks (free)
    char* wnext = wsm + ((ks + 1) & 1) * kWBytes;
    u32x4 af[2][MB], bf[2][NB];
    read_ab(ks, 0, af[0], bf[0]);
    read_w(csl_next, W);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st < 3) read_ab(ks, st + 1, af[(st + 1) & 1], bf[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (st == 0) tables(W, kd);
      decode_word(W, st, wnext);
      if (st < 3) {
#pragma unroll
        for (int i = st * kPerSub; i < (st + 1) * kPerSub && i < kLoads; ++i) dma_one(i, ky, ysl, kc, csl_far);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(af[st & 1][mb], bf[st & 1][nb], acc[mb][nb]);
#pragma unroll
      for (int i = 0; i < MB * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        if (st < 3 && i < kPerSub) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCodeLoads) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    csl_next = csl_next == 2 ? 0 : csl_next + 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // LoRA term: acc += U_tile . (s A)_tile^T, K = rp (At holds bf16(s A)^T),
  // accumulated straight into the MFMA accumulators.
  if (rp > 0) {
    const BufRsrc rk = make_rsrc(keep, DROP ? (uint64_t)M * k : 0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + wm * WM + mb * 32 + l32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int c = c0 + wn * WN + nb * 32 + l32;
        f32x16 t;
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e] = 0.0f;
        for (int jb = 0; jb < rp; jb += 16) {
          u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
          if (m < M) a = *reinterpret_cast<const u32x4*>(U + (size_t)m * rp + jb + half * 8);
          if (c < k) b = *reinterpret_cast<const u32x4*>(At + (size_t)c * rp + jb + half * 8);
          if (DROP)
            t = mfma32(a, b, t);
          else
            acc[mb][nb] = mfma32(a, b, acc[mb][nb]);
        }
        if (DROP) {
          drop_block(t, rk, m0 + wm * WM + mb * 32, c, M, k, half, dscale);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[mb][nb][e] += t[e];
        }
      }
    }
  }

  // Output through LDS: each wave stages WM x 64 bf16 (two 32-column blocks)
  // at a time and stores 16-byte row chunks.
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem) + wave * (WM * 64);
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

// Eight-wave form for the common shapes (d a multiple of 64, k a multiple of
// 256): 256 x 256 work-group tiles of 2 x 4 waves (each 128 x 64 outputs), so
// that every SIMD runs two waves and one wave's decode and LDS traffic
// overlap the other's MFMAs.  Per K step each wave fetches a quarter-eighth
// of the dY tile (four 1 KB fetches) and the packed codes it decodes itself
// (one 64-column block half per lane pair, one 1 KB fetch); waves 6 and 7
// also fetch the step's block constants for the whole tile (one c2 word and
// one c1 word per weight row: with k a multiple of 256 the four blocks of a
// row in the tile share one c2 word and one c1 group).  Fetch offsets are a
// per-lane constant plus a scalar per-step offset; there are no bounds
// checks in the K loop (rows past M repeat row M-1 and are never stored).
constexpr int kDx8Waves = 8;

template <int BM, bool DROP>
__global__ __launch_bounds__(64 * kDx8Waves) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dx8(
    const uint16_t* __restrict__ dY, int M, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ c2, const float* __restrict__ c1, const float* __restrict__ mean,
    int d, int k, int dsec, const uint16_t* __restrict__ U, const uint16_t* __restrict__ At, int rp,
    uint16_t* __restrict__ dX, Nf4Table tab, int cbase, int ntn,
    const uint8_t* __restrict__ keep, float dscale, int sps, float* __restrict__ part) {
  constexpr int BN = 256, WM = BM / 2, WN = 64;
  constexpr int YF = BM / 64;                       // 1 KB dY fetches per wave per step
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int ROWB = BN * 2;
  constexpr int kYBytes = BM * kDxBK * 2, kWBytes = kDxBK * BN * 2;
  constexpr int kCWave = 1024;                      // one wave's codes per step
  constexpr int kC2Off = kDx8Waves * kCWave;        // 64 c2 words, then 64 c1 words
  constexpr int kCSlot = kC2Off + 512;
  constexpr int kCOff = 2 * kYBytes;
  constexpr int kSmem = kCOff + 3 * kCSlot;
  constexpr int kStage = WM * WN * 2;               // one wave's output tile
  static_assert(4 * kStage <= kSmem && 4 * kStage <= 2 * kWBytes, "output staging must fit");
  static_assert(kSmem + 2 * kWBytes <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ __attribute__((aligned(16))) char wsm[2 * kWBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, ntn, tm, tn);
  const int m0 = tm * BM, c0 = cbase + tn * BN;  // this launch covers columns cbase .. cbase + ntn*BN
  // Split K (sps > 0): work-group column blockIdx.y takes K steps kbase ..
  // kbase + sps - 1 (64 weight rows each) and writes fp32 partials (split 0
  // also carries the LoRA term); k_dx_sum_splits adds them in order.
  const int split = blockIdx.y;
  const int kbase = sps > 0 ? split * sps : 0;
  const int ksteps = sps > 0 ? min(sps, d / kDxBK - kbase) : d / kDxBK;
  const int kblocks = k / 64;
  float mus[kMaxSections];  // means of the sections of weight rows
#pragma unroll
  for (int i = 0; i < kMaxSections; ++i) mus[i] = mean[min(i, d / dsec - 1)];
  float qh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qh[i] = half ? tab.q[8 + i] : tab.q[i];

  const BufRsrc ry = make_rsrc(dY, (uint64_t)M * d * 2);
  const BufRsrc rc = make_rsrc(codes, (uint64_t)d * k / 2);
  const uint32_t nblk = (uint32_t)d * (uint32_t)kblocks;
  const BufRsrc r2 = make_rsrc(c2, nblk);
  const BufRsrc r1 = make_rsrc(c1, (uint64_t)((nblk + 255) / 256) * 4);

  // dY: wave w fills tile rows [w*BM/8, (w+1)*BM/8), eight rows per fetch,
  // lane l -> row r0 + l/8, physical chunk l%8 (logical chunk (l%8) ^
  // swz_f(row)).
  uint32_t yoff[YF];
#pragma unroll
  for (int j = 0; j < YF; ++j) {
    const int row = wave * (BM / 8) + j * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ swz_f(row);
    yoff[j] = ((uint32_t)min(m0 + row, M - 1) * (uint32_t)d + (uint32_t)(lc * 8)) * 2u;
  }
  // This lane pair decodes weight row wrow of the step, 64-column block wblk
  // of the tile, column half `half`.
  const int wrow = (wave & 1) * 32 + l32, wblk = wave >> 1;
  const uint32_t coff = (uint32_t)wrow * (uint32_t)(k >> 1) + (uint32_t)((c0 + wblk * 64 + half * 32) >> 1);
  // block constants of row `lane` (waves 6 and 7)
  const uint32_t boff2 = (uint32_t)lane * (uint32_t)kblocks + (uint32_t)(c0 >> 6);
  const uint32_t boff1 = (boff2 >> 8) * 4u;
  const uint32_t sc = (uint32_t)k * 32u;            // code bytes per step
  const uint32_t s2 = (uint32_t)kblocks * 64u;      // c2 bytes per step
  const uint32_t s1 = (uint32_t)kblocks;            // c1 bytes per step (64 kblocks / 256 words)

  // Fetch i of this wave for dY tile ks (slot ysl) and codes of step kc
  // (slot csl): i = 0 block constants (waves 6, 7 only), 1..YF dY, YF+1
  // codes.
  // The codes come last so that one outstanding fetch at the end of a step
  // means everything else has landed.
  auto dma_one = [&](int i, int ks, int ysl, int kc, int csl) {
    char* cs = smem + kCOff + csl * kCSlot;
    ks += kbase;  // global K steps
    kc += kbase;
    if (i == 0) {
      if (wave_s == 6) dma_lds4s(r2, boff2, (uint32_t)kc * s2, cs + kC2Off);
      if (wave_s == 7) dma_lds4s(r1, boff1, (uint32_t)kc * s1, cs + kC2Off + 256);
    } else if (i <= YF) {
      dma_lds16s(ry, yoff[i - 1], (uint32_t)ks * (kDxBK * 2),
                 smem + ysl * kYBytes + (wave_s * (BM / 8) + (i - 1) * 8) * (kDxBK * 2));
    } else {
      dma_lds16s(rc, coff, (uint32_t)kc * sc, cs + wave_s * kCWave);
    }
  };
  constexpr int kLoads = YF + 2;
  constexpr int kFirst = kLoads / 2;               // fetches issued in substep 0

  struct WTile {
    u32x4 v;
    uint32_t q2;
    float q1;
  };
  auto read_w = [&](int csl, WTile& W) {
    const char* cs = smem + kCOff + csl * kCSlot;
    W.v = *reinterpret_cast<const u32x4*>(cs + wave_s * kCWave + lane * 16);
    W.q2 = *reinterpret_cast<const uint32_t*>(cs + kC2Off + wrow * 4);
    W.q1 = *reinterpret_cast<const float*>(cs + kC2Off + 256 + wrow * 4);
  };
  Lut lut;
  auto tables = [&](const WTile& W, int kc) {
    lut = build_lut_pair(qh, block_scale((W.q2 >> (wblk * 8)) & 0xFFu, W.q1, section_mean(mus, kbase + kc, dsec)));
  };
  uint32_t doff[4];
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) doff[wd] = (uint32_t)(wrow * ROWB + (wslot(wrow, wblk * 8 + half * 4 + wd) << 4));
  auto decode_word = [&](const WTile& W, int wd, char* ws) {
    *reinterpret_cast<u32x4*>(ws + doff[wd]) = dequant8(W.v[wd], lut);
  };

  uint32_t aoff[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int st = 0; st < 4; ++st) aoff[mb][st] = (uint32_t)(2 * swz(wm * WM + mb * 32 + l32, st * 2 + half));
  uint32_t boff[NB][2];
  {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = 8 * (g >> 1) + (sl >> 2) + 4 * q;
        const int col = wn * WN + nb * 32 + (g & 1) * 16 + 4 * (sl & 3);
        boff[nb][q] = (uint32_t)(r * ROWB + (wslot(r, col >> 3) << 4) + (col & 7) * 2);
      }
  }
  auto read_ab = [&](int ks, int st, u32x4 (&af)[MB], u32x4 (&bf)[NB]) {
    const char* ys = smem + (ks & 1) * kYBytes;
    const char* ws = wsm + (ks & 1) * kWBytes + st * 16 * ROWB;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u32x2 lo = lds_read_tr16(ws + boff[nb][0]);
      const u32x2 hi = lds_read_tr16(ws + boff[nb][1]);
      bf[nb] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const u32x4*>(ys + aoff[mb][st]);
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  // Pipeline as in k_dx: step ks multiplies dY tile ks by decoded tile ks,
  // decodes step ks+1 (codes fetched two steps earlier) and fetches dY tile
  // ks+1 and the codes of step ks+3 into the code slot step ks has freed.
  // The block constants are fetched by two waves for everyone: the barrier
  // at the end of each step publishes them (they land before the codes of
  // their step, which each wave waits for a step later).
  const auto clampk = [&](int x) { return x < ksteps ? x : ksteps - 1; };
  dma_one(0, 0, 0, 0, 0);
  dma_one(YF + 1, 0, 0, 0, 0);
#pragma unroll
  for (int i = 1; i <= YF; ++i) dma_one(i, 0, 0, 0, 0);
  dma_one(0, 0, 0, clampk(1), 1);
  dma_one(YF + 1, 0, 0, clampk(1), 1);
  dma_one(0, 0, 0, clampk(2), 2);
  dma_one(YF + 1, 0, 0, clampk(2), 2);
  // LoRA term first, while the first tiles land: acc = U_tile .
  // (s A)_tile^T from U (M x rp) and bf16(s A)^T (k x rp); token rows past M
  // load zeros.  With split K only the first split carries it.
  if (rp > 0 && split == 0) {
    const BufRsrc ru = make_rsrc(U, (uint64_t)M * rp * 2);
    const BufRsrc ra = make_rsrc(At, (uint64_t)k * rp * 2);
    for (int jb = 0; jb < rp; jb += 16) {
      u32x4 ua[MB], ab[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + wm * WM + mb * 32 + l32;
        const u32x4 v = ld_buf16(ru, ((uint32_t)min(m, M - 1) * (uint32_t)rp + (uint32_t)(jb + half * 8)) * 2u);
        ua[mb] = m < M ? v : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int c = c0 + wn * WN + nb * 32 + l32;
        ab[nb] = ld_buf16(ra, ((uint32_t)c * (uint32_t)rp + (uint32_t)(jb + half * 8)) * 2u);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(ua[mb], ab[nb], acc[mb][nb]);
    }
    if (DROP) {
      const BufRsrc rk = make_rsrc(keep, (uint64_t)M * k);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          drop_block(acc[mb][nb], rk, m0 + wm * WM + mb * 32, c0 + wn * WN + nb * 32 + l32, M, k, half, dscale);
    }
  }
  // codes and constants of step 0 and dY tile 0 landed (of every wave)
  if (wave_s >= 6)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  WTile W;
  read_w(0, W);
  tables(W, 0);
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) decode_word(W, wd, wsm);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  int csl_next = 1;
  for (int ks = 0; ks < ksteps; ++ks) {
    const int ky = clampk(ks + 1), kc = clampk(ks + 3), kd = clampk(ks + 1);  // kd: step decoded now
    const int ysl = (ks + 1) & 1;
    const int csl_far = csl_next == 0 ? 2 : csl_next - 1;
    char* wnext = wsm + ((ks + 1) & 1) * kWBytes;
    u32x4 af[2][MB], bf[2][NB];
    read_ab(ks, 0, af[0], bf[0]);
    read_w(csl_next, W);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st < 3) read_ab(ks, st + 1, af[(st + 1) & 1], bf[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      // the table is formed in substep 0 (its inputs arrive with this
      // step's first LDS reads) and the four words are decoded after it
      if (st == 0) tables(W, kd);
      if (st == 1) {
        decode_word(W, 0, wnext);
        decode_word(W, 1, wnext);
      }
      if (st >= 2) decode_word(W, st, wnext);
      // fetches: the first half in substep 0, the rest of dY in substep 1,
      // the codes (last) in substep 2
      if (st == 0) {
#pragma unroll
        for (int i = 0; i < kFirst; ++i) dma_one(i, ky, ysl, kc, csl_far);
      } else if (st == 1) {
#pragma unroll
        for (int i = kFirst; i < kLoads - 1; ++i) dma_one(i, ky, ysl, kc, csl_far);
      } else if (st == 2) {
        dma_one(kLoads - 1, ky, ysl, kc, csl_far);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(af[st & 1][mb], bf[st & 1][nb], acc[mb][nb]);
#pragma unroll
      for (int i = 0; i < MB * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        if (st < 3 && i < 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    csl_next = csl_next == 2 ? 0 : csl_next + 1;
  }
  (void)kLoads;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  if (part != nullptr) {
    // fp32 partial of this split (element e of a 32 x 32 block: row
    // 8*(e/4) + 4*half + e%4, column l32; 32 lanes store 128 contiguous bytes)
    float* pp = part + (size_t)split * M * k;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * WM + mb * 32 + 8 * (e / 4) + 4 * half + e % 4;
          if (m < M) pp[(size_t)m * k + c0 + wn * WN + nb * 32 + l32] = acc[mb][nb][e];
        }
    return;
  }
  // Output: each wave stages its WM x 64 tile (waves 0-3 in the fetch
  // area, 4-7 in the decoded-weight area) and stores 16-byte row chunks.
  uint16_t* stage = reinterpret_cast<uint16_t*>(wave < 4 ? smem : wsm) + (wave & 3) * (WM * 64);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mb * 32 + blk * 8 + half * 4 + i, col = q * 32 + l32;
          stage[swz(row, col >> 3) + (col & 7)] = (uint16_t)pack_bf16x2(acc[mb][q][blk * 4 + i], 0.0f);
        }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < WM / 8; ++i) {
    const int c = i * 64 + lane, row = c >> 3, ch = c & 7;
    const int m = m0 + wm * WM + row, col = c0 + wn * WN + ch * 8;
    if (m < M)
      *reinterpret_cast<u32x4*>(dX + (size_t)m * k + col) = *reinterpret_cast<const u32x4*>(&stage[swz(row, ch)]);
  }
}

// dX = bf16(sum over splits of the fp32 partials, in split order).
__global__ __launch_bounds__(256) void k_dx_sum_splits(const float* __restrict__ part, int ns, int64_t n,
                                                       uint16_t* __restrict__ dX) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 a = *reinterpret_cast<const f32x4*>(part + 4 * i);
    for (int sp = 1; sp < ns; ++sp) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(part + (size_t)sp * n + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += b[e];
    }
    *reinterpret_cast<u32x2*>(dX + 4 * i) = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  }
}

// Split K for dX when its tiles would leave CUs idle: the grid gets up to
// eight columns of K ranges (whole K steps, at least four each), every
// split writes fp32 partials and k_dx_sum_splits adds them in split order.
//  - Few tokens (16 work-groups at k = 4096 below 129 tokens, each running
//    the whole d loop): 128-row tiles, up to eight splits (four past 256
//    tokens, where the partials grow).
//  - 1024 tokens and more with fewer than 256 tiles of 256 rows (2048
//    tokens at k = 4096: 128 tiles): 256-row tiles in up to four splits
//    instead of 128-row tiles, which do half the MFMA work per decoded
//    weight and per LDS read (r = 16, 4096 x 4096: 2048 tokens 100 -> 74 +
//    12 us for the sum, 1536 tokens 92 -> 67 + 9, 1024 tokens 64 + 7 ->
//    47 + 11; 11008 x 4096: 2048 tokens 236 -> 174 + 13).
struct DxSplit {
  int S;   // K splits (1: none)
  int bm;  // token rows per tile of the split launch
};
static DxSplit dx_split(int M, int d, int k) {
  if (tile_override() != 0 || d % kDxBK != 0 || k % 256 != 0 || (uint64_t)M * d * 2 >= (1ull << 32)) return {1, 0};
  const int tiles256 = ((M + 255) / 256) * (k / 256);
  if (tiles256 >= 256) return {1, 0};  // 256-row tiles fill the chip
  const int steps = (d / kDxBK) / 4;  // splits of at least four K steps
  if (M >= 1024) {
    const int S = min(min(256 / tiles256, 4), steps);
    return S > 1 ? DxSplit{S, 256} : DxSplit{1, 0};
  }
  const int tiles = ((M + 127) / 128) * (k / 256);
  if (tiles > 128) return {1, 0};  // (128 tiles: one per two CUs, split in two)
  const int cap = M <= 256 ? 8 : 4;
  const int S = max(1, min(min(256 / tiles, cap), steps));
  return {S, S > 1 ? 128 : 0};
}

size_t dx_ws_bytes(int M, int d, int k) {
  const int S = dx_split(M, d, k).S;
  return S > 1 ? (size_t)S * M * k * sizeof(float) : 0;
}

template <bool DROP>
static hipError_t launch_dx_t(const uint16_t* dY, int M, const Nf4Dev& w, const uint16_t* U,
                              const uint16_t* At, int r, float s, uint16_t* dX, const Nf4Table& t,
                              hipStream_t st, const uint8_t* keep, float dscale, float* part) {
  const int rp = r > 0 ? padded_rank(r) : 0;
  const int tiles256 = ((M + 255) / 256) * ((w.k + 255) / 256);
  const int forced = tile_override();
  const bool even = w.d % kDxBK == 0 && w.k % 256 == 0 && (uint64_t)M * w.d * 2 < (1ull << 32);
  const DxSplit sp = dx_split(M, w.d, w.k);
  if (sp.S > 1 && part != nullptr) {
    const int ksteps = w.d / kDxBK;
    const int sps = (ksteps + sp.S - 1) / sp.S;
    const int ns = (ksteps + sps - 1) / sps;
    const int ntn = w.k / 256;
    if (sp.bm == 256)
      QLORA_LAUNCH("dx", st, (k_dx8<256, DROP>), dim3((unsigned)(ntn * ((M + 255) / 256)), (unsigned)ns),
                   dim3(64 * kDx8Waves), 0, st, dY, M, w.codes, w.c2, w.c1, w.mean, w.d, w.k, w.dsec, U, At, rp, dX, t,
                   0, ntn, keep, dscale, sps, part);
    else
      QLORA_LAUNCH("dx", st, (k_dx8<128, DROP>), dim3((unsigned)(ntn * ((M + 127) / 128)), (unsigned)ns),
                   dim3(64 * kDx8Waves), 0, st, dY, M, w.codes, w.c2, w.c1, w.mean, w.d, w.k, w.dsec, U, At, rp, dX, t,
                   0, ntn, keep, dscale, sps, part);
    const int64_t n = (int64_t)M * w.k;
    const int64_t blocks = (n / 4 + 255) / 256;
    QLORA_LAUNCH("dx_sum_splits", st, k_dx_sum_splits, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                 st, part, ns, n, dX);
    return hipGetLastError();
  }
  if (even && forced == 0) {
    // Whole rounds of 256-row tiles; the column tiles that would make a
    // last, partial round run as 128-row tiles in a second launch when those
    // fit in one round (as in the forward).
    const int ntn = w.k / 256;
    int c256 = 0;
    if (tiles256 >= 256) {
      const int ntm = (M + 255) / 256;
      c256 = ntn;
      if (tiles256 % 256 != 0 && tiles256 < 3 * 256) {  // with more full rounds the tail overlaps them (measured)
        const int full = (tiles256 / 256) * 256 / ntm;
        if ((ntn - full) * ((M + 127) / 128) <= 256) c256 = full;
      }
    }
    const int c128 = ntn - c256;
    if (c256 > 0)
      QLORA_LAUNCH("dx", st, (k_dx8<256, DROP>), dim3((unsigned)(c256 * ((M + 255) / 256))), dim3(64 * kDx8Waves), 0,
                   st, dY, M, w.codes, w.c2, w.c1, w.mean, w.d, w.k, w.dsec, U, At, rp, dX, t, 0, c256, keep, dscale, 0,
                   nullptr);
    if (c128 > 0)
      QLORA_LAUNCH("dx", st, (k_dx8<128, DROP>), dim3((unsigned)(c128 * ((M + 127) / 128))), dim3(64 * kDx8Waves), 0,
                   st, dY, M, w.codes, w.c2, w.c1, w.mean, w.d, w.k, w.dsec, U, At, rp, dX, t, c256 * 256, c128, keep,
                   dscale, 0, nullptr);
  } else if (forced == 256 || (forced == 0 && tiles256 >= 256)) {
    dim3 grid((unsigned)tiles256);
    QLORA_LAUNCH("dx", st, (k_dx<256, 256, DROP>), grid, dim3(256), 0, st, dY, M, w.codes, w.c2, w.c1, w.mean,
                 w.d, w.k, w.dsec, U, At, rp, s, dX, t, keep, dscale);
  } else {
    dim3 grid((unsigned)(((M + 127) / 128) * ((w.k + 127) / 128)));
    QLORA_LAUNCH("dx", st, (k_dx<128, 128, DROP>), grid, dim3(256), 0, st, dY, M, w.codes, w.c2, w.c1, w.mean,
                 w.d, w.k, w.dsec, U, At, rp, s, dX, t, keep, dscale);
  }
  return hipGetLastError();
}

hipError_t launch_dx(const uint16_t* dY, int M, const Nf4Dev& w, const uint16_t* U,
                     const uint16_t* At, int r, float s, uint16_t* dX, const Nf4Table& t,
                     hipStream_t st, const uint8_t* keep, float dscale, float* part) {
  if (keep != nullptr && r > 0) return launch_dx_t<true>(dY, M, w, U, At, r, s, dX, t, st, keep, dscale, part);
  return launch_dx_t<false>(dY, M, w, U, At, r, s, dX, t, st, nullptr, 1.0f, part);
}

}  // namespace qlora
