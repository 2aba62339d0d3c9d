// lora.hip -- the rank-r pieces of the adapted linear (page "LoRA and QLoRA
// fine-tuning: mechanics, and when not to fine-tune", section "The update
// LoRA is allowed to learn"; page "Fine-Tuning on a Budget", "The LoRA
// hypothesis"):
//
//   k_prep          B^T (rp x d), zero-padded, for ranks that are not a
//                   multiple of 8 (and the scaled copies of older callers).
//   k_proj          P = V L^T for a skinny L: the down-projection T = X A^T
//                   (L = A, r x K) and the backward vector U = dY B (L = B as
//                   stored, K x r, staged and read back transposed).  HBM-
//                   bound on V; MFMA 16x16x32 with V rows as the 16-row
//                   operand.  Writes P (M x rp, bf16) and optionally P^T
//                   (r x ldt); the U launch also writes bf16(s A)^T.
//   k_proj2         The same product with V (and L = A) fetched to LDS in
//                   whole-row chunks, for more than 16 ranks or few row
//                   blocks.
//   k_tokred        out = s Z^T V summed over tokens for Z^T (r x ldz):
//                   dA = s U^T X and dB^T = s T^T dY in one launch.  The
//                   contraction runs over tokens, the row index of V, so V
//                   is staged in LDS and read back with transposing reads.
//                   Work-groups own a column strip and every token; no
//                   partial sums leave a work-group (deterministic, no
//                   atomics).
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace qlora {

// Bp = bf16(s B) and At = bf16(s A)^T carry the LoRA scale, so the
// up-projections accumulate into the GEMM accumulators with no extra
// arithmetic; the rounding is exact when s is a power of two and otherwise
// at most half a bf16 ulp of each scaled adapter entry.  Bt = B^T (unscaled).
// One work-group per 64 rows i (of B and of A^T): the 64 x r slab of B and
// the r x 64 slab of A are contiguous in memory, staged through LDS, and
// every output row segment is written contiguously.
__global__ __launch_bounds__(256) void k_prep(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                             int d, int k, int r, int rp, float s,
                                             uint16_t* __restrict__ Bp, uint16_t* __restrict__ Bt,
                                             uint16_t* __restrict__ At) {
  __shared__ uint16_t tb[64][kMaxRank + 1];  // [i][j]: B slab, then A^T slab
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * 64;
  if ((Bp || Bt) && i0 < d) {
    const int rows = min(64, d - i0);
    for (int e = tid; e < 64 * rp; e += 256) {
      const int i = e / rp, j = e % rp;
      tb[i][j] = (i < rows && j < r) ? B[(size_t)(i0 + i) * r + j] : (uint16_t)0;
    }
    __syncthreads();
    if (Bp)
      for (int e = tid; e < rows * rp; e += 256) {
        const int i = e / rp, j = e % rp;
        Bp[(size_t)(i0 + i) * rp + j] = (uint16_t)pack_bf16x2(s * bf16_to_f32(tb[i][j]), 0.0f);
      }
    if (Bt)
      for (int e = tid; e < rp * 64; e += 256) {
        const int j = e / 64, i = e % 64;
        if (i < rows) Bt[(size_t)j * d + i0 + i] = tb[i][j];
      }
    __syncthreads();
  }
  if (At && i0 < k) {
    const int rows = min(64, k - i0);
    for (int e = tid; e < rp * 64; e += 256) {
      const int j = e / 64, i = e % 64;
      tb[i][j] = (i < rows && j < r) ? A[(size_t)j * k + i0 + i] : (uint16_t)0;
    }
    __syncthreads();
    for (int e = tid; e < rows * rp; e += 256) {
      const int i = e / rp, j = e % rp;
      At[(size_t)(i0 + i) * rp + j] = (uint16_t)pack_bf16x2(s * bf16_to_f32(tb[i][j]), 0.0f);
    }
  }
}

hipError_t launch_prep_adapters(const uint16_t* A, const uint16_t* B, int d, int k, int r, float s,
                                uint16_t* Bp, uint16_t* Bt, uint16_t* At, hipStream_t st) {
  const int rp = padded_rank(r);
  const int n = ((d > k ? d : k) + 63) / 64;
  QLORA_LAUNCH("prep_adapters", st, k_prep, dim3((unsigned)n), dim3(256), 0, st, A, B, d, k, r, rp, s, Bp, Bt, At);
  return hipGetLastError();
}

// ------------------------------------------------------------- lora_proj --
//
// P = V L^T, V (M x K) and L (r x K) bf16, K contiguous in both: each
// work-group owns 16 rows of V and a range of K (the whole of K unless M is
// small), its eight waves (two per SIMD) taking interleaved 32-wide K
// steps.  One MFMA 16x16x32 per step and 16 ranks: A = 16 rows of V, B = 16
// rows of L, so D holds (row, rank).  HBM-bound on V: each wave keeps two
// steps' loads in flight (registers double-buffered).  Rows past M
// and ranks past r read clamped addresses and are never stored; K lanes
// past K read zeros.  The waves' sums are added in a fixed order.

constexpr int kProjStep = 32;

constexpr int kLoraWaves = 8;  // waves per work-group of the projection kernel

// LT: L is given transposed (Lt, K x r row-major -- the adapter B as
// stored, for U = dY B), r a multiple of 8.  Per step and 16-rank block a
// lane loads 16 bytes of Lt (row st*32 + l/2, ranks jb*16 + 8*(l%2) .. +7),
// the wave stages the 32 x 16 piece in LDS (32-byte rows; rows 8..15 and
// 24..31 of the piece move by 128 bytes so that a transposing read's 32
// lanes meet distinct banks) and reads its B operand back with two
// transposing reads (rank l%16, eight consecutive k).
//
// Extra work-groups (blockIdx.x >= the row blocks, first split only) write
// At = bf16(s A)^T, zero-padded to rp ranks (k x rp), for the dX epilogue:
// one work-group per 64 rows of At.
struct AtJob {
  const uint16_t* A;
  int k;
  float s;
  uint16_t* At;
  int r, ld;  // ranks of A, row stride of At (r padded to 16)
};

template <int NJ, bool LT>
__global__ __launch_bounds__(64 * kLoraWaves) void k_proj(const uint16_t* __restrict__ V, int M, int K, int ldv,
                                             const uint16_t* __restrict__ L, int r, int rp, int rl, int dsec,
                                             int steps_per_split, float* __restrict__ part,
                                             uint16_t* __restrict__ P, int ldp, uint16_t* __restrict__ Pt,
                                             int ldt, AtJob aj) {
  constexpr int B = 1;  // steps per batch (shallow batches measured fastest; two batches in flight)
  constexpr int W = kLoraWaves;
  __shared__ float red[W - 1][NJ][64][4];
  __shared__ __attribute__((aligned(16))) char lst[LT ? W : 1][LT ? B * NJ : 1][1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int mt = (M + 15) / 16;
  if ((int)blockIdx.x >= mt) {
    if (blockIdx.y != 0) return;
    const int i0 = ((int)blockIdx.x - mt) * 64;
    const int rows = min(64, aj.k - i0);
    for (int e = tid; e < rows * aj.ld; e += 64 * W) {
      const int i = e / aj.ld, j = e % aj.ld;
      const float a = j < aj.r ? aj.s * bf16_to_f32(aj.A[(size_t)j * aj.k + i0 + i]) : 0.0f;
      aj.At[(size_t)(i0 + i) * aj.ld + j] = (uint16_t)pack_bf16x2(a, 0.0f);
    }
    return;
  }
  const int m = blockIdx.x * 16 + l16;
  const int mc = m < M ? m : M - 1;
  const int split = blockIdx.y;
  const int nsteps = (K + kProjStep - 1) / kProjStep;
  const int s0 = split * steps_per_split;
  const int s1 = min(nsteps, s0 + steps_per_split);
  const BufRsrc rv = make_rsrc(V, ((uint64_t)(M - 1) * ldv + K) * 2);
  const BufRsrc rlr = make_rsrc(L, (uint64_t)(LT ? rl : r) * K * 2);
  const uint32_t vb = ((uint32_t)mc * (uint32_t)ldv + 8u * g) * 2u;
  uint32_t lb[NJ];
  int slo[NJ];  // LT: first K row of the section that feeds rank block jb
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    if (LT) {
      const int rbl = (rl + 15) >> 4;  // rank blocks per section
      lb[jb] = ((uint32_t)(lane >> 1) * (uint32_t)rl + (uint32_t)((jb % rbl) * 16 + 8 * (lane & 1))) * 2u;
      slo[jb] = (jb / rbl) * dsec;
    } else {
      slo[jb] = 0;
      const int j = jb * 16 + l16;
      lb[jb] = ((uint32_t)(j < r ? j : r - 1) * (uint32_t)K + 8u * g) * 2u;
    }
  }
  // LT staging: write position of this lane's 16 bytes, transposing-read
  // positions of its operand (rows 8g + l16/4 (+4), ranks 4*(l16%4) .. +3)
  const uint32_t lwr = (uint32_t)(lane * 16) ^ ((uint32_t)((lane >> 4) & 1) << 7);
  auto lpos = [](int row, int col) { return (uint32_t)((row * 32 + col * 2) ^ (((row >> 3) & 1) << 7)); };
  const uint32_t tro0 = lpos(8 * g + (l16 >> 2), 4 * (l16 & 3));
  const uint32_t tro1 = lpos(8 * g + (l16 >> 2) + 4, 4 * (l16 & 3));

  f32x4 acc[NJ];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // batch starting at this wave's step index t (steps s0 + wave + W*(t+u))
  auto load = [&](int t, u32x4 (&a)[B], u32x4 (&b)[B][NJ]) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int st = s0 + wave + W * (t + u);
      const int kk = st * kProjStep + 8 * g;
      const bool ok = st < s1 && kk < K;
      const uint32_t o = ok ? (uint32_t)st * (kProjStep * 2) : 0u;
      const u32x4 v = ld_buf16(rv, vb + o);
      a[u] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      // LT: rows past K read zeros (past the end of Lt) or rows of the next
      // steps, which meet zeroed V lanes
      const uint32_t ol = LT ? (st < s1 ? (uint32_t)st * (uint32_t)(kProjStep * 2) * (uint32_t)rl : 0u) : o;
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        b[u][jb] = ld_buf16(rlr, lb[jb] + ol);
        // LT with sections: rank block jb only sees the K rows of its own
        // section (block-diagonal adapter); other steps add exact zeros
        if (LT && (uint32_t)(st * kProjStep - slo[jb]) >= (uint32_t)dsec) b[u][jb] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto compute = [&](const u32x4 (&a)[B], const u32x4 (&b)[B][NJ]) {
#pragma unroll
    for (int u = 0; u < B; ++u)
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        u32x4 bop = b[u][jb];
        if (LT) {
          char* c = &lst[LT ? wave : 0][LT ? u * NJ + jb : 0][0];
          *reinterpret_cast<u32x4*>(c + lwr) = b[u][jb];
          const u32x2 lo = lds_read_tr16(c + tro0);
          const u32x2 hi = lds_read_tr16(c + tro1);
          bop = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        acc[jb] = mfma16(a[u], bop, acc[jb]);
      }
  };
  const int nw = (s1 - s0 - wave + W - 1) / W;  // steps of this wave
  u32x4 a0[B], b0[B][NJ], a1[B], b1[B][NJ];
  load(0, a0, b0);
  for (int t = 0; t < nw; t += 2 * B) {
    load(t + B, a1, b1);
    compute(a0, b0);
    load(t + 2 * B, a0, b0);
    compute(a1, b1);
  }

  // Fixed-order sum of the waves: (((w0 + w1) + w2) + ...).
  if (wave > 0) {
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave - 1][jb][lane][i] = acc[jb][i];
  }
  __syncthreads();
  if (wave != 0) return;
  // lane holds rows 4g+i of the 16-row block and rank column jb*16 + l16
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jb * 16 + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = blockIdx.x * 16 + 4 * g + i;
      float v = acc[jb][i];
#pragma unroll
      for (int w = 0; w < W - 1; ++w) v += red[w][jb][lane][i];
      if (mm >= M) continue;
      if (part != nullptr) {
        part[((size_t)split * M + mm) * rp + j] = j < r ? v : 0.0f;
      } else {
        const uint16_t h = j < r ? (uint16_t)pack_bf16x2(v, 0.0f) : (uint16_t)0;
        P[(size_t)mm * ldp + j] = h;
        if (Pt != nullptr && j < r) Pt[(size_t)j * ldt + mm] = h;
      }
    }
  }
}

// Staged form (all shapes): the same product, with V (and L unless given
// transposed) fetched global->LDS in chunks of CK columns of K.  A fetch
// covers 1 KB of whole row segments (at least 256 bytes of one row), so a
// fetch touches a quarter of the 128-byte lines that a register load of 16
// rows x 64 bytes -- the MFMA operand layout -- would touch; the operands
// are read back from LDS, the 16-byte pieces of row t placed at piece ^
// (t % 16) so that those reads are free of bank conflicts.  Two slots: the
// next chunk is in flight while this one is multiplied.  Wave w takes the
// 32-wide K sub-steps w, w+8, ... of each chunk.  With L transposed (Lt, K
// x r, rows of r bf16 -- already contiguous) each wave loads its pieces of
// Lt into registers one chunk ahead and transposes them through LDS as in
// k_proj.
template <int NJ>
constexpr int proj_chunk() { return NJ == 1 ? 1024 : NJ == 4 ? 256 : 512; }

// NR row blocks of 16 tokens per work-group (NR > 1 only with L as stored):
// each L chunk then serves 16 NR rows of V, so L -- read whole by every
// work-group -- moves NR times less over the grid.
template <int NJ, bool LT, int NR>
__global__ __launch_bounds__(64 * kLoraWaves) void k_proj2(const uint16_t* __restrict__ V, int M, int K, int ldv,
                                              const uint16_t* __restrict__ L, int r, int rp, int rl, int dsec,
                                              int chunks_per_split, float* __restrict__ part,
                                              uint16_t* __restrict__ P, int ldp, uint16_t* __restrict__ Pt,
                                              int ldt, AtJob aj) {
  static_assert(NR == 1 || !LT, "row blocks with L as stored only");
  constexpr int W = kLoraWaves;
  constexpr int RM = 16 * NR;                 // token rows per work-group
  constexpr int CK = proj_chunk<NJ>();
  constexpr int PR = CK / 8;                  // 16-byte pieces per row segment
  constexpr int SUB = CK / 32 / W;            // sub-steps per wave per chunk
  constexpr int FV = NR * CK / 256;           // V fetches per wave per chunk (RM rows)
  constexpr int FL = LT ? 0 : NJ * CK / 256;  // L fetches per wave per chunk (16 NJ rows)
  constexpr int kVBytes = RM * CK * 2;
  constexpr int kLBytes = LT ? 0 : 16 * NJ * CK * 2;
  constexpr int kSlot = kVBytes + kLBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * kSlot];
  // the waves' sums: their own array with one row block, else the slots
  // (free once the K loop is done)
  constexpr int kRedBytes = (W - 1) * NR * NJ * 64 * 16;
  static_assert(NR == 1 || kRedBytes <= 2 * kSlot, "sums fit the slots");
  __shared__ __attribute__((aligned(16))) char red_own[NR == 1 ? kRedBytes : 16];
  __shared__ __attribute__((aligned(16))) char lst[LT ? W : 1][LT ? NJ : 1][1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 4, l16 = lane & 15;
  const int mt = (M + RM - 1) / RM;
  if ((int)blockIdx.x >= mt) {
    if (blockIdx.y != 0) return;
    const int i0 = ((int)blockIdx.x - mt) * 64;
    const int rows = min(64, aj.k - i0);
    for (int e = tid; e < rows * aj.ld; e += 64 * W) {
      const int i = e / aj.ld, j = e % aj.ld;
      const float a = j < aj.r ? aj.s * bf16_to_f32(aj.A[(size_t)j * aj.k + i0 + i]) : 0.0f;
      aj.At[(size_t)(i0 + i) * aj.ld + j] = (uint16_t)pack_bf16x2(a, 0.0f);
    }
    return;
  }
  const int m0 = blockIdx.x * RM;
  const int split = blockIdx.y;
  const int nch = (K + CK - 1) / CK;
  const int c0 = split * chunks_per_split;
  const int nc = min(chunks_per_split, nch - c0);
  const BufRsrc rv = make_rsrc(V, ((uint64_t)(M - 1) * ldv + K) * 2);
  const BufRsrc rlr = make_rsrc(L, (uint64_t)(LT ? rl : r) * K * 2);
  const uint32_t voob = ((uint32_t)(M - 1) * (uint32_t)ldv + (uint32_t)K) * 2u;  // offsets here read zeros
  const uint32_t loob = (uint32_t)(LT ? rl : r) * (uint32_t)K * 2u;

  // fetch lanes: global piece q = f*64 + lane of the chunk's row segments
  int vrow[FV], vpc[FV];
#pragma unroll
  for (int i = 0; i < FV; ++i) {
    const int q = (wave + W * i) * 64 + lane;
    vrow[i] = q / PR;
    vpc[i] = (q % PR) ^ (vrow[i] & 15);
  }
  int lrow[FL > 0 ? FL : 1], lpc[FL > 0 ? FL : 1];
#pragma unroll
  for (int i = 0; i < FL; ++i) {
    const int q = (wave + W * i) * 64 + lane;
    lrow[i] = q / PR;
    lpc[i] = (q % PR) ^ (lrow[i] & 15);
  }
  // LT: this lane's 16 bytes of Lt per sub-step and rank block (row kk +
  // lane/2, ranks jb*16 + 8*(lane%2) .. +7), as in k_proj
  // With sections (LT), rank block jb belongs to section jb / rbl and reads
  // only the K rows of that section (block-diagonal adapter).
  uint32_t lb[NJ];
  int slo[NJ];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int rbl = (rl + 15) >> 4;
    lb[jb] = ((uint32_t)(lane >> 1) * (uint32_t)rl + (uint32_t)((jb % rbl) * 16 + 8 * (lane & 1))) * 2u;
    slo[jb] = (jb / rbl) * dsec;
  }
  const uint32_t lwr = (uint32_t)(lane * 16) ^ ((uint32_t)((lane >> 4) & 1) << 7);
  auto lpos = [](int row, int col) { return (uint32_t)((row * 32 + col * 2) ^ (((row >> 3) & 1) << 7)); };
  const uint32_t tro0 = lpos(8 * g + (l16 >> 2), 4 * (l16 & 3));
  const uint32_t tro1 = lpos(8 * g + (l16 >> 2) + 4, 4 * (l16 & 3));

  u32x4 lr[2][LT ? SUB : 1][NJ];  // LT: Lt pieces of the current and next chunk
  auto fetch = [&](int c, int sl, u32x4 (&lreg)[LT ? SUB : 1][NJ]) {
    const int kb = (c0 + c) * CK;
    char* slot = smem + sl * kSlot;
    if (LT) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int kk = kb + 32 * (wave + W * u);
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
          lreg[LT ? u : 0][jb] = ld_buf16(rlr, kk < K && (uint32_t)(kk - slo[jb]) < (uint32_t)dsec
                                                   ? lb[jb] + (uint32_t)kk * (uint32_t)rl * 2u
                                                   : loob);
      }
    }
#pragma unroll
    for (int i = 0; i < FV; ++i) {
      const int kp = kb + vpc[i] * 8;
      const int m = m0 + vrow[i];
      dma_lds16(rv, m < M && kp < K ? ((uint32_t)m * (uint32_t)ldv + (uint32_t)kp) * 2u : voob,
                slot + (wave_s + W * i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < FL; ++i) {
      const int kp = kb + lpc[i] * 8;
      const int j = lrow[i];
      dma_lds16(rlr, j < r && kp < K ? ((uint32_t)j * (uint32_t)K + (uint32_t)kp) * 2u : loob,
                slot + kVBytes + (wave_s + W * i) * 1024);
    }
  };

  f32x4 acc[NR][NJ];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb)
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) acc[rb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // chunk c uses slot c % 2 and (LT) register set c % 2; chunks are taken in
  // pairs so that the register sets are named statically
  auto chunk = [&](int c, auto par) {
    constexpr int PB = decltype(par)::value;
    // this wave's loads of chunk c are done once only chunk c+1's are in
    // flight
    if (c + 1 < nc)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(FV + FL + (LT ? SUB * NJ : 0)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* slot = smem + PB * kSlot;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int piece = 4 * (wave + W * u) + g;
      u32x4 a[NR];
#pragma unroll
      for (int rb = 0; rb < NR; ++rb)
        a[rb] = *reinterpret_cast<const u32x4*>(slot + (rb * 16 + l16) * (CK * 2) + ((piece ^ l16) << 4));
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        u32x4 bop;
        if (LT) {
          char* cst = &lst[LT ? wave : 0][LT ? jb : 0][0];
          *reinterpret_cast<u32x4*>(cst + lwr) = lr[PB][LT ? u : 0][jb];
          const u32x2 lo = lds_read_tr16(cst + tro0);
          const u32x2 hi = lds_read_tr16(cst + tro1);
          bop = u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
          bop = *reinterpret_cast<const u32x4*>(slot + kVBytes + (jb * 16 + l16) * (CK * 2) + ((piece ^ l16) << 4));
        }
#pragma unroll
        for (int rb = 0; rb < NR; ++rb) acc[rb][jb] = mfma16(a[rb], bop, acc[rb][jb]);
      }
    }
    if (c + 2 < nc) {
      __syncthreads();
      fetch(c + 2, PB, lr[PB]);
    }
  };
  if (nc > 0) fetch(0, 0, lr[0]);
  if (nc > 1) fetch(1, 1, lr[1]);
  for (int c = 0; c < nc; c += 2) {
    chunk(c, std::integral_constant<int, 0>{});
    if (c + 1 < nc) chunk(c + 1, std::integral_constant<int, 1>{});
  }

  // Fixed-order sum of the waves: (((w0 + w1) + w2) + ...).
  char* redb = red_own;
  if constexpr (NR > 1) {
    __syncthreads();  // every wave is done with the slots
    redb = smem;
  }
  float(*red)[NR][NJ][64][4] = reinterpret_cast<float(*)[NR][NJ][64][4]>(redb);
  if (wave > 0) {
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][rb][jb][lane][i] = acc[rb][jb][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int rb = 0; rb < NR; ++rb)
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jb * 16 + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = m0 + rb * 16 + 4 * g + i;
      float v = acc[rb][jb][i];
#pragma unroll
      for (int w = 0; w < W - 1; ++w) v += red[w][rb][jb][lane][i];
      if (mm >= M) continue;
      if (part != nullptr) {
        part[((size_t)split * M + mm) * rp + j] = j < r ? v : 0.0f;
      } else {
        const uint16_t h = j < r ? (uint16_t)pack_bf16x2(v, 0.0f) : (uint16_t)0;
        P[(size_t)mm * ldp + j] = h;
        if (Pt != nullptr && j < r) Pt[(size_t)j * ldt + mm] = h;
      }
    }
  }
}

// LoRA dropout of the adapter input: Xd = bf16(fl32(x * scale)) where keep
// is nonzero, else 0 (scale = 1/(1-p)); eight elements per thread and step.
__global__ __launch_bounds__(256) void k_drop_input(const uint16_t* __restrict__ X,
                                                    const uint8_t* __restrict__ keep, int64_t n8, float scale,
                                                    uint16_t* __restrict__ Xd) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(X + 8 * i);
    const u32x2 kp = *reinterpret_cast<const u32x2*>(keep + 8 * i);
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t kb = (p < 2 ? kp.x : kp.y) >> (16 * (p & 1));
      const float lo = (kb & 0xFFu) ? __fmul_rn(bf16_lo(x[p]), scale) : 0.0f;
      const float hi = (kb & 0xFF00u) ? __fmul_rn(bf16_hi(x[p]), scale) : 0.0f;
      o[p] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(Xd + 8 * i) = o;
  }
}

hipError_t launch_drop_input(const uint16_t* X, const uint8_t* keep, int64_t n, float scale, uint16_t* Xd,
                             hipStream_t st) {
  const int64_t n8 = n / 8;
  const int64_t blocks = (n8 + 255) / 256;
  QLORA_LAUNCH("drop_input", st, k_drop_input, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, X,
               keep, n8, scale, Xd);
  return hipGetLastError();
}

__global__ void k_lora_proj_finish(const float* __restrict__ part, int nsplit, int M, int r, int rp,
                                   uint16_t* __restrict__ P, int ldp, uint16_t* __restrict__ Pt, int ldt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * rp) return;
  const int mm = (int)(idx / rp), j = (int)(idx % rp);
  const float v = sum_strided(part + (size_t)mm * rp + j, (size_t)M * rp, nsplit);
  const uint16_t h = (uint16_t)pack_bf16x2(v, 0.0f);
  P[(size_t)mm * ldp + j] = h;
  if (Pt != nullptr && j < r) Pt[(size_t)j * ldt + mm] = h;
}

// Split K only when the 16-row blocks alone would leave most CUs idle
// (splits are whole chunks of the staged kernel).
static int proj_chunk_host(int rp) { return rp <= 16 ? 1024 : rp > 48 ? 256 : 512; }

// Token rows per work-group of the staged kernel: 64 for 64 ranks of L as
// stored (k_proj2<4, false, 4>), else 16.
static int proj_rows(int rp, bool lt) { return rp == 64 && !lt ? 64 : 16; }

static void proj_split(int M, int K, int rp, bool lt, int* ns, int* cps) {
  const int mt = (M + proj_rows(rp, lt) - 1) / proj_rows(rp, lt);
  const int ck = proj_chunk_host(rp);
  const int nch = (K + ck - 1) / ck;
  int want = mt >= 128 ? 1 : (256 + mt - 1) / mt;
  if (want > nch) want = nch;
  if (want > 64) want = 64;
  if (want < 1) want = 1;
  *cps = (nch + want - 1) / want;
  *ns = (nch + *cps - 1) / *cps;
}

// A projection with more than kMaxRank ranks (row sections: nsec * r of
// them) runs as one launch per group of at most kMaxRank ranks, in order on
// the stream: whole sections when L is given transposed (a group reads only
// its sections' columns of V), else consecutive 64-rank slices of L's rows
// (every group reads all of V).  One group otherwise.
struct ProjGroup {
  int koff, K;  // columns of V (and rows of a transposed L) the group reads
  int j0, r;    // output ranks j0 .. j0 + r - 1
  int nsec;     // sections within the group (transposed L)
};

static int proj_groups(int K, int r, int nsec, bool lt, ProjGroup (&g)[kMaxSections]) {
  if (padded_rank(r) <= kMaxRank) {
    g[0] = ProjGroup{0, K, 0, r, nsec};
    return 1;
  }
  int n = 0;
  if (lt) {
    const int rl = r / nsec, dsec = K / nsec, per = kMaxRank / rl;
    for (int p0 = 0; p0 < nsec; p0 += per) {
      const int np = min(per, nsec - p0);
      g[n++] = ProjGroup{p0 * dsec, np * dsec, p0 * rl, np * rl, np};
    }
  } else {
    for (int j0 = 0; j0 < r; j0 += kMaxRank) g[n++] = ProjGroup{0, K, j0, min(kMaxRank, r - j0), 1};
  }
  return n;
}

static bool proj_groups_valid(int K, int r, int nsec, bool lt) {
  if (r < 1 || r > kMaxSections * kMaxRank || nsec < 1 || nsec > kMaxSections) return false;
  if (r % nsec != 0 || K % nsec != 0 || (nsec > 1 && !lt)) return false;
  if (nsec > 1 && ((r / nsec) % 16 != 0 || (K / nsec) % kProjStep != 0 || r / nsec > kMaxRank)) return false;
  return !(padded_rank(r) > kMaxRank && lt && nsec == 1);
}

size_t lora_proj_ws_bytes(int M, int K, int r, int nsec, bool l_transposed) {
  if (!proj_groups_valid(K, r, nsec, l_transposed)) return 0;
  ProjGroup g[kMaxSections];
  const int n = proj_groups(K, r, nsec, l_transposed, g);
  size_t bytes = 0;
  for (int i = 0; i < n; ++i) {
    int ns, cps;
    proj_split(M, g[i].K, padded_rank(g[i].r), l_transposed, &ns, &cps);
    const size_t b = ns > 1 ? (size_t)ns * M * padded_rank(g[i].r) * sizeof(float) : 0;
    bytes = b > bytes ? b : bytes;
  }
  return bytes;
}

// One launch (at most kMaxRank ranks): V (M x K, rows ldv apart), P rows
// ldp apart.
static hipError_t proj_launch(const uint16_t* V, int M, int K, int ldv, const uint16_t* L, bool lt, int r,
                              int nsec, uint16_t* P, int ldp, uint16_t* Pt, int ldt, float* partial, AtJob aj,
                              hipStream_t st) {
  const int rp = padded_rank(r);
  const int rl = r / nsec, dsec = K / nsec;
  int ns, sps;
  proj_split(M, K, rp, lt, &ns, &sps);
  const int mt = (M + proj_rows(rp, lt) - 1) / proj_rows(rp, lt);
  const int naux = aj.At != nullptr ? (aj.k + 63) / 64 : 0;
  dim3 grid((unsigned)(mt + naux), (unsigned)ns);
  float* part = ns > 1 ? partial : nullptr;
  // The register-load kernel is as fast as the staged one for one 16-rank
  // block over many row blocks (measured at 4096 x 4096, M = 4096); the
  // staged kernel is faster for more ranks and for fewer row blocks.
  const bool staged = !(rp == 16 && mt >= 256);
  const int steps = (K + kProjStep - 1) / kProjStep;  // register-load kernel: no split (ns == 1 here)
#define QLORA_PROJ(NJ, LT)                                                                                      \
  do {                                                                                                          \
    if (staged)                                                                                                 \
      QLORA_LAUNCH("lora_proj", st, (k_proj2<NJ, LT, (NJ == 4 && !LT) ? 4 : 1>), grid, dim3(64 * kLoraWaves), 0, \
                   st, V, M, K, ldv, L, r, rp, rl, dsec, sps, part, P, ldp, Pt, ldt, aj);                       \
    else                                                                                                        \
      QLORA_LAUNCH("lora_proj", st, (k_proj<NJ, LT>), grid, dim3(64 * kLoraWaves), 0, st, V, M, K, ldv, L, r,   \
                   rp, rl, dsec, steps, part, P, ldp, Pt, ldt, aj);                                             \
  } while (0)
  if (lt) {
    switch (rp / 16) {
      case 1: QLORA_PROJ(1, true); break;
      case 2: QLORA_PROJ(2, true); break;
      case 3: QLORA_PROJ(3, true); break;
      default: QLORA_PROJ(4, true); break;
    }
  } else {
    switch (rp / 16) {
      case 1: QLORA_PROJ(1, false); break;
      case 2: QLORA_PROJ(2, false); break;
      case 3: QLORA_PROJ(3, false); break;
      default: QLORA_PROJ(4, false); break;
    }
  }
#undef QLORA_PROJ
  if (ns > 1) {
    const int64_t n = (int64_t)M * rp;
    QLORA_LAUNCH("lora_proj_finish", st, k_lora_proj_finish, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                 partial, ns, M, r, rp, P, ldp, Pt, ldt);
  }
  return hipGetLastError();
}

hipError_t launch_lora_proj(const uint16_t* V, int M, int K, const uint16_t* L, bool l_transposed, int r,
                            int nsec, uint16_t* P, uint16_t* Pt, int ldt, float* partial, const uint16_t* A_for_at,
                            int k_at, float s_at, uint16_t* At, hipStream_t st) {
  // Sections (transposed L only): L is K x (r / nsec), and rank block j of
  // the output sees only the K rows of its own section.
  if (!proj_groups_valid(K, r, nsec, l_transposed)) return hipErrorInvalidValue;
  if (l_transposed && r % 8 != 0) return hipErrorInvalidValue;
  const int rp = padded_rank(r);
  const int rl = r / nsec;
  ProjGroup g[kMaxSections];
  const int n = proj_groups(K, r, nsec, l_transposed, g);
  hipError_t e = hipSuccess;
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    // the first launch also writes bf16(s A)^T for all r ranks
    const AtJob aj{A_for_at, k_at, s_at, i == 0 ? At : nullptr, r, rp};
    const uint16_t* Lg = l_transposed ? L + (size_t)g[i].koff * rl : L + (size_t)g[i].j0 * K;
    e = proj_launch(V + g[i].koff, M, g[i].K, K, Lg, l_transposed, g[i].r, g[i].nsec, P + g[i].j0, rp,
                    Pt != nullptr ? Pt + (size_t)g[i].j0 * ldt : nullptr, ldt, partial, aj, st);
  }
  return e;
}

// ----------------------------------------------------------- token_reduce --
//
// out = s Z^T V over tokens: dA = s U^T X (r x k) and dB = s dY^T T (d x r,
// written transposed).  Z^T (r x ldz, tokens contiguous) is the MFMA A
// operand as stored; V (M x N) is read down its columns.  A work-group owns
// a 32-column strip of V and every token: its eight waves take equal token
// ranges, in steps of 32 tokens, and the strip's two 16-column MFMA blocks
// share each Z operand.  A wave fetches each step global->LDS (two 1 KB
// fetches of V -- 32 tokens x 64 bytes -- and one 1 KB piece of Z^T per 16
// ranks) into its own ring of R steps, R-1 steps ahead, and reads the V
// operands back with the transposing LDS read (one column per lane, eight
// tokens per two reads).  The 16-byte chunks of a staged V row are XOR-ed
// with bit 3 of the row so that the 32 lanes of a transposing read hit 32
// distinct bank pairs.  No partial sums leave the work-group; the waves are
// added in a fixed order.  V rows past M repeat row M-1 and columns past N
// repeat earlier columns (never stored); Z tokens past M are zeroed on the
// last step (the padding of Z^T is unspecified).  Ranks past r read rank
// r-1 and are never stored.

constexpr int kRedStep = 32;  // tokens per wave step
constexpr int kRedWaves = 8;

// The four transposing reads of a step (two per 16-column block) in one
// block that also waits for them.  Written out because the compiler drains
// every outstanding global->LDS fetch (vmcnt(0)) before a transposing read
// of an LDS buffer that such fetches target, which would serialize the
// ring; the explicit vmcnt wait before this block orders it after the
// step's own fetches.
__device__ __forceinline__ void tr_reads4(const char* slot, const uint32_t (&off)[2][2], u32x4 (&vb)[2]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base = (uint32_t)(uintptr_t)slot;
  u32x2 a, b, c, e;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(e)
      : "v"(base + off[0][0]), "v"(base + off[0][1]), "v"(base + off[1][0]), "v"(base + off[1][1])
      : "memory");
  vb[0] = u32x4{a.x, a.y, b.x, b.y};
  vb[1] = u32x4{c.x, c.y, e.x, e.y};
#else
  (void)slot; (void)off;
  vb[0] = vb[1] = u32x4{0u, 0u, 0u, 0u};
#endif
}

// One reduction of a launch: out = s Z^T V with V (M x N), r output ranks.
// Sections: the columns of V fall into sections of dsec columns, and
// section p reads ranks p*zsec .. p*zsec + r - 1 of Z (zsec = 0, dsec = N:
// one section).
struct RedJob {
  const uint16_t* Zt;
  const uint16_t* V;
  int N;
  int ldv;  // row stride of V (>= N)
  uint16_t* out;
  int out_transposed;
  int r;
  int zsec;
  int dsec;
};

// Two reductions share one launch (dA and dB of a backward): work-groups
// [0, nstrips of job 0) serve job 0, the rest job 1.
template <int NJ, int R, int CB>
__global__ __launch_bounds__(64 * kRedWaves) void k_tokred(RedJob j0, RedJob j1, int ldz, int M, int rz, float s) {
  constexpr int W = kRedWaves;
  constexpr int SW = 16 * CB;                         // strip width (columns)
  constexpr int RB = 2 * SW;                          // bytes per staged token row
  constexpr int CPR = RB / 16;                        // 16-byte chunks per staged row
  constexpr int kStepB = 1024 * CB + 1024 * NJ;       // V chunk, then NJ Z pieces
  constexpr int kRing = R * kStepB;                   // per wave
  constexpr int kRedB = (W - 1) * CB * NJ * 64 * 16;  // wave partial sums
  constexpr int kLds = W * kRing > kRedB ? W * kRing : kRedB;
  static_assert(kLds <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, sl = lane & 15;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int ns0 = (j0.N + SW - 1) / SW;
  const bool second = (int)blockIdx.x >= ns0;
  const RedJob& J = second ? j1 : j0;
  const uint16_t* __restrict__ Zt = J.Zt;
  const uint16_t* __restrict__ V = J.V;
  const int N = J.N, out_transposed = J.out_transposed, r = J.r;
  uint16_t* __restrict__ out = J.out;
  const int nstrips = (N + SW - 1) / SW;
  int tm, strip;
  tile_of(second ? (int)blockIdx.x - ns0 : (int)blockIdx.x, 1, nstrips, tm, strip);
  const int n0 = strip * SW;
  const int per = ((M + W - 1) / W + kRedStep - 1) / kRedStep * kRedStep;
  const int tb = wave_s * per;
  const int nsw = max(0, (min(M, tb + per) - tb + kRedStep - 1) / kRedStep);  // this wave's steps
  const int ldv = J.ldv;
  const BufRsrc rv = make_rsrc(V, ((uint64_t)(M - 1) * ldv + N) * 2);
  const BufRsrc rzb = make_rsrc(Zt, (uint64_t)rz * ldz * 2);
  // Staged rows: the 16-byte chunk c of token row t sits at chunk c ^ f(t),
  // f spreading the rows that one transposing read takes (t, t+1, t+2, t+3
  // and t+8 .. t+11) over distinct banks.
  auto fsw = [](int t) { return CB == 2 ? ((t >> 3) & 1) << 1 : (((t >> 1) & 1) | (((t >> 3) & 1) << 1)) << 1; };
  // V fetch u of a step (1 KB): lane l -> token row (1024/RB)*u + l/CPR,
  // physical chunk l%CPR, logical chunk (l%CPR) ^ f(row).
  int vrow[CB];
  uint32_t vcol[CB];
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    vrow[u] = (1024 / RB) * u + lane / CPR;
    const int lc = (lane % CPR) ^ fsw(vrow[u]);
    vcol[u] = (uint32_t)min(n0 + lc * 8, N - 8) * 2u;
  }
  uint32_t zrow[NJ];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb)
    zrow[jb] = (uint32_t)((n0 / J.dsec) * J.zsec + min(jb * 16 + sl, r - 1)) * (uint32_t)ldz * 2u;

  char* ring = lds + wave_s * kRing;
  auto fetch = [&](int i) {
    i = min(i, nsw > 0 ? nsw - 1 : 0);
    char* slot = ring + (i % R) * kStepB;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int m = min(tb + i * kRedStep + vrow[u], M - 1);
      dma_lds16(rv, (uint32_t)m * (uint32_t)ldv * 2u + vcol[u], slot + u * 1024);
    }
    const int mz = min(tb + i * kRedStep + 8 * g, ldz - 8);
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) dma_lds16(rzb, zrow[jb] + (uint32_t)mz * 2u, slot + 1024 * CB + jb * 1024);
  };
  constexpr int kPer = CB + NJ;

  // transposing-read byte offsets in a staged V chunk: block cb, tokens
  // 8g + 4*part + (0..3); lane sl loads row 8g + sl/4 + 4*part, columns
  // cb*16 + 4*(sl%4) .. +3.
  uint32_t troff[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const int row = 8 * g + (sl >> 2) + 4 * part, c = sl & 3;
      const int pc = (2 * cb + (c >> 1)) ^ fsw(row);
      troff[cb][part] = (uint32_t)(row * RB + pc * 16 + (c & 1) * 8);
    }

  f32x4 acc[CB][NJ];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) acc[cb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < R - 1; ++p) fetch(p);
  for (int i = 0; i < nsw; ++i) {
    // the slot refilled now was read in the previous step
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    fetch(i + R - 1);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((R - 1) * kPer) : "memory");
    const char* slot = ring + (i % R) * kStepB;
    u32x4 vb[CB];
#pragma unroll
    for (int cb = 0; cb < CB; cb += 2) tr_reads4(slot, *reinterpret_cast<const uint32_t(*)[2][2]>(&troff[cb][0]), *reinterpret_cast<u32x4(*)[2]>(&vb[cb]));
    const int nvalid = M - (tb + i * kRedStep + 8 * g);  // valid tokens of this lane's Z operand
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      u32x4 zz = *reinterpret_cast<const u32x4*>(slot + 1024 * CB + jb * 1024 + lane * 16);
      if (tb + (i + 1) * kRedStep > M) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          zz[p] &= 2 * p + 1 < nvalid ? 0xFFFFFFFFu : (2 * p < nvalid ? 0x0000FFFFu : 0u);
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb][jb] = mfma16(zz, vb[cb], acc[cb][jb]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Fixed-order sum of the waves: (((w0 + w1) + w2) + ...).
  float* red = reinterpret_cast<float*>(lds);
  if (wave > 0) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb)
        *reinterpret_cast<f32x4*>(red + ((((wave - 1) * CB + cb) * NJ + jb) * 64 + lane) * 4) = acc[cb][jb];
  }
  __syncthreads();
  if (wave != 0) return;
  // lane holds ranks jb*16 + 4g + i of column n0 + cb*16 + sl
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = n0 + cb * 16 + sl;
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      f32x4 v = acc[cb][jb];
#pragma unroll
      for (int w = 0; w < W - 1; ++w) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(red + (((w * CB + cb) * NJ + jb) * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += o[i];
      }
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jb * 16 + 4 * g + i;
        if (j >= r) continue;
        const uint16_t h = (uint16_t)pack_bf16x2(s * v[i], 0.0f);
        if (out_transposed) out[(size_t)n * r + j] = h;
        else out[(size_t)j * N + n] = h;
      }
    }
  }
}

static hipError_t token_reduce_launch(const RedJob& j0, const RedJob& j1, bool has1, int ldz, int M, int r,
                                      float s, hipStream_t st) {
  const int rp = padded_rank(r);
  // 64-column strips (Z read half as often) when they still give at least
  // one work-group per CU, else 32-column strips.
  const int wide = (j0.N + 63) / 64 + (has1 ? (j1.N + 63) / 64 : 0);
  const bool cb4 = wide >= 256;
  const int sw = cb4 ? 64 : 32;
  dim3 grid((unsigned)((j0.N + sw - 1) / sw + (has1 ? (j1.N + sw - 1) / sw : 0)));
#define QLORA_RED(NJ, R, CB)                                                                              \
  QLORA_LAUNCH("token_reduce", st, (k_tokred<NJ, R, CB>), grid, dim3(64 * kRedWaves), 0, st, j0, j1, ldz, M, r, s)
  if (cb4) {
    switch (rp / 16) {
      case 1: QLORA_RED(1, 3, 4); break;
      case 2: QLORA_RED(2, 3, 4); break;
      case 3: QLORA_RED(3, 2, 4); break;
      default: QLORA_RED(4, 2, 4); break;
    }
  } else {
    switch (rp / 16) {
      case 1: QLORA_RED(1, 3, 2); break;
      case 2: QLORA_RED(2, 3, 2); break;
      case 3: QLORA_RED(3, 3, 2); break;
      default: QLORA_RED(4, 3, 2); break;
    }
  }
#undef QLORA_RED
  return hipGetLastError();
}

hipError_t launch_token_reduce2(const uint16_t* Zt0, const uint16_t* V0, int N0, uint16_t* out0, bool tr0,
                                const uint16_t* Zt1, const uint16_t* V1, int N1, uint16_t* out1, bool tr1,
                                int ldz, int M, int r, int nsec1, float s, hipStream_t st) {
  // Job 0 reduces against all r ranks of Zt0; job 1's columns fall into
  // nsec1 sections, section p against ranks p*r/nsec1 .. of Zt1 (r rows).
  if (nsec1 < 1 || nsec1 > kMaxSections || r % nsec1 != 0 || (V1 && N1 % nsec1 != 0)) return hipErrorInvalidValue;
  const int r1 = r / nsec1, dsec1 = V1 ? N1 / nsec1 : 1;
  if (nsec1 > 1 && dsec1 % 64 != 0) return hipErrorInvalidValue;  // strips stay inside one section
  if (padded_rank(r) <= kMaxRank) {
    const RedJob j0{Zt0, V0, N0, N0, out0, tr0 ? 1 : 0, r, 0, N0 > 0 ? N0 : 1};
    const RedJob j1{Zt1, V1, N1, N1, out1, tr1 ? 1 : 0, r1, r1, dsec1};
    return token_reduce_launch(j0, j1, V1 != nullptr, ldz, M, r, s, st);
  }
  // More ranks: one launch per group of whole sections (at most kMaxRank
  // ranks), in order on the stream.  Group [p0, p0 + np): ranks p0*r1 ..
  // of both jobs -- rows of out0, and job 1's sections, whose columns of V1
  // start at p0*dsec1 (rows of out1, written transposed).
  if (V1 == nullptr || tr0 || !tr1 || r1 > kMaxRank || r > kMaxSections * kMaxRank) return hipErrorInvalidValue;
  const int per = kMaxRank / r1;
  hipError_t e = hipSuccess;
  for (int p0 = 0; p0 < nsec1 && e == hipSuccess; p0 += per) {
    const int np = min(per, nsec1 - p0);
    const int j = p0 * r1, rg = np * r1;
    const RedJob j0{Zt0 + (size_t)j * ldz, V0, N0, N0, out0 + (size_t)j * N0, 0, rg, 0, N0 > 0 ? N0 : 1};
    const RedJob j1{Zt1 + (size_t)j * ldz, V1 + (size_t)p0 * dsec1, np * dsec1, N1,
                    out1 + (size_t)p0 * dsec1 * r1, 1, r1, r1, dsec1};
    e = token_reduce_launch(j0, j1, true, ldz, M, rg, s, st);
  }
  return e;
}

}  // namespace qlora
