// merge.hip -- deploy-time merge W = w~ + s B A and task-switch unmerge
// W0 = W - s B A (page "LoRA and QLoRA fine-tuning: mechanics, and when not
// to fine-tune", section "The update LoRA is allowed to learn"; the merge
// target is the 16-bit dequantised base, page "Fine-Tuning on a Budget",
// "What actually goes wrong").
//
// One pass over d x k, HBM-bound: per element 0.5 B of codes (merge) or 2 B
// of bf16 (unmerge) read and 2 B written.  A work-group owns a 128 x 128
// tile.  The rank-r product B A of the tile is one MFMA pass (32x32x16,
// K = r padded to 16): B rows are one operand as stored, and the tile's
// r x 128 slab of A is staged in LDS (rows padded to 320 bytes) and read
// back with the transposing LDS read as the other.  In k_merge (unmerge,
// the r = 0 merge, grids of at most one tile per work-group slot) the fp32
// product goes through LDS and so do the 16-entry tables (one per row and
// 64-column block, built once); each thread then decodes eight code words
// (or takes eight bf16 words of the input), adds s times the product with
// one fused multiply-add per element and rounds once to bf16.  k_merge_runs
// (the merge with adapters over larger grids) keeps the product in
// registers instead, below.  A wave's stores cover whole 256-byte row
// segments.  The output is written with
// non-temporal stores, so that its stream does not push out of L2 the A
// slabs and B rows that later tiles read again.
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

constexpr int kMergeTile = 128;
constexpr int kMergeARow = 320;                 // bytes per staged row of A (256 + padding)
constexpr int kMergeDRow = kMergeTile + 4;      // floats per row of the staged product
constexpr int kMergeSRow = kMergeTile * 2 + 16;  // bytes per staged output row (bf16, padded)

template <bool kFromNf4>
__global__ __launch_bounds__(256) void k_merge(const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ c2,
                                              const float* __restrict__ c1,
                                              const float* __restrict__ mean,
                                              const uint16_t* __restrict__ Win, int d, int k,
                                              const uint16_t* __restrict__ A,
                                              const uint16_t* __restrict__ B, int r, int rp, float s,
                                              uint16_t* __restrict__ Wout, Nf4Table t) {
  __shared__ __attribute__((aligned(16))) char lds[kMergeTile * kMergeDRow * 4];
  __shared__ __attribute__((aligned(16))) Lut tabs[kMergeTile * 2];  // per (row, 64-column block)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int i0 = blockIdx.y * kMergeTile, c0 = blockIdx.x * kMergeTile;
  float* D = reinterpret_cast<float*>(lds);

  // Inputs of this thread's eight output words (word it*256 + tid of the
  // tile: row (it*256 + tid) / 16, 8-column word (tid % 16), so a wave's
  // loads and stores cover four full 256-byte row segments), issued first so
  // that they land while the product is formed.
  const int wc = tid & 15;
  uint32_t cw[8];
  u32x4 win[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int row = it * 16 + (tid >> 4);
    const int i = min(i0 + row, d - 1), c = min(c0 + wc * 8, k - 8);
    const size_t flat = (size_t)i * k + c;
    if (kFromNf4) cw[it] = *reinterpret_cast<const uint32_t*>(codes + (flat >> 1));
    else win[it] = *reinterpret_cast<const u32x4*>(Win + flat);
  }
  // block constants of (row tid / 2, 64-column block tid % 2) for the tables
  uint32_t q2 = 0;
  float q1 = 0.0f;
  if (kFromNf4) {
    const int i = min(i0 + (tid >> 1), d - 1), c = min(c0 + (tid & 1) * 64, k - 64);
    const size_t flat = (size_t)i * k + c;
    q2 = c2[flat >> 6];
    q1 = c1[flat >> 14];
  }

  if (r > 0) {
    // Every global load of the product is issued here, before any of them
    // is used: this thread's four 16-byte pieces of the A slab (rp x 128,
    // zero past r and past k) and, per 16 ranks, the B operand of this
    // wave's rows i0 + 32*wave + l32 (ranks 8*half .. +7).  (Loaded inside
    // the rank loop, each 16 ranks cost one dependent round trip: 57 -> 49
    // us at 8192 x 8192, r = 64.)
    constexpr int kAPieces = kMaxRank * 16 / 256;
    u32x4 av[kAPieces];
#pragma unroll
    for (int q = 0; q < kAPieces; ++q) {
      const int e = tid + 256 * q, j = e >> 4, c = c0 + (e & 15) * 8;
      av[q] = (j < r && c < k) ? *reinterpret_cast<const u32x4*>(A + (size_t)j * k + c) : u32x4{0u, 0u, 0u, 0u};
    }
    const int ib = min(i0 + wave * 32 + l32, d - 1);
    u32x4 bo[kMaxRank / 16];
#pragma unroll
    for (int q = 0; q < kMaxRank / 16; ++q) {
      const int j0 = 16 * q + half * 8;
      bo[q] = u32x4{0u, 0u, 0u, 0u};
      if ((r & 7) == 0) {
        if (j0 < r) bo[q] = *reinterpret_cast<const u32x4*>(B + (size_t)ib * r + j0);
      } else if (16 * q < r) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = j0 + 2 * p < r ? B[(size_t)ib * r + j0 + 2 * p] : 0u;
          const uint32_t hi = j0 + 2 * p + 1 < r ? B[(size_t)ib * r + j0 + 2 * p + 1] : 0u;
          bo[q][p] = lo | (hi << 16);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kAPieces; ++q) {
      const int e = tid + 256 * q;
      if ((e >> 4) < rp) *reinterpret_cast<u32x4*>(lds + (e >> 4) * kMergeARow + (e & 15) * 16) = av[q];
    }
    __syncthreads();
    f32x16 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[cb][e] = 0.0f;
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int q = 0; q < kMaxRank / 16; ++q) {
      if (16 * q >= rp) break;
      const int jb = 16 * q;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        // B operand: ranks jb + 8*half .. +7 of column cb*32 + l32, from
        // two transposing reads (16-lane group g: rows 8*(g>>1) + sl/4 + 4q,
        // columns (g&1)*16 + 4*(sl%4) .. +3 of the 32-column block)
        const int row = jb + 8 * (g >> 1) + (sl >> 2);
        const int col = cb * 32 + (g & 1) * 16 + 4 * (sl & 3);
        const char* p0 = lds + row * kMergeARow + col * 2;
        const u32x2 lo = lds_read_tr16(p0);
        const u32x2 hi = lds_read_tr16(p0 + 4 * kMergeARow);
        acc[cb] = mfma32(bo[q], u32x4{lo.x, lo.y, hi.x, hi.y}, acc[cb]);
      }
    }
    __syncthreads();
    // product to LDS: lane holds rows 8*blk + 4*half + q, column cb*32 + l32
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          D[(wave * 32 + blk * 8 + half * 4 + q) * kMergeDRow + cb * 32 + l32] = acc[cb][blk * 4 + q];
    __syncthreads();
  }

  if (kFromNf4) {
    tabs[tid] = build_lut(t, block_scale(q2, q1, mean[0]));
    __syncthreads();
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int row = it * 16 + (tid >> 4);
    const int i = i0 + row, c = c0 + wc * 8;
    if (i >= d || c >= k) continue;
    const u32x4 base = kFromNf4 ? dequant8(cw[it], tabs[row * 2 + (wc >> 3)]) : win[it];
    u32x4 out = base;
    if (r > 0) {
      const float* dp = D + row * kMergeDRow + wc * 8;
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(dp);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(dp + 4);
      out.x = pack_bf16x2(fmaf(s, p0[0], bf16_lo(base.x)), fmaf(s, p0[1], bf16_hi(base.x)));
      out.y = pack_bf16x2(fmaf(s, p0[2], bf16_lo(base.y)), fmaf(s, p0[3], bf16_hi(base.y)));
      out.z = pack_bf16x2(fmaf(s, p1[0], bf16_lo(base.z)), fmaf(s, p1[1], bf16_hi(base.z)));
      out.w = pack_bf16x2(fmaf(s, p1[2], bf16_lo(base.w)), fmaf(s, p1[3], bf16_hi(base.w)));
    }
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(Wout + (size_t)i * k + c));
  }
}

// Merge with adapters over runs of tiles: a work-group takes a run of
// consecutive tiles in row-major tile order (two work-groups per CU),
// mostly along one row of tiles, keeps the B operand of its tile row in
// registers from one tile to the next (the product's operands that come
// from L2 -- the tile's A slab and B rows, 32 KB per tile at r = 64 -- cost
// more than its arithmetic; a run of n tiles in one row loads B once
// instead of n times), and has the next tile's global inputs in flight
// while it works on the current one.  The product is formed transposed
// (A^T B^T: the slab is the MFMA's first operand), so that a lane's outputs
// run along a row of the tile: each lane decodes exactly the weights its
// accumulators hold and adds the product in registers, and only the bf16
// result goes through LDS (for stores of whole 256-byte row segments) --
// half the LDS bytes of staging the fp32 product, and a quarter of the
// table reads (measured 40-51 -> 36-40 us at 8192 x 8192, r = 64).  Tiles
// as in k_merge.
constexpr int kMergeWgPerCu = 2;  // resident work-groups per CU (registers, LDS)

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_merge_runs(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ c2,
                                                   const float* __restrict__ c1,
                                                   const float* __restrict__ mean, int d, int k,
                                                   const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ B, int r, int rp, float s,
                                                   uint16_t* __restrict__ Wout, Nf4Table t, int ntx,
                                                   int ntiles, int per) {
  // the A slab during the product, then the tile's bf16 output rows
  // (kMergeSRow bytes apart) for the coalesced stores
  constexpr int kLds = kMergeTile * kMergeSRow > kMaxRank * kMergeARow ? kMergeTile * kMergeSRow
                                                                      : kMaxRank * kMergeARow;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ __attribute__((aligned(16))) Lut tabs[kMergeTile * 2];  // per (row, 64-column block)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wc = tid & 15;
  const float mu = mean[0];
  constexpr int kAPieces = kMaxRank * 16 / 256;

  u32x4 bo[kMaxRank / 16];  // B operand of the current tile row (ranks 16 q + 8 half .. + 7)
  int bo_row = -1;
  // Global inputs of tile tt, loaded one tile ahead, from clamped addresses
  // with no branch, so that the wait before their use counts only the loads
  // issued after them: this thread's four 16-byte pieces of the A slab
  // (rp x 128; pieces past r or past k are replaced by zeros where the slab
  // is written to LDS), the code words of its eight output words (word
  // it*256 + tid of the tile: row (it*256 + tid) / 16, 8-column word
  // tid % 16, so a wave's loads and stores cover four full 256-byte row
  // segments) and the block constants of (row tid / 2, 64-column block
  // tid % 2) for the tables.
  struct TileIn {
    u32x4 av[kAPieces];
    uint32_t cw[8];
    uint32_t q2;
    float q1;
  };
  auto load_in = [&](int tt, TileIn& in) {
    const int ty = tt / ntx;
    const int i0 = ty * kMergeTile, c0 = (tt - ty * ntx) * kMergeTile;
#pragma unroll
    for (int q = 0; q < kAPieces; ++q) {
      const int e = tid + 256 * q, j = e >> 4, c = c0 + (e & 15) * 8;
      in.av[q] = *reinterpret_cast<const u32x4*>(A + (size_t)min(j, r - 1) * k + min(c, k - 8));
    }
    {
      // this lane's half of its weight row in the tile: 64 columns, words
      // 8*half .. 8*half + 7 (clamped into the row at a ragged right edge:
      // those columns are never stored)
      const int i = min(i0 + wave * 32 + l32, d - 1), c = min(c0 + 64 * half, k - 64);
      const uint8_t* pc = codes + (((size_t)i * k + c) >> 1);
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(pc);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(pc + 16);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        in.cw[p] = v0[p];
        in.cw[4 + p] = v1[p];
      }
    }
    const int i = min(i0 + (tid >> 1), d - 1), c = min(c0 + (tid & 1) * 64, k - 64);
    const size_t flat = (size_t)i * k + c;
    in.q2 = c2[flat >> 6];
    in.q1 = c1[flat >> 14];
  };
  auto tile = [&](int tt, const TileIn& in, bool live) {
    const int ty = tt / ntx;
    const int i0 = ty * kMergeTile, c0 = (tt - ty * ntx) * kMergeTile;
    const u32x4(&av)[kAPieces] = in.av;
    const uint32_t(&cw)[8] = in.cw;
    const uint32_t q2 = in.q2;
    const float q1 = in.q1;
    f32x16 acc[4];

    {
      // When the tile row changes, the B operand of this wave's rows i0 +
      // 32*wave + l32.
      if (ty != bo_row) {  // uniform over the work-group
        bo_row = ty;
        const int ib = min(i0 + wave * 32 + l32, d - 1);
#pragma unroll
        for (int q = 0; q < kMaxRank / 16; ++q) {
          const int j0 = 16 * q + half * 8;
          bo[q] = u32x4{0u, 0u, 0u, 0u};
          if ((r & 7) == 0) {
            if (j0 < r) bo[q] = *reinterpret_cast<const u32x4*>(B + (size_t)ib * r + j0);
          } else if (16 * q < r) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t lo = j0 + 2 * p < r ? B[(size_t)ib * r + j0 + 2 * p] : 0u;
              const uint32_t hi = j0 + 2 * p + 1 < r ? B[(size_t)ib * r + j0 + 2 * p + 1] : 0u;
              bo[q][p] = lo | (hi << 16);
            }
          }
        }
        // wait for B here, on the rare path that loads it, so that the
        // common path does not wait for everything in flight at the join
#pragma unroll
        for (int q = 0; q < kMaxRank / 16; ++q) asm volatile("" ::"v"(bo[q]));
      }
      // every piece is written (rows past rp too: they are not read), so
      // that every loaded register is used on every path
#pragma unroll
      for (int q = 0; q < kAPieces; ++q) {
        const int e = tid + 256 * q, j = e >> 4;
        const bool in = j < r && c0 + (e & 15) * 8 < k;
        *reinterpret_cast<u32x4*>(lds + j * kMergeARow + (e & 15) * 16) = in ? av[q] : u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[cb][e] = 0.0f;
      const int g = lane >> 4, sl = lane & 15;
#pragma unroll
      for (int q = 0; q < kMaxRank / 16; ++q) {
        if (16 * q >= rp) break;
        const int jb = 16 * q;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          // slab operand: ranks jb + 8*half .. +7 of column cb*32 + l32, from
          // two transposing reads (16-lane group g: rows 8*(g>>1) + sl/4 +
          // 4q, columns (g&1)*16 + 4*(sl%4) .. +3 of the 32-column block)
          const int row = jb + 8 * (g >> 1) + (sl >> 2);
          const int col = cb * 32 + (g & 1) * 16 + 4 * (sl & 3);
          const char* p0 = lds + row * kMergeARow + col * 2;
          const u32x2 lo = lds_read_tr16(p0);
          const u32x2 hi = lds_read_tr16(p0 + 4 * kMergeARow);
          acc[cb] = mfma32(u32x4{lo.x, lo.y, hi.x, hi.y}, bo[q], acc[cb]);
        }
      }
    }

    tabs[tid] = build_lut(t, block_scale(q2, q1, mu));
    // the slab has been read and the tables are written once every thread
    // is here
    __syncthreads();
    // The product stays in registers: lane (l32, half) holds weight row
    // R = 32*wave + l32 of the tile, columns cb*32 + 8*blk + 4*half .. +3 in
    // acc[cb][4*blk ..], i.e. elements 4*half .. +3 of code word 4*cb + blk
    // of its row (low nibbles for half 0, high for half 1).  It takes its
    // row's sixteen words (its own eight and, through the lane swap, its
    // partner's), decodes those four elements of each, adds s times the
    // product with one fused multiply-add, rounds once and writes the bf16
    // results to the staging rows; the stores to HBM then read whole
    // 256-byte row segments back.
    {
      const int R = wave * 32 + l32;
      uint32_t wd[16];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
#if defined(__HIP_DEVICE_COMPILE__)  // device-only builtin; the host pass never runs this
        const auto sw = __builtin_amdgcn_permlane32_swap(cw[jj], cw[jj], false, false);
        wd[jj] = sw[0];      // lanes 0-31 hold words 0..7
        wd[8 + jj] = sw[1];  // lanes 32-63 words 8..15
#else
        wd[jj] = wd[8 + jj] = cw[jj];
#endif
      }
      const Lut tl[2] = {tabs[R * 2], tabs[R * 2 + 1]};
      char* srow = lds + R * kMergeSRow + half * 8;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t w = wd[j];
        const uint32_t x = half ? w : (w << 4);  // bit 7 of each byte: top bit of this lane's nibbles
        uint32_t la, ha;
        lut4((half ? (w >> 4) : w) & 0x07070707u, perm(x << 8, x, 0x090B080Au), tl[j >> 3], la, ha);
        const uint32_t b01 = perm(ha, la, 0x05010400u), b23 = perm(ha, la, 0x07030602u);
        const f32x16& a = acc[j >> 2];
        const int e = (j & 3) * 4;
        const uint32_t o0 = pack_bf16x2(fmaf(s, a[e], bf16_lo(b01)), fmaf(s, a[e + 1], bf16_hi(b01)));
        const uint32_t o1 = pack_bf16x2(fmaf(s, a[e + 2], bf16_lo(b23)), fmaf(s, a[e + 3], bf16_hi(b23)));
        *reinterpret_cast<u32x2*>(srow + j * 16) = u32x2{o0, o1};
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = it * 16 + (tid >> 4);
      const int i = i0 + row, c = c0 + wc * 8;
      const u32x4 out = *reinterpret_cast<const u32x4*>(lds + row * kMergeSRow + wc * 16);
      if (live && i < d && c < k) __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(Wout + (size_t)i * k + c));
    }
  };
  // The next tile's inputs are in flight while a tile is worked on (two
  // register sets, named statically by taking the tiles in pairs).  Every
  // pass issues the same loads and runs both tiles of its pair -- past the
  // run's end the last tile again, without storing it -- so that every path
  // has the same loads in flight and each wait covers only the tile about to
  // be used.  After each tile a barrier: the next one rewrites the slab, the
  // product and the tables.
  const int t0 = (int)blockIdx.x * per;
  const int t_end = min(ntiles, t0 + per);
  if (t0 >= t_end) return;
  TileIn in0, in1;
  load_in(t0, in0);
  for (int tt = t0; tt < t_end; tt += 2) {
    load_in(min(tt + 1, t_end - 1), in1);
    tile(tt, in0, true);
    __syncthreads();
    load_in(min(tt + 2, t_end - 1), in0);
    tile(min(tt + 1, t_end - 1), in1, tt + 1 < t_end);
    __syncthreads();
  }
}

hipError_t launch_merge(const Nf4Dev& w, const uint16_t* Win, int d, int k, const uint16_t* A,
                        const uint16_t* B, int r, float s_signed, uint16_t* Wout, const Nf4Table& t,
                        hipStream_t st) {
  const int rp = r > 0 ? padded_rank(r) : 0;
  const int ntx = (k + kMergeTile - 1) / kMergeTile, nty = (d + kMergeTile - 1) / kMergeTile;
  const int ntiles = ntx * nty;
  int cus = 256;  // CUs of the stream's GPU (only sizes the runs; any value is correct)
  {
    int dev = 0, n = 0;
    hipDevice_t sd = 0;
    const bool ok = st != nullptr ? hipStreamGetDevice(st, &sd) == hipSuccess : hipGetDevice(&dev) == hipSuccess;
    if (st != nullptr) dev = (int)sd;
    if (ok && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
  }
  // The merge with adapters takes runs of tiles (k_merge_runs); unmerge and
  // the r = 0 merge stream faster with one tile per work-group (measured
  // side by side at 8192 x 8192, r = 64: merge 49.3 -> 46.3 us with runs,
  // unmerge 51.1 -> 54.8 us with runs).
  const int slots = kMergeWgPerCu * cus;
  const int per = (ntiles + slots - 1) / slots;  // tiles per work-group
  if (Win == nullptr && r > 0 && per > 1) {
    const int nwg = (ntiles + per - 1) / per;
    QLORA_LAUNCH("merge", st, k_merge_runs, dim3((unsigned)nwg), dim3(256), 0, st, w.codes, w.c2, w.c1, w.mean, d, k,
                 A, B, r, rp, s_signed, Wout, t, ntx, ntiles, per);
    return hipGetLastError();
  }
  dim3 grid((unsigned)ntx, (unsigned)nty);
  if (Win == nullptr)
    QLORA_LAUNCH("merge", st, k_merge<true>, grid, dim3(256), 0, st, w.codes, w.c2, w.c1, w.mean, nullptr,
                       d, k, A, B, r, rp, s_signed, Wout, t);
  else
    QLORA_LAUNCH("unmerge", st, k_merge<false>, grid, dim3(256), 0, st, nullptr, nullptr, nullptr, nullptr,
                       Win, d, k, A, B, r, rp, s_signed, Wout, t);
  return hipGetLastError();
}

}  // namespace qlora
