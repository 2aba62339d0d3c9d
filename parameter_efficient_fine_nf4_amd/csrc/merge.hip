// merge.hip -- deploy-time merge W = w~ + s B A and task-switch unmerge
// W0 = W - s B A (page "LoRA and QLoRA fine-tuning: mechanics, and when not
// to fine-tune", section "The update LoRA is allowed to learn"; the merge
// target is the 16-bit dequantised base, page "Fine-Tuning on a Budget",
// "What actually goes wrong").
//
// One pass over d x k, HBM-bound: per element 0.5 B of codes (merge) or 2 B
// of bf16 (unmerge) read and 2 B written.  A work-group owns a 128 x 128
// tile.  The rank-r product B A of the tile is one MFMA pass (32x32x16,
// K = r padded to 16): B rows are the A operand as stored, and the tile's
// r x 128 slab of A is staged in LDS (rows padded to 320 bytes) and read
// back with the transposing LDS read.  The fp32 product goes through LDS
// and so do the 16-entry tables (one per row and 64-column block, built
// once); each thread then decodes eight code words (or takes eight bf16
// words of the input), adds s times the product with one fused
// multiply-add per element and rounds once to bf16.  A wave's loads and
// stores cover whole 256-byte row segments.
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

constexpr int kMergeTile = 128;
constexpr int kMergeARow = 320;                 // bytes per staged row of A (256 + padding)
constexpr int kMergeDRow = kMergeTile + 4;      // floats per row of the staged product

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
    *reinterpret_cast<u32x4*>(Wout + (size_t)i * k + c) = out;
  }
}

// Merge with adapters over runs of tiles: a work-group takes a run of
// consecutive tiles in row-major tile order (two work-groups per CU),
// mostly along one row of tiles, and keeps the B operand of its tile row in
// registers from one tile to the next.  The product's operands that come
// from L2 (the tile's A slab and B rows, 32 KB per tile at r = 64) cost
// more than its arithmetic (a timing-only build without those loads ran
// 8192 x 8192, r = 64, in 38 us against 49), and a run of n tiles in one
// row loads B once instead of n times.  Tiles as in k_merge.
constexpr int kMergeWgPerCu = 2;  // resident work-groups per CU (registers, LDS)

__global__ __launch_bounds__(256) void k_merge_runs(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ c2,
                                                   const float* __restrict__ c1,
                                                   const float* __restrict__ mean, int d, int k,
                                                   const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ B, int r, int rp, float s,
                                                   uint16_t* __restrict__ Wout, Nf4Table t, int ntx,
                                                   int ntiles, int per) {
  __shared__ __attribute__((aligned(16))) char lds[kMergeTile * kMergeDRow * 4];
  __shared__ __attribute__((aligned(16))) Lut tabs[kMergeTile * 2];  // per (row, 64-column block)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wc = tid & 15;
  float* D = reinterpret_cast<float*>(lds);
  const float mu = mean[0];
  constexpr int kAPieces = kMaxRank * 16 / 256;

  u32x4 bo[kMaxRank / 16];  // B operand of the current tile row (ranks 16 q + 8 half .. + 7)
  int bo_row = -1;
  auto tile = [&](int tt) {
    const int ty = tt / ntx;
    const int i0 = ty * kMergeTile, c0 = (tt - ty * ntx) * kMergeTile;

    // Inputs of this thread's eight output words (word it*256 + tid of the
    // tile: row (it*256 + tid) / 16, 8-column word (tid % 16), so a wave's
    // loads and stores cover four full 256-byte row segments), issued first
    // so that they land while the product is formed.
    uint32_t cw[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = it * 16 + (tid >> 4);
      const int i = min(i0 + row, d - 1), c = min(c0 + wc * 8, k - 8);
      const size_t flat = (size_t)i * k + c;
      cw[it] = *reinterpret_cast<const uint32_t*>(codes + (flat >> 1));
    }
    // block constants of (row tid / 2, 64-column block tid % 2) for the tables
    uint32_t q2;
    float q1;
    {
      const int i = min(i0 + (tid >> 1), d - 1), c = min(c0 + (tid & 1) * 64, k - 64);
      const size_t flat = (size_t)i * k + c;
      q2 = c2[flat >> 6];
      q1 = c1[flat >> 14];
    }

    {
      // This thread's four 16-byte pieces of the A slab (rp x 128, zero
      // past r and past k) and, when the tile row changes, the B operand of
      // its wave's rows i0 + 32*wave + l32, issued before any is used.
      u32x4 av[kAPieces];
#pragma unroll
      for (int q = 0; q < kAPieces; ++q) {
        const int e = tid + 256 * q, j = e >> 4, c = c0 + (e & 15) * 8;
        av[q] = (j < r && c < k) ? *reinterpret_cast<const u32x4*>(A + (size_t)j * k + c) : u32x4{0u, 0u, 0u, 0u};
      }
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
          // two transposing reads (16-lane group g: rows 8*(g>>1) + sl/4 +
          // 4q, columns (g&1)*16 + 4*(sl%4) .. +3 of the 32-column block)
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
    }

    tabs[tid] = build_lut(t, block_scale(q2, q1, mu));
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = it * 16 + (tid >> 4);
      const int i = i0 + row, c = c0 + wc * 8;
      if (i >= d || c >= k) continue;
      const u32x4 base = dequant8(cw[it], tabs[row * 2 + (wc >> 3)]);
      u32x4 out;
      {
        const float* dp = D + row * kMergeDRow + wc * 8;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(dp);
        const f32x4 p1 = *reinterpret_cast<const f32x4*>(dp + 4);
        out.x = pack_bf16x2(fmaf(s, p0[0], bf16_lo(base.x)), fmaf(s, p0[1], bf16_hi(base.x)));
        out.y = pack_bf16x2(fmaf(s, p0[2], bf16_lo(base.y)), fmaf(s, p0[3], bf16_hi(base.y)));
        out.z = pack_bf16x2(fmaf(s, p1[0], bf16_lo(base.z)), fmaf(s, p1[1], bf16_hi(base.z)));
        out.w = pack_bf16x2(fmaf(s, p1[2], bf16_lo(base.w)), fmaf(s, p1[3], bf16_hi(base.w)));
      }
      *reinterpret_cast<u32x4*>(Wout + (size_t)i * k + c) = out;
    }
  };
  const int t_end = min(ntiles, ((int)blockIdx.x + 1) * per);
  for (int tt = (int)blockIdx.x * per; tt < t_end; ++tt) {
    tile(tt);
    __syncthreads();  // the next tile rewrites the slab, the product and the tables
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
