// merge.hip -- deploy-time merge W = w~ + s B A and task-switch unmerge
// W0 = W - s B A (page "LoRA and QLoRA fine-tuning: mechanics, and when not
// to fine-tune", section "The update LoRA is allowed to learn"; the merge
// target is the 16-bit dequantised base, page "Fine-Tuning on a Budget",
// "What actually goes wrong").
//
// One pass over d x k, HBM-bound for small r: per element 0.5 B of codes
// (merge) or 2 B of bf16 (unmerge) read and 2 B written.  Each thread owns
// 8 consecutive columns (one packed code word) of 8 consecutive rows; the
// rank-r product is accumulated in fp32 from A (16-byte loads, reused for
// the 8 rows) and B (uniform across the work-group: scalar loads), then
// added to the base before a single bf16 rounding.
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

constexpr int kMergeRows = 8;

template <bool kFromNf4>
__global__ __launch_bounds__(256) void k_merge(const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ c2,
                                              const float* __restrict__ c1,
                                              const float* __restrict__ mean,
                                              const uint16_t* __restrict__ Win, int d, int k,
                                              const uint16_t* __restrict__ A,
                                              const uint16_t* __restrict__ B, int r, float s,
                                              uint16_t* __restrict__ Wout, Nf4Table t) {
  const int words_per_row = k >> 3;
  const int cw = blockIdx.x * 256 + threadIdx.x;
  if (cw >= words_per_row) return;
  const int c0 = cw * 8;
  const int row0 = blockIdx.y * kMergeRows;

  float acc[kMergeRows][8];
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;

  for (int j = 0; j < r; ++j) {
    const u32x4 av = *reinterpret_cast<const u32x4*>(A + (size_t)j * k + c0);
    const float a[8] = {bf16_lo(av.x), bf16_hi(av.x), bf16_lo(av.y), bf16_hi(av.y),
                        bf16_lo(av.z), bf16_hi(av.z), bf16_lo(av.w), bf16_hi(av.w)};
#pragma unroll
    for (int i = 0; i < kMergeRows; ++i) {
      const int row = row0 + i;
      const float b = (row < d) ? bf16_to_f32(B[(size_t)row * r + j]) : 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(b, a[e], acc[i][e]);
    }
  }

  const float mu = kFromNf4 ? mean[0] : 0.0f;
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) {
    const int row = row0 + i;
    if (row >= d) break;
    const size_t flat = (size_t)row * k + c0;
    u32x4 base;
    if (kFromNf4) {
      const uint32_t word = reinterpret_cast<const uint32_t*>(codes)[flat >> 3];
      const size_t blk = flat >> 6;
      const float ah = block_scale(c2[blk], c1[blk >> 8], mu);
      base = dequant8(word, build_lut(t, ah));
    } else {
      base = *reinterpret_cast<const u32x4*>(Win + flat);
    }
    u32x4 out = base;
    if (r > 0) {
      const float w[8] = {bf16_lo(base.x), bf16_hi(base.x), bf16_lo(base.y), bf16_hi(base.y),
                          bf16_lo(base.z), bf16_hi(base.z), bf16_lo(base.w), bf16_hi(base.w)};
      out.x = pack_bf16x2(fmaf(s, acc[i][0], w[0]), fmaf(s, acc[i][1], w[1]));
      out.y = pack_bf16x2(fmaf(s, acc[i][2], w[2]), fmaf(s, acc[i][3], w[3]));
      out.z = pack_bf16x2(fmaf(s, acc[i][4], w[4]), fmaf(s, acc[i][5], w[5]));
      out.w = pack_bf16x2(fmaf(s, acc[i][6], w[6]), fmaf(s, acc[i][7], w[7]));
    }
    *reinterpret_cast<u32x4*>(Wout + flat) = out;
  }
}

hipError_t launch_merge(const Nf4Dev& w, const uint16_t* Win, int d, int k, const uint16_t* A,
                        const uint16_t* B, int r, float s_signed, uint16_t* Wout, const Nf4Table& t,
                        hipStream_t st) {
  const int words = k / 8;
  dim3 grid((unsigned)((words + 255) / 256), (unsigned)((d + kMergeRows - 1) / kMergeRows));
  if (Win == nullptr)
    QLORA_LAUNCH("merge", st, k_merge<true>, grid, dim3(256), 0, st, w.codes, w.c2, w.c1, w.mean, nullptr,
                       d, k, A, B, r, s_signed, Wout, t);
  else
    QLORA_LAUNCH("unmerge", st, k_merge<false>, grid, dim3(256), 0, st, nullptr, nullptr, nullptr, nullptr,
                       Win, d, k, A, B, r, s_signed, Wout, t);
  return hipGetLastError();
}

}  // namespace qlora
