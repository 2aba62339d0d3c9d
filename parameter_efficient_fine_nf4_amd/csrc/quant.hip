// quant.hip -- blockwise NF4 quantisation with double-quantised block
// constants (page "LoRA and QLoRA fine-tuning: mechanics, and when not to
// fine-tune", paragraphs "4-bit NormalFloat" and "Double quantisation").
//
// Three passes, all deterministic and bit-exact with the definition in
// include/qlora.h:
//   1. k_quant_blocks  absmax of each block of 64, codes, nibble packing;
//   2. k_group_sums    float64 sum of each group of 256 absmax values,
//      sequential inside the group;  k_mean (one wave): sequential sum of
//      the group sums (one chain of adds passed from lane to lane), divided
//      by n_b, rounded to fp32 (mu);
//   3. k_dq            per group: c1 = max|a - mu| / 448, c2 = e4m3((a-mu)/c1).
// One-time work per weight; HBM-bound (4 bytes read per weight in pass 1).
#include "common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace qlora {

// 16 lanes per block of 64 (one float4 each), 4 blocks per wave.
__global__ __launch_bounds__(256) void k_quant_blocks(const float* __restrict__ W, int64_t n_b,
                                                     Nf4Table t, uint8_t* __restrict__ codes,
                                                     float* __restrict__ absmax) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  if (blk >= n_b) return;  // whole 16-lane groups leave together
  const int sub = lane & 15;
  const float4 x = reinterpret_cast<const float4*>(W)[blk * 16 + sub];
  float m = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
  const float v[4] = {x.x, x.y, x.z, x.w};
  uint32_t mine = 0;  // one code per byte
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t code = 7u;
    if (m != 0.0f) {
      const float n = __fdiv_rn(v[e], m);
      code = 0u;
#pragma unroll
      for (int j = 0; j < 15; ++j) code += (n > t.mid[j]) ? 1u : 0u;
    }
    mine |= code << (8 * e);
  }
  // Lanes 2i and 2i+1 hold elements 0..3 and 4..7 of one group of 8: byte j
  // of the group's word is element j (low nibble) | element j+4 (high).
  const uint32_t other = (uint32_t)__shfl_xor((int)mine, 1, 16);
  if ((sub & 1) == 0) reinterpret_cast<uint32_t*>(codes)[blk * 8 + (sub >> 1)] = mine | (other << 4);
  if (sub == 0) absmax[blk] = m;
}

// One work-group per group of 256 constants; thread 0 adds them in order.
__global__ __launch_bounds__(256) void k_group_sums(const float* __restrict__ absmax, int64_t n_b,
                                                   double* __restrict__ gsum) {
  __shared__ double s[kGroup];
  const int64_t g = blockIdx.x;
  const int64_t i = g * kGroup + threadIdx.x;
  s[threadIdx.x] = (i < n_b) ? (double)absmax[i] : 0.0;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t cnt = (n_b - g * kGroup) < kGroup ? (n_b - g * kGroup) : kGroup;
    double acc = 0.0;
    for (int64_t j = 0; j < cnt; ++j) acc += s[j];
    gsum[g] = acc;
  }
}

// One wave, one chain of float64 additions in index order (the same
// sequential sum as one thread reading the group sums one by one).  The sums
// come in 512 at a time, lane l holding the eight consecutive terms
// 8l .. 8l+7 of the batch in registers (the next batch in flight).  The
// running sum moves from lane to lane: at hop l every lane takes its left
// neighbour's sum (lane 0 the sum carried over from the previous batch;
// DPP wave_shr:1) and adds its eight terms in order, so after hop l lane l
// holds the sum through its last term and, after hop 63, lane 63 the sum of
// the batch.  Terms past n_g are zeros (x + 0.0 == x for the non-negative
// sums here).
__device__ __forceinline__ double shr1(double x, double lane0) {
  const uint64_t xb = __builtin_bit_cast(uint64_t, x), ob = __builtin_bit_cast(uint64_t, lane0);
  // wave_shr:1 (DPP control 0x138): lane i receives lane i - 1; lane 0 keeps `old`
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)ob, (int)(uint32_t)xb, 0x138, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(ob >> 32), (int)(uint32_t)(xb >> 32), 0x138, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(64) void k_mean(const double* __restrict__ gsum, int64_t n_g, int64_t n_b,
                                             float* __restrict__ mean) {
  const int lane = threadIdx.x;
  constexpr int64_t kStep = 512;
  auto load = [&](int64_t b0, double (&v)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // unconditional (clamped) loads: the wait before the first use then
      // counts only the loads that were issued before them
      const int64_t i = b0 + 8 * lane + u;
      const double x = gsum[i < n_g ? i : n_g - 1];
      v[u] = i < n_g ? x : 0.0;
    }
  };
  double carry = 0.0;  // uniform: the sum of all earlier batches
  double cur[8], nxt[8];
  load(0, cur);
  for (int64_t b0 = 0; b0 < n_g; b0 += kStep) {
    load(b0 + kStep, nxt);
    double acc = 0.0;
#pragma unroll
    for (int hop = 0; hop < 64; ++hop) {
      acc = shr1(acc, carry);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += cur[u];
    }
    // lane 63's sum, to every lane
    const uint64_t ab = __builtin_bit_cast(uint64_t, acc);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)ab, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(ab >> 32), 63);
    carry = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
#pragma unroll
    for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
  }
  if (lane == 0) mean[0] = (float)(carry / (double)n_b);
}

__global__ __launch_bounds__(256) void k_dq(const float* __restrict__ absmax, int64_t n_b,
                                           const float* __restrict__ mean,
                                           uint8_t* __restrict__ c2, float* __restrict__ c1) {
  __shared__ float red[4];
  const int64_t g = blockIdx.x;
  const int64_t i = g * kGroup + threadIdx.x;
  const bool valid = i < n_b;
  const float mu = mean[0];
  const float e = valid ? __fsub_rn(absmax[i], mu) : 0.0f;
  float am = wave_max(fabsf(e));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = __fdiv_rn(am, 448.0f);
  if (threadIdx.x == 0) c1[g] = scale;
  if (valid) c2[i] = (uint8_t)(scale != 0.0f ? f32_to_e4m3(__fdiv_rn(e, scale)) : 0u);
}

hipError_t launch_quantize(const float* W, int64_t d, int64_t k, const Nf4Table& t, uint8_t* codes,
                           uint8_t* c2, float* c1, float* mean, void* ws, hipStream_t st) {
  const int64_t n_b = d * k / kBlock;
  const int64_t n_g = (n_b + kGroup - 1) / kGroup;
  float* absmax = reinterpret_cast<float*>(ws);
  double* gsum = reinterpret_cast<double*>(reinterpret_cast<char*>(ws) + align_up(n_b * 4, 256));
  QLORA_LAUNCH("quant_blocks", st, k_quant_blocks, dim3((unsigned)((n_b + 15) / 16)), dim3(256), 0, st, W, n_b, t,
                     codes, absmax);
  QLORA_LAUNCH("quant_group_sums", st, k_group_sums, dim3((unsigned)n_g), dim3(256), 0, st, absmax, n_b, gsum);
  QLORA_LAUNCH("quant_mean", st, k_mean, dim3(1), dim3(64), 0, st, gsum, n_g, n_b, mean);
  QLORA_LAUNCH("quant_dq", st, k_dq, dim3((unsigned)n_g), dim3(256), 0, st, absmax, n_b, mean, c2, c1);
  return hipGetLastError();
}

size_t quantize_ws_bytes(int64_t d, int64_t k) {
  const int64_t n_b = d * k / kBlock;
  const int64_t n_g = (n_b + kGroup - 1) / kGroup;
  return (size_t)(align_up(n_b * 4, 256) + align_up(n_g * 8, 256));
}

}  // namespace qlora
