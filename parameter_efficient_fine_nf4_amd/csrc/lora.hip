// lora.hip -- the rank-r pieces of the adapted linear (page "LoRA and QLoRA
// fine-tuning: mechanics, and when not to fine-tune", section "The update
// LoRA is allowed to learn"; page "Fine-Tuning on a Budget", "The LoRA
// hypothesis"):
//
//   k_prep          zero-padded copies of the adapters in the layouts the
//                   MFMA tiles read: s B (d x rp), B^T (rp x d), s A^T (k x rp).
//   k_lora_proj     P = V L^T for a skinny L (r x K): the down-projection
//                   T = X A^T and the backward vector U = dY B.  HBM-bound
//                   on V; MFMA 16x16x32 with V rows as the 16-row operand.
//                   Writes P (M x rp, bf16) and optionally P^T (r x ldt).
//   k_token_reduce  out = s Z^T V summed over tokens for Z^T (r x ldz):
//                   dA = s U^T X and dB^T = s T^T dY.  The contraction runs
//                   over tokens, the row index of V, so each lane loads an
//                   8 x 8 block of V (8 tokens x 8 columns) and transposes it
//                   in registers into 8 MFMA operands.  Work-groups own a
//                   128-column tile and a token range; partial sums go to
//                   the workspace and a second kernel adds them in a fixed
//                   order (deterministic, no atomics).
#include "common.hpp"
#include "launch.hpp"

namespace qlora {

// Bp = bf16(s B) and At = bf16(s A)^T carry the LoRA scale, so the
// up-projections accumulate into the GEMM accumulators with no extra
// arithmetic; the rounding is exact when s is a power of two and otherwise
// at most half a bf16 ulp of each scaled adapter entry.  Bt = B^T (unscaled).
__global__ void k_prep(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int d, int k,
                       int r, int rp, float s, uint16_t* __restrict__ Bp, uint16_t* __restrict__ Bt,
                       uint16_t* __restrict__ At) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)(d > k ? d : k) * rp;
  if (idx >= n) return;
  const int i = (int)(idx / rp), j = (int)(idx % rp);
  if (i < d) {
    const uint16_t b = j < r ? B[(size_t)i * r + j] : (uint16_t)0;
    if (Bp) Bp[(size_t)i * rp + j] = (uint16_t)pack_bf16x2(s * bf16_to_f32(b), 0.0f);
    if (Bt) Bt[(size_t)j * d + i] = b;
  }
  if (At && i < k) {
    const uint16_t a = j < r ? A[(size_t)j * k + i] : (uint16_t)0;
    At[(size_t)i * rp + j] = (uint16_t)pack_bf16x2(s * bf16_to_f32(a), 0.0f);
  }
}

hipError_t launch_prep_adapters(const uint16_t* A, const uint16_t* B, int d, int k, int r, float s,
                                uint16_t* Bp, uint16_t* Bt, uint16_t* At, hipStream_t st) {
  const int rp = padded_rank(r);
  const int64_t n = (int64_t)(d > k ? d : k) * rp;
  QLORA_LAUNCH("prep_adapters", st, k_prep, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, A, B, d, k, r, rp, s,
                     Bp, Bt, At);
  return hipGetLastError();
}

// ------------------------------------------------------------- lora_proj --

constexpr int kProjStep = 32;

__global__ __launch_bounds__(256) void k_lora_proj(const uint16_t* __restrict__ V, int M, int K,
                                                  const uint16_t* __restrict__ L, int r, int rp,
                                                  int steps_per_split, float* __restrict__ part,
                                                  uint16_t* __restrict__ P, uint16_t* __restrict__ Pt,
                                                  int ldt) {
  __shared__ float red[4][4][64][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int m = blockIdx.x * 16 + l16;
  const int split = blockIdx.y;
  const int nsteps = (K + kProjStep - 1) / kProjStep;
  const int s0 = split * steps_per_split;
  const int s1 = min(nsteps, s0 + steps_per_split);
  const int nj = rp / 16;

  f32x4 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = s0 + wave; st < s1; st += 4) {
    const int kk = st * kProjStep + 8 * g;
    const bool kval = kk < K;
    u32x4 a = {0u, 0u, 0u, 0u};
    if (kval && m < M) a = *reinterpret_cast<const u32x4*>(V + (size_t)m * K + kk);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (jb < nj) {
        const int j = jb * 16 + l16;
        u32x4 b = {0u, 0u, 0u, 0u};
        if (kval && j < r) b = *reinterpret_cast<const u32x4*>(L + (size_t)j * K + kk);
        acc[jb] = mfma16(a, b, acc[jb]);
      }
    }
  }
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][jb][lane][i] = acc[jb][i];
  __syncthreads();
  if (wave != 0) return;
  // lane holds rows 4g+i (tokens), column l16 of each 16x16 block (rank index)
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    if (jb >= nj) break;
    const int j = jb * 16 + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = blockIdx.x * 16 + 4 * g + i;
      const float v = ((red[0][jb][lane][i] + red[1][jb][lane][i]) + red[2][jb][lane][i]) + red[3][jb][lane][i];
      if (mm >= M) continue;
      if (part != nullptr) {
        part[((size_t)split * M + mm) * rp + j] = v;
      } else {
        const uint16_t h = (uint16_t)pack_bf16x2(v, 0.0f);
        P[(size_t)mm * rp + j] = h;
        if (Pt != nullptr && j < r) Pt[(size_t)j * ldt + mm] = h;
      }
    }
  }
}

__global__ void k_lora_proj_finish(const float* __restrict__ part, int nsplit, int M, int r, int rp,
                                   uint16_t* __restrict__ P, uint16_t* __restrict__ Pt, int ldt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * rp) return;
  const int mm = (int)(idx / rp), j = (int)(idx % rp);
  float v = 0.0f;
  for (int sp = 0; sp < nsplit; ++sp) v += part[((size_t)sp * M + mm) * rp + j];
  const uint16_t h = (uint16_t)pack_bf16x2(v, 0.0f);
  P[(size_t)mm * rp + j] = h;
  if (Pt != nullptr && j < r) Pt[(size_t)j * ldt + mm] = h;
}

static void proj_split(int M, int K, int* nsplit, int* sps) {
  const int mt = (M + 15) / 16;
  const int nsteps = (K + kProjStep - 1) / kProjStep;
  int want = (256 + mt - 1) / mt;
  int maxs = (nsteps + 3) / 4;
  if (maxs < 1) maxs = 1;
  int ns = want < maxs ? want : maxs;
  if (ns < 1) ns = 1;
  const int per = (nsteps + ns - 1) / ns;
  *nsplit = (nsteps + per - 1) / per;
  *sps = per;
}

static void proj_split_final(int M, int K, int* ns, int* sps) {
  proj_split(M, K, ns, sps);
  if (*ns > 64) *ns = 64;
  const int nsteps = (K + kProjStep - 1) / kProjStep;
  *sps = (nsteps + *ns - 1) / *ns;
  *ns = (nsteps + *sps - 1) / *sps;
}

size_t lora_proj_ws_bytes(int M, int K, int r) {
  int ns, sps;
  proj_split_final(M, K, &ns, &sps);
  return ns > 1 ? (size_t)ns * M * padded_rank(r) * sizeof(float) : 0;
}

hipError_t launch_lora_proj(const uint16_t* V, int M, int K, const uint16_t* L, int r, uint16_t* P,
                            uint16_t* Pt, int ldt, float* partial, hipStream_t st) {
  const int rp = padded_rank(r);
  int ns, sps;
  proj_split_final(M, K, &ns, &sps);
  dim3 grid((unsigned)((M + 15) / 16), (unsigned)ns);
  QLORA_LAUNCH("lora_proj", st, k_lora_proj, grid, dim3(256), 0, st, V, M, K, L, r, rp, sps,
                     ns > 1 ? partial : nullptr, P, Pt, ldt);
  if (ns > 1) {
    const int64_t n = (int64_t)M * rp;
    QLORA_LAUNCH("lora_proj_finish", st, k_lora_proj_finish, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, partial,
                       ns, M, r, rp, P, Pt, ldt);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------- token_reduce --

constexpr int kRedCols = 128;  // columns per work-group (16 lanes x 8)
constexpr int kRedStep = 32;   // tokens per wave step (4 lane quarters x 8)

// In-register transpose of an 8 x 8 block of bf16: rows[i] holds 8 columns
// of token i; cols[c] receives the 8 tokens of column c.
__device__ __forceinline__ void transpose8x8(const u32x4 (&rows)[8], u32x4 (&cols)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) cols[c][p] = perm(rows[2 * p + 1][c >> 1], rows[2 * p][c >> 1], sel);
  }
}

__global__ __launch_bounds__(256) void k_token_reduce(const uint16_t* __restrict__ Zt, int ldz, int M,
                                                     const uint16_t* __restrict__ V, int N, int r,
                                                     int rp, int steps_per_chunk, float s,
                                                     float* __restrict__ part,
                                                     uint16_t* __restrict__ out, int out_transposed) {
  __shared__ float red[4 * 8 * 64 * 4];  // one wave's accumulators (rp <= 64)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int n0 = blockIdx.x * kRedCols + 8 * l16;  // this lane's 8 columns
  const bool nval = n0 < N;
  const int chunk = blockIdx.y;
  const int nsteps = (M + kRedStep - 1) / kRedStep;
  const int s0 = chunk * steps_per_chunk;
  const int s1 = min(nsteps, s0 + steps_per_chunk);
  const int nj = rp / 16;

  f32x4 acc[4][8];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[jb][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = s0 + wave; st < s1; st += 4) {
    const int mb = st * kRedStep + 8 * g;  // this lane's 8 tokens
    u32x4 rows[8], cols[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (nval && mb + i < M) v = *reinterpret_cast<const u32x4*>(V + (size_t)(mb + i) * N + n0);
      rows[i] = v;
    }
    transpose8x8(rows, cols);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (jb >= nj) break;
      const int j = jb * 16 + l16;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (j < r && mb < M) {
        z = *reinterpret_cast<const u32x4*>(Zt + (size_t)j * ldz + mb);
        if (mb + 8 > M) {  // ragged token tail: zero the entries past M
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (mb + e >= M) z[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[jb][c] = mfma16(z, cols[c], acc[jb][c]);
    }
  }

  // Fixed-order sum of the four waves: ((w0 + w1) + w2) + w3.
  for (int w = 1; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((jb * 8 + c) * 64 + lane) * 4 + i] = acc[jb][c][i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[jb][c][i] += red[((jb * 8 + c) * 64 + lane) * 4 + i];
    }
    __syncthreads();
  }
  if (wave != 0 || !nval) return;
  // lane holds rank rows jb*16 + 4g + i and columns n0 + c (c = 0..7)
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    if (jb >= nj) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = jb * 16 + 4 * g + i;
      if (j >= r) continue;
      if (part != nullptr) {
        float* dst = part + ((size_t)chunk * rp + j) * N + n0;
#pragma unroll
        for (int c = 0; c < 8; ++c) dst[c] = acc[jb][c][i];
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint16_t h = (uint16_t)pack_bf16x2(s * acc[jb][c][i], 0.0f);
          if (out_transposed) out[(size_t)(n0 + c) * r + j] = h;
          else out[(size_t)j * N + n0 + c] = h;
        }
      }
    }
  }
}

__global__ void k_token_reduce_finish(const float* __restrict__ part, int nchunk, int N, int r, int rp,
                                      float s, uint16_t* __restrict__ out, int out_transposed) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)r * N) return;
  const int j = (int)(idx / N), n = (int)(idx % N);
  float v = 0.0f;
  for (int c = 0; c < nchunk; ++c) v += part[((size_t)c * rp + j) * N + n];
  const uint16_t h = (uint16_t)pack_bf16x2(s * v, 0.0f);
  if (out_transposed) out[(size_t)n * r + j] = h;
  else out[(size_t)j * N + n] = h;
}

static void reduce_split(int M, int N, int* nchunk, int* spc) {
  const int nt = (N + kRedCols - 1) / kRedCols;
  const int nsteps = (M + kRedStep - 1) / kRedStep;
  int want = (512 + nt - 1) / nt;
  int maxc = (nsteps + 3) / 4;
  if (maxc < 1) maxc = 1;
  int nc = want < maxc ? want : maxc;
  if (nc > 32) nc = 32;
  if (nc < 1) nc = 1;
  const int per = (nsteps + nc - 1) / nc;
  *nchunk = (nsteps + per - 1) / per;
  *spc = per;
}

size_t token_reduce_ws_bytes(int M, int N, int r) {
  int nc, spc;
  reduce_split(M, N, &nc, &spc);
  return nc > 1 ? (size_t)nc * padded_rank(r) * N * sizeof(float) : 0;
}

hipError_t launch_token_reduce(const uint16_t* Zt, int ldz, const uint16_t* V, int M, int N, int r,
                               float s, uint16_t* out, bool out_transposed, float* partial,
                               hipStream_t st) {
  const int rp = padded_rank(r);
  int nc, spc;
  reduce_split(M, N, &nc, &spc);
  dim3 grid((unsigned)((N + kRedCols - 1) / kRedCols), (unsigned)nc);
  QLORA_LAUNCH("token_reduce", st, k_token_reduce, grid, dim3(256), 0, st, Zt, ldz, M, V, N, r, rp, spc, s,
                     nc > 1 ? partial : nullptr, out, out_transposed ? 1 : 0);
  if (nc > 1) {
    const int64_t n = (int64_t)r * N;
    QLORA_LAUNCH("token_reduce_finish", st, k_token_reduce_finish, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       partial, nc, N, r, rp, s, out, out_transposed ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace qlora
