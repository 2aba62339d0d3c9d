// common.hpp -- device helpers shared by the gfx950 kernels of libqlora.
//
// Number formats of the layer (page "LoRA and QLoRA fine-tuning: mechanics,
// and when not to fine-tune", section "What QLoRA freezes, and in how many
// bits"): NF4 codes in blocks of 64, FP8 (E4M3FN) second-level constants in
// groups of 256 with an fp32 scale and a subtracted mean, bf16 compute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// No implicit multiply-add contraction in any kernel of the library: the
// storage format fixes two separate fp32 roundings in the block constant
// (fl32(fl32(c2 c1) + mu)) and the optimiser rounds every operation, while
// __fmul_rn / __fadd_rn are plain products and sums that the compiler would
// otherwise fuse.  The library is built with -ffp-contract=off (hipcc's
// default mode fuses across statements and does not honour this pragma,
// which states the same intent for other builds); fused operations are
// written out as fmaf.
#pragma clang fp contract(off)

namespace qlora {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kBlock = 64;    // weights per NF4 block constant
constexpr int kGroup = 256;   // block constants per second-level scale
constexpr int kMaxRank = 64;
// Row sections of one stored weight (projections sharing an input, each
// with its own mean and adapter): at most four, since every section carries
// at least 16 adapter ranks and the ranks of all sections fit kMaxRank.
constexpr int kMaxSections = 4;

// The 16 NF4 levels (ascending) and the 15 decision thresholds between
// neighbours, passed by value as kernel arguments.
struct Nf4Table {
  float q[16];
  float mid[16];  // mid[0..14] used
};

// ---------------------------------------------------------------- bf16 ----

// Two fp32 -> packed bf16 pair with round-to-nearest-even
// (v_cvt_pk_bf16_f32); a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ---------------------------------------------------------------- E4M3 ----

// OCP FP8 E4M3FN byte (low 8 bits of b) -> fp32, exact:
// |v| = (m + 8 [e > 0]) * 2^(max(e, 1) - 10) with the sign of bit 7.  On
// gfx950 v_cvt_f32_fp8 decodes this OCP format (earlier CDNA parts decoded
// the FNUZ variant), one instruction in place of the ten-odd of a bitwise
// decode; the GPU tests dequantise blocks carrying every finite code.  NaN
// patterns are never produced by the quantiser.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)(b & 0xFFu), 0);
}

// fp32 -> E4M3FN, round to nearest even, saturating at +-448, sign of zero
// kept.  Integer arithmetic on the fp32 encoding.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t ax = u & 0x7FFFFFFFu;
  uint32_t code;
  if (ax >= 0x43E00000u) {                 // |x| >= 448
    code = 0x7Eu;
  } else if (ax < 0x3C800000u) {           // |x| < 2^-6: subnormal grid 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(ax) * 512.0f);  // 0..8
  } else {                                  // keep 3 fraction bits, RNE
    uint32_t r = (ax + 0x7FFFFu + ((ax >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// Double-dequantised block constant a^ = fl32(fl32(e4m3(c2) * c1) + mu):
// two separate roundings, no fused multiply-add.
__device__ __forceinline__ float block_scale(uint32_t c2, float c1, float mu) {
  return __fadd_rn(__fmul_rn(e4m3_to_f32(c2), c1), mu);
}

// ------------------------------------------------------ NF4 block LUT ----
//
// For one block with constant a^, the 16 possible outputs
// bf16_rne(fl32(level[c] * a^)) are formed once and kept as two byte planes
// (low bytes L, high bytes H) of 4 dwords each, so that four codes are
// decoded by byte permutes (v_perm_b32) instead of per-element multiplies.
struct Lut {
  uint32_t L0, L1, L2, L3, H0, H1, H2, H3;
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ Lut build_lut(const Nf4Table& t, float ah) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(__fmul_rn(t.q[2 * i], ah), __fmul_rn(t.q[2 * i + 1], ah));
  Lut r;
  r.L0 = perm(w[1], w[0], 0x06040200u); r.H0 = perm(w[1], w[0], 0x07050301u);
  r.L1 = perm(w[3], w[2], 0x06040200u); r.H1 = perm(w[3], w[2], 0x07050301u);
  r.L2 = perm(w[5], w[4], 0x06040200u); r.H2 = perm(w[5], w[4], 0x07050301u);
  r.L3 = perm(w[7], w[6], 0x06040200u); r.H3 = perm(w[7], w[6], 0x07050301u);
  return r;
}

// Four 3-bit table indices (one per byte) and a per-byte mask (0xFF where
// the code is >= 8) -> low and high bf16 bytes of the four values.
__device__ __forceinline__ void lut4(uint32_t s, uint32_t m, const Lut& t, uint32_t& lo, uint32_t& hi) {
  const uint32_t la = perm(t.L1, t.L0, s), lb = perm(t.L3, t.L2, s);
  const uint32_t ha = perm(t.H1, t.H0, s), hb = perm(t.H3, t.H2, s);
  lo = (lb & m) | (la & ~m);
  hi = (hb & m) | (ha & ~m);
}

// One packed word (8 consecutive elements: byte j holds element j in its
// low nibble and element j + 4 in its high nibble) -> 8 bf16 in element
// order (dword j = e[2j] | e[2j+1] << 16).  The code's top bit selects the
// upper half of the table; v_perm's sign-replicating selectors (8..11 copy
// bit 7 of bytes 1, 3, 5, 7 of the 8-byte pool) turn those bits into byte
// masks: bit 7 of byte j of w is bit 3 of element j + 4, and of w << 4 is
// bit 3 of element j.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, const Lut& t) {
  const uint32_t w4 = w << 4;
  const uint32_t m_lo = perm(w4 << 8, w4, 0x090B080Au);
  const uint32_t m_hi = perm(w << 8, w, 0x090B080Au);
  uint32_t la, ha, lb, hb;
  lut4(w & 0x07070707u, m_lo, t, la, ha);           // elements 0..3
  lut4((w >> 4) & 0x07070707u, m_hi, t, lb, hb);    // elements 4..7
  u32x4 r;
  r.x = perm(ha, la, 0x05010400u);  // e0 | e1
  r.y = perm(ha, la, 0x07030602u);  // e2 | e3
  r.z = perm(hb, lb, 0x05010400u);  // e4 | e5
  r.w = perm(hb, lb, 0x07030602u);  // e6 | e7
  return r;
}

// Table of one block built jointly by lanes l and l + 32 (same block): each
// lane forms the products of its half of the levels (qh = levels 8h..8h+7
// for lane half h), and v_permlane32_swap hands each lane the other half.
__device__ __forceinline__ Lut build_lut_pair(const float (&qh)[8], float ah) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(__fmul_rn(qh[2 * i], ah), __fmul_rn(qh[2 * i + 1], ah));
  const uint32_t pl0 = perm(w[1], w[0], 0x06040200u), pl1 = perm(w[3], w[2], 0x06040200u);
  const uint32_t ph0 = perm(w[1], w[0], 0x07050301u), ph1 = perm(w[3], w[2], 0x07050301u);
  // lanes 0-31 hold planes 0,1 (levels 0..7), lanes 32-63 planes 2,3
  // (levels 8..15); the swap exchanges the first operand of the upper half
  // with the second operand of the lower half.
  Lut r;
#if defined(__HIP_DEVICE_COMPILE__)  // device-only builtin; the host pass never runs this
  const auto s0 = __builtin_amdgcn_permlane32_swap(pl0, pl0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(pl1, pl1, false, false);
  const auto s2 = __builtin_amdgcn_permlane32_swap(ph0, ph0, false, false);
  const auto s3 = __builtin_amdgcn_permlane32_swap(ph1, ph1, false, false);
  r.L0 = s0[0]; r.L2 = s0[1];
  r.L1 = s1[0]; r.L3 = s1[1];
  r.H0 = s2[0]; r.H2 = s2[1];
  r.H1 = s3[0]; r.H3 = s3[1];
#else
  r.L0 = r.L2 = pl0; r.L1 = r.L3 = pl1; r.H0 = r.H2 = ph0; r.H1 = r.H3 = ph1;
#endif
  return r;
}

// LDS tiles of 64 bf16 per row (128 B, no padding).  The 16-byte chunk c of
// row r is stored at chunk c ^ f(r), f(r) = (r ^ (r >> 3)) & 7: among any 8
// consecutive rows f is a permutation (conflict-free when a 128-bit LDS
// access serves 8 lanes per cycle), and among the even (odd) rows of any 16
// consecutive rows it is one too (conflict-free when it serves 16 lanes, two
// rows per 256-byte bank line).  Element offset.
__device__ __forceinline__ int swz_f(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ swz_f(row)) << 3); }

// Work-group index -> (m tile, n tile).  Work-groups are dealt to the eight
// XCDs round-robin; the remap gives each XCD a contiguous run of tiles in
// row-major tile order, so the tiles of one XCD share their activation rows
// in that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int ntm, int ntn, int& tm, int& tn) {
  const int total = ntm * ntn;
  int t = bid;
  if ((total & 7) == 0) t = (bid & 7) * (total >> 3) + (bid >> 3);
  tm = t / ntn;
  tn = t - tm * ntn;
}

// ----------------------------------------------- global -> LDS fetches ----
//
// Buffer-addressed direct-to-LDS loads (buffer_load_* ... lds): 64 lanes
// each fetch `size` bytes at base + voffset and the wave writes them to LDS
// contiguously (lane i at lds + i*size; lds must be wave-uniform).  Reads
// past the buffer's byte size return zeros.  These are tracked by vmcnt
// alone; the FLAT form (global_load_lds) would also make the compiler treat
// every later LDS read result as waiting on all outstanding LDS reads.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
// The LDS destination is passed as a bare 32-bit LDS address turned back
// into a pointer, so the compiler does not tie the fetch to an LDS object:
// it then never inserts its own (full) vmcnt drains before LDS reads.  The
// kernels order every fetch against its readers with explicit vmcnt waits
// and barriers.
// (The low 32 bits of a generic address of LDS are its LDS address: the
// shared aperture is 4 GB aligned.)
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_untracked(void* p) {
  const uint32_t a = (uint32_t)(uintptr_t)p;
  return (__attribute__((address_space(3))) void*)(uintptr_t)a;
}
__device__ __forceinline__ void dma_lds16(BufRsrc r, uint32_t voffset, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_untracked(lds), 16, (int)voffset, 0, 0, 0);
}
__device__ __forceinline__ void dma_lds4(BufRsrc r, uint32_t voffset, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_untracked(lds), 4, (int)voffset, 0, 0, 0);
}
// Same with a wave-uniform byte offset added in the scalar unit (soffset):
// a per-lane offset that is fixed for the kernel plus a per-step scalar one
// needs no vector arithmetic per fetch.
__device__ __forceinline__ void dma_lds16s(BufRsrc r, uint32_t voffset, uint32_t soffset, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_untracked(lds), 16, (int)voffset, (int)soffset, 0, 0);
}
__device__ __forceinline__ void dma_lds4s(BufRsrc r, uint32_t voffset, uint32_t soffset, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_untracked(lds), 4, (int)voffset, (int)soffset, 0, 0);
}
// 16-byte buffer load into registers; offsets at or past the buffer's byte
// size read zeros (used to zero out-of-range lanes without branches).
__device__ __forceinline__ u32x4 ld_buf16(BufRsrc r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, 0, 0);
}
__device__ __forceinline__ uint32_t ld_buf4(BufRsrc r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voffset, 0, 0);
}
__device__ __forceinline__ uint32_t ld_buf1(BufRsrc r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voffset, 0, 0);
}
__device__ __forceinline__ u32x2 ld_buf8(BufRsrc r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voffset, 0, 0);
}
#else  // host pass: never executed
struct BufRsrc {
  const void* p;
};
__device__ inline BufRsrc make_rsrc(const void* base, uint64_t) { return BufRsrc{base}; }
__device__ inline void dma_lds16(BufRsrc, uint32_t, void*) {}
__device__ inline void dma_lds4(BufRsrc, uint32_t, void*) {}
__device__ inline void dma_lds16s(BufRsrc, uint32_t, uint32_t, void*) {}
__device__ inline void dma_lds4s(BufRsrc, uint32_t, uint32_t, void*) {}
__device__ inline u32x4 ld_buf16(BufRsrc, uint32_t) { return u32x4{0u, 0u, 0u, 0u}; }
__device__ inline uint32_t ld_buf4(BufRsrc, uint32_t) { return 0u; }
__device__ inline uint32_t ld_buf1(BufRsrc, uint32_t) { return 0u; }
__device__ inline u32x2 ld_buf8(BufRsrc, uint32_t) { return u32x2{0u, 0u}; }
#endif

// Transposing 8-byte LDS read (ds_read_b64_tr_b16; lds is an LDS byte
// address): within each 16-lane group, lane i receives element i % 4 of the
// 8-byte (four bf16) loads of lanes 4q + i/4, q = 0..3.  With those lanes
// pointing at four consecutive rows of a row-major bf16 tile (four columns
// each), lane i gets column i of the four rows.
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(lds));
  return __builtin_bit_cast(u32x2, v);
#else
  return u32x2{0u, 0u};
#endif
}

// ------------------------------------------------------------- MFMA ----

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Sum of n floats at p, p + stride, ... in index order.  The loads go out
// eight at a time before they are added, so a long sum costs a few memory
// round trips rather than one per term.
__device__ __forceinline__ float sum_strided(const float* __restrict__ p, size_t stride, int n) {
  float acc = 0.0f;
  for (int base = 0; base < n; base += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = base + u < n ? p[(size_t)(base + u) * stride] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + u < n) acc += v[u];
  }
  return acc;
}

// Wave-wide sum / max helpers (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qlora
