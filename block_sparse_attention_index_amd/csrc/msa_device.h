// msa_device.h -- device helpers of the gfx950 MSA kernels: format codecs,
// slab addressing, wave reductions.  Internal to the HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

constexpr int kPage = MSA_PAGE_TOKENS;
constexpr int kDim = MSA_HEAD_DIM;
constexpr int kHpg = MSA_HEADS_PER_GROUP;
constexpr int kGroups = 4;  // KV heads = GQA groups
constexpr int kNvSlab = MSA_NVFP4_SLAB_BYTES;
constexpr int kScaleOff = 8192;  // scales follow the 128 x 64 B of codes
constexpr int kF32Slab = MSA_F32_SLAB_BYTES;
constexpr int kFp8Slab = MSA_FP8_SLAB_BYTES;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- codecs
// E4M3 (OCP): decode with the gfx950 conversion (checked against every code
// by the dequantisation tests).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

// FP32 -> E4M3, round to nearest even, saturating to +-448; NaN -> 0x7F.
// Written from the format: for |x| >= 2^-6 the exponent is read from the
// FP32 bits and the 3 mantissa bits are rounded with rint (RNE); below 2^-6
// the value is a multiple of 2^-9.  A rounded mantissa of 8 carries into the
// exponent field by the addition.
// Both candidate encodings are computed and the right one selected, so the
// function has no branches.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  // subnormal range (a < 2^-6): multiples of 2^-9, exact power-of-two scaling;
  // a rounded value of 8 is the smallest normal, code 0x08
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(a, 0.015625f) * 512.0f);
  // normal range: a in [2^e, 2^(e+1)), e = -6..8; a / 2^e in [1, 2) is exact
  const int e = max((int)((bits >> 23) & 0xff) - 127, -6);
  const float f = fminf(a, 464.0f) * __uint_as_float((uint32_t)(127 - e) << 23);
  const uint32_t m = (uint32_t)__builtin_rintf(f * 8.0f) - 8u;  // 0..8, 8 carries into the exponent
  const uint32_t nrm = min(((uint32_t)(e + 7) << 3) + m, 0x7Eu);
  uint32_t code = a < 0.015625f ? sub : nrm;
  code = a >= 464.0f ? 0x7Eu : code;  // 464 = midpoint 448|480: the tie goes to 448 (even); beyond saturates
  code = (a == a) ? code : 0x7Fu;
  return sign | code;
}

// |y| -> E2M1 magnitude code (0..7), round to nearest, ties to the even code,
// saturating at 6.  Grid 0, .5, 1, 1.5, 2, 3, 4, 6; NaN -> 7.
// Branch-free: the code is the number of rounding thresholds below |y|, with
// "<=" at the thresholds that are ties going down (to an even code) and "<" at
// those going up.
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return (a == a) ? c : 7u;
}

// Two E2M1 codes (low and high nibble of byte `sel` of w) -> exact FP16 pair.
// The scale operand of this conversion only applies its exponent, so it is
// kept at 1 and the E4M3 block scale is multiplied separately.
template <int sel>
__device__ __forceinline__ h2 e2m1x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, sel);
}

// Two E4M3 bytes (bytes 0,1 or 2,3 of w) -> exact FP16 pair.
template <bool hi>
__device__ __forceinline__ h2 e4m3x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, hi);
}

// 8 packed E2M1 codes (one dword, element 0 in the low nibble) -> 8 FP16.
__device__ __forceinline__ h8 e2m1x8_to_h8(uint32_t w) {
  h2 a = e2m1x2_to_h2<0>(w), b = e2m1x2_to_h2<1>(w), c = e2m1x2_to_h2<2>(w), d = e2m1x2_to_h2<3>(w);
  h8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// ---------------------------------------------------------------- slabs
// Byte of token t (0..127), dim d of an FP8 slab in each layout: token-major
// [t][d], dim-major [d][t], half rows [t/16][d/64][t%16][d%64].
__device__ __forceinline__ int fp8_offset(int layout, int t, int d) {
  if (layout == MSA_DIM_MAJOR) return d * kPage + t;
  if (layout == MSA_HALF_ROWS) return (t >> 4) * 2048 + (d >> 6) * 1024 + (t & 15) * 64 + (d & 63);
  return t * kDim + d;
}

// 16-byte load with the streaming (non-temporal) hint: data read once per step.
__device__ __forceinline__ uint4 nt_load4(const uint8_t* p) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ const uint8_t* slab_ptr(const uint8_t* pages, int64_t page, int heads, int head,
                                                   int slab_bytes) {
  return pages + (page * heads + head) * (int64_t)slab_bytes;
}

// ---------------------------------------------------------------- wave ops
// DPP lane moves (VALU, no LDS round trip).  Lanes outside row_mask keep
// their own value.
template <int ctrl, int row_mask>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, ctrl, row_mask, 0xf, false);
}

// Running maximum of a max-pool: m (which starts at -inf and so is never NaN)
// against a score x, skipping a NaN x.  The median of (m, x, +inf) is
// max(m, x) for a number x, and the hardware median of operands that include
// a NaN is the minimum of the others, m; the compiler folds chains of these
// into v_max3_f32, whose IEEE-mode result skips quiet NaN operands the same
// way.  (fmaxf means the same, but its lowering first quiets every operand
// that is not known to be canonical -- one extra instruction per matrix-core
// result.)
__device__ __forceinline__ float pool_max(float m, float x) { return __builtin_amdgcn_fmed3f(m, x, __builtin_inff()); }

// fmaxf over lanes l, l^16, l^32 and l^48 (the four 16-lane rows) in every
// lane: gfx950's row swaps, which run on the vector ALU, instead of permutes
// through the LDS unit.  Swapping the upper half of one copy with the lower
// half of another leaves each lane's partner l^32 in one of the two results
// and the lane's own value in the other (likewise odd and even rows for
// l^16), so the max of the pair is the max over both lanes.
__device__ __forceinline__ float rows_max4(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max within each 16-lane row, in every lane of the row (no lane NaN): pairs
// and quads by quad permutes, then half-row and row mirrors.
__device__ __forceinline__ float wave_max16(float v) {
  v = pool_max(v, __uint_as_float(dpp_mov<0xB1, 0xf>(__float_as_uint(v))));   // quad_perm [1,0,3,2]
  v = pool_max(v, __uint_as_float(dpp_mov<0x4E, 0xf>(__float_as_uint(v))));   // quad_perm [2,3,0,1]
  v = pool_max(v, __uint_as_float(dpp_mov<0x141, 0xf>(__float_as_uint(v))));  // row_half_mirror
  v = pool_max(v, __uint_as_float(dpp_mov<0x140, 0xf>(__float_as_uint(v))));  // row_mirror
  return v;
}

// Wave-wide unsigned max: the row max as above, then rows 0->1, 2->3 and
// 1->2,3 by row broadcasts; lane 63 ends with the maximum, read back as a
// scalar so every lane gets it.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_mov<0xB1, 0xf>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_mov<0x4E, 0xf>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_mov<0x141, 0xf>(v));  // row_half_mirror
  v = max(v, dpp_mov<0x140, 0xf>(v));  // row_mirror
  v = max(v, dpp_mov<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_mov<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ---------------------------------------------------------------- NVFP4 quantiser
// One 16-element group on one 16-lane DPP row, element i in lane i of the
// row: returns the E4M3 group scale and sets this lane's E2M1 code (sign in
// bit 3), by the amax recipe -- every step one FP32 operation with
// round-to-nearest-even:
//   s = E4M3_sat((amax / 6) / ts);  s == 0 -> code +0;
//   else code = sign(x) | E2M1_sat(|x / (s * ts)|).
// NaN elements count as 0 in the amax (max(|x|, 0) drops them).
__device__ __forceinline__ uint32_t nvfp4_row_quantize(float x, float ts, uint32_t& code) {
  const float amax = wave_max16(fmaxf(fabsf(x), 0.0f));
  const float t1 = amax / 6.0f;
  const float s32 = t1 / ts;
  const uint32_t sc = e4m3_encode(s32);
  const float sv = e4m3_to_f32(sc);
  code = 0;
  if (sv != 0.0f) {
    const float denom = sv * ts;
    const float y = x / denom;
    code = e2m1_mag(fabsf(y)) | ((__float_as_uint(x) >> 28) & 0x8u);
  }
  return sc;
}

// Store a row's group (token `off` of the slab, 16-dim group `grp`, this
// lane's element i).  Token-major: adjacent lanes pair their nibbles into a
// byte (element 2j in the low nibble of byte j) and the even lanes store it.
// Dim-major: dim 16 grp + i holds the token's nibble (off & 7) in dword
// off/8 of its 64-byte row; the nibble is cleared then set with atomic AND /
// OR (other tokens of the dword may be written at the same time).  Lane 0
// stores the scale.  `valid` (uniform over the row) suppresses every store.
__device__ __forceinline__ void nvfp4_row_store(uint8_t* slab, int off, int grp, int i, uint32_t code, uint32_t sc,
                                                bool dim_major, bool valid) {
  if (!dim_major) {
    const uint32_t hi = dpp_mov<0xB1, 0xf>(code);  // quad_perm [1,0,3,2]: lane 2j gets lane 2j+1's code
    if (valid) {
      if ((i & 1) == 0) slab[off * 64 + grp * 8 + (i >> 1)] = (uint8_t)(code | (hi << 4));
      if (i == 0) slab[kScaleOff + off * 8 + grp] = (uint8_t)sc;
    }
  } else if (valid) {
    const unsigned int sh = 4u * (unsigned)(off & 7);
    unsigned int* word = reinterpret_cast<unsigned int*>(slab + (grp * 16 + i) * 64 + (off >> 3) * 4);
    atomicAnd(word, ~(0xFu << sh));
    atomicOr(word, code << sh);
    if (i == 0) slab[kScaleOff + grp * 128 + off] = (uint8_t)sc;
  }
}

// Context length clamped to the block-table capacity; negative read as 0.
__device__ __forceinline__ int clamp_len(int L, int max_pages) {
  int cap = max_pages * kPage;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

}  // namespace msa
