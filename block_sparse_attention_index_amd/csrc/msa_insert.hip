// msa_insert.hip -- step 0 (cache insert with NVFP4 or FP8 quantisation),
// the FP8 query quantiser and the dequantisation test aid.
//
// Insert: one 16-lane row (a DPP row) per (token, cache head, 16-dim
// group), one element per lane.  The row reduces the group's amax with DPP,
// every lane derives the E4M3 group scale and its own E2M1 code with the amax
// recipe below (every step an FP32 operation with round-to-nearest-even, no
// contraction), and the codes go into the page slab of the token's slot.
// Token-major slabs: adjacent lanes pair their nibbles into a byte (one DPP
// swap) and the even lanes store the bytes.  Dim-major (value) slabs hold the
// codes of 8 consecutive tokens of one dim in a dword, so each lane replaces
// its nibble with an atomic AND then OR (vector memory atomics, no read round
// trip) -- tokens inserted together may share that dword.  One element per
// lane keeps each lane's dependency chain to one quantisation (a single
// IEEE division instead of sixteen in a row).  FP8 caches: each lane stores
// its own element, E4M3(x / tensor_scale), one byte, where its slab layout
// puts it (keys [token][dim], values [dim][token], index keys in half rows).
#pragma clang fp contract(off)

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

// Up to three target caches (keys, values, index keys), passed as scalars so
// that choosing one per thread is a register select, not a memory load.
struct InsertArgs {
  uint8_t* pages0;
  uint8_t* pages1;
  uint8_t* pages2;
  const float* src0;
  const float* src1;
  const float* src2;
  int32_t np0, np1, np2;     // page-pool sizes
  int32_t h0, h1, h2;        // heads
  int32_t nv0, nv1, nv2;     // msa_dtype: MSA_NVFP4, MSA_FP8_E4M3 or MSA_F32
  int32_t dm0, dm1, dm2;     // msa_layout of the slab
  float ts0, ts1, ts2;       // tensor scales
  int32_t u0, u1, u2;        // 16-dim groups per token (heads * 8), 0 if absent
};

__global__ __launch_bounds__(256) void kv_insert_kernel(InsertArgs A, const int64_t* __restrict__ slots, int32_t n) {
  const int32_t units = A.u0 + A.u1 + A.u2;  // 16-dim groups per token over all caches
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gunit = gid >> 4;  // (token, group) of this 16-lane row
  const int i = (int)(gid & 15);   // element within the group
  if (gunit >= (int64_t)n * units) return;  // whole rows leave together (blockDim is a multiple of 16)
  const int32_t tok = (int32_t)(gunit / units);
  int32_t u = (int32_t)(gunit - (int64_t)tok * units);
  const int c = u < A.u0 ? 0 : (u < A.u0 + A.u1 ? 1 : 2);
  u -= c == 0 ? 0 : (c == 1 ? A.u0 : A.u0 + A.u1);
  uint8_t* pages = c == 0 ? A.pages0 : (c == 1 ? A.pages1 : A.pages2);
  const float* src = c == 0 ? A.src0 : (c == 1 ? A.src1 : A.src2);
  const int32_t num_pages = c == 0 ? A.np0 : (c == 1 ? A.np1 : A.np2);
  const int32_t heads = c == 0 ? A.h0 : (c == 1 ? A.h1 : A.h2);
  const int32_t fmt = c == 0 ? A.nv0 : (c == 1 ? A.nv1 : A.nv2);
  const int32_t layout = c == 0 ? A.dm0 : (c == 1 ? A.dm1 : A.dm2);
  const float ts = c == 0 ? A.ts0 : (c == 1 ? A.ts1 : A.ts2);
  const int head = u >> 3, grp = u & 7;

  // Both loads go out before anything waits on them: an invalid slot only
  // predicates the stores (an early return would let the compiler sink the
  // row load behind the slot load).
  const int64_t slot = slots[tok];
  const float x = src[((int64_t)tok * heads + head) * kDim + grp * 16 + i];
  const bool valid = slot >= 0 && slot < (int64_t)num_pages * kPage;
  const int64_t page = valid ? slot >> 7 : 0;
  const int off = (int)(slot & 127);
  if (fmt == MSA_F32) {
    float* dst = reinterpret_cast<float*>(pages + (page * heads + head) * (int64_t)kF32Slab);
    if (valid) dst[off * kDim + grp * 16 + i] = x;
    return;
  }
  if (fmt == MSA_FP8_E4M3) {
    uint8_t* slab = pages + (page * heads + head) * (int64_t)kFp8Slab;
    const int d = grp * 16 + i;
    if (valid) slab[fp8_offset(layout, off, d)] = (uint8_t)e4m3_encode(x / ts);
    return;
  }
  if (layout == MSA_DIM_MAJOR) {
    // A value byte holds the nibbles of tokens 2k and 2k+1 of one dim.  When the
    // token of an even slot is followed in the batch by the token of the next
    // slot (a prompt chunk, tokens in order), this row quantises both and
    // writes whole bytes; the follower's row writes nothing.  Other tokens
    // merge their nibble into the shared dword with atomics.
    const int64_t nxt = tok + 1 < n ? slots[tok + 1] : -1;
    const int64_t prv = tok > 0 ? slots[tok - 1] : -1;
    if (valid && (slot & 1) && prv == slot - 1) return;  // written by the previous token's row
    if (valid && !(slot & 1) && nxt == slot + 1) {
      const float x1 = src[((int64_t)(tok + 1) * heads + head) * kDim + grp * 16 + i];
      uint32_t c0, c1;
      const uint32_t s0 = nvfp4_row_quantize(x, ts, c0);
      const uint32_t s1 = nvfp4_row_quantize(x1, ts, c1);
      uint8_t* slab = pages + (page * heads + head) * (int64_t)kNvSlab;
      slab[(grp * 16 + i) * 64 + (off >> 1)] = (uint8_t)(c0 | (c1 << 4));
      if (i == 0) {
        slab[kScaleOff + grp * 128 + off] = (uint8_t)s0;
        slab[kScaleOff + grp * 128 + off + 1] = (uint8_t)s1;
      }
      return;
    }
  }
  uint32_t code;
  const uint32_t sc = nvfp4_row_quantize(x, ts, code);
  nvfp4_row_store(pages + (page * heads + head) * (int64_t)kNvSlab, off, grp, i, code, sc, layout == MSA_DIM_MAJOR,
                  valid);
}

// The same NVFP4 insert with one lane per 16-element group, for large
// batches (a prompt chunk): the group's amax and E4M3 scale are derived once
// per group instead of once per element, so the vector work per element is
// about a quarter.  Every step is the same FP32 operation on the same
// values as nvfp4_row_quantize (the maximum of |x| over the group does not
// depend on the order), so the bytes written are identical.  All three
// caches NVFP4.
__device__ __forceinline__ uint32_t nvfp4_group_quantize(const float (&x)[16], float ts, uint32_t (&code)[16]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(x[i]), 0.0f));
  const float t1 = amax / 6.0f;
  const float s32 = t1 / ts;
  const uint32_t sc = e4m3_encode(s32);
  const float sv = e4m3_to_f32(sc);
#pragma unroll
  for (int i = 0; i < 16; ++i) code[i] = 0;
  if (sv != 0.0f) {
    const float denom = sv * ts;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float y = x[i] / denom;
      code[i] = e2m1_mag(fabsf(y)) | ((__float_as_uint(x[i]) >> 28) & 0x8u);
    }
  }
  return sc;
}

__device__ __forceinline__ void load_group(const float* __restrict__ p, float (&x)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = reinterpret_cast<const float4*>(p)[q];
    x[4 * q] = v.x, x[4 * q + 1] = v.y, x[4 * q + 2] = v.z, x[4 * q + 3] = v.w;
  }
}

__global__ __launch_bounds__(256) void kv_insert_group_kernel(InsertArgs A, const int64_t* __restrict__ slots,
                                                              int32_t n) {
  const int32_t units = A.u0 + A.u1 + A.u2;
  const int64_t gunit = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (token, group)
  if (gunit >= (int64_t)n * units) return;
  const int32_t tok = (int32_t)(gunit / units);
  int32_t u = (int32_t)(gunit - (int64_t)tok * units);
  const int c = u < A.u0 ? 0 : (u < A.u0 + A.u1 ? 1 : 2);
  u -= c == 0 ? 0 : (c == 1 ? A.u0 : A.u0 + A.u1);
  uint8_t* pages = c == 0 ? A.pages0 : (c == 1 ? A.pages1 : A.pages2);
  const float* src = c == 0 ? A.src0 : (c == 1 ? A.src1 : A.src2);
  const int32_t num_pages = c == 0 ? A.np0 : (c == 1 ? A.np1 : A.np2);
  const int32_t heads = c == 0 ? A.h0 : (c == 1 ? A.h1 : A.h2);
  const int32_t layout = c == 0 ? A.dm0 : (c == 1 ? A.dm1 : A.dm2);
  const float ts = c == 0 ? A.ts0 : (c == 1 ? A.ts1 : A.ts2);
  const int head = u >> 3, grp = u & 7;
  const int64_t slot = slots[tok];
  const bool valid = slot >= 0 && slot < (int64_t)num_pages * kPage;
  if (!valid) return;
  const int64_t page = slot >> 7;
  const int off = (int)(slot & 127);
  uint8_t* slab = pages + (page * heads + head) * (int64_t)kNvSlab;
  float x[16];
  load_group(src + ((int64_t)tok * heads + head) * kDim + grp * 16, x);
  uint32_t code[16];
  if (layout != MSA_DIM_MAJOR) {
    const uint32_t sc = nvfp4_group_quantize(x, ts, code);
    uint2 w = make_uint2(0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) w.x |= code[i] << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) w.y |= code[8 + i] << (4 * i);
    *reinterpret_cast<uint2*>(slab + off * 64 + grp * 8) = w;
    slab[kScaleOff + off * 8 + grp] = (uint8_t)sc;
    return;
  }
  // dim-major values: as kv_insert_kernel, a token of an even slot followed in
  // the batch by the next slot writes both tokens' nibbles as whole bytes
  const int64_t nxt = tok + 1 < n ? slots[tok + 1] : -1;
  const int64_t prv = tok > 0 ? slots[tok - 1] : -1;
  if ((slot & 1) && prv == slot - 1) return;  // written by the previous token's lane
  const uint32_t sc = nvfp4_group_quantize(x, ts, code);
  if (!(slot & 1) && nxt == slot + 1) {
    float x1[16];
    load_group(src + ((int64_t)(tok + 1) * heads + head) * kDim + grp * 16, x1);
    uint32_t code1[16];
    const uint32_t sc1 = nvfp4_group_quantize(x1, ts, code1);
#pragma unroll
    for (int i = 0; i < 16; ++i) slab[(grp * 16 + i) * 64 + (off >> 1)] = (uint8_t)(code[i] | (code1[i] << 4));
    slab[kScaleOff + grp * 128 + off] = (uint8_t)sc;
    slab[kScaleOff + grp * 128 + off + 1] = (uint8_t)sc1;
    return;
  }
  const unsigned int sh = 4u * (unsigned)(off & 7);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    unsigned int* word = reinterpret_cast<unsigned int*>(slab + (grp * 16 + i) * 64 + (off >> 3) * 4);
    atomicAnd(word, ~(0xFu << sh));
    atomicOr(word, code[i] << sh);
  }
  slab[kScaleOff + grp * 128 + off] = (uint8_t)sc;
}

__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const float* __restrict__ x, int64_t n, float scale,
                                                            uint8_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)e4m3_encode(x[i] / scale);
}

// One thread per (page, head, token, 8-dim chunk): decodes 8 elements.
__global__ __launch_bounds__(256) void debug_dequant_kernel(const uint8_t* __restrict__ pages, int32_t num_pages,
                                                            int32_t heads, int32_t fmt, int32_t layout,
                                                            float ts, const int32_t* __restrict__ page_ids,
                                                            int32_t n_pages, int32_t mode, float* __restrict__ out) {
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)n_pages * heads * kPage * (kDim / 8);
  if (gid >= total) return;
  int chunk = (int)(gid % (kDim / 8));
  int t = (int)((gid / (kDim / 8)) % kPage);
  int head = (int)((gid / (kDim / 8 * kPage)) % heads);
  int i = (int)(gid / ((int64_t)kDim / 8 * kPage * heads));
  int64_t page = page_ids[i];
  float* o = out + (((int64_t)i * heads + head) * kPage + t) * kDim + chunk * 8;
  if (page < 0 || page >= num_pages) {
    for (int e = 0; e < 8; ++e) o[e] = __builtin_nanf("");
    return;
  }
  if (fmt == MSA_F32) {
    const float* s = reinterpret_cast<const float*>(pages + (page * heads + head) * (int64_t)kF32Slab) + t * kDim;
    for (int e = 0; e < 8; ++e) o[e] = s[chunk * 8 + e];
    return;
  }
  if (fmt == MSA_FP8_E4M3) {
    // both modes: E4M3 is exact in FP32 and FP16, one FP32 multiply by the tensor scale
    const uint8_t* slab = pages + (page * heads + head) * (int64_t)kFp8Slab;
    for (int e = 0; e < 8; ++e) {
      const int d = chunk * 8 + e;
      o[e] = e4m3_to_f32(slab[fp8_offset(layout, t, d)]) * ts;
    }
    return;
  }
  const uint8_t* slab = pages + (page * heads + head) * (int64_t)kNvSlab;
  uint32_t codes = 0;  // 8 nibbles, dim chunk*8 + e at nibble e
  uint8_t sc;
  if (layout != MSA_DIM_MAJOR) {
    codes = *reinterpret_cast<const uint32_t*>(slab + t * 64 + chunk * 4);
    sc = slab[kScaleOff + t * 8 + chunk / 2];
  } else {
    for (int e = 0; e < 8; ++e) {
      int d = chunk * 8 + e;
      uint32_t byte = slab[d * 64 + t / 2];
      codes |= ((byte >> (4 * (t & 1))) & 0xFu) << (4 * e);
    }
    sc = slab[kScaleOff + (chunk / 2) * 128 + t];
  }
  h8 c = e2m1x8_to_h8(codes);
  if (mode == 0) {
    float s = e4m3_to_f32(sc);
    for (int e = 0; e < 8; ++e) o[e] = ((float)c[e] * s) * ts;
  } else {
    h2 s2 = e4m3x2_to_h2<false>((uint32_t)sc | ((uint32_t)sc << 8));
    for (int e = 0; e < 8; ++e) {
      _Float16 v = c[e] * s2[0];  // exact in FP16
      o[e] = (float)v * ts;
    }
  }
}

}  // namespace msa

using namespace msa;

extern "C" int msa_launch_kv_insert(const float* k, const float* v, const float* idx_k, const int64_t* slots,
                                    int32_t n, const msa_cache* kc, const msa_cache* vc, const msa_cache* ic,
                                    hipStream_t stream) {
  InsertArgs A{};
  auto fill = [](const msa_cache* c, const float* src, uint8_t*& pg, const float*& s, int32_t& np, int32_t& h,
                 int32_t& nv, int32_t& dm, float& ts, int32_t& u) {
    if (!c || !src) return;
    pg = (uint8_t*)c->pages;
    s = src;
    np = c->num_pages;
    h = c->num_heads;
    nv = c->dtype;
    dm = c->layout;
    ts = c->tensor_scale;
    u = c->num_heads * 8;
  };
  fill(kc, k, A.pages0, A.src0, A.np0, A.h0, A.nv0, A.dm0, A.ts0, A.u0);
  fill(vc, v, A.pages1, A.src1, A.np1, A.h1, A.nv1, A.dm1, A.ts1, A.u1);
  fill(ic, idx_k, A.pages2, A.src2, A.np2, A.h2, A.nv2, A.dm2, A.ts2, A.u2);
  const int64_t groups = (int64_t)n * (A.u0 + A.u1 + A.u2);
  if (groups == 0) return 0;
  // a prompt chunk with every cache NVFP4: one lane per group; otherwise (and
  // for a decode step's few tokens, where a 16-lane row per group is faster)
  // one 16-lane row per (token, group)
  const bool nv = (!A.pages0 || A.nv0 == MSA_NVFP4) && (!A.pages1 || A.nv1 == MSA_NVFP4) &&
                  (!A.pages2 || A.nv2 == MSA_NVFP4);
  if (nv && n >= 512) {
    hipLaunchKernelGGL(kv_insert_group_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream, A,
                       slots, n);
  } else {
    const int64_t total = groups * 16;
    hipLaunchKernelGGL(kv_insert_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, A, slots, n);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int msa_launch_quantize_e4m3(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t stream) {
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int msa_launch_debug_dequant(const msa_cache* c, const int32_t* pages, int32_t n_pages, int32_t mode,
                                        float* out, hipStream_t stream) {
  int64_t total = (int64_t)n_pages * c->num_heads * kPage * (kDim / 8);
  if (total == 0) return 0;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(debug_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint8_t*)c->pages,
                     c->num_pages, c->num_heads, (int32_t)c->dtype,
                     (int32_t)c->layout, c->tensor_scale, pages, n_pages, mode, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
