// Device-side helpers shared by the ftmoe kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ftmoe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

// Weight format tags (values match ftmoe_wfmt).
constexpr int kMXFP4 = 1;
constexpr int kNVFP4 = 2;
constexpr int kFP8 = 3;
constexpr int kBF16 = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the default cache policy.  (Measured on MI355X for the
// decode weight streams: the non-temporal hint made them about 13% slower.)
__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- bf16 ----

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ------------------------------------------------------------- codecs -----

// E8M0 scale code -> the fp32 whose exponent field is that code.  The gfx950
// scaled conversions read only the exponent field of their scale operand, so
// this encodes 2^(code - 127) for every code 0..254 (code 0 included).
__device__ __forceinline__ float e8m0_as_scale(uint32_t code) {
  return __uint_as_float(code << 23);
}

// E4M3FN byte -> fp32 value (exact; hardware decode of the OCP format).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code & 0xFFu, 1.0f, false);
  return v[0];
}

// Eight packed E2M1 nibbles (one dword, element 0 in the low nibble) times a
// power-of-two scale given as an E8M0-style float -> four bf16 pairs.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t w, float scale, uint32_t out[4]) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  out[0] = __builtin_bit_cast(uint32_t, p0);
  out[1] = __builtin_bit_cast(uint32_t, p1);
  out[2] = __builtin_bit_cast(uint32_t, p2);
  out[3] = __builtin_bit_cast(uint32_t, p3);
}

// Two fp32 values that are exactly representable in bf16 -> their bf16
// pair, by the hardware conversion (one instruction; no rounding happens).
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float lo, float hi) {
  const bf16x2 r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, r);
}

// The significand of an NVFP4 block scale s (decoded E4M3, finite) with its
// sign, as an fp32 in [1, 2) (0 for a zero scale): s = 2^floor(log2|s|) times it.
__device__ __forceinline__ float nv_scale_significand(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x7FFFFFFFu) ? __uint_as_float((b & 0x807FFFFFu) | 0x3F800000u) : 0.0f;
}

// Eight E2M1 nibbles times an NVFP4 block scale s -> four bf16 pairs, exactly.
// The scaled conversion applies s's power of two (it reads only the exponent
// field of its scale operand), one multiply its significand `sig`
// (nv_scale_significand(s)); E2M1 has 2 significant bits and E4M3 4, so each
// product fits bf16's 8 and the final conversion does not round.
__device__ __forceinline__ void fp4x8_to_bf16_nv(uint32_t w, float s, float sig, uint32_t out[4]) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
  out[0] = pack_exact_bf16x2(v0[0] * sig, v0[1] * sig);
  out[1] = pack_exact_bf16x2(v1[0] * sig, v1[1] * sig);
  out[2] = pack_exact_bf16x2(v2[0] * sig, v2[1] * sig);
  out[3] = pack_exact_bf16x2(v3[0] * sig, v3[1] * sig);
}

// Four E4M3 codes (one dword) -> two bf16 pairs, exactly (every E4M3 value is
// a bf16 value).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, uint32_t out[2]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// fp32 -> E4M3FN code: round to nearest even, saturate to +-448.  The
// hardware conversion rounds to nearest even but does not saturate, so the
// input is clamped first.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// ------------------------------------------- split FP8 activation blocks ----
// For the MX-scaled MFMA (FP8 activations x MXFP4 weights) a block of 32
// activations is carried as two E4M3 vectors sharing one power-of-two scale
// 2^e:  x ~= 2^e * (hi + lo / 16)  with  hi = E4M3(x / 2^e) and
// lo = E4M3(16 (x / 2^e - hi)).  e = floor(log2 amax) - 7 keeps |x / 2^e| below
// 256 (no saturation), so the pair keeps about 8 significant bits -- the
// precision of the bf16 input -- while the weights stay as 4-bit codes.
// The scale is returned as its E8M0 code (e + 127, clamped to [4, 254]).
// The code is at least 4, so that the lo codes' scale (code - 4) is a valid
// E8M0 code and can be formed by a plain subtraction; this only matters for
// blocks whose largest magnitude is below 2^-116.
__device__ __forceinline__ uint32_t mx_split_scale_code(float amax) {
  const int ebits = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF);
  int code = ebits - 7;
  code = code < 4 ? 4 : (code > 254 ? 254 : code);
  return static_cast<uint32_t>(code);
}

// 2^(127 - code): multiplying by it divides by the block scale exactly.
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// hi and lo E4M3 codes of two adjacent values already divided by the scale.
// Such values lie in (-256, 256): the scale code is at least floor(log2
// amax) - 7, and its lower clamp only makes them smaller.  The lo input,
// 16 (a - hi), is at most 16 times half an E4M3 step at 128..256, i.e. 128.
// Neither conversion can therefore leave E4M3's range (448), and the
// hardware's nearest-even conversion needs no clamp in front of it.
__device__ __forceinline__ void mx_split_pair(float a, float b, uint32_t* hi2, uint32_t* lo2) {
  const uint32_t h = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false));
  const f32x2 dh = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 1.0f, false);
  *hi2 = h;
  *lo2 = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32((a - dh[0]) * 16.0f, (b - dh[1]) * 16.0f, 0, false));
}

// The same for four adjacent values, codes packed as one dword each (the
// second conversion of each writes the upper half of the first's dword).
__device__ __forceinline__ void mx_split_quad(float a0, float a1, float a2, float a3, uint32_t& hi4, uint32_t& lo4) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, h, true);
  const f32x2 d01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(static_cast<uint32_t>(h), 1.0f, false);
  const f32x2 d23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(static_cast<uint32_t>(h), 1.0f, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32((a0 - d01[0]) * 16.0f, (a1 - d01[1]) * 16.0f, 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32((a2 - d23[0]) * 16.0f, (a3 - d23[1]) * 16.0f, l, true);
  hi4 = static_cast<uint32_t>(h);
  lo4 = static_cast<uint32_t>(l);
}

// Largest magnitude of the bf16 values in n vectors of 8.  With the sign bit
// cleared, the bits of finite bf16 values order as their magnitudes, so the
// maximum is taken on the 16-bit patterns, two per packed integer max.
template <int N>
__device__ __forceinline__ float bf16_amax(const uint4 (&v)[N]) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = {0, 0};
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  }
  return bf16_to_f32(m.x > m.y ? m.x : m.y);
}

// Half of a 32-block (16 bf16 values, 2 vectors of 8) in the split form, given
// the maximum over the whole block: 16 hi codes, 16 lo codes; returns the
// block's scale code.
__device__ __forceinline__ uint32_t mx_split_half(const uint4 (&v)[2], float amax, uint4& hi, uint4& lo) {
  const uint32_t code = mx_split_scale_code(amax);
  const float inv = mx_inv_scale(code);
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
    for (int i = 0; i < 4; i += 2)
      mx_split_quad(bf16_to_f32(w[i] & 0xFFFF) * inv, bf16_to_f32(w[i] >> 16) * inv,
                    bf16_to_f32(w[i + 1] & 0xFFFF) * inv, bf16_to_f32(w[i + 1] >> 16) * inv, hw[2 * q + i / 2],
                    lw[2 * q + i / 2]);
  }
  hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  return code;
}

// Splits one 32-block of bf16 values (4 vectors of 8) into 32 hi codes, 32
// lo codes (16-byte aligned destinations, global or LDS) and the scale code.
__device__ __forceinline__ void mx_split_block(const uint4 (&v)[4], uint8_t* hi, uint8_t* lo, uint8_t* sc) {
  const float amax = bf16_amax(v);
  const uint4 a[2] = {v[0], v[1]}, b[2] = {v[2], v[3]};
  uint4 h0, l0, h1, l1;
  const uint32_t code = mx_split_half(a, amax, h0, l0);
  mx_split_half(b, amax, h1, l1);
  reinterpret_cast<uint4*>(hi)[0] = h0;
  reinterpret_cast<uint4*>(hi)[1] = h1;
  reinterpret_cast<uint4*>(lo)[0] = l0;
  reinterpret_cast<uint4*>(lo)[1] = l1;
  *sc = static_cast<uint8_t>(code);
}

// ------------------------------------------------ MXFP8 activation blocks --
// OCP Microscaling v1.0 conversion of a block of 32 values to E4M3 elements
// under one E8M0 scale 2^X: X = floor(log2 amax) - 8 (8 being E4M3's largest
// exponent), at least -127; each element is the nearest E4M3 of v / 2^X,
// saturating at 448.  The scale is returned as its E8M0 code X + 127 (the
// biased exponent field of amax minus 8, clamped at 0).
__device__ __forceinline__ uint32_t mxfp8_scale_code(float amax) {
  const int ebits = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF);
  return static_cast<uint32_t>(ebits > 8 ? ebits - 8 : 0);
}

// Half of a 32-block (16 bf16 values) as E4M3 codes under the block's scale,
// given the maximum over the whole block; returns the scale code.
__device__ __forceinline__ uint32_t mxfp8_half(const uint4 (&v)[2], float amax, uint4& q) {
  const uint32_t code = mxfp8_scale_code(amax);
  const float inv = mx_inv_scale(code);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    const uint32_t p0 = f32x2_to_e4m3x2(bf16_to_f32(w[0] & 0xFFFF) * inv, bf16_to_f32(w[0] >> 16) * inv);
    const uint32_t p1 = f32x2_to_e4m3x2(bf16_to_f32(w[1] & 0xFFFF) * inv, bf16_to_f32(w[1] >> 16) * inv);
    const uint32_t p2 = f32x2_to_e4m3x2(bf16_to_f32(w[2] & 0xFFFF) * inv, bf16_to_f32(w[2] >> 16) * inv);
    const uint32_t p3 = f32x2_to_e4m3x2(bf16_to_f32(w[3] & 0xFFFF) * inv, bf16_to_f32(w[3] >> 16) * inv);
    o[2 * i] = p0 | (p1 << 16);
    o[2 * i + 1] = p2 | (p3 << 16);
  }
  q = make_uint4(o[0], o[1], o[2], o[3]);
  return code;
}

// Converts one 32-block of bf16 values (4 vectors of 8) to 32 E4M3 codes
// (16-byte aligned destination, global or LDS) and the scale code.
__device__ __forceinline__ void mxfp8_block(const uint4 (&v)[4], uint8_t* q, uint8_t* sc) {
  const float amax = bf16_amax(v);
  const uint4 a[2] = {v[0], v[1]}, b[2] = {v[2], v[3]};
  uint4 q0, q1;
  const uint32_t code = mxfp8_half(a, amax, q0);
  mxfp8_half(b, amax, q1);
  reinterpret_cast<uint4*>(q)[0] = q0;
  reinterpret_cast<uint4*>(q)[1] = q1;
  *sc = static_cast<uint8_t>(code);
}

// ------------------------------------------------------------ wave ops ----

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// DPP lane permutations within 16-lane rows (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within each 16 lanes

// Largest value over the 32 lanes of each half-wave: DPP within each 16-lane
// row, then one swizzle exchanging rows 0 <-> 1 and 2 <-> 3 (lane ^ 16).
__device__ __forceinline__ float half_wave_max(float v) {
  v = __builtin_fmaxf(v, dpp_f<kDppXor1>(v));
  v = __builtin_fmaxf(v, dpp_f<kDppXor2>(v));
  v = __builtin_fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = __builtin_fmaxf(v, dpp_f<kDppMirror>(v));
  return __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Wave-wide reductions with a fixed combination order (deterministic): DPP
// within each 16-lane row, then the four row results in lane order.
__device__ __forceinline__ float wave_sum_fixed(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max_fast(float v) {
  v = __builtin_fmaxf(v, dpp_f<kDppXor1>(v));
  v = __builtin_fmaxf(v, dpp_f<kDppXor2>(v));
  v = __builtin_fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = __builtin_fmaxf(v, dpp_f<kDppMirror>(v));
  return __builtin_fmaxf(__builtin_fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
                         __builtin_fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  v = min(v, dpp_i<kDppMirror>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Wave argmax: the largest value, equal values resolved to the lowest index.
// Every lane gets (value, index).
__device__ __forceinline__ void wave_argmax(float v, int idx, float* best_v, int* best_i) {
  const float m = wave_max_fast(v);
  const unsigned long long mask = __ballot(v == m);
  int wi;
  if (__popcll(mask) == 1) {
    wi = __builtin_amdgcn_readlane(idx, __ffsll(static_cast<long long>(mask)) - 1);
  } else {
    wi = wave_min_int(v == m ? idx : 0x7FFFFFFF);
  }
  *best_v = m;
  *best_i = wi;
}

// Per-call maximum of |h| for the FP8 per-tensor scale.  Many workgroups
// contribute, and atomics on one address serialise, so each workgroup first
// reduces in LDS and then updates one of kAmaxSlots words kAmaxStride words
// apart (different cache lines); a one-wave pass folds the slots afterwards.
constexpr int kAmaxSlots = 64;
constexpr int kAmaxStride = 32;

// All threads of the workgroup must call it.  `red` is >= 16 floats of LDS.
__device__ __forceinline__ void wg_amax_to_slots(float m, uint32_t* slots, float* red) {
  m = wave_max_fast(m);
  const int wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  if (lane_id() == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.f;
    for (int i = 0; i < nw; ++i) r = __builtin_fmaxf(r, red[i]);
    const unsigned slot = (blockIdx.x + blockIdx.y * gridDim.x) % kAmaxSlots;
    atomicMax(slots + slot * kAmaxStride, __float_as_uint(r));
  }
}

// The same from one wave, without LDS: its lane 0 updates the slot of
// (workgroup, wave).
__device__ __forceinline__ void wave_amax_to_slots(float m, uint32_t* slots) {
  m = wave_max_fast(m);
  if (lane_id() == 0) {
    const unsigned slot = (blockIdx.x * 8u + (threadIdx.x >> 6)) % kAmaxSlots;
    atomicMax(slots + slot * kAmaxStride, __float_as_uint(m));
  }
}

// silu(g) * u with the hardware exponential and reciprocal (about 1 ulp
// each), instead of an IEEE division.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

}  // namespace ftmoe
