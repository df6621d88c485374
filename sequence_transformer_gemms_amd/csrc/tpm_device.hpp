// Device-side helpers shared by the gfx950 kernels of libtpmlp: vector types,
// bf16 / e4m3fn conversions, activations, buffer-resource loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

// Raw buffer descriptor (gfx9 family: 32-bit data format, no swizzle).
// A load whose byte offset is past `bytes` returns zeros, which is how every
// tile edge (ragged M, N or K) is predicated.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOOB = 0xFFFFFFF0u;  // an offset no descriptor here covers

// The 32-bit LDS byte address of a generic pointer into LDS.  Callers take
// it once and form every DMA destination from it with 32-bit arithmetic: a
// generic pointer cast per load costs a 64-bit add and a null check in
// scalar instructions, in the instruction stream that feeds the matrix cores.
__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// 16 bytes per lane from global memory straight into LDS; lane i of the wave
// writes bytes [16 i, 16 i + 16) after the wave-uniform LDS byte address
// `lds`.  The address passes through an empty asm statement, so the compiler
// cannot tie these DMA writes to the LDS block the kernel reads through a
// restrict-qualified pointer, and does not drain every DMA in flight before
// each such read: callers order DMA writes and LDS reads themselves (a
// vmcnt wait and a work-group barrier), and wait for vmcnt(0) before they
// write LDS that a DMA may still target.
__device__ inline lds_void* lds_dma_address(uint32_t lds) {
  uint32_t a = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("" : "+s"(a));
  return (lds_void*)(uintptr_t)a;
}
__device__ inline void load16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dma_address(lds), 16, voff, 0, 0, 0);
}

// The same with a uniform part of the offset in the scalar offset register.
// The hardware range check covers the vector offset only, so the sum must be
// known to lie inside the buffer (callers use it for whole tiles only).
__device__ inline void load16_to_lds_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_dma_address(lds), 16, voff, soff, 0, 0);
}

__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// ---------------------------------------------------------------- formats
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// Two fp32 values rounded to bf16 (nearest, ties to even) and packed, a in
// the low half: one v_cvt_pk_bf16_f32.  Equal to f32_to_bf16_rne on every
// non-NaN input (a NaN stays a quiet NaN, not necessarily 0x7FC0).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Decodes of the fp8 formats from their bit fields.  e4m3fn: bias 7, field
// 0 subnormal (m * 2^-9), S.1111.111 NaN, no infinity.  e5m2: bias 15,
// field 0 subnormal (m * 2^-16), field 31 infinity (m = 0) or NaN.
__device__ inline float e4m3_to_f32(uint8_t c) {
  const uint32_t sign = (uint32_t)(c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 15u && m == 7u) return __builtin_nanf("");
  const float mag = e == 0u ? (float)m * 0.001953125f : __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, mag) | sign);
}
__device__ inline float e5m2_to_f32(uint8_t c) {
  const uint32_t sign = (uint32_t)(c & 0x80u) << 24;
  const uint32_t e = (c >> 2) & 0x1Fu, m = c & 3u;
  float mag;
  if (e == 31u) mag = m == 0u ? __builtin_inff() : __builtin_nanf("");
  else mag = e == 0u ? (float)m * 1.52587890625e-05f : __builtin_bit_cast(float, ((e + 112u) << 23) | (m << 21));
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, mag) | sign);
}

// OCP e4m3fn encode of an fp32 value: nearest, ties to even, saturating to
// +-448, NaN -> 0x7F, sign kept for zero.  Integer arithmetic on the fp32
// bits, so the result does not depend on any hardware conversion mode.
__device__ inline uint8_t f32_to_e4m3_rne_sat(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7F;
  // 448 = 1.75 * 2^8 -> fp32 bits 0x43E00000; the rounding midpoint to the
  // (non-existent) next value 480 is 464 (0x43E80000): everything at or
  // above 448 after rounding saturates.
  if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7E);
  int e = (int)(a >> 23) - 127;  // unbiased exponent
  uint8_t code;
  if (e >= -6) {
    // normal e4m3: keep 3 mantissa bits, round the 20 dropped bits
    uint32_t mant = a & 0x7FFFFFu;
    uint32_t keep = mant >> 20;
    uint32_t rest = mant & 0xFFFFFu;
    uint32_t half = 0x80000u;
    uint32_t q = ((uint32_t)(e + 7) << 3) | keep;
    if (rest > half || (rest == half && (keep & 1u))) q += 1;  // may carry into exponent
    if (q > 0x7E) q = 0x7E;
    code = (uint8_t)q;
  } else {
    // subnormal e4m3: value = m * 2^-9, m in 0..7 (m = 8 rounds up to the
    // smallest normal, code 0x08).  x / 2^-9 = significand * 2^(e + 9).
    if (e < -10) return (uint8_t)sign;  // below half the smallest subnormal
    uint32_t sig = (a & 0x7FFFFFu) | 0x800000u;  // 24-bit significand, value sig * 2^(e-23)
    int shift = 14 - e;                          // m = sig >> shift (shift in 21..24)
    uint32_t m = sig >> shift;
    uint32_t rest = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rest > half || (rest == half && (m & 1u))) m += 1;
    code = (uint8_t)m;
  }
  return (uint8_t)(sign | code);
}

// OCP e5m2 encode of an fp32 value: nearest, ties to even, saturating to
// +-57344 (1.75 * 2^15, fp32 bits 0x47600000: every larger finite value,
// and inf, rounds past it), NaN -> 0x7F, sign kept for zero.
__device__ inline uint8_t f32_to_e5m2_rne_sat(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7F;
  if (a >= 0x47600000u) return (uint8_t)(sign | 0x7B);
  int e = (int)(a >> 23) - 127;
  uint8_t code;
  if (e >= -14) {
    // normal e5m2: keep 2 mantissa bits, round the 21 dropped bits
    uint32_t mant = a & 0x7FFFFFu;
    uint32_t keep = mant >> 21;
    uint32_t rest = mant & 0x1FFFFFu;
    uint32_t half = 0x100000u;
    uint32_t q = ((uint32_t)(e + 15) << 2) | keep;
    if (rest > half || (rest == half && (keep & 1u))) q += 1;  // may carry into exponent
    if (q > 0x7B) q = 0x7B;
    code = (uint8_t)q;
  } else {
    // subnormal e5m2: value = m * 2^-16, m in 0..3 (m = 4 is the smallest
    // normal, code 0x04).  x / 2^-16 = significand * 2^(e + 16 - 23).
    if (e < -17) return (uint8_t)sign;           // below half the smallest subnormal
    uint32_t sig = (a & 0x7FFFFFu) | 0x800000u;
    int shift = 7 - e;                           // 22 .. 24
    uint32_t m = sig >> shift;
    uint32_t rest = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rest > half || (rest == half && (m & 1u))) m += 1;
    code = (uint8_t)m;
  }
  return (uint8_t)(sign | code);
}

// Four fp32 values to four OCP fp8 codes (e4m3fn, or e5m2 when E5M2), byte e
// of the result holding value e: the same codes as the integer encoders
// above.  The hardware pack conversion (two values per instruction) rounds to
// nearest-even and keeps the sign of zero, but turns a finite magnitude past
// the format's largest value into NaN instead of saturating, so each input is
// clamped to +-largest first; a group holding a NaN takes the integer
// encoders.  The two agree on every fp32 bit pattern (checked exhaustively).
template <bool E5M2>
__device__ inline uint32_t fp8x4(float a, float b, float c, float d) {
  if (__builtin_expect((a != a) | (b != b) | (c != c) | (d != d), 0)) {
    if (E5M2)
      return (uint32_t)f32_to_e5m2_rne_sat(a) | (uint32_t)f32_to_e5m2_rne_sat(b) << 8 |
             (uint32_t)f32_to_e5m2_rne_sat(c) << 16 | (uint32_t)f32_to_e5m2_rne_sat(d) << 24;
    return (uint32_t)f32_to_e4m3_rne_sat(a) | (uint32_t)f32_to_e4m3_rne_sat(b) << 8 |
           (uint32_t)f32_to_e4m3_rne_sat(c) << 16 | (uint32_t)f32_to_e4m3_rne_sat(d) << 24;
  }
  constexpr float kMax = E5M2 ? 57344.0f : 448.0f;
  a = fminf(fmaxf(a, -kMax), kMax);
  b = fminf(fmaxf(b, -kMax), kMax);
  c = fminf(fmaxf(c, -kMax), kMax);
  d = fminf(fmaxf(d, -kMax), kMax);
  int w;
  if (E5M2) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// ------------------------------------------------------------ activations
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_ERF = 2, ACT_GELU_TANH = 3, ACT_SILU = 4 };

// Elementary functions of the epilogues on the hardware transcendental
// units (v_exp_f32 = 2^x, v_rcp_f32 = 1/x, each within about one ulp):
// exp(x) = 2^(x log2 e) and a / b = a * (1 / b), a few instructions where
// the library's correctly rounded forms take dozens per element.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Standard normal tail Q(z) = P(Z > z) = erfc(z / sqrt 2) / 2 for z >= 0, and
// exp(-z^2 / 2) beside it, with erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 +
// t a5)))) exp(-x^2), t = 1 / (1 + p x): Hastings' approximation as given
// by Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26
// (absolute error below 1.5e-7 for x >= 0).  Q carries that absolute
// error, so Phi(z) = 1 - Q(z) (z >= 0) and Phi(z) = Q(-z) (z < 0) are
// accurate to about 2e-7 absolute, GeLU(z) = z Phi(z) to 3e-6 relative for
// z >= -2 and 2.2e-7 absolute below.
__device__ __forceinline__ float normal_tail(float az, float& e) {
  const float x = az * 0.70710678118654752f;
  const float t = fast_rcp(1.f + 0.3275911f * x);
  e = fast_exp(-x * x);
  const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f +
                                                                                 t * 1.061405429f))));
  return 0.5f * poly * e;
}

// Activation and its derivative with the activation fixed at compile time,
// so that element loops carry no per-element dispatch; act_fwd / act_grad
// take it at run time.
template <int ACT>
__device__ inline float act_fwd_c(float z) {
  if constexpr (ACT == ACT_RELU) {
    return z > 0.f ? z : 0.f;
  } else if constexpr (ACT == ACT_GELU_ERF) {
    // z * Phi(z), Phi from the normal tail: no cancellation in 1 + erf(.)
    // for negative z, where the product is small
    float e;
    const float q = normal_tail(fabsf(z), e);
    return z * (z >= 0.f ? 1.f - q : q);
  } else if constexpr (ACT == ACT_GELU_TANH) {
    // 0.5 z (1 + tanh u) = z / (1 + exp(-2u)), free of the same cancellation
    float u = 0.79788456080286536f * (z + 0.044715f * z * z * z);
    return z * fast_rcp(1.f + fast_exp(-2.f * u));
  } else if constexpr (ACT == ACT_SILU) {
    return z * fast_rcp(1.f + fast_exp(-z));  // z sigma(z); -0 once exp overflows
  } else {
    return z;
  }
}

template <int ACT>
__device__ inline float act_grad_c(float z) {
  if constexpr (ACT == ACT_RELU) {
    return z > 0.f ? 1.f : 0.f;
  } else if constexpr (ACT == ACT_GELU_ERF) {
    // Phi(z) + z phi(z), phi(z) = exp(-z^2 / 2) / sqrt(2 pi)
    float e;
    const float q = normal_tail(fabsf(z), e);
    const float cdf = z >= 0.f ? 1.f - q : q;
    return cdf + z * (e * 0.39894228040143268f);
  } else if constexpr (ACT == ACT_GELU_TANH) {
    // with s = (1 + tanh u) / 2 = sigma(2u): d/dz = s + 2 z s (1 - s) du/dz,
    // 1 - s = sigma(-2u) taken directly (no inf * 0 once exp(-2u) overflows)
    float u = 0.79788456080286536f * (z + 0.044715f * z * z * z);
    float sg = fast_rcp(1.f + fast_exp(-2.f * u));
    float sn = fast_rcp(1.f + fast_exp(2.f * u));
    float du = 0.79788456080286536f * (1.f + 3.f * 0.044715f * z * z);
    return sg + 2.f * z * sg * sn * du;
  } else if constexpr (ACT == ACT_SILU) {
    // sigma(z) (1 + z sigma(-z)), both logistic values taken directly so
    // that neither 1 - sigma nor inf * 0 appears at large |z|
    const float sp = fast_rcp(1.f + fast_exp(-z)), sn = fast_rcp(1.f + fast_exp(z));
    return sp * (1.f + z * sn);
  } else {
    return 1.f;
  }
}

__device__ inline float act_fwd(float z, int act) {
  switch (act) {
    case ACT_RELU: return act_fwd_c<ACT_RELU>(z);
    case ACT_GELU_ERF: return act_fwd_c<ACT_GELU_ERF>(z);
    case ACT_GELU_TANH: return act_fwd_c<ACT_GELU_TANH>(z);
    case ACT_SILU: return act_fwd_c<ACT_SILU>(z);
    default: return z;
  }
}

__device__ inline float act_grad(float z, int act) {
  switch (act) {
    case ACT_RELU: return act_grad_c<ACT_RELU>(z);
    case ACT_GELU_ERF: return act_grad_c<ACT_GELU_ERF>(z);
    case ACT_GELU_TANH: return act_grad_c<ACT_GELU_TANH>(z);
    case ACT_SILU: return act_grad_c<ACT_SILU>(z);
    default: return 1.f;
  }
}

// Calls f(std::integral_constant-like tag) with the activation as a
// compile-time value: one branch per epilogue pass instead of per element.
template <int N>
struct ActTag {
  static constexpr int value = N;
};
template <class F>
__device__ __forceinline__ void with_act(int act, F&& f) {
  switch (act) {
    case ACT_RELU: f(ActTag<ACT_RELU>{}); break;
    case ACT_GELU_ERF: f(ActTag<ACT_GELU_ERF>{}); break;
    case ACT_GELU_TANH: f(ActTag<ACT_GELU_TANH>{}); break;
    case ACT_SILU: f(ActTag<ACT_SILU>{}); break;
    default: f(ActTag<ACT_NONE>{}); break;
  }
}

}  // namespace tpm
