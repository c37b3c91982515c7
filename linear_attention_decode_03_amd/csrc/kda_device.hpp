// Device helpers shared by the KDA kernels for MI355X (gfx950, CDNA4):
// BF16 storage, the page's scalar helpers (SiLU with its BF16 rounding,
// sigmoid, the gate decay), DPP row and wave reductions, and the state-page
// access forms (buffer loads through a per-page resource, non-temporal
// global stores).
//
// Operation: the helpers section and kernel body of the vLLM API page
// vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide.
#ifndef KDA_DEVICE_HPP
#define KDA_DEVICE_HPP

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

namespace {

constexpr int kD = 128;         // head dimension
constexpr int kThreads = 256;   // 4 wave64s
constexpr int kMaxT = 8;

// ---- BF16 storage --------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // nearest even
  const uint32_t quiet = (u >> 16) | 0x40u;                         // NaN stays NaN
  return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;
}

__device__ __forceinline__ float round_bf16(float f) {
  return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

// ---- the page's helpers --------------------------------------------------

// exp and sigmoid on the hardware exp2 (v_exp_f32, 1 ulp) and reciprocal
// (v_rcp_f32, 1 ulp): within |x|/2 + 2 FP32 ulps (exp; the argument's own
// rounding grows with |x|) or a few ulps (sigmoid) of the correctly rounded
// values.  Used where the result stays FP32 (beta, the decay, the output
// gate), whose rounding order is free; the exact special values hold:
// exp(0) = 1, sigmoid(+-large) = 1 or 0.
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp_fast(-x));
}

// SiLU x / (1 + exp(-x)) as three FP32 operations (exp rounded to FP32, then
// the add and the IEEE divide), stored BF16: the value the oracle defines.
// Fast path: exp from v_exp_f32 (2^(-x log2 e)) and the quotient as
// x * rcp(1 + e).  Its result y_f differs from the value y_c of the exactly
// rounded steps by at most (1.5|x| + 12) FP32 ulps (argument rounding
// 0.61|x| 2^-23 relative, v_exp_f32 and v_rcp_f32 within 4 and 1 ulps, the
// roundings of the add and the product; a relative error r is at most
// 2^24 r ulps of y), so when y_f is more than 2|x| + 16 ulps away from a
// BF16 rounding midpoint both round to the same BF16 value.  Otherwise, and
// for |x| >= 80 (near exp over/underflow), the steps are redone with exp in
// FP64 rounded once to FP32 and an IEEE divide.
__device__ __forceinline__ float silu_bf16_exact(float x) {
  const float e = static_cast<float>(exp(-static_cast<double>(x)));
  const float d = 1.0f + e;
  return round_bf16(x / d);
}

__device__ __forceinline__ float silu_bf16(float x) {
  const float ax = fabsf(x);
  const float ef = __builtin_amdgcn_exp2f(x * -1.44269504088896341f);
  const float yf = x * __builtin_amdgcn_rcpf(1.0f + ef);
  const uint32_t bits = __float_as_uint(yf);
  const int dist = abs(static_cast<int>(bits & 0xffffu) - 0x8000);
  // Both tests without a branch between them (the fast value is computed
  // for every x; v_exp_f32 and v_rcp_f32 take any argument).
  const bool fast = (ax < 80.0f) & (static_cast<float>(dist) > fmaf(2.0f, ax, 16.0f));
  // Fast: yf is finite and its low 16 bits are far from 0x8000, so rounding
  // to nearest is adding half a BF16 ulp and truncating (no tie, no NaN).
  if (fast) return __uint_as_float((bits + 0x8000u) & 0xffff0000u);
  return silu_bf16_exact(x);
}

// exp(lower_bound * sigmoid(exp(A_log) * (raw_g + dt_bias))); e = exp(A_log).
__device__ __forceinline__ float decay_f32(float e, float raw_g, float dt, float lower_bound) {
  const float y = e * (raw_g + dt);
  return exp_fast(lower_bound * sigmoid_fast(y));
}

// ---- cross-lane reductions -----------------------------------------------

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Sum over each 16-lane DPP row, result in every lane of the row:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xffffffffu), kCtrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), kCtrl, 0xf, 0xf, false);
  return __longlong_as_double(static_cast<long long>(
      (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo)));
}

// The same 16-lane row sum for FP64 values (each half moved by DPP).
__device__ __forceinline__ double row_sum16_f64(double v) {
  v += dpp_f64<0xb1>(v);
  v += dpp_f64<0x4e>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Element e (0-7) of eight BF16 values packed in a uint4, as a float.
__device__ __forceinline__ float bf16_at(const uint4& p, int e) {
  const uint32_t w = e < 2 ? p.x : e < 4 ? p.y : e < 6 ? p.z : p.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// ---- state pages through buffer resources ---------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kPageBytes = kD * kD * 4;      // one (slot, head) page: 64 KiB
constexpr int kRsrcWord3 = 0x00020000;       // gfx9 raw-buffer format word
constexpr int kStream = 2;                   // cache policy: non-temporal (nt)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(float* state, int slot, int h, int H) {
  float* page = state + (static_cast<size_t>(slot) * H + h) * (kD * kD);
  return __builtin_amdgcn_make_buffer_rsrc(page, static_cast<short>(0), kPageBytes, kRsrcWord3);
}

__device__ __forceinline__ float4 load_f4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStream);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// State stores go through a global pointer (uniform page base + per-lane byte
// offset), not a buffer resource.  A buffer store whose offset sits in an
// SGPR gets no wait state before a VALU write of its data registers, and on
// gfx950 such a write in the next cycle changes the stored data; the global
// form keeps that wait.
__device__ __forceinline__ float* page_ptr(float* state, int slot, int h, int H) {
  return state + (static_cast<size_t>(slot) * H + h) * (kD * kD);
}

__device__ __forceinline__ void store_f4(float* page, int byte_off, float4 f) {
  f32x4 v;
  v.x = f.x; v.y = f.y; v.z = f.z; v.w = f.w;
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(reinterpret_cast<char*>(page) + byte_off));
}

__device__ __forceinline__ float f4_at(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}
}  // namespace

#endif  // KDA_DEVICE_HPP
