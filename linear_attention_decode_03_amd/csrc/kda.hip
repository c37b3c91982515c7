// KDA decode / verify step for MI355X (gfx950, CDNA4): kernels and C ABI.
//
// Operation: the KdaWide step of the vLLM API page
// vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide (class
// docstring, constructor, kernel body, helpers silu / decay); the argument
// contract is in include/kda.h.
//
// Design (one workgroup of 4 wave64s per (request, head) item):
//  * The item's 128x128 FP32 state page (64 KiB) lives in VGPRs for every
//    token of the step: thread (wave w, lane l) owns value rows
//    32w + 4i + (l >> 4), i < 8, and keys 4(l & 15) + [0, 4) and
//    64 + 4(l & 15) + [0, 4): 64 floats.  Each 16-byte load or store of a
//    wave covers four 256-byte row segments, so every HBM line is used whole.
//    The loads are issued first and land while the inputs are prepared.
//  * A row's 128 keys sit in one 16-lane DPP row, so the two row reductions
//    per token (S.k and S.q) are four DPP adds each, with no LDS traffic.
//  * The BF16 rounding points that feed the state (SiLU outputs and the raw
//    gate) are computed so that they are the correctly rounded values of the
//    page's FP32 operations: the SiLU's exp is evaluated in FP64 and rounded
//    once, and the gate projection (products of BF16 values, exact in FP64)
//    is accumulated in FP64 and rounded once.  Only the recurrence's dot
//    products keep an FP32 reduction order of their own.
//  * Items are numbered head-fastest; with H a multiple of 8 the
//    round-robin dispatch over the 8 XCDs sends every head to one XCD, so
//    each XCD's L2 keeps only its heads' 32 KiB F_B blocks.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "kda.h"

namespace {

constexpr int kD = 128;         // head dimension
constexpr int kThreads = 256;   // 4 wave64s
constexpr int kMaxT = 8;

struct Args {
  const uint16_t* x;
  const uint16_t* conv_w;
  const uint16_t* conv_b;
  uint16_t* conv_state;
  const uint16_t* f_a;
  const uint16_t* beta;
  const float* a_log;
  const float* dt_bias;
  const int32_t* slots;
  float* state;
  uint16_t* out;
  const uint16_t* gate;
  const uint16_t* norm_w;
  const uint16_t* f_b;
  const int32_t* accepted;
  float* rec_u;
  uint16_t* rec_kg;
  float lower_bound, scale, eps;
  int B, H, N, W, slot_stride;
};

// ---- BF16 storage --------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                  // nearest even
  return u >> 16;
}

__device__ __forceinline__ float round_bf16(float f) {
  return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

// ---- the page's helpers --------------------------------------------------

// SiLU x / (1 + exp(-x)) as FP32 operations, stored BF16.  exp is evaluated in
// FP64 and rounded once, which gives the correctly rounded FP32 exp; the add
// and the divide are IEEE FP32 operations.
__device__ __forceinline__ float silu_bf16(float x) {
  const float e = static_cast<float>(exp(-static_cast<double>(x)));
  const float d = 1.0f + e;
  return round_bf16(x / d);
}

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

// exp(lower_bound * sigmoid(exp(A_log) * (raw_g + dt_bias))); e = exp(A_log).
__device__ __forceinline__ float decay_f32(float e, float raw_g, float dt, float lower_bound) {
  const float y = e * (raw_g + dt);
  return expf(lower_bound * sigmoid_f32(y));
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

// ---- state pages through buffer resources ---------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ void store_f4(__amdgpu_buffer_rsrc_t r, int voff, int soff, float4 f) {
  u32x4 v;
  v.x = __float_as_uint(f.x); v.y = __float_as_uint(f.y);
  v.z = __float_as_uint(f.z); v.w = __float_as_uint(f.w);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kStream);
}

// ---- the step kernel -----------------------------------------------------

template <int T, bool kRecord, bool kBias>
__global__ __launch_bounds__(kThreads) void kda_step_kernel(const Args A) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int H = A.H;
  const int item = blockIdx.x;
  const int h = item % H;
  const int b = item / H;
  const int dim = H * kD;
  const size_t token0 = static_cast<size_t>(b) * T;

  // Slot resolution (uniform over the workgroup).
  int rs, cs, off = 0;
  bool live;
  if constexpr (T == 1) {
    rs = A.slots[b];
    cs = rs;
    live = rs > 0 && rs < A.N;
  } else {
    const int acc = A.accepted[b];
    const int lim = T < A.slot_stride ? T : A.slot_stride;
    live = acc >= 1 && acc <= lim;
    rs = 0;
    cs = 0;
    if (live) {
      off = acc - 1;
      rs = A.slots[static_cast<size_t>(b) * A.slot_stride + off];
      cs = A.slots[static_cast<size_t>(b) * A.slot_stride];
      live = rs > 0 && rs < A.N && cs >= 0 && cs < A.N;
    }
  }
  if (!live) {  // padding: BF16 zeros, nothing else touched
    if (tid < kD) {
#pragma unroll
      for (int t = 0; t < T; ++t) A.out[(token0 + t) * dim + static_cast<size_t>(h) * kD + tid] = 0;
    }
    return;
  }

  __shared__ float sh_q[T][kD], sh_k[T][kD], sh_v[T][kD], sh_a[T][kD], sh_o[T][kD];
  __shared__ float sh_g[T][kD];      // FP32 gate projection before BF16 rounding
  __shared__ float sh_beta[kMaxT];
  __shared__ float sh_sq[T][2][2];  // [token][q, k][wave 0, 1]
  __shared__ float sh_os[T][2];     // [token][wave 0, 1]

  // 1. State page into registers: one buffer resource per 64 KiB page, a
  //    per-lane byte offset in one VGPR and the (i, j) offsets as immediates.
  //    Thread (wave w, lane l) owns rows 32(l >> 4) + 8w + i, i < 8: every
  //    16-byte access of a wave covers four 256-byte row segments 16 KiB
  //    apart, which spreads each instruction over more HBM channels.
  const int c16 = lane & 15;
  const int row0 = 32 * (lane >> 4) + 8 * wave;
  const int lane_off = (row0 * kD + 4 * c16) * 4;
  float4 st[8][2];
  {
    const __amdgpu_buffer_rsrc_t page = page_rsrc(A.state, rs, h, H);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) st[i][j] = load_f4(page, lane_off, i * kD * 4 + j * 256);
  }

  // 2. Convolution + SiLU.  Threads 0-127 make q and k of channel tid,
  //    threads 128-255 make v of channel tid - 128.
  {
    const int c = tid & (kD - 1);
    const int nparts = tid < kD ? 2 : 1;
    for (int s = 0; s < nparts; ++s) {
      const int part = tid < kD ? s : 2;
      const size_t ch = static_cast<size_t>(part) * dim + static_cast<size_t>(h) * kD + c;
      uint16_t* col = A.conv_state + (static_cast<size_t>(cs) * 3 * dim + ch) * A.W;
      float win[3 + T];
      uint16_t raw[3 + T];
#pragma unroll
      for (int i = 0; i < 3; ++i) raw[i] = col[off + i];
#pragma unroll
      for (int t = 0; t < T; ++t) raw[3 + t] = A.x[(token0 + t) * 3 * dim + ch];
#pragma unroll
      for (int i = 0; i < 3 + T; ++i) win[i] = bf16_bits_to_f32(raw[i]);
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = bf16_bits_to_f32(A.conv_w[(static_cast<size_t>(part) * 4 + i) * dim +
                                         static_cast<size_t>(h) * kD + c]);
      const float bias = kBias ? bf16_bits_to_f32(A.conv_b[ch]) : 0.0f;
      // The window is read above; rewrite it in place: [tap1, tap2, x_0 ..].
      col[0] = raw[1];
      col[1] = raw[2];
#pragma unroll
      for (int t = 0; t < T; ++t) col[2 + t] = raw[3 + t];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float acc = bias;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(win[t + i], w[i], acc);
        const float y = silu_bf16(acc);
        if (part == 0) sh_q[t][c] = y;
        if (part == 1) {
          sh_k[t][c] = y;
          if constexpr (kRecord)
            A.rec_kg[((static_cast<size_t>(b) * H + h) * T + t) * (2 * kD) + c] =
                static_cast<uint16_t>(f32_to_bf16_bits(y));
        }
        if (part == 2) sh_v[t][c] = y;
      }
    }
  }
  // Sums of squares of q and k (waves 0 and 1 hold channels 0-63, 64-127).
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float q = sh_q[t][tid], k = sh_k[t][tid];
      const float sq = wave_sum(q * q), sk = wave_sum(k * k);
      if (lane == 0) {
        sh_sq[t][0][wave] = sq;
        sh_sq[t][1][wave] = sk;
      }
    }
  }
  if (tid < T)
    sh_beta[tid] = sigmoid_f32(bf16_bits_to_f32(A.beta[(token0 + tid) * H + h]));

  // 3. Gate projection raw_g[t][f] = BF16(sum_j F_B[h*128+f][j] f_a[t][j]),
  //    exact in FP64.  Thread holds features 16i + (tid >> 4) and columns
  //    8(tid & 15) .. +7, so every 16-byte load of the workgroup is
  //    contiguous; the 16 partial sums of a feature sit in one 16-lane row.
  {
    const int fsub = tid >> 4;
    const int j0 = 8 * (tid & 15);
    // Feature groups of G: all eight loads at once for decode; pairs for
    // verify, where the state page occupies the registers longer.
    constexpr int G = T == 1 ? 8 : 2;
#pragma unroll 1
    for (int i0 = 0; i0 < 8; i0 += G) {
      uint4 fb[G];
#pragma unroll
      for (int g = 0; g < G; ++g)
        fb[g] = *reinterpret_cast<const uint4*>(
            A.f_b + (static_cast<size_t>(h) * kD + 16 * (i0 + g) + fsub) * kD + j0);
#pragma unroll 1
      for (int t = 0; t < T; ++t) {
        const uint4 fa4 = *reinterpret_cast<const uint4*>(A.f_a + (token0 + t) * kD + j0);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          // A product of two BF16 values is exact in FP32; the sum is kept in FP64.
          double acc = static_cast<double>(bf16_lo(fb[g].x) * bf16_lo(fa4.x));
          acc += static_cast<double>(bf16_hi(fb[g].x) * bf16_hi(fa4.x));
          acc += static_cast<double>(bf16_lo(fb[g].y) * bf16_lo(fa4.y));
          acc += static_cast<double>(bf16_hi(fb[g].y) * bf16_hi(fa4.y));
          acc += static_cast<double>(bf16_lo(fb[g].z) * bf16_lo(fa4.z));
          acc += static_cast<double>(bf16_hi(fb[g].z) * bf16_hi(fa4.z));
          acc += static_cast<double>(bf16_lo(fb[g].w) * bf16_lo(fa4.w));
          acc += static_cast<double>(bf16_hi(fb[g].w) * bf16_hi(fa4.w));
          acc = row_sum16_f64(acc);
          if ((tid & 15) == 0) sh_g[t][16 * (i0 + g) + fsub] = static_cast<float>(acc);
        }
      }
    }
  }
  __syncthreads();
  // Raw gate to BF16, then the decay of key channel f = tid (threads 0-127).
  if (tid < kD) {
    const float e = expf(A.a_log[h]);
    const float dt = A.dt_bias[static_cast<size_t>(h) * kD + tid];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float raw_g = round_bf16(sh_g[t][tid]);
      sh_a[t][tid] = decay_f32(e, raw_g, dt, A.lower_bound);
      if constexpr (kRecord)
        A.rec_kg[((static_cast<size_t>(b) * H + h) * T + t) * (2 * kD) + kD + tid] =
            static_cast<uint16_t>(f32_to_bf16_bits(raw_g));
    }
  }
  __syncthreads();

  // 4. The recurrence, token by token.
#pragma unroll 1
  for (int t = 0; t < T; ++t) {
    const float fq = 1.0f / sqrtf((sh_sq[t][0][0] + sh_sq[t][0][1]) + 1.0e-6f);
    const float fk = 1.0f / sqrtf((sh_sq[t][1][0] + sh_sq[t][1][1]) + 1.0e-6f);
    float kh[8], qh[8], a[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 k4 = *reinterpret_cast<const float4*>(&sh_k[t][64 * j + 4 * c16]);
      const float4 q4 = *reinterpret_cast<const float4*>(&sh_q[t][64 * j + 4 * c16]);
      const float4 a4 = *reinterpret_cast<const float4*>(&sh_a[t][64 * j + 4 * c16]);
      kh[4 * j + 0] = k4.x * fk; kh[4 * j + 1] = k4.y * fk;
      kh[4 * j + 2] = k4.z * fk; kh[4 * j + 3] = k4.w * fk;
      qh[4 * j + 0] = (q4.x * fq) * A.scale; qh[4 * j + 1] = (q4.y * fq) * A.scale;
      qh[4 * j + 2] = (q4.z * fq) * A.scale; qh[4 * j + 3] = (q4.w * fq) * A.scale;
      a[4 * j + 0] = a4.x; a[4 * j + 1] = a4.y; a[4 * j + 2] = a4.z; a[4 * j + 3] = a4.w;
    }
    const float beta = sh_beta[t];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float* s = reinterpret_cast<float*>(&st[i][0]);  // 8 contiguous floats
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[e] = s[e] * a[e];
        dot = fmaf(s[e], kh[e], dot);
      }
      dot = row_sum16(dot);
      const int v = row0 + i;
      const float u = (sh_v[t][v] - dot) * beta;
      float o = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[e] = fmaf(kh[e], u, s[e]);
        o = fmaf(s[e], qh[e], o);
      }
      o = row_sum16(o);
      if (c16 == 0) {
        sh_o[t][v] = round_bf16(o);
        if constexpr (kRecord)
          A.rec_u[((static_cast<size_t>(b) * H + h) * T + t) * kD + v] = u;
      }
    }
    if constexpr (!kRecord) {
      const int target = T == 1 ? rs : A.slots[static_cast<size_t>(b) * A.slot_stride + t];
      if (target > 0 && target < A.N) {
        const __amdgpu_buffer_rsrc_t page = page_rsrc(A.state, target, h, H);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) store_f4(page, lane_off, i * kD * 4 + j * 256, st[i][j]);
      }
    }
  }
  __syncthreads();

  // 5. Gated RMSNorm: threads 0-127, channel tid.
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float o = sh_o[t][tid];
      const float ss = wave_sum(o * o);
      if (lane == 0) sh_os[t][wave] = ss;
    }
  }
  __syncthreads();
  if (wave < 2) {
    const float nw = bf16_bits_to_f32(A.norm_w[tid]);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float variance = (sh_os[t][0] + sh_os[t][1]) * (1.0f / 128.0f) + A.eps;
      const float rstd = 1.0f / sqrtf(variance);
      const size_t idx = (token0 + t) * dim + static_cast<size_t>(h) * kD + tid;
      const float sg = sigmoid_f32(bf16_bits_to_f32(A.gate[idx]));
      A.out[idx] = static_cast<uint16_t>(f32_to_bf16_bits(((sh_o[t][tid] * rstd) * nw) * sg));
    }
  }
}

// ---- host side -------------------------------------------------------------

kda_status check(const Args& A, int T, int record, int gate_mode) {
  if (T < 1 || T > kMaxT) return KDA_ERR_TOKENS;
  if (gate_mode != 0 && gate_mode != 1) return KDA_ERR_GATE_MODE;
  if (record && T == 1) return KDA_ERR_RECORD_T1;
  if (A.B < 0 || A.H < 1 || A.N < 1) return KDA_ERR_SHAPE;
  if (A.W < (T == 1 ? 3 : T + 2)) return KDA_ERR_SHAPE;
  if (T > 1 && A.slot_stride < T) return KDA_ERR_SHAPE;
  if (!isfinite(A.lower_bound) || !isfinite(A.scale) || !isfinite(A.eps)) return KDA_ERR_SHAPE;
  // Grid and 32-bit index limits: B*H workgroups; H*128 channels per row.
  if (static_cast<long long>(A.B) * A.H > 0x7fffffffLL) return KDA_ERR_SHAPE;
  if (static_cast<long long>(A.H) * 3 * kD * (T + 3) > 0x7fffffffLL) return KDA_ERR_SHAPE;
  if (A.B == 0) return KDA_OK;
  if (!A.x || !A.conv_w || !A.conv_state || !A.f_a || !A.beta || !A.a_log || !A.dt_bias ||
      !A.slots || !A.state || !A.out || !A.gate || !A.norm_w || !A.f_b)
    return KDA_ERR_NULL;
  if (T > 1 && !A.accepted) return KDA_ERR_NULL;
  if (record && (!A.rec_u || !A.rec_kg)) return KDA_ERR_NULL;
  return KDA_OK;
}

template <int T, bool kRecord>
kda_status launch_t(const Args& A, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(A.B * A.H));
  const dim3 block(kThreads);
  if (A.conv_b)
    hipLaunchKernelGGL((kda_step_kernel<T, kRecord, true>), grid, block, 0, stream, A);
  else
    hipLaunchKernelGGL((kda_step_kernel<T, kRecord, false>), grid, block, 0, stream, A);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

template <bool kRecord>
kda_status launch(const Args& A, int T, hipStream_t stream) {
  switch (T) {
    case 1: if constexpr (!kRecord) return launch_t<1, false>(A, stream); else return KDA_ERR_RECORD_T1;
    case 2: return launch_t<2, kRecord>(A, stream);
    case 3: return launch_t<3, kRecord>(A, stream);
    case 4: return launch_t<4, kRecord>(A, stream);
    case 5: return launch_t<5, kRecord>(A, stream);
    case 6: return launch_t<6, kRecord>(A, stream);
    case 7: return launch_t<7, kRecord>(A, stream);
    case 8: return launch_t<8, kRecord>(A, stream);
    default: return KDA_ERR_TOKENS;
  }
}

Args pack(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
          uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta, const float* a_log,
          const float* dt_bias, const int32_t* slots, float* state, uint16_t* out,
          const uint16_t* gate, const uint16_t* norm_w, float lower_bound, float scale,
          float eps, const uint16_t* f_b, const int32_t* accepted, float* rec_u,
          uint16_t* rec_kg, int B, int H, int N, int W, int slot_stride) {
  Args A;
  A.x = x; A.conv_w = conv_w; A.conv_b = conv_b; A.conv_state = conv_state; A.f_a = f_a;
  A.beta = beta; A.a_log = a_log; A.dt_bias = dt_bias; A.slots = slots; A.state = state;
  A.out = out; A.gate = gate; A.norm_w = norm_w; A.f_b = f_b; A.accepted = accepted;
  A.rec_u = rec_u; A.rec_kg = rec_kg;
  A.lower_bound = lower_bound; A.scale = scale; A.eps = eps;
  A.B = B; A.H = H; A.N = N; A.W = W; A.slot_stride = slot_stride;
  return A;
}

}  // namespace

extern "C" {

kda_status kda_validate(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                        uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                        const float* a_log, const float* dt_bias, const int32_t* slots,
                        float* state, uint16_t* out, const uint16_t* gate,
                        const uint16_t* norm_w, float lower_bound, float scale, float eps,
                        const uint16_t* f_b, const int32_t* accepted, float* rec_u,
                        uint16_t* rec_kg, int B, int H, int N, int W, int T, int slot_stride,
                        int record, int gate_mode) {
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, accepted, rec_u, rec_kg,
                      B, H, N, W, T == 1 ? 1 : slot_stride);
  return check(A, T, record, gate_mode);
}

kda_status kda_decode(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                      uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                      const float* a_log, const float* dt_bias, const int32_t* slots,
                      float* state, uint16_t* out, const uint16_t* gate,
                      const uint16_t* norm_w, float lower_bound, float scale, float eps,
                      const uint16_t* f_b, int B, int H, int N, int W, int gate_mode, int ahead,
                      void* stream) {
  (void)ahead;
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, nullptr, nullptr,
                      nullptr, B, H, N, W, 1);
  const kda_status s = check(A, 1, 0, gate_mode);
  if (s != KDA_OK || B == 0) return s;
  return launch<false>(A, 1, static_cast<hipStream_t>(stream));
}

kda_status kda_verify(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                      uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                      const float* a_log, const float* dt_bias, const int32_t* slots,
                      float* state, uint16_t* out, const uint16_t* gate,
                      const uint16_t* norm_w, float lower_bound, float scale, float eps,
                      const uint16_t* f_b, const int32_t* accepted, float* rec_u,
                      uint16_t* rec_kg, int B, int H, int N, int W, int T, int slot_stride,
                      int record, int gate_mode, int ahead, void* stream) {
  (void)ahead;
  if (T == 1) return KDA_ERR_TOKENS;  // a one-token step is kda_decode
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, accepted, rec_u, rec_kg,
                      B, H, N, W, slot_stride);
  const kda_status s = check(A, T, record, gate_mode);
  if (s != KDA_OK || B == 0) return s;
  return record ? launch<true>(A, T, static_cast<hipStream_t>(stream))
                : launch<false>(A, T, static_cast<hipStream_t>(stream));
}

const char* kda_status_string(kda_status status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_TOKENS: return "tokens per request must be in [1, 8] (verify: [2, 8])";
    case KDA_ERR_GATE_MODE: return "gate_mode must be 0 or 1";
    case KDA_ERR_RECORD_T1: return "record mode needs more than one token";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "invalid sizes or scalars";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
