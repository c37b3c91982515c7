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
  int ahead;  // prefetch distance in items (0: off), a multiple of 8
};

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

// SiLU x / (1 + exp(-x)) as three FP32 operations (exp rounded to FP32, then
// the add and the IEEE divide), stored BF16: the value the oracle defines.
// Fast path: exp from v_exp_f32 (2^(-x log2 e)).  Its result y_f differs from
// the value y_c of the exactly rounded steps by at most (1.5|x| + 10) FP32
// ulps (argument rounding |x| 1.3e-7 relative, v_exp_f32 within 4 ulps, three
// roundings), so when y_f is more than 2|x| + 16 ulps away from a BF16
// rounding midpoint both round to the same BF16 value.  Otherwise, and for
// |x| >= 80 (near exp over/underflow), the steps are redone with exp in FP64
// rounded once to FP32.
__device__ __forceinline__ float silu_bf16_exact(float x) {
  const float e = static_cast<float>(exp(-static_cast<double>(x)));
  const float d = 1.0f + e;
  return round_bf16(x / d);
}

__device__ __forceinline__ float silu_bf16(float x) {
  const float ax = fabsf(x);
  const float ef = __builtin_amdgcn_exp2f(x * -1.44269504088896341f);
  const float yf = x / (1.0f + ef);
  const uint32_t bits = __float_as_uint(yf);
  const int dist = abs(static_cast<int>(bits & 0xffffu) - 0x8000);
  const int margin = static_cast<int>(2.0f * fminf(ax, 80.0f)) + 16;
  if (ax < 80.0f && dist > margin) return round_bf16(yf);
  return silu_bf16_exact(x);
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

// ---- shared memory -----------------------------------------------------------

// Per-item tables.  q, k, a and g are dead once the inputs are reduced to
// what the body needs; the record-mode body reuses their space for P, C and o.
template <int T>
struct Inputs {
  float q[T][kD], k[T][kD], a[T][kD];
  float g[T][kD];  // FP32 gate projection before BF16 rounding
};
template <int T>
struct RecordOut {
  float P[16][kD];  // S0 W
  float C[16][16];  // W X^T
  float o[T][kD];
};
template <int T, bool kRecordBody>
struct Shared {
  union {
    Inputs<T> in;
    RecordOut<T> out;
  } u;
  float v[T][kD];
  float o[kRecordBody ? 1 : T][kD];  // token-by-token body's outputs
  float beta[kMaxT];
  float sq[T][2][2];  // [token][q, k][wave 0, 1]
  float os[T][2];     // [token][wave 0, 1]
};

// Record-mode operand tables: W rows A_t k_hat_t (t < T) and A_t q_hat_t
// (T + t), X rows k_hat_t / A_t; rows beyond are zero.
constexpr int kPad = kD + 4;  // W row pitch: the 16 rows read together fall in different banks
struct RecordTables {
  float W[16][kPad];
  float X[16][kD];
};

// ---- item resolution -----------------------------------------------------

struct Item {
  int b, h, rs, cs, off;
  size_t token0;
  int dim;
};

// Slot resolution (uniform over the workgroup); false means padding.
template <int T>
__device__ __forceinline__ bool resolve(const Args& A, Item& it) {
  const int H = A.H;
  it.h = blockIdx.x % H;
  it.b = blockIdx.x / H;
  it.dim = H * kD;
  it.token0 = static_cast<size_t>(it.b) * T;
  it.off = 0;
  if constexpr (T == 1) {
    it.rs = A.slots[it.b];
    it.cs = it.rs;
    return it.rs > 0 && it.rs < A.N;
  } else {
    const int acc = A.accepted[it.b];
    const int lim = T < A.slot_stride ? T : A.slot_stride;
    it.rs = 0;
    it.cs = 0;
    if (acc < 1 || acc > lim) return false;
    it.off = acc - 1;
    it.rs = A.slots[static_cast<size_t>(it.b) * A.slot_stride + it.off];
    it.cs = A.slots[static_cast<size_t>(it.b) * A.slot_stride];
    return it.rs > 0 && it.rs < A.N && it.cs >= 0 && it.cs < A.N;
  }
}

// Prefetch (the page's prefetch_next): touch every 128-byte line of the
// state page that item blockIdx + ahead will read, so that it is on its way
// into the L2 of the XCD that runs that item (workgroups go round-robin to
// the 8 XCDs; ahead is a multiple of 8) and into the memory-side cache.  Two
// 4-byte loads per thread with the default cache policy (so the lines are
// kept), issued after the item's own page loads so that the in-order
// retirement of loads does not hold up the input phase; the values are only
// kept alive by a test that is never true at run time.  Measured on MI355X
// this never pays: at 8 MiB of pages in flight per XCD against a 4 MB L2 the
// touched lines are mostly gone before use, so it adds reads (decode B=256:
// +5 % at ahead 256, +28 % at 1024); the default is off.
template <int T>
__device__ __forceinline__ void prefetch_page(const Args& A, float& sink) {
  sink = 0.0f;
  const int item = static_cast<int>(blockIdx.x) + A.ahead;
  if (A.ahead <= 0 || item >= static_cast<int>(gridDim.x)) return;
  const int b = item / A.H, h = item % A.H;
  int slot;
  if constexpr (T == 1) {
    slot = A.slots[b];
  } else {
    const int acc = A.accepted[b];
    const int lim = T < A.slot_stride ? T : A.slot_stride;
    if (acc < 1 || acc > lim) return;
    slot = A.slots[static_cast<size_t>(b) * A.slot_stride + acc - 1];
  }
  if (slot <= 0 || slot >= A.N) return;
  const float* page = A.state + (static_cast<size_t>(slot) * A.H + h) * (kD * kD);
  const int line = 64 * static_cast<int>(threadIdx.x);  // floats: 256 B per thread
  sink = page[line] + page[line + 32];
}

__device__ __forceinline__ void keep_alive(const Args& A, float sink) {
  if (A.B < 0 && sink == 0.0f) A.out[0] = 0;  // B < 0 never reaches a kernel
}

template <int T>
__device__ __forceinline__ void write_padding(const Args& A, const Item& it) {
  const int tid = threadIdx.x;
  if (tid < kD) {
#pragma unroll
    for (int t = 0; t < T; ++t)
      A.out[(it.token0 + t) * it.dim + static_cast<size_t>(it.h) * kD + tid] = 0;
  }
}

// Output-gate logits and norm weight of channel tid (threads 0-127), loaded
// at the start so that the last phase does not wait on memory.
template <int T>
struct OutputOperands {
  uint16_t gate[T];
  float nw;
};

template <int T>
__device__ __forceinline__ void load_output_operands(const Args& A, const Item& it,
                                                     OutputOperands<T>& oo) {
  const int tid = threadIdx.x;
  if (tid < kD) {
#pragma unroll
    for (int t = 0; t < T; ++t)
      oo.gate[t] = A.gate[(it.token0 + t) * it.dim + static_cast<size_t>(it.h) * kD + tid];
    oo.nw = bf16_bits_to_f32(A.norm_w[tid]);
  }
}

// ---- prologue: convolution, SiLU, norms, gate projection, decay -------------

// Convolution + SiLU.  Threads 0-127 make q and k of channel tid, threads
// 128-255 make v of channel tid - 128.  Split in two so that the operand
// loads can be issued before the state page: loads of a wave retire in issue
// order, so inputs loaded after the page could not be used before all of it
// has arrived.
template <int T>
struct ConvOperands {
  uint16_t raw[2][3 + T];  // [part slot][tap0, tap1, tap2, x_0 .. x_{T-1}]
  float w[2][4];
  float bias[2];
};

template <int T, bool kBias>
__device__ __forceinline__ void conv_load(const Args& A, const Item& it, ConvOperands<T>& co) {
  const int tid = threadIdx.x;
  const int c = tid & (kD - 1);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (s == 1 && tid >= kD) break;
    const int part = tid < kD ? s : 2;
    const size_t ch = static_cast<size_t>(part) * it.dim + static_cast<size_t>(it.h) * kD + c;
    const uint16_t* col = A.conv_state + (static_cast<size_t>(it.cs) * 3 * it.dim + ch) * A.W;
#pragma unroll
    for (int i = 0; i < 3; ++i) co.raw[s][i] = col[it.off + i];
#pragma unroll
    for (int t = 0; t < T; ++t) co.raw[s][3 + t] = A.x[(it.token0 + t) * 3 * it.dim + ch];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      co.w[s][i] = bf16_bits_to_f32(A.conv_w[(static_cast<size_t>(part) * 4 + i) * it.dim +
                                             static_cast<size_t>(it.h) * kD + c]);
    co.bias[s] = kBias ? bf16_bits_to_f32(A.conv_b[ch]) : 0.0f;
  }
}

// The window is rewritten in place after it was read: [tap1, tap2, x_0 ..];
// record mode stores k.
template <int T, bool kRecord, class SH>
__device__ __forceinline__ void conv_compute(const Args& A, const Item& it, SH& sh,
                                             const ConvOperands<T>& co) {
  const int tid = threadIdx.x;
  const int c = tid & (kD - 1);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (s == 1 && tid >= kD) break;
    const int part = tid < kD ? s : 2;
    const size_t ch = static_cast<size_t>(part) * it.dim + static_cast<size_t>(it.h) * kD + c;
    uint16_t* col = A.conv_state + (static_cast<size_t>(it.cs) * 3 * it.dim + ch) * A.W;
    col[0] = co.raw[s][1];
    col[1] = co.raw[s][2];
#pragma unroll
    for (int t = 0; t < T; ++t) col[2 + t] = co.raw[s][3 + t];
    float* dst = part == 0 ? &sh.u.in.q[0][0] : part == 1 ? &sh.u.in.k[0][0] : &sh.v[0][0];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float acc = co.bias[s];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(bf16_bits_to_f32(co.raw[s][t + i]), co.w[s][i], acc);
      const float y = silu_bf16(acc);
      dst[t * kD + c] = y;
      if constexpr (kRecord) {
        if (part == 1)
          A.rec_kg[((static_cast<size_t>(it.b) * A.H + it.h) * T + t) * (2 * kD) + c] =
              static_cast<uint16_t>(f32_to_bf16_bits(y));
      }
    }
  }
}

template <int T, bool kRecord, bool kBias, class SH>
__device__ __forceinline__ void conv_silu(const Args& A, const Item& it, SH& sh) {
  ConvOperands<T> co;
  conv_load<T, kBias>(A, it, co);
  conv_compute<T, kRecord>(A, it, sh, co);
}

// Sums of squares of q and k (waves 0 and 1 hold channels 0-63, 64-127) and
// beta = sigmoid(logit).
template <int T, class SH>
__device__ __forceinline__ void norms_beta(const Args& A, const Item& it, SH& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float q = sh.u.in.q[t][tid], k = sh.u.in.k[t][tid];
      const float sq = wave_sum(q * q), sk = wave_sum(k * k);
      if (lane == 0) {
        sh.sq[t][0][wave] = sq;
        sh.sq[t][1][wave] = sk;
      }
    }
  }
  if (tid < T)
    sh.beta[tid] = sigmoid_f32(bf16_bits_to_f32(A.beta[(it.token0 + tid) * A.H + it.h]));
}

// Gate projection raw_g[t][f] = BF16(sum_j F_B[h*128+f][j] f_a[t][j]), exact:
// the products of two BF16 values are exact and are summed in FP64.
// One token (decode): on the vector ALUs.  Thread holds features
// 16i + (tid >> 4) and columns 8(tid & 15) .. +7 (every 16-byte load of the
// workgroup contiguous); a feature's 16 partial sums sit in one 16-lane row.
struct GateOperands {
  uint4 fb[8];
  uint4 fa;
};

__device__ __forceinline__ void gate_load(const Args& A, const Item& it, GateOperands& go) {
  const int tid = threadIdx.x;
  const int fsub = tid >> 4;
  const int j0 = 8 * (tid & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    go.fb[i] = *reinterpret_cast<const uint4*>(
        A.f_b + (static_cast<size_t>(it.h) * kD + 16 * i + fsub) * kD + j0);
  go.fa = *reinterpret_cast<const uint4*>(A.f_a + it.token0 * kD + j0);
}

template <class SH>
__device__ __forceinline__ void gate_valu(const GateOperands& go, SH& sh) {
  const int tid = threadIdx.x;
  const int fsub = tid >> 4;
  const uint4 fa4 = go.fa;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 fb = go.fb[i];
    double acc = static_cast<double>(bf16_lo(fb.x) * bf16_lo(fa4.x));
    acc += static_cast<double>(bf16_hi(fb.x) * bf16_hi(fa4.x));
    acc += static_cast<double>(bf16_lo(fb.y) * bf16_lo(fa4.y));
    acc += static_cast<double>(bf16_hi(fb.y) * bf16_hi(fa4.y));
    acc += static_cast<double>(bf16_lo(fb.z) * bf16_lo(fa4.z));
    acc += static_cast<double>(bf16_hi(fb.z) * bf16_hi(fa4.z));
    acc += static_cast<double>(bf16_lo(fb.w) * bf16_lo(fa4.w));
    acc += static_cast<double>(bf16_hi(fb.w) * bf16_hi(fa4.w));
    acc = row_sum16_f64(acc);
    if ((tid & 15) == 0) sh.u.in.g[0][16 * i + fsub] = static_cast<float>(acc);
  }
}

// Several tokens: FP64 MFMA 16x16x4, D[feature][token] over K = 128 columns
// (tokens >= T are zero columns).  Wave w computes feature tiles 32w and
// 32w + 16.  Lane (g = l >> 4, c = l & 15) feeds A[c][g] = F_B[f0 + c][k] and
// B[g][c] = f_a[token c][k] with k = 32q + 8g + e at step (q, e): each lane's
// operands are 16-byte loads; the 128 columns are visited in that order.  D layout of this instruction: lane l,
// element r holds D[l/16 + 4r][l%16].
template <int T, class SH>
__device__ __forceinline__ void gate_mfma(const Args& A, const Item& it, SH& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
#pragma unroll 1
  for (int tile = 0; tile < 2; ++tile) {
    const int f0 = 32 * wave + 16 * tile;
    // Two independent accumulation chains (even and odd 32-column quarters);
    // the sums are exact in FP64, so the chain structure does not change a bit.
    f64x4 acc[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
#pragma unroll 1
    for (int q0 = 0; q0 < 4; q0 += 2) {
      uint4 fb[2], fa[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = q0 + j;
        fb[j] = *reinterpret_cast<const uint4*>(
            A.f_b + (static_cast<size_t>(it.h) * kD + f0 + c) * kD + 32 * q + 8 * g);
        fa[j] = make_uint4(0, 0, 0, 0);
        if (c < T)
          fa[j] = *reinterpret_cast<const uint4*>(A.f_a + (it.token0 + c) * kD + 32 * q + 8 * g);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(bf16_at(fb[j], e)),
                                                         static_cast<double>(bf16_at(fa[j], e)),
                                                         acc[j], 0, 0, 0);
    }
    if (c < T) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sh.u.in.g[c][f0 + g + 4 * r] = static_cast<float>(acc[0][r] + acc[1][r]);
    }
  }
}

// Raw gate to BF16, then the decay of key channel f = tid (threads 0-127);
// record mode stores raw_g.
template <int T, bool kRecord, class SH>
__device__ __forceinline__ void decay(const Args& A, const Item& it, SH& sh) {
  const int tid = threadIdx.x;
  if (tid < kD) {
    const float e = expf(A.a_log[it.h]);
    const float dt = A.dt_bias[static_cast<size_t>(it.h) * kD + tid];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float raw_g = round_bf16(sh.u.in.g[t][tid]);
      sh.u.in.a[t][tid] = decay_f32(e, raw_g, dt, A.lower_bound);
      if constexpr (kRecord)
        A.rec_kg[((static_cast<size_t>(it.b) * A.H + it.h) * T + t) * (2 * kD) + kD + tid] =
            static_cast<uint16_t>(f32_to_bf16_bits(raw_g));
    }
  }
}

template <int T, class SH>
__device__ __forceinline__ void norm_factors(const SH& sh, int t, float& fq, float& fk) {
  fq = 1.0f / sqrtf((sh.sq[t][0][0] + sh.sq[t][0][1]) + 1.0e-6f);
  fk = 1.0f / sqrtf((sh.sq[t][1][0] + sh.sq[t][1][1]) + 1.0e-6f);
}

// ---- epilogue: gated RMSNorm --------------------------------------------------

template <int T, class SH>
__device__ __forceinline__ void gated_rmsnorm(const Args& A, const Item& it, SH& sh,
                                              const float (*o)[kD],
                                              const OutputOperands<T>& oo) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float ot = o[t][tid];
      const float ss = wave_sum(ot * ot);
      if (lane == 0) sh.os[t][wave] = ss;
    }
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float variance = (sh.os[t][0] + sh.os[t][1]) * (1.0f / 128.0f) + A.eps;
      const float rstd = 1.0f / sqrtf(variance);
      const float sg = sigmoid_f32(bf16_bits_to_f32(oo.gate[t]));
      const size_t idx = (it.token0 + t) * it.dim + static_cast<size_t>(it.h) * kD + tid;
      A.out[idx] = static_cast<uint16_t>(f32_to_bf16_bits(((o[t][tid] * rstd) * oo.nw) * sg));
    }
  }
}

// ---- decode / verify: the recurrence token by token ------------------------

// Thread (wave w, lane l) owns rows 32(l >> 4) + 8w + i (i < 8) and keys
// 4(l & 15) + [0, 4) and 64 + 4(l & 15) + [0, 4): 64 floats in VGPRs.  Every
// 16-byte access of a wave covers four 256-byte row segments 16 KiB apart,
// which spreads each instruction over more HBM channels; a row's keys sit in
// one 16-lane DPP row.
template <int T, bool kRecord, bool kBias>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void kda_step_kernel(const Args A) {
  Item it;
  if (!resolve<T>(A, it)) {  // padding: BF16 zeros, nothing else touched
    write_padding<T>(A, it);
    return;
  }
  __shared__ Shared<T, false> sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15;
  const int row0 = 32 * (lane >> 4) + 8 * wave;
  const int lane_off = (row0 * kD + 4 * c16) * 4;

  // 1. Input operands first, then the state page (one buffer resource per
  //    64 KiB page): the inputs are used while the page is still arriving.
  ConvOperands<T> co;
  conv_load<T, kBias>(A, it, co);
  GateOperands go;
  if constexpr (T == 1) gate_load(A, it, go);
  OutputOperands<T> oo;
  float4 st[8][2];
  {
    const __amdgpu_buffer_rsrc_t page = page_rsrc(A.state, it.rs, it.h, A.H);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) st[i][j] = load_f4(page, lane_off, i * kD * 4 + j * 256);
  }
  float sink;
  prefetch_page<T>(A, sink);

  // 2. Inputs.
  conv_compute<T, kRecord>(A, it, sh, co);
  norms_beta<T>(A, it, sh);
  if constexpr (T == 1) gate_valu(go, sh); else gate_mfma<T>(A, it, sh);
  __syncthreads();
  decay<T, kRecord>(A, it, sh);
  __syncthreads();

  // 3. The recurrence, token by token.
#pragma unroll 1
  for (int t = 0; t < T; ++t) {
    float fq, fk;
    norm_factors<T>(sh, t, fq, fk);
    float kh[8], qh[8], a[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 k4 = *reinterpret_cast<const float4*>(&sh.u.in.k[t][64 * j + 4 * c16]);
      const float4 q4 = *reinterpret_cast<const float4*>(&sh.u.in.q[t][64 * j + 4 * c16]);
      const float4 a4 = *reinterpret_cast<const float4*>(&sh.u.in.a[t][64 * j + 4 * c16]);
      kh[4 * j + 0] = k4.x * fk; kh[4 * j + 1] = k4.y * fk;
      kh[4 * j + 2] = k4.z * fk; kh[4 * j + 3] = k4.w * fk;
      qh[4 * j + 0] = (q4.x * fq) * A.scale; qh[4 * j + 1] = (q4.y * fq) * A.scale;
      qh[4 * j + 2] = (q4.z * fq) * A.scale; qh[4 * j + 3] = (q4.w * fq) * A.scale;
      a[4 * j + 0] = a4.x; a[4 * j + 1] = a4.y; a[4 * j + 2] = a4.z; a[4 * j + 3] = a4.w;
    }
    const float beta = sh.beta[t];
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
      const float u = (sh.v[t][v] - dot) * beta;
      float o = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[e] = fmaf(kh[e], u, s[e]);
        o = fmaf(s[e], qh[e], o);
      }
      o = row_sum16(o);
      if (c16 == 0) {
        sh.o[t][v] = round_bf16(o);
        if constexpr (kRecord)
          A.rec_u[((static_cast<size_t>(it.b) * A.H + it.h) * T + t) * kD + v] = u;
      }
    }
    if constexpr (!kRecord) {
      const int target = T == 1 ? it.rs : A.slots[static_cast<size_t>(it.b) * A.slot_stride + t];
      if (target > 0 && target < A.N) {
        float* page = page_ptr(A.state, target, it.h, A.H);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) store_f4(page, lane_off + i * kD * 4 + j * 256, st[i][j]);
      }
    }
  }
  load_output_operands<T>(A, it, oo);
  __syncthreads();

  // 4. Gated RMSNorm.
  gated_rmsnorm<T>(A, it, sh, sh.o, oo);
  keep_alive(A, sink);
}

// ---- record mode (RecoverSSM verify): all tokens from one pass over S0 -------
//
// With no state to store, the outputs and records follow from the page read,
// S0, in closed form.  Let A_t be the running product of the decays
// a_1 ... a_t (per key).  Then S_t = diag(A_t) (S0 + sum_{s<=t} (k_s / A_s) u_s^T)
// and, per value row v,
//   u_t = beta_t (v_t - P[t] - sum_{s<t} C[t][s] u_s),
//   o_t = P[T + t] + sum_{s<=t} C[T + t][s] u_s,
// with W_t = A_t (.) k_t, W_{T+t} = A_t (.) q_t, X_s = k_s / A_s,
// P[m][v] = sum_key S0[v][key] W_m[key] and C[m][s] = W_m . X_s.
// P is a 128 x 128 x 2T contraction and C a 2T x T x 128 one: both run on
// FP32 MFMA 16x16x4; the state page is loaded straight into the B operand
// layout (lane (g, c) of wave w holds rows 32w + 16 tile + c, keys
// 16q + 4g + [0, 4)).  Used when |lower_bound| <= 10, so that every A_t and
// 1 / A_t stays a normal FP32 number (|log A_t| <= 80).
template <int T, bool kBias>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void kda_record_kernel(const Args A) {
  Item it;
  if (!resolve<T>(A, it)) {
    write_padding<T>(A, it);
    return;
  }
  __shared__ Shared<T, true> sh;
  __shared__ RecordTables rt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;

  // 1. S0 into the MFMA B-operand layout: [tile][q] = rows 32w + 16 tile + c,
  //    keys 16q + 4g .. +3 (each instruction: 16 rows x 64 contiguous bytes).
  float4 st[2][8];
  {
    const __amdgpu_buffer_rsrc_t page = page_rsrc(A.state, it.rs, it.h, A.H);
    const int voff = (32 * wave + c) * kD * 4 + 16 * g;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int q = 0; q < 8; ++q) st[tile][q] = load_f4(page, voff, tile * 16 * kD * 4 + 64 * q);
  }
  float sink;
  prefetch_page<T>(A, sink);

  // 2. Inputs.
  conv_silu<T, true, kBias>(A, it, sh);
  norms_beta<T>(A, it, sh);
  gate_mfma<T>(A, it, sh);
  __syncthreads();
  decay<T, true>(A, it, sh);
  __syncthreads();

  // 3. W and X (thread = key channel), zero rows beyond 2T and T.
  if (tid < kD) {
    const int key = tid;
    float acc = 1.0f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float fq, fk;
      norm_factors<T>(sh, t, fq, fk);
      acc = acc * sh.u.in.a[t][key];
      const float kh = sh.u.in.k[t][key] * fk;
      const float qh = (sh.u.in.q[t][key] * fq) * A.scale;
      rt.W[t][key] = acc * kh;
      rt.W[T + t][key] = acc * qh;
      rt.X[t][key] = kh / acc;
    }
#pragma unroll
    for (int m = 2 * T; m < 16; ++m) rt.W[m][key] = 0.0f;
#pragma unroll
    for (int m = T; m < 16; ++m) rt.X[m][key] = 0.0f;
  }
  __syncthreads();  // from here q, k, a and g are dead: P, C and o take their space
  OutputOperands<T> oo;
  load_output_operands<T>(A, it, oo);

  // 4. P = S0 W (two 16-row tiles per wave) and, on wave 0, C = W X^T.
  //    A operand lane (g, c): W[c][16q + 4g + e]; the K order is shared by
  //    both operands of each product.
  {
    f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 w4 = *reinterpret_cast<const float4*>(&rt.W[c][16 * q + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0 = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(st[0][q], e), p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(st[1][q], e), p1, 0, 0, 0);
      }
    }
    // D layout (f32 16x16x4): lane l, element r holds D[4(l/16) + r][l%16].
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sh.u.out.P[4 * g + r][32 * wave + c] = p0[r];
      sh.u.out.P[4 * g + r][32 * wave + 16 + c] = p1[r];
    }
    if (wave == 0) {
      f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 w4 = *reinterpret_cast<const float4*>(&rt.W[c][16 * q + 4 * g]);
        const float4 x4 = *reinterpret_cast<const float4*>(&rt.X[c][16 * q + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cc = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(x4, e), cc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.u.out.C[4 * g + r][c] = cc[r];
    }
  }
  __syncthreads();

  // 5. Per value row v = tid (threads 0-127): the triangular solve for u and o.
  if (tid < kD) {
    const int v = tid;
    float u[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float dot = sh.u.out.P[t][v];
#pragma unroll
      for (int s = 0; s < t; ++s) dot = fmaf(sh.u.out.C[t][s], u[s], dot);
      u[t] = (sh.v[t][v] - dot) * sh.beta[t];
      float o = sh.u.out.P[T + t][v];
#pragma unroll
      for (int s = 0; s <= t; ++s) o = fmaf(sh.u.out.C[T + t][s], u[s], o);
      sh.u.out.o[t][v] = round_bf16(o);
      A.rec_u[((static_cast<size_t>(it.b) * A.H + it.h) * T + t) * kD + v] = u[t];
    }
  }
  __syncthreads();

  // 6. Gated RMSNorm.
  gated_rmsnorm<T>(A, it, sh, sh.u.out.o, oo);
  keep_alive(A, sink);
}

// ---- RecoverSSM replay: checkpoint + records -> the state after n tokens ----
//
// After a record-mode verify, the state after the first n accepted tokens is
// rebuilt from the checkpoint page that verify read and its records, with
// the step's own operations per token: k_hat = k (sum k^2 + 1e-6)^-1/2 from
// the recorded key, a = decay(raw_g) per key, then s <- k_hat u_v + s a for
// every element (one multiply and one FMA).  Same thread layout, access
// shape and store form as the decode kernel.

struct ReplayArgs {
  const float* rec_u;
  const uint16_t* rec_kg;
  const float* a_log;
  const float* dt_bias;
  const int32_t* src;
  const int32_t* dst;
  const int32_t* n;
  float* state;
  float lower_bound;
  int B, H, N, T;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void kda_replay_kernel(const ReplayArgs R) {
  const int h = blockIdx.x % R.H, b = blockIdx.x / R.H;
  const int src = R.src[b], dst = R.dst[b], n = R.n[b];
  if (src <= 0 || src >= R.N || dst <= 0 || dst >= R.N || n < 0 || n > R.T) return;
  __shared__ float sh_k[kMaxT][kD], sh_a[kMaxT][kD], sh_u[kMaxT][kD];
  __shared__ float sh_sq[kMaxT][2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15;
  const int row0 = 32 * (lane >> 4) + 8 * wave;
  const int lane_off = (row0 * kD + 4 * c16) * 4;
  const size_t rec0 = (static_cast<size_t>(b) * R.H + h) * R.T;

  // 1. Records first (threads 0-127: k and raw_g of channel tid; 128-255: u
  //    of row tid - 128), then the checkpoint page.
  const int c = tid & (kD - 1);
  uint16_t kraw[kMaxT], graw[kMaxT];
  float uval[kMaxT];
#pragma unroll
  for (int t = 0; t < kMaxT; ++t) {
    if (t < n) {
      if (tid < kD) {
        kraw[t] = R.rec_kg[(rec0 + t) * (2 * kD) + c];
        graw[t] = R.rec_kg[(rec0 + t) * (2 * kD) + kD + c];
      } else {
        uval[t] = R.rec_u[(rec0 + t) * kD + c];
      }
    }
  }
  float4 st[8][2];
  {
    const __amdgpu_buffer_rsrc_t page = page_rsrc(R.state, src, h, R.H);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) st[i][j] = load_f4(page, lane_off, i * kD * 4 + j * 256);
  }

  // 2. k, decay and u tables; per-token sums of squares of k.
  if (tid < kD) {
    const float e = expf(R.a_log[h]);
    const float dt = R.dt_bias[static_cast<size_t>(h) * kD + c];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t < n) {
        const float k = bf16_bits_to_f32(kraw[t]);
        sh_k[t][c] = k;
        sh_a[t][c] = decay_f32(e, bf16_bits_to_f32(graw[t]), dt, R.lower_bound);
        const float sk = wave_sum(k * k);
        if (lane == 0) sh_sq[t][wave] = sk;
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < kMaxT; ++t)
      if (t < n) sh_u[t][c] = uval[t];
  }
  __syncthreads();

  // 3. Apply the n tokens.
#pragma unroll 1
  for (int t = 0; t < n; ++t) {
    const float fk = 1.0f / sqrtf((sh_sq[t][0] + sh_sq[t][1]) + 1.0e-6f);
    float kh[8], a[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 k4 = *reinterpret_cast<const float4*>(&sh_k[t][64 * j + 4 * c16]);
      const float4 a4 = *reinterpret_cast<const float4*>(&sh_a[t][64 * j + 4 * c16]);
      kh[4 * j + 0] = k4.x * fk; kh[4 * j + 1] = k4.y * fk;
      kh[4 * j + 2] = k4.z * fk; kh[4 * j + 3] = k4.w * fk;
      a[4 * j + 0] = a4.x; a[4 * j + 1] = a4.y; a[4 * j + 2] = a4.z; a[4 * j + 3] = a4.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float* s = reinterpret_cast<float*>(&st[i][0]);
      const float u = sh_u[t][row0 + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = fmaf(kh[e], u, s[e] * a[e]);
    }
  }

  // 4. The state after n tokens.
  float* page = page_ptr(R.state, dst, h, R.H);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) store_f4(page, lane_off + i * kD * 4 + j * 256, st[i][j]);
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

// Record mode takes the closed-form kernel when the running decay products
// stay normal FP32 numbers (|lower_bound| <= 10, at most 8 tokens: |log A_t| <= 80).
constexpr float kRecordBound = 10.0f;

template <int T, bool kRecord>
kda_status launch_t(const Args& A, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(A.B * A.H));
  const dim3 block(kThreads);
  const bool bias = A.conv_b != nullptr;
  if constexpr (kRecord && T > 1) {
    if (fabsf(A.lower_bound) <= kRecordBound) {
      if (bias)
        hipLaunchKernelGGL((kda_record_kernel<T, true>), grid, block, 0, stream, A);
      else
        hipLaunchKernelGGL((kda_record_kernel<T, false>), grid, block, 0, stream, A);
      return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
  }
  if (bias)
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

// The prefetch distance: -1 takes the library default (off: the step is at
// its measured HBM ceiling without it), other values are rounded up to a
// multiple of 8 so that the prefetching workgroup and the one that reads the
// page sit on the same XCD.
constexpr int kDefaultAhead = 0;

int resolve_ahead(int ahead) {
  if (ahead < 0) ahead = kDefaultAhead;
  return (ahead + 7) & ~7;
}

Args pack(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
          uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta, const float* a_log,
          const float* dt_bias, const int32_t* slots, float* state, uint16_t* out,
          const uint16_t* gate, const uint16_t* norm_w, float lower_bound, float scale,
          float eps, const uint16_t* f_b, const int32_t* accepted, float* rec_u,
          uint16_t* rec_kg, int B, int H, int N, int W, int slot_stride, int ahead) {
  Args A;
  A.x = x; A.conv_w = conv_w; A.conv_b = conv_b; A.conv_state = conv_state; A.f_a = f_a;
  A.beta = beta; A.a_log = a_log; A.dt_bias = dt_bias; A.slots = slots; A.state = state;
  A.out = out; A.gate = gate; A.norm_w = norm_w; A.f_b = f_b; A.accepted = accepted;
  A.rec_u = rec_u; A.rec_kg = rec_kg;
  A.lower_bound = lower_bound; A.scale = scale; A.eps = eps;
  A.B = B; A.H = H; A.N = N; A.W = W; A.slot_stride = slot_stride;
  A.ahead = resolve_ahead(ahead);
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
                      B, H, N, W, T == 1 ? 1 : slot_stride, 0);
  return check(A, T, record, gate_mode);
}

kda_status kda_decode(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                      uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                      const float* a_log, const float* dt_bias, const int32_t* slots,
                      float* state, uint16_t* out, const uint16_t* gate,
                      const uint16_t* norm_w, float lower_bound, float scale, float eps,
                      const uint16_t* f_b, int B, int H, int N, int W, int gate_mode, int ahead,
                      void* stream) {
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, nullptr, nullptr,
                      nullptr, B, H, N, W, 1, ahead);
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
  if (T == 1) return KDA_ERR_TOKENS;  // a one-token step is kda_decode
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, accepted, rec_u, rec_kg,
                      B, H, N, W, slot_stride, ahead);
  const kda_status s = check(A, T, record, gate_mode);
  if (s != KDA_OK || B == 0) return s;
  return record ? launch<true>(A, T, static_cast<hipStream_t>(stream))
                : launch<false>(A, T, static_cast<hipStream_t>(stream));
}

kda_status kda_replay(const float* rec_u, const uint16_t* rec_kg, const float* a_log,
                      const float* dt_bias, const int32_t* src_slots, const int32_t* dst_slots,
                      const int32_t* n_tokens, float* state, float lower_bound, int B, int H,
                      int N, int T, void* stream) {
  if (T < 1 || T > kMaxT) return KDA_ERR_TOKENS;
  if (B < 0 || H < 1 || N < 1 || !isfinite(lower_bound)) return KDA_ERR_SHAPE;
  if (static_cast<long long>(B) * H > 0x7fffffffLL) return KDA_ERR_SHAPE;
  if (B == 0) return KDA_OK;
  if (!rec_u || !rec_kg || !a_log || !dt_bias || !src_slots || !dst_slots || !n_tokens || !state)
    return KDA_ERR_NULL;
  ReplayArgs R;
  R.rec_u = rec_u; R.rec_kg = rec_kg; R.a_log = a_log; R.dt_bias = dt_bias;
  R.src = src_slots; R.dst = dst_slots; R.n = n_tokens; R.state = state;
  R.lower_bound = lower_bound; R.B = B; R.H = H; R.N = N; R.T = T;
  hipLaunchKernelGGL(kda_replay_kernel, dim3(static_cast<unsigned>(B * H)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), R);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
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
