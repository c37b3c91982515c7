// The stages of one KDA step item shared by the step kernels: operands,
// slot resolution and padding, the prologue (causal convolution + SiLU,
// L2 norms, beta, gate projection, decay) and the epilogue (gated RMSNorm).
//
// Operation: the KdaWide kernel body of the vLLM API page
// vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide; the
// argument contract is in include/kda.h.
#ifndef KDA_STAGES_HPP
#define KDA_STAGES_HPP

#include "kda_device.hpp"

namespace {

struct Args {
  const uint16_t* x;
  const uint16_t* conv_w;
  const uint16_t* conv_b;
  void* conv_state;  // BF16 bits, or FP32 when conv_f32
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
  int conv_f32;  // the convolution pool holds FP32 values
};

// ---- shared memory -----------------------------------------------------------

// Row pitch of the record tables: lanes (g, c) of an MFMA operand read row c
// at column 4g, and P is stored at rows 4g + r, column c; with 132 floats
// per row both patterns fall in distinct banks.
constexpr int kPad = kD + 4;
// Per-item tables.  q, k, a and g are dead once the inputs are reduced to
// what the body needs; the record-mode body reuses their space for P, C and
// o, and the space of g (dead after the decay) for its X table.
template <int T>
struct Inputs {
  float q[T][kD], k[T][kD], a[T][kD];
  float g[T][kPad];  // FP32 gate projection before BF16 rounding
};
template <int T>
struct RecordOut {
  float P[16][kPad];  // S0 W
  float C[16][16];    // W X^T
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
  float sq[T][2];     // [token][q, k]: sums of squares
  float os[T][2];     // [token][wave 0, 1]
};

// Record-mode operand table W: rows A_t k_hat_t (t < T) and A_t q_hat_t
// (T + t); rows beyond are zero.  (Its X rows, k_hat_t / A_t, live in the
// space of Inputs::g.)  Until W is written its space holds the item's f_a
// rows in FP64 for the gate projection.
struct alignas(16) RecordTables {
  float W[16][kPad];
};

// ---- item resolution -----------------------------------------------------

struct Item {
  int b, h, rs, cs, off;
  size_t token0;
  int dim;
};

// Verify: the request's slot row, slots[b, 0 .. T-1], read once.
template <int T>
struct SlotRow {
  int s[T];
};

// Entry t of the slot row (t uniform): a chain of selects, so the row stays
// in scalar registers (the readfirstlane keeps the compiler from turning the
// chain into an indexed table in scratch memory).
template <int T>
__device__ __forceinline__ int row_slot(const SlotRow<T>& row, int t) {
  int s = row.s[0];
#pragma unroll
  for (int u = 1; u < T; ++u) s = __builtin_amdgcn_readfirstlane(t == u ? row.s[u] : s);
  return s;
}

// Item `item` (head-fastest numbering: item = b * H + h) and its token rows.
template <int T>
__device__ __forceinline__ void locate_item(const Args& A, Item& it, int item) {
  const int H = A.H;
  it.h = item % H;
  it.b = item / H;
  it.dim = H * kD;
  it.token0 = static_cast<size_t>(it.b) * T;
  it.off = 0;
  it.rs = 0;
  it.cs = 0;
}

// The item of this workgroup.
template <int T>
__device__ __forceinline__ void locate(const Args& A, Item& it) {
  locate_item<T>(A, it, blockIdx.x);
}

// Slot resolution (uniform over the workgroup); false means padding.  Verify
// reads the request's slot row (T entries, slot_stride >= T) together with
// its accepted count, one round trip instead of two dependent ones, and
// selects the read slot from the row.
template <int T>
__device__ __forceinline__ bool resolve(const Args& A, Item& it, SlotRow<T>& slot_row) {
  if constexpr (T == 1) {
    it.rs = A.slots[it.b];
    it.cs = it.rs;
    return it.rs > 0 && it.rs < A.N;
  } else {
    const int acc = A.accepted[it.b];
    const int32_t* row = A.slots + static_cast<size_t>(it.b) * A.slot_stride;
#pragma unroll
    for (int t = 0; t < T; ++t) slot_row.s[t] = row[t];
    // One test of everything (no branch between the two loads and their use).
    const int lim = T < A.slot_stride ? T : A.slot_stride;
    it.off = acc - 1;
    const int rs = row_slot<T>(slot_row, it.off);
    it.rs = rs;
    it.cs = slot_row.s[0];
    return (acc >= 1) & (acc <= lim) & (rs > 0) & (rs < A.N) & (it.cs >= 0) & (it.cs < A.N);
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
  const long long next = static_cast<long long>(blockIdx.x) + A.ahead;
  if (A.ahead <= 0 || next >= static_cast<long long>(gridDim.x)) return;
  const int item = static_cast<int>(next);
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
  uint32_t gate[T];  // BF16 bits, one per register: packing would consume the load
  float nw;
};

// Channel tid & 127 on every thread (threads 128-255 repeat 0-127, unused):
// a load under a divergent branch would be waited for inside the branch.
template <int T>
__device__ __forceinline__ void load_output_operands(const Args& A, const Item& it,
                                                     OutputOperands<T>& oo) {
  const int c = threadIdx.x & (kD - 1);
#pragma unroll
  for (int t = 0; t < T; ++t)
    oo.gate[t] = A.gate[(it.token0 + t) * it.dim + static_cast<size_t>(it.h) * kD + c];
  oo.nw = bf16_bits_to_f32(A.norm_w[c]);
}

// ---- prologue: convolution, SiLU, norms, gate projection, decay -------------

// Convolution + SiLU.  Wave w < 3 makes part w of the q | k | v channels,
// lane l channels 2l and 2l + 1 of the head: inputs, weights and bias arrive
// as one 4-byte pair per lane.  Every operand load is issued unconditionally
// (the compiler waits for a load under a branch inside the branch) and ahead
// of the state page (loads of a wave retire in issue order, so an input
// loaded after the page could not be used before all of the page has
// arrived).  Wave 3 therefore issues the same loads as wave 2 and uses none
// of them: a window column must be read and rewritten by one wave only, as
// another wave's read could land after the rewrite.  Waves 0 and 1 hold all
// of q and all of k and reduce their sums of squares alone.
template <int T>
struct ConvOperands {
  uint32_t tap[2][3];  // [channel 2l, 2l + 1][tap]: the pool's type (BF16 or FP32 bits)
  uint32_t x[T];       // BF16 pair of each token's input (low half: channel 2l)
  uint32_t w[4];       // BF16 pair of each tap's weight
  uint32_t bias;       // BF16 pair of the bias (0: none)
};

__device__ __forceinline__ int conv_wave() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
}

__device__ __forceinline__ uint32_t load_pair(const uint16_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

template <bool kConvF32>
__device__ __forceinline__ float tap_value(uint32_t bits) {
  return kConvF32 ? __uint_as_float(bits) : bf16_bits_to_f32(bits);
}

// Inputs, weights and bias: independent of the slot tables, so they are
// issued before the slots are read.
template <int T, bool kBias>
__device__ __forceinline__ void conv_load_inputs(const Args& A, const Item& it,
                                                 ConvOperands<T>& co) {
  const int wave = conv_wave();
  const int part = wave < 2 ? wave : 2;
  const size_t hc = static_cast<size_t>(it.h) * kD + 2 * (threadIdx.x & 63);
  const size_t ch = static_cast<size_t>(part) * it.dim + hc;
#pragma unroll
  for (int t = 0; t < T; ++t) co.x[t] = load_pair(A.x + (it.token0 + t) * 3 * it.dim + ch);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    co.w[i] = load_pair(A.conv_w + (static_cast<size_t>(part) * 4 + i) * it.dim + hc);
  co.bias = kBias ? load_pair(A.conv_b + ch) : 0u;
}

// The three taps of the window (columns off .. off + 2) of the resolved
// convolution slot.
template <int T, bool kConvF32>
__device__ __forceinline__ void conv_load_taps(const Args& A, const Item& it,
                                               ConvOperands<T>& co) {
  const int wave = conv_wave();
  const int part = wave < 2 ? wave : 2;
  const size_t ch = static_cast<size_t>(part) * it.dim + static_cast<size_t>(it.h) * kD +
                    2 * (threadIdx.x & 63);
  const size_t base = (static_cast<size_t>(it.cs) * 3 * it.dim + ch) * A.W + it.off;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const size_t at = base + static_cast<size_t>(j) * A.W + i;
      co.tap[j][i] = kConvF32 ? static_cast<const uint32_t*>(A.conv_state)[at]
                              : static_cast<const uint16_t*>(A.conv_state)[at];
    }
}

// The window is rewritten in place after it was read: [tap1, tap2, x_0 ..]
// in the pool's type (an FP32 pool receives the inputs' exact FP32 values).
// Part `part` (wave), channel pair of lane `lane`.
template <int T, bool kConvF32>
__device__ __forceinline__ void conv_window_store(const Args& A, const Item& it,
                                                  const ConvOperands<T>& co, int part, int lane) {
  const size_t ch = static_cast<size_t>(part) * it.dim + static_cast<size_t>(it.h) * kD + 2 * lane;
  {
    const size_t base = (static_cast<size_t>(it.cs) * 3 * it.dim + ch) * A.W;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const size_t at = base + static_cast<size_t>(j) * A.W;
      if constexpr (kConvF32) {
        uint32_t* col = static_cast<uint32_t*>(A.conv_state) + at;
        col[0] = co.tap[j][1];
        col[1] = co.tap[j][2];
#pragma unroll
        for (int t = 0; t < T; ++t) col[2 + t] = j ? co.x[t] & 0xffff0000u : co.x[t] << 16;
      } else {
        uint16_t* col = static_cast<uint16_t*>(A.conv_state) + at;
        col[0] = static_cast<uint16_t>(co.tap[j][1]);
        col[1] = static_cast<uint16_t>(co.tap[j][2]);
#pragma unroll
        for (int t = 0; t < T; ++t) col[2 + t] = static_cast<uint16_t>(j ? co.x[t] >> 16 : co.x[t]);
      }
    }
  }
}

// The whole window of the item, by the three waves that hold its parts.
template <int T, bool kConvF32>
__device__ __forceinline__ void conv_write_window(const Args& A, const Item& it,
                                                  const ConvOperands<T>& co) {
  const int part = conv_wave();
  if (part == 3) return;
  conv_window_store<T, kConvF32>(A, it, co, part, threadIdx.x & 63);
}

// The convolution outputs go to the q, k and v tables; record mode stores k.
// kWindow: rewrite the window here (a kernel whose window another workgroup
// may still read rewrites it later with conv_write_window).
template <int T, bool kRecord, bool kConvF32, bool kWindow = true, class SH>
__device__ __forceinline__ void conv_compute(const Args& A, const Item& it, SH& sh,
                                             const ConvOperands<T>& co) {
  const int part = conv_wave();
  if (part == 3) return;  // issued copies of wave 2's loads only
  const int lane = threadIdx.x & 63;
  if constexpr (kWindow) conv_window_store<T, kConvF32>(A, it, co, part, lane);
  float* dst = part == 0 ? &sh.u.in.q[0][0] : part == 1 ? &sh.u.in.k[0][0] : &sh.v[0][0];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float y[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float acc = j ? bf16_hi(co.bias) : bf16_lo(co.bias);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = t + i;  // window position: taps 0-2, then the inputs
        const float term = r < 3 ? tap_value<kConvF32>(co.tap[j][r < 3 ? r : 0])
                                 : (j ? bf16_hi(co.x[r < 3 ? 0 : r - 3])
                                      : bf16_lo(co.x[r < 3 ? 0 : r - 3]));
        acc = fmaf(term, j ? bf16_hi(co.w[i]) : bf16_lo(co.w[i]), acc);
      }
      y[j] = silu_bf16(acc);
    }
    *reinterpret_cast<float2*>(&dst[t * kD + 2 * lane]) = make_float2(y[0], y[1]);
    if (part < 2) {
      const float ss = wave_sum(fmaf(y[1], y[1], y[0] * y[0]));
      if (lane == 0) sh.sq[t][part] = ss;
    }
    if constexpr (kRecord) {
      if (part == 1)
        __builtin_nontemporal_store(
            f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16),
            reinterpret_cast<uint32_t*>(
                &A.rec_kg[((static_cast<size_t>(it.b) * A.H + it.h) * T + t) * (2 * kD) + 2 * lane]));
    }
  }
}

// beta = sigmoid(logit).  The logit of token tid (tid < T) is loaded by
// load_beta with the other input operands, ahead of the state page.
template <int T>
__device__ __forceinline__ float load_beta(const Args& A, const Item& it) {
  const int t = threadIdx.x < T ? threadIdx.x : T - 1;  // no divergent load
  return bf16_bits_to_f32(A.beta[(it.token0 + t) * A.H + it.h]);
}

template <int T, class SH>
__device__ __forceinline__ void store_beta(SH& sh, float beta_logit) {
  if (threadIdx.x < T) sh.beta[threadIdx.x] = sigmoid_fast(beta_logit);
}

// Gate projection raw_g[t][f] = BF16(sum_j F_B[h*128+f][j] f_a[t][j]): the
// products of two BF16 values (16 significant bits) are exact in FP64 and
// are summed in FP64.  The sum is exact while the 128 products span fewer
// than 2^37 in magnitude (53 bits hold every partial sum); beyond that each
// addition errs by at most 2^-53 relative, so the order of the sum could
// change the FP32 rounding only within ~2^-45 of a rounding boundary.
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

// Both factors are widened to FP64 before they meet (an FP64 fma): the
// product of two BF16 values is then exact for every finite input, also
// where an FP32 product would underflow or overflow.
template <class SH>
__device__ __forceinline__ void gate_valu(const GateOperands& go, SH& sh) {
  const int tid = threadIdx.x;
  const int fsub = tid >> 4;
  double fa[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) fa[e] = static_cast<double>(bf16_at(go.fa, e));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fma(static_cast<double>(bf16_at(go.fb[i], e)), fa[e], acc);
    acc = row_sum16_f64(acc);
    if ((tid & 15) == 0) sh.u.in.g[0][16 * i + fsub] = static_cast<float>(acc);
  }
}

// Several tokens: the gate projection on FP64 MFMA 4x4x4 (four 4x4 blocks
// per instruction, 16 cycles; a 16x16x4 tile takes 64 and has 16 token
// columns, so this needs half its cycles at T = 8 and a quarter at T <= 4).
// Lane layout of the instruction: block b = (l >> 2) & 3; A: lane
// 16k + 4b + i holds A[i][k]; B: lane 16k + 4b + j holds B[k][j]; D: lane
// 16i + 4b + j holds D[i][j].  Block b = feature quad: A[i][k] =
// F_B[32w + 16 fg + 4b + i][K], B[k][j] = f_a[4 tg + j][K] (the same in every
// block), K = 32k + 8n + e at step (n, e); each D lane ends with a whole
// sum.  Token groups (tg) past T - 1 load token T - 1 and are discarded.
// The sums are exact in FP64, so the order changes no bit.
template <int T>
struct GateQuadOperands {
  static constexpr int kTokenGroups = (T + 3) / 4;
  uint4 fb[2][4];                 // [feature group fg][n]: 8 columns 32k + 8n ..
  uint4 fa[kTokenGroups][4];      // [token group tg][n]
};

// F_B rows of feature group fg (the second group can be loaded once the
// convolution operands are dead) and the f_a rows.
template <int T>
__device__ __forceinline__ void gate_quad_load_fb(const Args& A, const Item& it,
                                                  GateQuadOperands<T>& go, int fg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k = lane >> 4, b = (lane >> 2) & 3, i = lane & 3;
#pragma unroll
  for (int n = 0; n < 4; ++n)
    go.fb[fg][n] = *reinterpret_cast<const uint4*>(
        A.f_b + (static_cast<size_t>(it.h) * kD + 32 * wave + 16 * fg + 4 * b + i) * kD +
        32 * k + 8 * n);
}

template <int T>
__device__ __forceinline__ void gate_quad_load_fa(const Args& A, const Item& it,
                                                  GateQuadOperands<T>& go) {
  const int lane = threadIdx.x & 63;
  const int k = lane >> 4, j = lane & 3;
#pragma unroll
  for (int tg = 0; tg < GateQuadOperands<T>::kTokenGroups; ++tg) {
    const int tok = 4 * tg + j < T ? 4 * tg + j : T - 1;
#pragma unroll
    for (int n = 0; n < 4; ++n)
      go.fa[tg][n] = *reinterpret_cast<const uint4*>(A.f_a + (it.token0 + tok) * kD + 32 * k +
                                                     8 * n);
  }
}

template <int T, class SH>
__device__ __forceinline__ void gate_quad_compute(const GateQuadOperands<T>& go, SH& sh) {
  constexpr int kTG = GateQuadOperands<T>::kTokenGroups;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane >> 4, b = (lane >> 2) & 3, j = lane & 3;
  // Steps outside, (fg, tg) inside: each converted operand is used at once,
  // and the 2 kTG accumulators are independent chains.
  double acc[2][kTG];
#pragma unroll
  for (int fg = 0; fg < 2; ++fg)
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) acc[fg][tg] = 0.0;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double bv[kTG];
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg) bv[tg] = static_cast<double>(bf16_at(go.fa[tg][n], e));
#pragma unroll
      for (int fg = 0; fg < 2; ++fg) {
        const double av = static_cast<double>(bf16_at(go.fb[fg][n], e));
#pragma unroll
        for (int tg = 0; tg < kTG; ++tg)
          acc[fg][tg] = __builtin_amdgcn_mfma_f64_4x4x4f64(av, bv[tg], acc[fg][tg], 0, 0, 0);
      }
    }
#pragma unroll
  for (int fg = 0; fg < 2; ++fg) {
    const int f = 32 * wave + 16 * fg + 4 * b + i;
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) {
      const int t = 4 * tg + j;
      if (t < T) sh.u.in.g[t][f] = static_cast<float>(acc[fg][tg]);
    }
  }
}

// The same 4x4x4 product with its operands in rounds, for kernels that
// cannot hold the whole set: the operands of column step n (8 columns of
// each 32-column quarter) arrive in a round of their own, and the round for
// step n + 1 is requested before step n is computed, so at most two rounds
// are live (2 x (2 + kTG) 16-byte loads).  gate_rounds_begin issues round 0
// (early, where the kernel has registers to spare); gate_rounds_compute
// runs the four steps.  The last step requests its own columns again (cache
// hits, unused) so that no load sits under a branch.
template <int T>
struct GateRounds {
  static constexpr int kTG = GateQuadOperands<T>::kTokenGroups;
  const uint16_t* fb_base;  // wave-uniform bases ...
  const uint16_t* fa_base;
  uint32_t fb_off;          // ... and lane offsets in elements
  uint32_t fa_off[kTG];
  uint4 fb[2], fa[kTG];     // the current round
};

template <int T>
__device__ __forceinline__ void gate_rounds_begin(const Args& A, const Item& it,
                                                  GateRounds<T>& gr) {
  constexpr int kTG = GateRounds<T>::kTG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k = lane >> 4, b = (lane >> 2) & 3, i = lane & 3, j = lane & 3;
  gr.fb_base = A.f_b + static_cast<size_t>(it.h) * kD * kD;
  gr.fa_base = A.f_a + it.token0 * kD;
  gr.fb_off = (32 * wave + 4 * b + i) * kD + 32 * k;  // feature group 1: 16 rows on
#pragma unroll
  for (int tg = 0; tg < kTG; ++tg) {
    const int tok = 4 * tg + j < T ? 4 * tg + j : T - 1;
    gr.fa_off[tg] = tok * kD + 32 * k;
  }
#pragma unroll
  for (int fg = 0; fg < 2; ++fg)
    gr.fb[fg] = *reinterpret_cast<const uint4*>(gr.fb_base + gr.fb_off + 16 * kD * fg);
#pragma unroll
  for (int tg = 0; tg < kTG; ++tg)
    gr.fa[tg] = *reinterpret_cast<const uint4*>(gr.fa_base + gr.fa_off[tg]);
}

template <int T, class SH>
__device__ __forceinline__ void gate_rounds_compute(GateRounds<T>& gr, SH& sh) {
  constexpr int kTG = GateRounds<T>::kTG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = (lane >> 2) & 3, j = lane & 3;
  double acc[2][kTG];
#pragma unroll
  for (int fg = 0; fg < 2; ++fg)
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) acc[fg][tg] = 0.0;
#pragma unroll 1
  for (int n = 0; n < 4; ++n) {
    const uint32_t col = 8 * (n < 3 ? n + 1 : n);
    uint4 fb_next[2], fa_next[kTG];
#pragma unroll
    for (int fg = 0; fg < 2; ++fg)
      fb_next[fg] = *reinterpret_cast<const uint4*>(gr.fb_base + gr.fb_off + 16 * kD * fg + col);
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg)
      fa_next[tg] = *reinterpret_cast<const uint4*>(gr.fa_base + gr.fa_off[tg] + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double bv[kTG];
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg) bv[tg] = static_cast<double>(bf16_at(gr.fa[tg], e));
#pragma unroll
      for (int fg = 0; fg < 2; ++fg) {
        const double av = static_cast<double>(bf16_at(gr.fb[fg], e));
#pragma unroll
        for (int tg = 0; tg < kTG; ++tg)
          acc[fg][tg] = __builtin_amdgcn_mfma_f64_4x4x4f64(av, bv[tg], acc[fg][tg], 0, 0, 0);
      }
    }
#pragma unroll
    for (int fg = 0; fg < 2; ++fg) gr.fb[fg] = fb_next[fg];
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) gr.fa[tg] = fa_next[tg];
  }
#pragma unroll
  for (int fg = 0; fg < 2; ++fg) {
    const int f = 32 * wave + 16 * fg + 4 * b + (lane >> 4);
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) {
      const int t = 4 * tg + j;
      if (t < T) sh.u.in.g[t][f] = static_cast<float>(acc[fg][tg]);
    }
  }
}

// The record kernel's variant: the f_a rows of the item are converted to
// FP64 once, into an LDS table shared by the four waves, so the B operand
// of every gate step is one 8-byte LDS read instead of a global load and
// two conversions per lane; the F_B rows stay in registers.  Column
// 32k + r of token t sits at t * kFaPitch + 33k + r (doubles): the 16
// distinct addresses of one read (4 tokens x 4 column quarters) fall in
// distinct banks.
constexpr int kFaPitch = 4 * 33;

template <int T>
struct FaPairs {
  static constexpr int kPer = (T + 3) / 4;  // tokens per thread
  uint32_t v[kPer];                         // two BF16 columns of one token
};

// Thread tid: columns 2(tid & 63) and 2(tid & 63) + 1 of tokens
// (tid >> 6) + 4m.  Tokens past T - 1 load token T - 1 (no load under a
// branch) and are not stored.
template <int T>
__device__ __forceinline__ void fa_pairs_load(const Args& A, const Item& it, FaPairs<T>& fp) {
  const int pc = threadIdx.x & 63, tt = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < FaPairs<T>::kPer; ++m) {
    const int t = tt + 4 * m;
    const int tok = t < T ? t : T - 1;
    fp.v[m] = *reinterpret_cast<const uint32_t*>(A.f_a + (it.token0 + tok) * kD + 2 * pc);
  }
}

template <int T>
__device__ __forceinline__ void fa_pairs_store(const FaPairs<T>& fp, double* fa64) {
  const int pc = threadIdx.x & 63, tt = threadIdx.x >> 6;
  const int col = 2 * pc;
  const int at = 33 * (col >> 5) + (col & 31);
#pragma unroll
  for (int m = 0; m < FaPairs<T>::kPer; ++m) {
    const int t = tt + 4 * m;
    if (t < T) {
      fa64[t * kFaPitch + at] = static_cast<double>(bf16_lo(fp.v[m]));
      fa64[t * kFaPitch + at + 1] = static_cast<double>(bf16_hi(fp.v[m]));
    }
  }
}

// All four column rounds of the F_B rows at once, loaded with the other
// input operands so that the gate waits on no memory (a load issued after
// the state page would retire after it).
template <int T>
struct GateFBAll {
  uint4 fb[4][2];  // [column step n][feature group fg]
};

template <int T>
__device__ __forceinline__ void gate_fb_all_load(const Args& A, const Item& it, GateFBAll<T>& gf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k = lane >> 4, b = (lane >> 2) & 3, i = lane & 3;
  const uint16_t* base = A.f_b + static_cast<size_t>(it.h) * kD * kD +
                         (32 * wave + 4 * b + i) * kD + 32 * k;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int fg = 0; fg < 2; ++fg)
      gf.fb[n][fg] = *reinterpret_cast<const uint4*>(base + 16 * kD * fg + 8 * n);
}

// The 4x4x4 FP64 projection (the lane layout of gate_quad_compute) with F_B
// in registers and f_a from the FP64 table in LDS: each B operand is one
// 8-byte LDS read.
template <int T, class SH>
__device__ __forceinline__ void gate_fb_all_compute(const GateFBAll<T>& gf, const double* fa64,
                                                    SH& sh) {
  constexpr int kTG = GateQuadOperands<T>::kTokenGroups;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k = lane >> 4, b = (lane >> 2) & 3, j = lane & 3;
  int row[kTG];
#pragma unroll
  for (int tg = 0; tg < kTG; ++tg) {
    const int tok = 4 * tg + j < T ? 4 * tg + j : T - 1;
    row[tg] = tok * kFaPitch + 33 * k;
  }
  double acc[2][kTG];
#pragma unroll
  for (int fg = 0; fg < 2; ++fg)
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) acc[fg][tg] = 0.0;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double bv[kTG];
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg) bv[tg] = fa64[row[tg] + 8 * n + e];
#pragma unroll
      for (int fg = 0; fg < 2; ++fg) {
        const double av = static_cast<double>(bf16_at(gf.fb[n][fg], e));
#pragma unroll
        for (int tg = 0; tg < kTG; ++tg)
          acc[fg][tg] = __builtin_amdgcn_mfma_f64_4x4x4f64(av, bv[tg], acc[fg][tg], 0, 0, 0);
      }
    }
#pragma unroll
  for (int fg = 0; fg < 2; ++fg) {
    const int f = 32 * wave + 16 * fg + 4 * b + (lane >> 4);
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) {
      const int t = 4 * tg + j;
      if (t < T) sh.u.in.g[t][f] = static_cast<float>(acc[fg][tg]);
    }
  }
}

// Raw gate to BF16, then the decay of key channel f = tid (threads 0-127);
// record mode stores raw_g.
template <int T, bool kRecord, class SH>
__device__ __forceinline__ void decay(const Args& A, const Item& it, SH& sh, float dt,
                                      float a_log) {
  const int tid = threadIdx.x;
  if (tid < kD) {
    const float e = expf(a_log);
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

// Token halves for the per-channel stages of the record kernel: thread tid
// takes channel tid & 127 and, in step j < kHalfTokens, token
// half_token<T>(j) of its half (tid >> 7: the first (T + 1) / 2 tokens, or
// the rest), so all four waves share the work that threads 0-127 would do
// alone.  Each value is computed by the same operations as with one thread
// per channel, so the results are the same bits.  Steps and register
// indices stay compile-time constants (a select by the wave-uniform half).
template <int T>
constexpr int kHalfTokens = (T + 1) / 2;

__device__ __forceinline__ bool second_half() { return (threadIdx.x >> 7) != 0; }

template <int T>
__device__ __forceinline__ int half_token(int j) {
  return second_half() ? kHalfTokens<T> + j : j;
}

// Step j exists in both halves, or only in the first (odd T).
template <int T>
__device__ __forceinline__ bool half_step_live(int j) {
  return !second_half() || kHalfTokens<T> + j < T;
}

// The decay (and the record of raw_g) of decay<T, true>, by token halves.
template <int T, class SH>
__device__ __forceinline__ void decay_halves(const Args& A, const Item& it, SH& sh, float dt,
                                             float a_log) {
  const int f = threadIdx.x & (kD - 1);
  const float e = expf(a_log);
#pragma unroll
  for (int j = 0; j < kHalfTokens<T>; ++j) {
    if (half_step_live<T>(j)) {
      const int t = half_token<T>(j);
      const float raw_g = round_bf16(sh.u.in.g[t][f]);
      sh.u.in.a[t][f] = decay_f32(e, raw_g, dt, A.lower_bound);
      __builtin_nontemporal_store(
          static_cast<uint16_t>(f32_to_bf16_bits(raw_g)),
          &A.rec_kg[((static_cast<size_t>(it.b) * A.H + it.h) * T + t) * (2 * kD) + kD + f]);
    }
  }
}

// dt_bias of key channel tid (threads 0-127), loaded with the input operands.
__device__ __forceinline__ float load_dt(const Args& A, const Item& it) {
  return A.dt_bias[static_cast<size_t>(it.h) * kD + (threadIdx.x & (kD - 1))];
}

// A_log of the item's head (a scalar load), read in the prologue: a load
// after a barrier cannot be issued before it, and the decay sits after one.
__device__ __forceinline__ float load_a_log(const Args& A, const Item& it) {
  return A.a_log[it.h];
}

template <int T, class SH>
__device__ __forceinline__ void norm_factors(const SH& sh, int t, float& fq, float& fk) {
  // v_rsq_f32 (1 ulp): the sums are >= 1e-6, normal numbers.
  fq = __builtin_amdgcn_rsqf(sh.sq[t][0] + 1.0e-6f);
  fk = __builtin_amdgcn_rsqf(sh.sq[t][1] + 1.0e-6f);
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
      // v_rsq_f32: 1 ulp for normal arguments (variance >= eps, 1e-6 in use);
      // 0 and negative arguments give inf and NaN as 1 / sqrt would.
      const float rstd = __builtin_amdgcn_rsqf(variance);
      const float sg = sigmoid_fast(bf16_bits_to_f32(oo.gate[t]));
      const size_t idx = (it.token0 + t) * it.dim + static_cast<size_t>(it.h) * kD + tid;
      A.out[idx] = static_cast<uint16_t>(f32_to_bf16_bits(((o[t][tid] * rstd) * oo.nw) * sg));
    }
  }
}

// The gated RMSNorm of gated_rmsnorm by token halves: waves 0-1 take the
// first half of the tokens, waves 2-3 the second, each pair summing o^2
// over the 128 channels (64 per wave) in the same order.
template <int T, class SH>
__device__ __forceinline__ void gated_rmsnorm_halves(const Args& A, const Item& it, SH& sh,
                                                     const float (*o)[kD],
                                                     const OutputOperands<T>& oo) {
  const int tid = threadIdx.x, lane = tid & 63, pw = (tid >> 6) & 1;
  const int c = tid & (kD - 1);
#pragma unroll
  for (int j = 0; j < kHalfTokens<T>; ++j) {
    if (half_step_live<T>(j)) {
      const float ot = o[half_token<T>(j)][c];
      const float ss = wave_sum(ot * ot);
      if (lane == 0) sh.os[half_token<T>(j)][pw] = ss;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kHalfTokens<T>; ++j) {
    if (half_step_live<T>(j)) {
      const int t = half_token<T>(j);
      const int kHi = kHalfTokens<T> + j < T ? kHalfTokens<T> + j : j;  // constant once unrolled
      const uint32_t gbits = second_half() ? oo.gate[kHi] : oo.gate[j];
      const float variance = (sh.os[t][0] + sh.os[t][1]) * (1.0f / 128.0f) + A.eps;
      const float rstd = __builtin_amdgcn_rsqf(variance);
      const float sg = sigmoid_fast(bf16_bits_to_f32(gbits));
      const size_t idx = (it.token0 + t) * it.dim + static_cast<size_t>(it.h) * kD + c;
      A.out[idx] = static_cast<uint16_t>(f32_to_bf16_bits(((o[t][c] * rstd) * oo.nw) * sg));
    }
  }
}

}  // namespace

#endif  // KDA_STAGES_HPP
