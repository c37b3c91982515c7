// KDA decode / verify step for MI355X (gfx950, CDNA4): the step kernels and
// the C ABI of kda_decode, kda_verify and kda_validate.
//
// Operation: the KdaWide step of the vLLM API page
// vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide (class
// docstring, constructor, kernel body, helpers silu / decay); the argument
// contract is in include/kda.h.
//
// Design (one workgroup of 4 wave64s per (request, head) item):
//  * The item's 128x128 FP32 state page (64 KiB) lives in VGPRs for every
//    token of the step: thread (wave w, lane l) owns value rows
//    32(l >> 4) + 8w + i, i < 8, and keys 4(l & 15) + [0, 4) and
//    64 + 4(l & 15) + [0, 4): 64 floats.  Each 16-byte load or store of a
//    wave covers four 256-byte row segments 16 KiB apart, so every HBM line
//    is used whole and each instruction spreads over more channels.  The
//    loads are issued after the input loads and land while the inputs are
//    prepared.
//  * A row's 128 keys sit in one 16-lane DPP row, so the two row reductions
//    per token (S.k and S.q) are four DPP adds each, with no LDS traffic.
//  * The BF16 rounding points that feed the state (SiLU outputs and the raw
//    gate) are the correctly rounded values of the page's FP32 operations:
//    the SiLU takes a fast FP32 path whose error bound decides the BF16
//    value unless it lies near a rounding midpoint (then exp is evaluated in
//    FP64), and the gate projection (products of BF16 values, exact in FP64)
//    is accumulated in FP64 and rounded once.  Only the recurrence's dot
//    products keep an FP32 reduction order of their own.
//  * Record mode (no state written) runs in closed form on FP32 MFMA from
//    one pass over the page read.
//  * Items are numbered head-fastest; with H a multiple of 8 the
//    round-robin dispatch over the 8 XCDs sends every head to one XCD, so
//    each XCD's L2 keeps only its heads' 32 KiB F_B blocks.
#include "kda.h"
#include "kda_host.hpp"

namespace {

// ---- decode / verify: the recurrence token by token ------------------------

// Thread (wave w, lane l) owns rows 32(l >> 4) + 8w + i (i < 8) and keys
// 4(l & 15) + [0, 4) and 64 + 4(l & 15) + [0, 4): 64 floats in VGPRs.  Every
// 16-byte access of a wave covers four 256-byte row segments 16 KiB apart,
// which spreads each instruction over more HBM channels; a row's keys sit in
// one 16-lane DPP row.
//
// kLatency: the variant for batches small enough that every workgroup is
// resident at 2 per CU (512 items).  There occupancy buys nothing and each
// item's chain of memory round trips is the launch time, so the kernel takes
// up to 256 VGPRs and issues every operand (beta, dt_bias, the output-norm
// operands and, for T > 1, the whole gate operand set of the 4x4x4 FP64
// projection) ahead of the state page: one round trip before the page
// instead of one per gate step.
template <int T, bool kRecord, bool kBias, bool kConvF32, bool kLatency>
__device__ __forceinline__ void step_body(const Args& A) {
  // 1. Input operands first, then the state page (one buffer resource per
  //    64 KiB page): the inputs are used while the page is still arriving.
  //    The operands that do not depend on the slot tables are issued before
  //    the tables are read.
  Item it;
  locate<T>(A, it);
  ConvOperands<T> co;
  conv_load_inputs<T, kBias>(A, it, co);
  GateOperands go;
  if constexpr (T == 1) gate_load(A, it, go);
  GateQuadOperands<T> gq;
  if constexpr (T > 1 && kLatency) {
    gate_quad_load_fb<T>(A, it, gq, 0);
    gate_quad_load_fb<T>(A, it, gq, 1);
    gate_quad_load_fa<T>(A, it, gq);
  }
  // beta and dt ahead of the page, so that nothing before the recurrence
  // waits for it and the recurrence starts on the first rows of the page
  // while the rest arrive (loads retire in order).  Decode at full occupancy
  // with a bias or an FP32 pool has no VGPRs to spare for them at the start
  // (they would spill); there they are loaded after the convolution.
  constexpr bool kEarlyScalars = T > 1 || kLatency || (!kBias && !kConvF32);
  float beta_logit = 0.0f, dt = 0.0f;
  if constexpr (kEarlyScalars) {
    beta_logit = load_beta<T>(A, it);
    dt = load_dt(A, it);
  }
  const float a_log = load_a_log(A, it);
  OutputOperands<T> oo;
  if constexpr (kLatency) load_output_operands<T>(A, it, oo);
  __builtin_amdgcn_sched_barrier(0);  // not sunk below the slot reads
  SlotRow<T> slot_row;
  if (!resolve<T>(A, it, slot_row)) {  // padding: BF16 zeros, nothing else touched
    write_padding<T>(A, it);
    return;
  }
  __shared__ Shared<T, false> sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15;
  const int row0 = 32 * (lane >> 4) + 8 * wave;
  const int lane_off = (row0 * kD + 4 * c16) * 4;
  conv_load_taps<T, kConvF32>(A, it, co);
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
  conv_compute<T, kRecord, kConvF32>(A, it, sh, co);
  if constexpr (!kEarlyScalars) {
    // Behind the page (loads retire in order), so they arrive with it.
    beta_logit = load_beta<T>(A, it);
    dt = load_dt(A, it);
  }
  store_beta<T>(sh, beta_logit);
  if constexpr (T == 1)
    gate_valu(go, sh);
  else if constexpr (kLatency)
    gate_quad_compute<T>(gq, sh);
  else {
    GateRounds<T> gr;
    gate_rounds_begin<T>(A, it, gr);
    gate_rounds_compute<T>(gr, sh);
  }
  __syncthreads();
  decay<T, kRecord>(A, it, sh, dt, a_log);
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
      const int target = T == 1 ? it.rs : row_slot<T>(slot_row, t);
      if (target > 0 && target < A.N) {
        float* page = page_ptr(A.state, target, it.h, A.H);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) store_f4(page, lane_off + i * kD * 4 + j * 256, st[i][j]);
      }
    }
  }
  if constexpr (!kLatency) load_output_operands<T>(A, it, oo);
  __syncthreads();

  // 4. Gated RMSNorm.
  gated_rmsnorm<T>(A, it, sh, sh.o, oo);
  keep_alive(A, sink);
}

template <int T, bool kRecord, bool kBias, bool kConvF32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void kda_step_kernel(const Args A) {
  step_body<T, kRecord, kBias, kConvF32, false>(A);
}

template <int T, bool kRecord, bool kBias, bool kConvF32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void kda_step_latency_kernel(const Args A) {
  step_body<T, kRecord, kBias, kConvF32, true>(A);
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
template <int T, bool kBias, bool kConvF32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void kda_record_kernel(const Args A) {
  // The records (k, raw_g, u) are stored with the non-temporal policy: they
  // are read back only by a later replay, and a store that stays dirty in
  // the caches is written back during a later launch (measured: cold-clean
  // launches ~1 % faster, the others within run-to-run spread).
  // 1. Every input operand ahead of the state page (loads of a wave retire in
  //    issue order, so nothing that the prologue needs may queue behind the
  //    page): convolution inputs, all F_B rows of the gate, f_a, beta,
  //    dt_bias before the slot tables are read, the window taps after.  The
  //    page's first row tile is issued right after the taps and arrives
  //    during the convolution and the gate; the first half of the second
  //    (keys 0-63) after the convolution, when its operands are dead, and
  //    the rest after the gate, behind the output-norm operands.  The
  //    scheduling barriers keep the groups in this order.
  Item it;
  locate<T>(A, it);
  ConvOperands<T> co;
  conv_load_inputs<T, kBias>(A, it, co);
  GateFBAll<T> gf;
  gate_fb_all_load<T>(A, it, gf);
  FaPairs<T> fp;
  fa_pairs_load<T>(A, it, fp);
  const float beta_logit = load_beta<T>(A, it);
  const float dt = load_dt(A, it);
  const float a_log = load_a_log(A, it);
  __builtin_amdgcn_sched_barrier(0);
  SlotRow<T> slot_row;
  if (!resolve<T>(A, it, slot_row)) {
    write_padding<T>(A, it);
    return;
  }
  __shared__ Shared<T, true> sh;
  __shared__ RecordTables rt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  conv_load_taps<T, kConvF32>(A, it, co);
  __builtin_amdgcn_sched_barrier(0);
  // S0 in the MFMA B-operand layout: [tile][q] = rows 32w + 16 tile + c,
  // keys 16q + 4g .. +3 (each instruction: 16 rows x 64 contiguous bytes).
  float4 st[2][8];
  const __amdgpu_buffer_rsrc_t page = page_rsrc(A.state, it.rs, it.h, A.H);
  const int voff = (32 * wave + c) * kD * 4 + 16 * g;
#pragma unroll
  for (int q = 0; q < 8; ++q) st[0][q] = load_f4(page, voff, 64 * q);
  __builtin_amdgcn_sched_barrier(0);
  // f_a in FP64 for the gate, in the space of W (written only in step 4)
  static_assert(T * kFaPitch * sizeof(double) <= sizeof(rt.W), "f_a table exceeds W");
  double* fa64 = reinterpret_cast<double*>(&rt.W[0][0]);
  fa_pairs_store<T>(fp, fa64);
  __syncthreads();

  // 2. Convolution, norms, gate projection.
  conv_compute<T, true, kConvF32>(A, it, sh, co);
  store_beta<T>(sh, beta_logit);
#pragma unroll
  for (int q = 0; q < 4; ++q) st[1][q] = load_f4(page, voff, 16 * kD * 4 + 64 * q);
  gate_fb_all_compute<T>(gf, fa64, sh);
  OutputOperands<T> oo;
  load_output_operands<T>(A, it, oo);
  __syncthreads();

  // 3. The rest of the page's second row tile; the decay and the W and X
  //    tables are computed while it arrives.
#pragma unroll
  for (int q = 4; q < 8; ++q) st[1][q] = load_f4(page, voff, 16 * kD * 4 + 64 * q);
  float sink;
  prefetch_page<T>(A, sink);
  decay_halves<T>(A, it, sh, dt, a_log);
  __syncthreads();

  // 4. W and X (thread = key channel, token half), W zero beyond row 2T.  X
  //    takes the space of the FP32 gate projection, dead since the decay.
  //    The second half first forms the running product over the first
  //    half's tokens itself, with the same multiplications in order.
  float (&X)[T][kPad] = sh.u.in.g;
  {
    const int key = tid & (kD - 1);
    float acc = 1.0f;
    if (second_half()) {
#pragma unroll
      for (int t = 0; t < kHalfTokens<T>; ++t) acc = acc * sh.u.in.a[t][key];
    }
#pragma unroll
    for (int j = 0; j < kHalfTokens<T>; ++j) {
      if (half_step_live<T>(j)) {
        const int t = half_token<T>(j);
        float fq, fk;
        norm_factors<T>(sh, t, fq, fk);
        acc = acc * sh.u.in.a[t][key];
        const float kh = sh.u.in.k[t][key] * fk;
        const float qh = (sh.u.in.q[t][key] * fq) * A.scale;
        rt.W[t][key] = acc * kh;
        rt.W[T + t][key] = acc * qh;
        X[t][key] = kh * __builtin_amdgcn_rcpf(acc);  // acc a normal number (bound above)
      }
    }
    if (tid >= kD) {
#pragma unroll
      for (int m = 2 * T; m < 16; ++m) rt.W[m][key] = 0.0f;
    }
  }
  __syncthreads();  // from here q, k, a and g are dead: P, C and o take their space

  // 5. P = S0 W (two 16-row tiles per wave) and, on wave 0, C = W X^T.
  //    A operand lane (g, c): W[c][16q + 4g + e]; the K order is shared by
  //    both operands of each product.  The results stay in registers until
  //    every wave has passed a barrier: P overlaps the space of X (the gate
  //    projection's) when T < 6, and wave 0 reads X meanwhile.
  {
    // Tile 0's products first (two accumulators, alternating q, so that two
    // independent MFMA chains keep the pipe full), then C on wave 0, then
    // tile 1's, whose second half is the last of the page to arrive.
    f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, cc = p0, p0b = p0, p1b = p0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 w4 = *reinterpret_cast<const float4*>(&rt.W[c][16 * q + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (q & 1)
          p0b = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(st[0][q], e), p0b, 0, 0, 0);
        else
          p0 = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(st[0][q], e), p0, 0, 0, 0);
      }
    }
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 w4 = *reinterpret_cast<const float4*>(&rt.W[c][16 * q + 4 * g]);
        // X rows past T are zero operands (columns of C that are never read)
        const float4 x4 = c < T ? *reinterpret_cast<const float4*>(&X[c][16 * q + 4 * g])
                                : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cc = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(x4, e), cc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 w4 = *reinterpret_cast<const float4*>(&rt.W[c][16 * q + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (q & 1)
          p1b = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(st[1][q], e), p1b, 0, 0, 0);
        else
          p1 = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(w4, e), f4_at(st[1][q], e), p1, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p0[r] += p0b[r];
      p1[r] += p1b[r];
    }
    __syncthreads();
    // D layout (f32 16x16x4): lane l, element r holds D[4(l/16) + r][l%16].
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sh.u.out.P[4 * g + r][32 * wave + c] = p0[r];
      sh.u.out.P[4 * g + r][32 * wave + 16 + c] = p1[r];
    }
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.u.out.C[4 * g + r][c] = cc[r];
    }
  }
  __syncthreads();

  // 6. Per value row v = tid (threads 0-127): the triangular solve for u and o.
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
      __builtin_nontemporal_store(
          u[t], &A.rec_u[((static_cast<size_t>(it.b) * A.H + it.h) * T + t) * kD + v]);
    }
  }
  __syncthreads();

  // 7. Gated RMSNorm (token halves over the four waves).
  gated_rmsnorm_halves<T>(A, it, sh, sh.u.out.o, oo);
  keep_alive(A, sink);
}

// ---- host side -------------------------------------------------------------

// Up to this many items every workgroup of the latency variant is resident
// at once (2 per CU on 256 CUs).
constexpr long long kLatencyItems = 512;

// Record mode takes the closed-form kernel when the running decay products
// stay normal FP32 numbers (|lower_bound| <= 10, at most 8 tokens: |log A_t| <= 80).
constexpr float kRecordBound = 10.0f;

template <int T, bool kRecord, bool kBias, bool kConvF32>
kda_status launch_v(const Args& A, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(A.B * A.H));
  const dim3 block(kThreads);
  if constexpr (kRecord && T > 1) {
    if (fabsf(A.lower_bound) <= kRecordBound) {
      hipLaunchKernelGGL((kda_record_kernel<T, kBias, kConvF32>), grid, block, 0, stream, A);
      return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
  }
  if (static_cast<long long>(A.B) * A.H <= kLatencyItems)
    hipLaunchKernelGGL((kda_step_latency_kernel<T, kRecord, kBias, kConvF32>), grid, block, 0,
                       stream, A);
  else
    hipLaunchKernelGGL((kda_step_kernel<T, kRecord, kBias, kConvF32>), grid, block, 0, stream, A);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

template <int T, bool kRecord>
kda_status launch_t(const Args& A, hipStream_t stream) {
  const bool bias = A.conv_b != nullptr;
  if (A.conv_f32)
    return bias ? launch_v<T, kRecord, true, true>(A, stream)
                : launch_v<T, kRecord, false, true>(A, stream);
  return bias ? launch_v<T, kRecord, true, false>(A, stream)
              : launch_v<T, kRecord, false, false>(A, stream);
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

kda_status decode(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                  void* conv_state, int conv_f32, const uint16_t* f_a, const uint16_t* beta,
                  const float* a_log, const float* dt_bias, const int32_t* slots, float* state,
                  uint16_t* out, const uint16_t* gate, const uint16_t* norm_w,
                  float lower_bound, float scale, float eps, const uint16_t* f_b, int B, int H,
                  int N, int W, int gate_mode, int ahead, void* stream) {
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, nullptr, nullptr,
                      nullptr, B, H, N, W, 1, ahead, conv_f32);
  const kda_status s = check(A, 1, 0, gate_mode);
  if (s != KDA_OK || B == 0) return s;
  return launch<false>(A, 1, static_cast<hipStream_t>(stream));
}

kda_status verify(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                  void* conv_state, int conv_f32, const uint16_t* f_a, const uint16_t* beta,
                  const float* a_log, const float* dt_bias, const int32_t* slots, float* state,
                  uint16_t* out, const uint16_t* gate, const uint16_t* norm_w,
                  float lower_bound, float scale, float eps, const uint16_t* f_b,
                  const int32_t* accepted, float* rec_u, uint16_t* rec_kg, int B, int H, int N,
                  int W, int T, int slot_stride, int record, int gate_mode, int ahead,
                  void* stream) {
  if (T == 1) return KDA_ERR_TOKENS;  // a one-token step is kda_decode
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, accepted, rec_u, rec_kg,
                      B, H, N, W, slot_stride, ahead, conv_f32);
  const kda_status s = check(A, T, record, gate_mode);
  if (s != KDA_OK || B == 0) return s;
  return record ? launch<true>(A, T, static_cast<hipStream_t>(stream))
                : launch<false>(A, T, static_cast<hipStream_t>(stream));
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
  return decode(x, conv_w, conv_b, conv_state, 0, f_a, beta, a_log, dt_bias, slots, state, out,
                gate, norm_w, lower_bound, scale, eps, f_b, B, H, N, W, gate_mode, ahead,
                stream);
}

kda_status kda_decode_f32conv(const uint16_t* x, const uint16_t* conv_w,
                              const uint16_t* conv_b, float* conv_state, const uint16_t* f_a,
                              const uint16_t* beta, const float* a_log, const float* dt_bias,
                              const int32_t* slots, float* state, uint16_t* out,
                              const uint16_t* gate, const uint16_t* norm_w, float lower_bound,
                              float scale, float eps, const uint16_t* f_b, int B, int H, int N,
                              int W, int gate_mode, int ahead, void* stream) {
  return decode(x, conv_w, conv_b, conv_state, 1, f_a, beta, a_log, dt_bias, slots, state, out,
                gate, norm_w, lower_bound, scale, eps, f_b, B, H, N, W, gate_mode, ahead,
                stream);
}

kda_status kda_verify(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                      uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                      const float* a_log, const float* dt_bias, const int32_t* slots,
                      float* state, uint16_t* out, const uint16_t* gate,
                      const uint16_t* norm_w, float lower_bound, float scale, float eps,
                      const uint16_t* f_b, const int32_t* accepted, float* rec_u,
                      uint16_t* rec_kg, int B, int H, int N, int W, int T, int slot_stride,
                      int record, int gate_mode, int ahead, void* stream) {
  return verify(x, conv_w, conv_b, conv_state, 0, f_a, beta, a_log, dt_bias, slots, state, out,
                gate, norm_w, lower_bound, scale, eps, f_b, accepted, rec_u, rec_kg, B, H, N,
                W, T, slot_stride, record, gate_mode, ahead, stream);
}

kda_status kda_verify_f32conv(const uint16_t* x, const uint16_t* conv_w,
                              const uint16_t* conv_b, float* conv_state, const uint16_t* f_a,
                              const uint16_t* beta, const float* a_log, const float* dt_bias,
                              const int32_t* slots, float* state, uint16_t* out,
                              const uint16_t* gate, const uint16_t* norm_w, float lower_bound,
                              float scale, float eps, const uint16_t* f_b,
                              const int32_t* accepted, float* rec_u, uint16_t* rec_kg, int B,
                              int H, int N, int W, int T, int slot_stride, int record,
                              int gate_mode, int ahead, void* stream) {
  return verify(x, conv_w, conv_b, conv_state, 1, f_a, beta, a_log, dt_bias, slots, state, out,
                gate, norm_w, lower_bound, scale, eps, f_b, accepted, rec_u, rec_kg, B, H, N,
                W, T, slot_stride, record, gate_mode, ahead, stream);
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
    case KDA_ERR_ALIGN: return "a pointer is not aligned as its operand needs";
    case KDA_ERR_WORKSPACE: return "the split workspace is missing, too small or misaligned";
    case KDA_ERR_SCRATCH:
      return "the split needs more than the static scratch holds (B*H*(1 + 64*T) words > 1024*513)";
  }
  return "unknown status";
}

}  // extern "C"
