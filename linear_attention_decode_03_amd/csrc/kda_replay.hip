// KDA RecoverSSM replay for MI355X (gfx950, CDNA4): the replay kernel and
// the C ABI of kda_replay.
//
// Operation: the RecoverSSM mode of the KdaWide class docstring on the vLLM
// API page vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide
// (records written by the kernel body's record branches); the argument
// contract is in include/kda.h.
#include "kda.h"
#include "kda_device.hpp"

namespace {

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

  // 1. Records first, then the checkpoint page.  Thread (half = tid >> 7,
  //    channel c) takes tokens half, half + 2, ...: the k and raw_g of
  //    channel c and the u of value row c.  No load sits under a branch (the
  //    compiler would wait for each inside it, one round trip per token):
  //    tokens past n - 1 load token n - 1 again, which stays inside the
  //    record buffers, and are not used.  One value per register.
  constexpr int kPer = kMaxT / 2;
  const int c = tid & (kD - 1), half = tid >> 7;
  const int t_last = n > 0 ? n - 1 : 0;
  uint32_t kraw[kPer], graw[kPer];
  float uval[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int t = 2 * m + half;
    const size_t rec = rec0 + (t < t_last ? t : t_last);
    kraw[m] = R.rec_kg[rec * (2 * kD) + c];
    graw[m] = R.rec_kg[rec * (2 * kD) + kD + c];
    uval[m] = R.rec_u[rec * kD + c];
  }
  const float dt = R.dt_bias[static_cast<size_t>(h) * kD + c];
  __builtin_amdgcn_sched_barrier(0);  // every record load ahead of the page
  float4 st[8][2];
  {
    const __amdgpu_buffer_rsrc_t page = page_rsrc(R.state, src, h, R.H);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) st[i][j] = load_f4(page, lane_off, i * kD * 4 + j * 256);
  }

  // 2. k, decay and u tables; per-token sums of squares of k (the two waves
  //    of a half hold channels 0-63 and 64-127).
  const float e = expf(R.a_log[h]);
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int t = 2 * m + half;
    if (t < n) {
      const float k = bf16_bits_to_f32(kraw[m]);
      sh_k[t][c] = k;
      sh_a[t][c] = decay_f32(e, bf16_bits_to_f32(graw[m]), dt, R.lower_bound);
      sh_u[t][c] = uval[m];
      const float sk = wave_sum(k * k);
      if (lane == 0) sh_sq[t][wave & 1] = sk;
    }
  }
  __syncthreads();

  // 3. Apply the n tokens.
#pragma unroll 1
  for (int t = 0; t < n; ++t) {
    const float fk = __builtin_amdgcn_rsqf((sh_sq[t][0] + sh_sq[t][1]) + 1.0e-6f);
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

}  // namespace

extern "C" {

kda_status kda_replay(const float* rec_u, const uint16_t* rec_kg, const float* a_log,
                      const float* dt_bias, const int32_t* src_slots, const int32_t* dst_slots,
                      const int32_t* n_tokens, float* state, float lower_bound, int B, int H,
                      int N, int T, void* stream) {
  if (T < 1 || T > kMaxT) return KDA_ERR_TOKENS;
  if (B < 0 || H < 1 || N < 1 || !isfinite(lower_bound)) return KDA_ERR_SHAPE;
  // B*H workgroups of kThreads work-items: a dispatch counts its grid in
  // work-items, 32 bits.
  if (static_cast<long long>(B) * H * kThreads > 0xffffffffLL) return KDA_ERR_SHAPE;
  if (B == 0) return KDA_OK;
  if (!rec_u || !rec_kg || !a_log || !dt_bias || !src_slots || !dst_slots || !n_tokens || !state)
    return KDA_ERR_NULL;
  // 16-byte page loads and stores; the element size for everything else.
  const auto misaligned = [](const void* p, uintptr_t bytes) {
    return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) != 0;
  };
  if (misaligned(state, 16) || misaligned(rec_u, 4) || misaligned(rec_kg, 2) ||
      misaligned(a_log, 4) || misaligned(dt_bias, 4) || misaligned(src_slots, 4) ||
      misaligned(dst_slots, 4) || misaligned(n_tokens, 4))
    return KDA_ERR_ALIGN;
  ReplayArgs R;
  R.rec_u = rec_u; R.rec_kg = rec_kg; R.a_log = a_log; R.dt_bias = dt_bias;
  R.src = src_slots; R.dst = dst_slots; R.n = n_tokens; R.state = state;
  R.lower_bound = lower_bound; R.B = B; R.H = H; R.N = N; R.T = T;
  hipLaunchKernelGGL(kda_replay_kernel, dim3(static_cast<unsigned>(B * H)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), R);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}
}  // extern "C"
