// KDA decode / verify with each (request, head) item split over G
// workgroups, for batches too small to fill the GPU: the C ABI of
// kda_decode_split and kda_verify_split.
//
// Operation: the KdaWide step of the vLLM API page
// vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide (kernel
// body); the split follows the class docstring's KdaSplit, which spreads a
// head over several CTAs when there are few requests and repeats the
// convolution and the gate projection in each.  The argument contract is in
// include/kda.h.
//
// Design.  Workgroup (item, part), part < G, owns value rows
// 32(l >> 4) + 8w + (8/G) part + i, i < 8/G, of the item's page (the
// decode kernel's thread layout and access shape, 8/G rows per lane group
// instead of 8): it reads and writes only those rows of the state.  The rows
// of the recurrence are independent; only the output RMSNorm (a sum over
// all 128 rows) and the convolution window (read by every part, rewritten
// once) cross workgroups.  Both go to the part that finishes last, with no
// waiting, through atomics only:
//   * each part publishes its recurrence outputs o (BF16, two rows per
//     32-bit word) with returning atomic exchanges into the workspace, and
//     waits for their returns: a returned atomic has been performed at the
//     location's point of coherence;
//   * then one atomic add on the item's counter; the part that reads G - 1
//     is the last, and every other part published before it added;
//   * the last part resets the counter, reads the published words back
//     with returning atomics (performed after its counter add, so they see
//     every part's exchange), rewrites the window (every other part had
//     read it before it added), and writes the normalised output.
// No agent-scope fence is used: on gfx950 its L2 write-back (release) and
// invalidate (acquire) serialise across the device and cost more than the
// split gains.  Each part repeats the convolution, the gate projection and
// the decay, which need all 128 channels.
#include <mutex>

#include "kda.h"
#include "kda_host.hpp"

namespace {

// Workspace layout (32-bit words): the item counters [items], then the
// published outputs [items][T][64], word p holding rows 2p (low half) and
// 2p + 1 as BF16.
__device__ __forceinline__ uint32_t* split_words(uint32_t* ws, long long items, int item,
                                                 int T, int t) {
  return ws + items + (static_cast<long long>(item) * T + t) * (kD / 2);
}

// A register value that depends on `v` and is 0: the compiler must have v
// (the returns of the atomics folded into it) before it can use the result.
__device__ __forceinline__ uint32_t zero_after(uint32_t v) {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(v));
  return z;
}

template <int T, bool kBias, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void kda_split_kernel(const Args A, uint32_t* ws) {
  constexpr int kRows = 8 / G;  // rows per lane group
  static_assert(kRows % 2 == 0, "rows are published in pairs");
  const long long items = static_cast<long long>(A.B) * A.H;
  const int item = blockIdx.x / G;
  const int part = blockIdx.x % G;
  // 1. Every operand ahead of the state page (the latency kernel's order).
  Item it;
  locate_item<T>(A, it, item);
  ConvOperands<T> co;
  conv_load_inputs<T, kBias>(A, it, co);
  GateOperands go;
  if constexpr (T == 1) gate_load(A, it, go);
  GateQuadOperands<T> gq;
  if constexpr (T > 1) {
    gate_quad_load_fb<T>(A, it, gq, 0);
    gate_quad_load_fb<T>(A, it, gq, 1);
    gate_quad_load_fa<T>(A, it, gq);
  }
  const float beta_logit = load_beta<T>(A, it);
  const float dt = load_dt(A, it);
  const float a_log = load_a_log(A, it);
  OutputOperands<T> oo;
  load_output_operands<T>(A, it, oo);
  __builtin_amdgcn_sched_barrier(0);
  SlotRow<T> slot_row;
  if (!resolve<T>(A, it, slot_row)) {  // every part sees the same tables
    if (part == 0) write_padding<T>(A, it);
    return;
  }
  __shared__ Shared<T, false> sh;
  __shared__ int last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15;
  const int row0 = 32 * (lane >> 4) + 8 * wave + kRows * part;
  const int lane_off = (row0 * kD + 4 * c16) * 4;
  conv_load_taps<T, false>(A, it, co);
  float4 st[kRows][2];
  {
    const __amdgpu_buffer_rsrc_t page = page_rsrc(A.state, it.rs, it.h, A.H);
#pragma unroll
    for (int i = 0; i < kRows; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) st[i][j] = load_f4(page, lane_off, i * kD * 4 + j * 256);
  }

  // 2. Inputs (the window is left as read: other parts may still read it).
  conv_compute<T, false, false, false>(A, it, sh, co);
  store_beta<T>(sh, beta_logit);
  if constexpr (T == 1)
    gate_valu(go, sh);
  else
    gate_quad_compute<T>(gq, sh);
  __syncthreads();
  decay<T, false>(A, it, sh, dt, a_log);
  __syncthreads();

  // 3. The recurrence on this part's rows (o to the table); the last
  //    token's state is stored after the counter add.
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
    for (int i = 0; i < kRows; ++i) {
      float* s = reinterpret_cast<float*>(&st[i][0]);
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
      if (c16 == 0) sh.o[t][v] = round_bf16(o);
    }
    if (t + 1 < T) {
      const int target = row_slot<T>(slot_row, t);
      if (target > 0 && target < A.N) {
        float* page = page_ptr(A.state, target, it.h, A.H);
#pragma unroll
        for (int i = 0; i < kRows; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) store_f4(page, lane_off + i * kD * 4 + j * 256, st[i][j]);
      }
    }
  }

  // 4. Publish: the part's 64/G words (row pairs) of every token, one
  //    exchange per thread.  Word j of the part holds rows 2w_j, 2w_j + 1
  //    with w_j = 16 lg + 4 wave + (kRows/2) part + m for
  //    j = (4 lg + wave) (kRows/2) + m.  Then the hand-off: every exchange
  //    of the workgroup has returned (zero_after needs its value, and every
  //    wave passes it before the barrier), then one add on the counter.
  __syncthreads();
  constexpr int kWords = kD / 2 / G;
  uint32_t returned = 0;
  if (tid < T * kWords) {
    const int t = tid / kWords, j = tid % kWords;
    const int m = j % (kRows / 2), lw = j / (kRows / 2);  // lw = 4 lg + wave
    const int w = 16 * (lw >> 2) + 4 * (lw & 3) + (kRows / 2) * part + m;
    const uint32_t bits =
        f32_to_bf16_bits(sh.o[t][2 * w]) | (f32_to_bf16_bits(sh.o[t][2 * w + 1]) << 16);
    returned = __hip_atomic_exchange(&split_words(ws, items, item, T, t)[w], bits,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const uint32_t zero = __builtin_amdgcn_readfirstlane(zero_after(returned));
  __syncthreads();
  if (tid == 0) {
    const uint32_t before = __hip_atomic_fetch_add(&ws[item], 1u + zero, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    last = before == static_cast<uint32_t>(G - 1);
  }
  {
    const int target = T == 1 ? it.rs : row_slot<T>(slot_row, T - 1);
    if (target > 0 && target < A.N) {
      float* page = page_ptr(A.state, target, it.h, A.H);
#pragma unroll
      for (int i = 0; i < kRows; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) store_f4(page, lane_off + i * kD * 4 + j * 256, st[i][j]);
    }
  }
  __syncthreads();
  if (!last) return;
  if (tid == 0) __hip_atomic_store(&ws[item], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 5. The last part: the window, then the gated RMSNorm over all rows.
  conv_write_window<T, false>(A, it, co);
  {
    const int p = tid & 63;  // word p of tokens (tid >> 6) + 4m
#pragma unroll
    for (int m = 0; m < (T + 3) / 4; ++m) {
      const int t = (tid >> 6) + 4 * m;
      if (t < T) {
        const uint32_t w = __hip_atomic_fetch_add(&split_words(ws, items, item, T, t)[p], 0u,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.o[t][2 * p] = bf16_lo(w);
        sh.o[t][2 * p + 1] = bf16_hi(w);
      }
    }
  }
  __syncthreads();
  gated_rmsnorm<T>(A, it, sh, sh.o, oo);
}

// ---- host side -------------------------------------------------------------

// The automatic choice (split = 0), from graph-replayed launches at H = 32
// (us per launch, unsplit / 2 parts / 4 parts): T = 1 never pays (32 items
// 6.4 / 7.2 / 7.0: one token's chain is mostly the operand and page round
// trips, which the split does not shorten, plus the three atomic round trips
// of the hand-off); T = 2 breaks even at best (9.5 / 9.9 / 9.4); T = 4 at 32
// items 13.9 / 13.1 / 11.8, at 128 items 15.0 / 14.9 / 16.8; T = 8 at 32 items
// 23.6 / 20.8 / 18.3, at 128 items 24.4 / 23.0 / 25.2.
constexpr long long kSplit4Items = 64;
constexpr long long kSplit2Items = 128;
constexpr int kSplitMinTokens = 4;

int auto_split(long long items, int T) {
  if (T < kSplitMinTokens) return 1;
  if (items <= kSplit4Items) return 4;
  if (items <= kSplit2Items) return 2;
  return 1;
}

template <int T, bool kBias, int G>
kda_status launch_split_g(const Args& A, uint32_t* ws, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(A.B) * A.H * G));
  hipLaunchKernelGGL((kda_split_kernel<T, kBias, G>), grid, dim3(kThreads), 0, stream, A, ws);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

template <int T>
kda_status launch_split_t(const Args& A, int G, uint32_t* ws, hipStream_t stream) {
  const bool bias = A.conv_b != nullptr;
  if (G == 2)
    return bias ? launch_split_g<T, true, 2>(A, ws, stream)
                : launch_split_g<T, false, 2>(A, ws, stream);
  return bias ? launch_split_g<T, true, 4>(A, ws, stream)
              : launch_split_g<T, false, 4>(A, ws, stream);
}

kda_status launch_split(const Args& A, int T, int G, uint32_t* ws, hipStream_t stream) {
  switch (T) {
    case 1: return launch_split_t<1>(A, G, ws, stream);
    case 2: return launch_split_t<2>(A, G, ws, stream);
    case 3: return launch_split_t<3>(A, G, ws, stream);
    case 4: return launch_split_t<4>(A, G, ws, stream);
    case 5: return launch_split_t<5>(A, G, ws, stream);
    case 6: return launch_split_t<6>(A, G, ws, stream);
    case 7: return launch_split_t<7>(A, G, ws, stream);
    case 8: return launch_split_t<8>(A, G, ws, stream);
    default: return KDA_ERR_TOKENS;
  }
}

// Checks of the split arguments beyond the step's own; *G receives the
// workgroups per item (1: no split).
size_t split_bytes(long long B, long long H, int T) {
  return static_cast<size_t>(B * H) * (1 + (kD / 2) * static_cast<size_t>(T)) * sizeof(uint32_t);
}

kda_status check_split(const Args& A, int T, int split, const void* workspace,
                       size_t workspace_bytes, int* G) {
  if (split != 0 && split != 1 && split != 2 && split != 4) return KDA_ERR_SHAPE;
  const long long items = static_cast<long long>(A.B) * A.H;
  *G = split == 0 ? auto_split(items, T) : split;
  if (*G == 1) return KDA_OK;
  if (items * *G * kThreads > 0xffffffffLL) return KDA_ERR_SHAPE;
  if (!workspace || misaligned(workspace, 4) ||
      workspace_bytes < split_bytes(A.B, A.H, T))
    return KDA_ERR_WORKSPACE;
  return KDA_OK;
}

// The step's checks, then the split's; on success *G holds the workgroups
// per item (1: the unsplit kernels run, through kda_decode / kda_verify).
kda_status prepare_split(const Args& A, int T, int gate_mode, int split, const void* workspace,
                         size_t workspace_bytes, int* G) {
  *G = 1;
  const kda_status s = check(A, T, 0, gate_mode);
  if (s != KDA_OK || A.B == 0) return s;
  return check_split(A, T, split, workspace, workspace_bytes, G);
}

// ---- the entry point that allocates nothing ---------------------------------
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the split verify with its workspace in a file-scope device array.
// Each GPU the library runs on holds one copy until the process ends; the
// host finds that GPU's copy with hipGetSymbolAddress on the first call made
// with the device current, and passes that address to the kernels (the
// array's name in host code is only a host-side stand-in).  The counters
// (the first words) start at zero when the code object is loaded, and every
// completed launch leaves them at zero.  Every call on a GPU shares that
// GPU's array: calls that may overlap on one GPU (other streams) race.
constexpr long long kScratchItems = 1024;
constexpr size_t kScratchWords = static_cast<size_t>(kScratchItems) * (1 + (kD / 2) * kMaxT);
static __device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // per device, set once

// The current device's copy of `scratch`, or nullptr (status in *err).
uint32_t* device_scratch(kda_status* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = KDA_ERR_LAUNCH;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *err = KDA_ERR_LAUNCH;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return static_cast<uint32_t*>(g_scratch_ptr[dev]);
}

}  // namespace

extern "C" {

size_t kda_split_workspace_bytes(int B, int H, int T) {
  if (B <= 0 || H <= 0 || T < 1 || T > kMaxT) return 0;
  return split_bytes(B, H, T);
}

kda_status kda_decode_split(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                            uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                            const float* a_log, const float* dt_bias, const int32_t* slots,
                            float* state, uint16_t* out, const uint16_t* gate,
                            const uint16_t* norm_w, float lower_bound, float scale, float eps,
                            const uint16_t* f_b, int B, int H, int N, int W, int gate_mode,
                            int split, void* workspace, size_t workspace_bytes, void* stream) {
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, nullptr, nullptr,
                      nullptr, B, H, N, W, 1, 0);
  int G;
  const kda_status s = prepare_split(A, 1, gate_mode, split, workspace, workspace_bytes, &G);
  if (s != KDA_OK || B == 0) return s;
  if (G == 1)
    return kda_decode(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                      gate, norm_w, lower_bound, scale, eps, f_b, B, H, N, W, gate_mode, -1,
                      stream);
  return launch_split(A, 1, G, static_cast<uint32_t*>(workspace),
                      static_cast<hipStream_t>(stream));
}

kda_status kda_verify_split(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                            uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                            const float* a_log, const float* dt_bias, const int32_t* slots,
                            float* state, uint16_t* out, const uint16_t* gate,
                            const uint16_t* norm_w, float lower_bound, float scale, float eps,
                            const uint16_t* f_b, const int32_t* accepted, int B, int H, int N,
                            int W, int T, int slot_stride, int gate_mode, int split,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (T == 1) return KDA_ERR_TOKENS;  // a one-token step is kda_decode_split
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, accepted, nullptr,
                      nullptr, B, H, N, W, slot_stride, 0);
  int G;
  const kda_status s = prepare_split(A, T, gate_mode, split, workspace, workspace_bytes, &G);
  if (s != KDA_OK || B == 0) return s;
  if (G == 1)
    return kda_verify(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                      gate, norm_w, lower_bound, scale, eps, f_b, accepted, nullptr, nullptr, B,
                      H, N, W, T, slot_stride, 0, gate_mode, -1, stream);
  return launch_split(A, T, G, static_cast<uint32_t*>(workspace),
                      static_cast<hipStream_t>(stream));
}

kda_status kda_verify_split_noalloc(const uint16_t* x, const uint16_t* conv_w,
                                    const uint16_t* conv_b, uint16_t* conv_state,
                                    const uint16_t* f_a, const uint16_t* beta, const float* a_log,
                                    const float* dt_bias, const int32_t* slots, float* state,
                                    uint16_t* out, const uint16_t* gate, const uint16_t* norm_w,
                                    float lower_bound, float scale, float eps,
                                    const uint16_t* f_b, const int32_t* accepted, int B, int H,
                                    int N, int W, int T, int slot_stride, int gate_mode,
                                    int split, void* stream) {
  if (T == 1) return KDA_ERR_TOKENS;
  const Args A = pack(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                      out, gate, norm_w, lower_bound, scale, eps, f_b, accepted, nullptr,
                      nullptr, B, H, N, W, slot_stride, 0);
  kda_status s = check(A, T, 0, gate_mode);
  if (s != KDA_OK || B == 0) return s;
  if (split != 0 && split != 1 && split != 2 && split != 4) return KDA_ERR_SHAPE;
  const long long items = static_cast<long long>(B) * H;
  const int G = split == 0 ? auto_split(items, T) : split;
  if (G == 1)
    return kda_verify(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                      gate, norm_w, lower_bound, scale, eps, f_b, accepted, nullptr, nullptr, B,
                      H, N, W, T, slot_stride, 0, gate_mode, -1, stream);
  if (split_bytes(B, H, T) > sizeof(scratch)) return KDA_ERR_SCRATCH;
  uint32_t* ws = device_scratch(&s);
  if (!ws) return s;
  return launch_split(A, T, G, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
