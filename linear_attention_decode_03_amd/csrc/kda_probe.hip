// A measurement aid for MI355X (gfx950): the state-page traffic of the KDA
// step without its compute, to measure the ceiling that traffic reaches on
// this GPU.  The C ABI of kda_page_copy.
//
// What it reproduces: the kernel body's state load (the item's 64 KiB page
// read once) and state stores (the page written once per stored token), on
// the vLLM API page vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.
// kda.wide; the argument contract is in include/kda.h.  The access shape is
// the step kernels' own: thread (wave w, lane l) moves rows
// 32(l >> 4) + 8w + i (i < 8), keys 4(l & 15) + [0, 4) and 64 + the same,
// 16 bytes per access, non-temporal loads through a per-page buffer resource
// and non-temporal global stores.
#include "kda.h"
#include "kda_device.hpp"

namespace {

struct CopyArgs {
  float* state;
  const int32_t* src;
  const int32_t* dst;
  int n_dst, H, N;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void kda_page_copy_kernel(const CopyArgs C) {
  const int h = blockIdx.x % C.H, b = blockIdx.x / C.H;
  const int src = C.src[b];
  if (src <= 0 || src >= C.N) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = 32 * (lane >> 4) + 8 * wave;
  const int lane_off = (row0 * kD + 4 * (lane & 15)) * 4;
  float4 st[8][2];
  {
    const __amdgpu_buffer_rsrc_t page = page_rsrc(C.state, src, h, C.H);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) st[i][j] = load_f4(page, lane_off, i * kD * 4 + j * 256);
  }
  // With no write the loads still have to happen: their sum feeds a store
  // that a negative n_dst (refused on the host) would take.
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) sum += st[i][j].x + st[i][j].y + st[i][j].z + st[i][j].w;
  if (C.n_dst < 0 && sum == 0.0f) C.state[0] = sum;
  for (int w = 0; w < C.n_dst; ++w) {
    const int dst = C.dst[static_cast<size_t>(b) * C.n_dst + w];
    if (dst <= 0 || dst >= C.N) continue;
    float* page = page_ptr(C.state, dst, h, C.H);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) store_f4(page, lane_off + i * kD * 4 + j * 256, st[i][j]);
  }
}

}  // namespace

extern "C" {

kda_status kda_page_copy(float* state, const int32_t* src_slots, const int32_t* dst_slots,
                         int n_dst, int B, int H, int N, void* stream) {
  if (B < 0 || H < 1 || N < 1 || n_dst < 0 || n_dst > KDA_MAX_TOKENS) return KDA_ERR_SHAPE;
  if (static_cast<long long>(B) * H * kThreads > 0xffffffffLL) return KDA_ERR_SHAPE;
  if (B == 0) return KDA_OK;
  if (!state || !src_slots || (n_dst > 0 && !dst_slots)) return KDA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(state) & 15) || (reinterpret_cast<uintptr_t>(src_slots) & 3) ||
      (reinterpret_cast<uintptr_t>(dst_slots) & 3))
    return KDA_ERR_ALIGN;
  CopyArgs C;
  C.state = state; C.src = src_slots; C.dst = dst_slots; C.n_dst = n_dst; C.H = H; C.N = N;
  hipLaunchKernelGGL(kda_page_copy_kernel, dim3(static_cast<unsigned>(B * H)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), C);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // extern "C"
