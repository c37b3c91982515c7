// Host side shared by the entry points: packing the operands and the checks
// every call makes before it enqueues anything (the constructor's contract on
// the kda.wide page, plus NULL, shape and alignment checks).
#ifndef KDA_HOST_HPP
#define KDA_HOST_HPP

#include "kda.h"
#include "kda_stages.hpp"

namespace {

bool misaligned(const void* p, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) != 0;
}

kda_status check(const Args& A, int T, int record, int gate_mode) {
  if (T < 1 || T > kMaxT) return KDA_ERR_TOKENS;
  if (gate_mode != 0 && gate_mode != 1) return KDA_ERR_GATE_MODE;
  if (record && T == 1) return KDA_ERR_RECORD_T1;
  if (A.B < 0 || A.H < 1 || A.N < 1) return KDA_ERR_SHAPE;
  if (A.W < (T == 1 ? 3 : T + 2)) return KDA_ERR_SHAPE;
  if (T > 1 && A.slot_stride < T) return KDA_ERR_SHAPE;
  if (!isfinite(A.lower_bound) || !isfinite(A.scale) || !isfinite(A.eps)) return KDA_ERR_SHAPE;
  // Grid and 32-bit index limits: B*H workgroups of kThreads work-items (a
  // dispatch counts its grid in work-items, 32 bits); H*128 channels per row.
  if (static_cast<long long>(A.B) * A.H * kThreads > 0xffffffffLL) return KDA_ERR_SHAPE;
  if (static_cast<long long>(A.H) * 3 * kD * (T + 3) > 0x7fffffffLL) return KDA_ERR_SHAPE;
  if (A.B == 0) return KDA_OK;
  if (!A.x || !A.conv_w || !A.conv_state || !A.f_a || !A.beta || !A.a_log || !A.dt_bias ||
      !A.slots || !A.state || !A.out || !A.gate || !A.norm_w || !A.f_b)
    return KDA_ERR_NULL;
  if (T > 1 && !A.accepted) return KDA_ERR_NULL;
  if (record && (!A.rec_u || !A.rec_kg)) return KDA_ERR_NULL;
  // Alignment the kernels' accesses assume: 16 bytes for the state pool and
  // the gate projection operands (16-byte loads), 4 bytes for the BF16
  // operands moved as channel pairs, the element size for everything else.
  if (misaligned(A.state, 16) || misaligned(A.f_a, 16) || misaligned(A.f_b, 16) ||
      misaligned(A.x, 4) || misaligned(A.conv_w, 4) || misaligned(A.conv_b, 4) ||
      misaligned(A.conv_state, A.conv_f32 ? 4 : 2) || misaligned(A.beta, 2) ||
      misaligned(A.a_log, 4) || misaligned(A.dt_bias, 4) || misaligned(A.slots, 4) ||
      misaligned(A.out, 2) || misaligned(A.gate, 2) || misaligned(A.norm_w, 2) ||
      (T > 1 && misaligned(A.accepted, 4)) ||
      (record && (misaligned(A.rec_u, 4) || misaligned(A.rec_kg, 4))))
    return KDA_ERR_ALIGN;
  return KDA_OK;
}

// The prefetch distance: -1 takes the library default (off: the step is at
// its measured HBM ceiling without it), other values are rounded up to a
// multiple of 8 so that the prefetching workgroup and the one that reads the
// page sit on the same XCD.  A distance of a whole grid or more touches no
// page; it is capped well below the int range.
constexpr int kDefaultAhead = 0;
constexpr int kMaxAhead = 1 << 30;

int resolve_ahead(int ahead) {
  if (ahead < 0) ahead = kDefaultAhead;
  if (ahead > kMaxAhead) ahead = kMaxAhead;
  return (ahead + 7) & ~7;
}

Args pack(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
          void* conv_state, const uint16_t* f_a, const uint16_t* beta, const float* a_log,
          const float* dt_bias, const int32_t* slots, float* state, uint16_t* out,
          const uint16_t* gate, const uint16_t* norm_w, float lower_bound, float scale,
          float eps, const uint16_t* f_b, const int32_t* accepted, float* rec_u,
          uint16_t* rec_kg, int B, int H, int N, int W, int slot_stride, int ahead,
          int conv_f32 = 0) {
  Args A;
  A.x = x; A.conv_w = conv_w; A.conv_b = conv_b; A.conv_state = conv_state; A.f_a = f_a;
  A.beta = beta; A.a_log = a_log; A.dt_bias = dt_bias; A.slots = slots; A.state = state;
  A.out = out; A.gate = gate; A.norm_w = norm_w; A.f_b = f_b; A.accepted = accepted;
  A.rec_u = rec_u; A.rec_kg = rec_kg;
  A.lower_bound = lower_bound; A.scale = scale; A.eps = eps;
  A.B = B; A.H = H; A.N = N; A.W = W; A.slot_stride = slot_stride;
  A.ahead = resolve_ahead(ahead);
  A.conv_f32 = conv_f32;
  return A;
}

}  // namespace

#endif  // KDA_HOST_HPP
