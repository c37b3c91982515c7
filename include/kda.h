/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention decode / verify step.
 *
 * The operation is the one the vLLM API page
 * vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide (class KdaWide)
 * defines: for every (request b, head h) item, read the item's 128x128 FP32
 * recurrent state from a slot-indexed pool and advance it through T tokens
 * (T = 1: decode; T in [2, 8]: speculative verify).  Per token:
 *   - a 4-tap causal convolution over the q, k and v channels against the
 *     per-slot convolution window, then SiLU, rounded to BF16;
 *   - q and k L2-normalised (1e-6 added to the sum of squares), q scaled;
 *   - the gate projection raw_g = BF16(F_B[h] . f_a) and the per-key-channel
 *     decay a = exp(lower_bound * sigmoid(exp(A_log[h]) * (raw_g + dt_bias)));
 *   - beta = sigmoid(beta logit);
 *   - the gated delta rule on the state S[v][k] (value row v, key k):
 *       S <- S (.) a (along keys);  u_v = beta (v_v - S_v . k_hat);
 *       S_v <- S_v + u_v k_hat;    o_v = S_v . q_hat, rounded to BF16;
 *   - a gated RMSNorm: out = BF16(((o * rstd) * norm_w) * sigmoid(gate)),
 *     rstd = (sum(o^2) / 128 + eps)^-1/2.
 * The convolution window is rewritten to [tap1, tap2, x_0, ..., x_{T-1}].
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer owned by the caller; BF16 operands are
 *     passed as uint16_t bit patterns.  All tensors are contiguous, row-major,
 *     in the layouts given below.  The library allocates nothing, keeps no
 *     state between calls (kda_verify_split_noalloc's file-scope device
 *     array aside) and never synchronises.
 *   - `stream` is a hipStream_t (NULL = the default stream).  The call
 *     validates its arguments on the host, then enqueues one kernel on
 *     `stream` and returns; buffers must stay alive until the stream passes.
 *   - `state` and `conv_state` are updated in place; `out`, `rec_u` and
 *     `rec_kg` are written; everything else is read only.  `out`, `rec_u`
 *     and `rec_kg` must not alias any input.
 *   - Alignment: state, f_a and f_b on 16 bytes (16-byte vector accesses);
 *     x, conv_w, conv_b and rec_kg on 4 bytes (BF16 channel pairs moved as
 *     one 32-bit word); every other operand on its element size.  Tensors
 *     from a device allocator (and their row slices) satisfy this; a call
 *     that does not returns KDA_ERR_ALIGN.
 *   - Errors: on any non-OK status nothing is enqueued, except KDA_ERR_LAUNCH
 *     (the launch itself failed).  B = 0 is a successful no-op.
 *   - Caller contract, not checked on the device: the live read slots and
 *     write targets are pairwise distinct across requests (a request may read
 *     and write the same slot), and each live request's convolution slot is
 *     its own.  Tables that break the range rules below never make the kernel
 *     touch memory outside the pools: such an item is treated as padding.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128   /* dk = dv = 128 */
#define KDA_CONV_TAPS 4
#define KDA_MAX_TOKENS 8

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_TOKENS = 1,     /* T outside [1, 8] (the page's ValueError) */
  KDA_ERR_GATE_MODE = 2,  /* gate_mode not 0 or 1 (the page's assertion) */
  KDA_ERR_RECORD_T1 = 3,  /* record with T = 1 (the page's assertion) */
  KDA_ERR_NULL = 4,       /* a required pointer is NULL */
  KDA_ERR_SHAPE = 5,      /* B < 0, H < 1, N < 1, W too small, slot_stride < T,
                             non-finite scalar, or sizes beyond 32-bit grids
                             (B*H*256 work-items above 2^32 - 1) */
  KDA_ERR_LAUNCH = 6,     /* the kernel launch failed (hipGetLastError) */
  KDA_ERR_ALIGN = 7,      /* a pointer not aligned as its operand needs (see the
                             alignment convention above) */
  KDA_ERR_WORKSPACE = 8,  /* a split call's workspace is NULL, smaller than
                             kda_split_workspace_bytes or not 4-byte aligned */
  KDA_ERR_SCRATCH = 9     /* kda_verify_split_noalloc: the split the call needs
                             does not fit the library's static scratch
                             (B*H*(1 + 64*T) 32-bit words above 1024*(1 + 64*8)) */
} kda_status;

/*
 * kda_decode -- one decode step, T = 1 (KdaWide with tokens = 1).
 *
 * Slot resolution (the kernel body's first lines on the page): for request b,
 * slot = slots[b] is both the state slot and the convolution slot; slot <= 0
 * marks padding: the H*128 output values of the request are set to BF16 +0
 * and nothing else is read or written for it.  Live slots must lie in
 * [1, N); a slot >= N is treated as padding.
 *
 *   x          [B, 3*H*128]      BF16  q | k | v channels before the convolution
 *   conv_w     [3, 4, H*128]     BF16  (part, tap, channel); tap 0 multiplies the oldest entry
 *   conv_b     [3*H*128] or NULL BF16  convolution bias (NULL: none)
 *   conv_state [N, 3*H*128, W]   BF16  per-slot window, W >= 3, in place
 *   f_a        [B, 128]          BF16  low-rank gate input
 *   beta       [B, H]            BF16  beta logits
 *   a_log      [H]               FP32
 *   dt_bias    [H*128]           FP32
 *   slots      [B]               INT32
 *   state      [N, H, 128, 128]  FP32  (slot, head, value row, key), in place
 *   out        [B, H*128]        BF16
 *   gate       [B, H*128]        BF16  output-gate logits
 *   norm_w     [128]             BF16  RMSNorm weight
 *   lower_bound, scale, eps            decay bound, q scale (1/sqrt(128)), RMSNorm eps
 *   f_b        [H*128, 128]      BF16  gate projection
 *   gate_mode  0 or 1: the accumulation structure of the gate projection
 *              (0: one chain, 1: four chains over 32-column quarters).  This
 *              library accumulates the projection exactly, so both modes
 *              give the same bits (the correctly rounded FP32 sum).
 *   ahead      prefetch distance in items: each workgroup touches the state
 *              page of the item that many positions later (rounded up to a
 *              multiple of 8).  A hint only; results are identical for every
 *              value.  -1 takes the library default (off).
 */
kda_status kda_decode(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                      uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                      const float* a_log, const float* dt_bias, const int32_t* slots,
                      float* state, uint16_t* out, const uint16_t* gate,
                      const uint16_t* norm_w, float lower_bound, float scale, float eps,
                      const uint16_t* f_b, int B, int H, int N, int W, int gate_mode,
                      int ahead, void* stream);

/*
 * kda_verify -- one speculative-verify step over T in [2, 8] tokens
 * (KdaWide with tokens = T, optionally record = RecoverSSM).
 *
 * The same operands as kda_decode, with x, f_a, beta, gate and out holding
 * B*T rows (row b*T + t is token t of request b) and slots of shape
 * [B, slot_stride], slot_stride >= T.  Slot resolution (the page's verify
 * branch): offset = accepted[b] - 1, the state is read from
 * slots[b, offset], the convolution window of slots[b, 0] is read at columns
 * offset .. offset+2 and rewritten at columns 0 .. T+1 (so W >= T + 2).
 * A read slot <= 0 marks padding (B*T output rows of BF16 +0, nothing else
 * touched).  Without record, the state after token t is written to
 * slots[b, t] when that entry is in [1, N) and skipped otherwise.  With
 * record, no state is written; instead
 *   rec_u  [B, H, T, 128]  FP32  u of every value row and token
 *   rec_kg [B, H, T, 256]  BF16  k (after SiLU, before the norm) | raw_g
 * are written for live items (padded items leave them untouched), from which
 * the state after any accepted prefix can be rebuilt from the checkpoint page
 * that was read.
 *   accepted [B] INT32, 1 <= accepted[b] <= T (a value outside that range
 *            makes the item padding).
 */
kda_status kda_verify(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                      uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                      const float* a_log, const float* dt_bias, const int32_t* slots,
                      float* state, uint16_t* out, const uint16_t* gate,
                      const uint16_t* norm_w, float lower_bound, float scale, float eps,
                      const uint16_t* f_b, const int32_t* accepted, float* rec_u,
                      uint16_t* rec_kg, int B, int H, int N, int W, int T, int slot_stride,
                      int record, int gate_mode, int ahead, void* stream);

/*
 * kda_decode_f32conv, kda_verify_f32conv -- kda_decode and kda_verify for a
 * convolution pool held in FP32 (the kernel body reads the window taps in
 * the pool's element type and writes the window back in it).  Arguments as
 * for kda_decode / kda_verify except
 *   conv_state  [N, 3*H*128, W] FP32: taps enter the convolution unrounded;
 *               the window is rewritten [tap1, tap2, x_0, ..] with each BF16
 *               input stored as its exact FP32 value.
 * Everything else (layouts, ownership, errors, caller contract) is the same.
 */
kda_status kda_decode_f32conv(const uint16_t* x, const uint16_t* conv_w,
                              const uint16_t* conv_b, float* conv_state, const uint16_t* f_a,
                              const uint16_t* beta, const float* a_log, const float* dt_bias,
                              const int32_t* slots, float* state, uint16_t* out,
                              const uint16_t* gate, const uint16_t* norm_w, float lower_bound,
                              float scale, float eps, const uint16_t* f_b, int B, int H, int N,
                              int W, int gate_mode, int ahead, void* stream);

kda_status kda_verify_f32conv(const uint16_t* x, const uint16_t* conv_w,
                              const uint16_t* conv_b, float* conv_state, const uint16_t* f_a,
                              const uint16_t* beta, const float* a_log, const float* dt_bias,
                              const int32_t* slots, float* state, uint16_t* out,
                              const uint16_t* gate, const uint16_t* norm_w, float lower_bound,
                              float scale, float eps, const uint16_t* f_b,
                              const int32_t* accepted, float* rec_u, uint16_t* rec_kg, int B,
                              int H, int N, int W, int T, int slot_stride, int record,
                              int gate_mode, int ahead, void* stream);

/*
 * kda_decode_split, kda_verify_split -- kda_decode and kda_verify (plain
 * verify, no record mode) for small batches: each (request, head) item is
 * split over `split` workgroups, each owning 128/split value rows of the
 * state (the KdaSplit of the KdaWide class docstring, which spreads a head
 * over several CTAs when there are few requests).  The results are those of
 * kda_decode / kda_verify (the same roundings; only the FP32 order of the
 * recurrence's dot products may differ).  Operands, layouts, ownership,
 * errors and caller contract as for kda_decode / kda_verify, with a BF16
 * convolution pool, plus:
 *   split      workgroups per item: 2 or 4; 1 runs the unsplit kernels
 *              (kda_decode / kda_verify with the default prefetch); 0 lets
 *              the library choose from B*H and T (measured on MI355X: no
 *              split below 4 tokens; for T >= 4, 4 up to 64 items, 2 up to
 *              128, 1 above).  Other values: KDA_ERR_SHAPE.
 *   workspace  device memory of at least kda_split_workspace_bytes(B, H, T)
 *              bytes, 4-byte aligned.  Its first B*H 32-bit words are one
 *              counter per item and must be ZERO before the first use; every
 *              launch leaves them zero again when it completes, so one
 *              workspace serves any number of calls in a stream.  The rest
 *              holds the items' recurrence outputs between the workgroups of
 *              an item (no initial value needed).  Calls that may run at the
 *              same time (other streams) need workspaces of their own.  Not
 *              read when the chosen split is 1 (may then be NULL).
 * The last workgroup of an item to finish writes the item's convolution
 * window and its normalised output; the workgroups hand over through
 * atomics on the workspace, with no waiting.  kda_split_workspace_bytes
 * returns 0 for B or H below 1 or T outside [1, 8].
 */
size_t kda_split_workspace_bytes(int B, int H, int T);

kda_status kda_decode_split(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                            uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                            const float* a_log, const float* dt_bias, const int32_t* slots,
                            float* state, uint16_t* out, const uint16_t* gate,
                            const uint16_t* norm_w, float lower_bound, float scale, float eps,
                            const uint16_t* f_b, int B, int H, int N, int W, int gate_mode,
                            int split, void* workspace, size_t workspace_bytes, void* stream);

kda_status kda_verify_split(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                            uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                            const float* a_log, const float* dt_bias, const int32_t* slots,
                            float* state, uint16_t* out, const uint16_t* gate,
                            const uint16_t* norm_w, float lower_bound, float scale, float eps,
                            const uint16_t* f_b, const int32_t* accepted, int B, int H, int N,
                            int W, int T, int slot_stride, int gate_mode, int split,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_verify_split_noalloc -- kda_verify_split for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same operands and results without
 * the workspace argument.  The workspace is a file-scope device array of the
 * library, 1024*(1 + 64*8) 32-bit words (2.0 MiB) per GPU, held until the
 * process ends; its address is looked up (hipGetSymbolAddress) on the first
 * call made with a given device current, the only set-up, and nothing is
 * allocated or freed.  A call whose split needs more than the array holds
 * (B*H*(1 + 64*T) words) returns KDA_ERR_SCRATCH before any device work;
 * one that runs unsplit (split 1, or the library's choice) needs none and
 * runs kda_verify.  Every call on one GPU shares that GPU's array: calls that
 * may run at the same time on one GPU (other streams) race and must not
 * overlap.  The counters in the array start at zero and every completed
 * launch leaves them at zero.
 */
kda_status kda_verify_split_noalloc(const uint16_t* x, const uint16_t* conv_w,
                                    const uint16_t* conv_b, uint16_t* conv_state,
                                    const uint16_t* f_a, const uint16_t* beta, const float* a_log,
                                    const float* dt_bias, const int32_t* slots, float* state,
                                    uint16_t* out, const uint16_t* gate, const uint16_t* norm_w,
                                    float lower_bound, float scale, float eps,
                                    const uint16_t* f_b, const int32_t* accepted, int B, int H,
                                    int N, int W, int T, int slot_stride, int gate_mode,
                                    int split, void* stream);

/*
 * kda_replay -- RecoverSSM: the state after the first n accepted tokens of a
 * record-mode kda_verify, rebuilt from the checkpoint page that verify read
 * and the records it wrote (the KdaWide class docstring's RecoverSSM mode;
 * the replay itself is not shown on the page).  Per token t < n[b], with the
 * step's own operations:
 *   k_hat = k (sum k^2 + 1e-6)^-1/2      k = rec_kg[b, h, t, 0:128]
 *   a     = exp(lower_bound * sigmoid(exp(A_log[h]) * (raw_g + dt_bias)))
 *                                         raw_g = rec_kg[b, h, t, 128:256]
 *   S[v][key] <- k_hat[key] u[v] + S[v][key] a[key]   u = rec_u[b, h, t, :]
 *
 *   rec_u     [B, H, T, 128] FP32, rec_kg [B, H, T, 256] BF16 (as written
 *             by kda_verify with record; T its token count)
 *   a_log [H], dt_bias [H*128] FP32; lower_bound as given to kda_verify
 *   src_slots [B]  checkpoint slot of each request (the slot verify read)
 *   dst_slots [B]  slot that receives the state after n tokens (may equal
 *                  the request's own src_slots entry: in place)
 *   n_tokens  [B]  0 <= n <= T; n = 0 copies the checkpoint
 *   state     [N, H, 128, 128] FP32
 * A request whose src or dst lies outside [1, N) or whose n lies outside
 * [0, T] is skipped (nothing is written for it).  Caller contract: the dst
 * slots are distinct across requests and no dst is another request's src.
 * Status: KDA_ERR_TOKENS for T outside [1, 8]; KDA_ERR_SHAPE, KDA_ERR_NULL,
 * KDA_ERR_ALIGN (state on 16 bytes, the rest on their element size),
 * KDA_ERR_LAUNCH as for the other entry points.
 */
kda_status kda_replay(const float* rec_u, const uint16_t* rec_kg, const float* a_log,
                      const float* dt_bias, const int32_t* src_slots, const int32_t* dst_slots,
                      const int32_t* n_tokens, float* state, float lower_bound, int B, int H,
                      int N, int T, void* stream);

/*
 * kda_page_copy -- a measurement aid, not a step of the method: the state-page
 * traffic of the step (the kernel body's one read of an item's 64 KiB page
 * and one write per stored token) without the compute, in the step kernels'
 * access shape, to measure what that traffic alone reaches on the GPU.  For
 * every (request b, head h): read page state[src_slots[b], h] and write it
 * unchanged to state[dst_slots[b*n_dst + w], h] for w < n_dst (n_dst = 1:
 * the decode pattern, in place when dst = src; n_dst = T: the verify
 * pattern; 0: reads only).  A src slot outside [1, N) skips the request, a
 * dst slot outside [1, N) skips that write.  Caller contract: the dst pages
 * are distinct across requests and no dst is another request's src.
 * Status: KDA_ERR_SHAPE (B < 0, H < 1, N < 1, n_dst outside [0, 8], grid
 * beyond 32 bits), KDA_ERR_NULL, KDA_ERR_ALIGN (state on 16 bytes, tables on
 * 4), KDA_ERR_LAUNCH; B = 0 is a no-op.
 */
kda_status kda_page_copy(float* state, const int32_t* src_slots, const int32_t* dst_slots,
                         int n_dst, int B, int H, int N, void* stream);

/*
 * kda_validate -- the host-side checks of kda_verify (T = 1 checks a decode
 * call, with slot_stride and accepted ignored) without enqueuing anything.
 * Touches no device memory and makes no HIP call: usable without a GPU.
 */
kda_status kda_validate(const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                        uint16_t* conv_state, const uint16_t* f_a, const uint16_t* beta,
                        const float* a_log, const float* dt_bias, const int32_t* slots,
                        float* state, uint16_t* out, const uint16_t* gate,
                        const uint16_t* norm_w, float lower_bound, float scale, float eps,
                        const uint16_t* f_b, const int32_t* accepted, float* rec_u,
                        uint16_t* rec_kg, int B, int H, int N, int W, int T,
                        int slot_stride, int record, int gate_mode);

/* A static, human-readable name for a status code. */
const char* kda_status_string(kda_status status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
