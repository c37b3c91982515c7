/*
 * Plain CPU oracle for the Kimi Delta Attention (KDA) decode / verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  It shares no code, header,
 * table or constant with the GPU library, and the GPU library never calls it.
 *
 * What it follows: the vLLM API-reference page for the module
 * vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.wide, class
 * KdaWide -- its class docstring (one (request, head) item per CTA, state read
 * once, written once per token; BF16-rounded convolution outputs, raw gates
 * and recurrence outputs; only the FP32 reduction order is left free), its
 * constructor (tokens in [1, 8], record needs tokens > 1), its kernel body
 * (slot resolution, padding, convolution, gate projection, L2 norm,
 * recurrence, state write-back, convolution window, gated RMSNorm) and its
 * helpers silu and decay.
 *
 * How it computes (the plain reading of that page):
 *   - every FP32 operation the page performs element-wise (a multiply, an add,
 *     an fma) is one correctly rounded IEEE single operation here;
 *   - every transcendental (exp, the sigmoid, the reciprocal square root) is
 *     evaluated in double precision and rounded once to FP32;
 *   - every reduction (sums of squares, dot products, the gate projection) is
 *     accumulated in double precision and rounded once to FP32: the page fixes
 *     FP32 as the accumulation type but leaves the order free, and the nearly
 *     exact sum is the value every order approximates;
 *   - BF16 rounding is round-to-nearest-even from FP32.
 * gate_mode (the constructor's choice between one chain of eight MMAs and
 * four chains of two for the gate projection) selects an accumulation order
 * only: both modes take the exact sum here, so neither chained FP32 order is
 * reproduced -- parity unpinned for that order itself.
 * Built with -O2 -ffp-contract=off so the compiler adds no fused operations:
 * an fma appears only where the page writes one.
 *
 * Single-threaded, no blocking, no fusion: one (request, head) item at a time,
 * one token at a time, one value row at a time.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define D 128 /* head dimension, dk = dv = 128 */
#define TAPS 4
#define MAX_T 8

/* ---- BF16 storage (round-to-nearest-even) ---------------------------- */

static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t float_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static float round_bf16(float f) { return bf16_to_float(float_to_bf16(f)); }

/* ---- helpers of the page ---------------------------------------------- */

/* sigma(x) = 1 / (1 + exp(-x)), evaluated in double and rounded once. */
static float sigmoid_f32(float x) {
  return (float)(1.0 / (1.0 + exp(-(double)x)));
}

/* KdaWide.silu: x / (1 + exp(-x)) in FP32 (exp rounded to FP32, the add and
 * the full-precision divide each an FP32 operation), then stored BF16. */
float kda_oracle_silu_bf16(float x) {
  float e = (float)exp(-(double)x);
  float d = 1.0f + e;
  float y = x / d;
  return round_bf16(y);
}

/* KdaWide.decay: exp(lower_bound * sigmoid(exp(A_log) * (raw_g + dt_bias))),
 * each step an FP32 value. */
float kda_oracle_decay(float a_log, float raw_g, float dt, float lower_bound) {
  float e = (float)exp((double)a_log);
  float z = raw_g + dt;
  float y = e * z;
  float s = sigmoid_f32(y);
  float g = lower_bound * s;
  return (float)exp((double)g);
}

/* 1 / sqrt(x), evaluated in double and rounded once. */
static float rsqrt_f32(float x) { return (float)(1.0 / sqrt((double)x)); }

/* Gated RMSNorm of one token of one head (the kernel's last phase):
 * rstd = (sum(o^2) * (1/128) + eps)^-1/2, out = BF16(((o * rstd) * nw) * sigma(gate)).
 * o_bf: the 128 BF16-rounded recurrence outputs (as floats). */
void kda_oracle_gated_rmsnorm(const float* o_bf, const uint16_t* gate,
                              const uint16_t* norm_w, float eps, uint16_t* out) {
  double ss = 0.0;
  for (int c = 0; c < D; ++c) ss += (double)o_bf[c] * (double)o_bf[c];
  float variance = (float)ss * (1.0f / 128.0f) + eps;
  float rstd = rsqrt_f32(variance);
  for (int c = 0; c < D; ++c) {
    float sg = sigmoid_f32(bf16_to_float(gate[c]));
    float r = ((o_bf[c] * rstd) * bf16_to_float(norm_w[c])) * sg;
    out[c] = float_to_bf16(r);
  }
}

/* ---- the problem ------------------------------------------------------- */

typedef struct kda_oracle_problem {
  /* sizes and switches */
  int B, H, N, W, T, slot_stride, record, has_bias;
  int conv_f32;             /* 1: the convolution pool holds FP32, else BF16 */
  float lower_bound, scale, eps;
  /* operands: host memory, the same layouts as the device library */
  const uint16_t* x;        /* [B*T, 3*H*128] q|k|v before the convolution */
  const uint16_t* conv_w;   /* [3, 4, H*128] */
  const uint16_t* conv_b;   /* [3*H*128], read iff has_bias */
  void* conv_state;         /* [N, 3*H*128, W] BF16 or FP32 (conv_f32), in place */
  const uint16_t* f_a;      /* [B*T, 128] gate low-rank input */
  const uint16_t* beta;     /* [B*T, H] logits */
  const float* a_log;       /* [H] */
  const float* dt_bias;     /* [H*128] */
  const int32_t* slots;     /* [B] (T == 1) or [B, slot_stride] */
  const int32_t* accepted;  /* [B], T > 1 only */
  float* state;             /* [N, H, 128, 128]: [slot][head][value row][key] */
  uint16_t* out;            /* [B*T, H*128] */
  const uint16_t* gate;     /* [B*T, H*128] output-gate logits */
  const uint16_t* norm_w;   /* [128] */
  const uint16_t* f_b;      /* [H*128, 128] gate projection */
  float* rec_u;             /* [B, H, T, 128], record only */
  uint16_t* rec_kg;         /* [B, H, T, 256], record only: k | raw_g */
} kda_oracle_problem;

/* Optional intermediate values, each [B, H, T, 128] (beta: [B, H, T]); any
 * pointer may be NULL.  o_exact is the recurrence output before any rounding
 * (double), o_abs the sum of |S[v][k] * q_hat[k]| over k (its rounding scale). */
typedef struct kda_oracle_taps {
  float *q, *k, *v;        /* BF16-rounded SiLU outputs */
  float *raw_g, *decay;    /* BF16 raw gate, FP32 decay */
  float *beta;             /* FP32 sigmoid(beta logit), [B, H, T] */
  float *q_hat, *k_hat;    /* normalised q (with scale) and k */
  float *u;                /* FP32 delta-rule coefficient per value row */
  double *o_exact, *o_abs; /* recurrence output before rounding, its scale */
  float *o_bf;             /* BF16-rounded recurrence output */
} kda_oracle_taps;

/* Resolve the item's slots as the kernel does.  Returns 1 for a live item.
 * Beyond the page: slots >= N, a convolution slot outside [0, N) and an
 * accepted count outside [1, min(T, slot_stride)] make the item padding
 * (memory safety for tables that break the caller contract). */
static int resolve(const kda_oracle_problem* P, int b, int* read_slot,
                   int* conv_slot, int* offset) {
  if (P->T == 1) {
    *read_slot = P->slots[b];
    *conv_slot = *read_slot;
    *offset = 0;
  } else {
    int acc = P->accepted[b];
    int lim = P->T < P->slot_stride ? P->T : P->slot_stride;
    if (acc < 1 || acc > lim) return 0;
    *offset = acc - 1;
    *read_slot = P->slots[(size_t)b * P->slot_stride + *offset];
    *conv_slot = P->slots[(size_t)b * P->slot_stride];
  }
  if (*read_slot <= 0 || *read_slot >= P->N) return 0;
  if (*conv_slot < 0 || *conv_slot >= P->N) return 0;
  return 1;
}

static size_t tap_index(const kda_oracle_problem* P, int b, int h, int t) {
  return (((size_t)b * P->H + h) * P->T + t) * D;
}

/* One (request, head) item, following the kernel body in its order. */
static void run_item(const kda_oracle_problem* P, int b, int h,
                     const kda_oracle_taps* taps) {
  const int T = P->T, H = P->H, W = P->W;
  const size_t dim = (size_t)H * D;
  const size_t token0 = (size_t)b * T;
  int rs, cs, off;

  /* Slot resolution and padding: a padded item writes BF16 zeros to its T
   * output rows and touches nothing else. */
  if (!resolve(P, b, &rs, &cs, &off)) {
    for (int t = 0; t < T; ++t)
      for (int c = 0; c < D; ++c) P->out[(token0 + t) * dim + (size_t)h * D + c] = 0;
    return;
  }

  float S[D][D]; /* the item's state, [value row][key] */
  const float* page = P->state + (((size_t)rs * H + h) * D) * D;
  memcpy(S, page, sizeof(S));

  /* Short causal convolution over the window
   * [tap0, tap1, tap2, x_0, ..., x_{T-1}] and SiLU, BF16-rounded. */
  float Y[3][MAX_T][D]; /* q, k, v */
  /* The window holds values of the pool's element type (kernel body: the
   * taps are read in that type and the inputs are converted to it); the
   * arithmetic reads them as FP32, which both types convert to exactly. */
  float window[3][D][3 + MAX_T];
  for (int p = 0; p < 3; ++p) {
    for (int c = 0; c < D; ++c) {
      size_t ch = (size_t)p * dim + (size_t)h * D + c;
      size_t base = ((size_t)cs * 3 * dim + ch) * W;
      for (int i = 0; i < 3; ++i) {
        size_t at = base + off + i;
        if (P->conv_f32) window[p][c][i] = ((const float*)P->conv_state)[at];
        else window[p][c][i] = bf16_to_float(((const uint16_t*)P->conv_state)[at]);
      }
      for (int t = 0; t < T; ++t)
        window[p][c][3 + t] = bf16_to_float(P->x[(token0 + t) * 3 * dim + ch]);
      for (int t = 0; t < T; ++t) {
        float acc = P->has_bias ? bf16_to_float(P->conv_b[ch]) : 0.0f;
        for (int i = 0; i < TAPS; ++i) {
          float w = bf16_to_float(P->conv_w[((size_t)p * TAPS + i) * dim + (size_t)h * D + c]);
          acc = fmaf(window[p][c][t + i], w, acc);
        }
        Y[p][t][c] = kda_oracle_silu_bf16(acc);
      }
    }
  }

  /* Gate projection raw_g[t][f] = BF16(sum_j F_B[h*128+f][j] * f_a[t][j]),
   * then the per-key-channel decay, and beta = sigmoid(logit). */
  float raw_g[MAX_T][D], decay[MAX_T][D], beta[MAX_T];
  for (int t = 0; t < T; ++t) {
    const uint16_t* fa = P->f_a + (token0 + t) * D;
    for (int f = 0; f < D; ++f) {
      const uint16_t* row = P->f_b + ((size_t)h * D + f) * D;
      double g = 0.0;
      for (int j = 0; j < D; ++j) g += (double)bf16_to_float(row[j]) * (double)bf16_to_float(fa[j]);
      raw_g[t][f] = round_bf16((float)g);
      decay[t][f] = kda_oracle_decay(P->a_log[h], raw_g[t][f], P->dt_bias[(size_t)h * D + f],
                                     P->lower_bound);
    }
    beta[t] = sigmoid_f32(bf16_to_float(P->beta[(token0 + t) * H + h]));
  }

  /* L2 normalisation: q_hat = (q * (sum q^2 + 1e-6)^-1/2) * scale,
   * k_hat = k * (sum k^2 + 1e-6)^-1/2. */
  float q_hat[MAX_T][D], k_hat[MAX_T][D];
  for (int t = 0; t < T; ++t) {
    double sq = 0.0, sk = 0.0;
    for (int c = 0; c < D; ++c) {
      sq += (double)Y[0][t][c] * (double)Y[0][t][c];
      sk += (double)Y[1][t][c] * (double)Y[1][t][c];
    }
    float fq = rsqrt_f32((float)sq + 1.0e-6f);
    float fk = rsqrt_f32((float)sk + 1.0e-6f);
    for (int c = 0; c < D; ++c) {
      q_hat[t][c] = (Y[0][t][c] * fq) * P->scale;
      k_hat[t][c] = Y[1][t][c] * fk;
    }
  }

  /* The gated delta rule, token by token, value row by value row:
   * s <- s (.) a;  u = (v - s.k_hat) * beta;  s <- s + u k_hat;  o = s.q_hat. */
  float o_bf[MAX_T][D];
  for (int t = 0; t < T; ++t) {
    for (int v = 0; v < D; ++v) {
      float* s = S[v];
      for (int k = 0; k < D; ++k) s[k] = s[k] * decay[t][k];
      double dot = 0.0;
      for (int k = 0; k < D; ++k) dot += (double)s[k] * (double)k_hat[t][k];
      float u = (Y[2][t][v] - (float)dot) * beta[t];
      for (int k = 0; k < D; ++k) s[k] = fmaf(k_hat[t][k], u, s[k]);
      double o = 0.0, oa = 0.0;
      for (int k = 0; k < D; ++k) {
        o += (double)s[k] * (double)q_hat[t][k];
        oa += fabs((double)s[k] * (double)q_hat[t][k]);
      }
      o_bf[t][v] = round_bf16((float)o);
      if (P->record) P->rec_u[tap_index(P, b, h, t) + v] = u;
      if (taps) {
        size_t ti = tap_index(P, b, h, t) + v;
        if (taps->u) taps->u[ti] = u;
        if (taps->o_exact) taps->o_exact[ti] = o;
        if (taps->o_abs) taps->o_abs[ti] = oa;
        if (taps->o_bf) taps->o_bf[ti] = o_bf[t][v];
      }
    }
    if (P->record) {
      /* RecoverSSM records: k (post-SiLU, before the norm) and raw_g, BF16. */
      uint16_t* kg = P->rec_kg + (((size_t)b * H + h) * T + t) * 2 * D;
      for (int c = 0; c < D; ++c) {
        kg[c] = float_to_bf16(Y[1][t][c]);
        kg[D + c] = float_to_bf16(raw_g[t][c]);
      }
    } else {
      /* State write-back: in place for decode, to slots[b, t] for verify;
       * a target <= 0 (or >= N) skips this token's write. */
      int target = T == 1 ? rs : P->slots[(size_t)b * P->slot_stride + t];
      if (target > 0 && target < P->N)
        memcpy(P->state + (((size_t)target * H + h) * D) * D, S, sizeof(S));
    }
  }

  /* Convolution window [tap1, tap2, x_0, ..., x_{T-1}] in the pool's type:
   * every value came from that type or from BF16, so the conversion back is
   * exact and the bits are those read. */
  for (int p = 0; p < 3; ++p) {
    for (int c = 0; c < D; ++c) {
      size_t ch = (size_t)p * dim + (size_t)h * D + c;
      size_t base = ((size_t)cs * 3 * dim + ch) * W;
      for (int j = 0; j < 2 + T; ++j) {
        float v = window[p][c][1 + j];
        if (P->conv_f32) ((float*)P->conv_state)[base + j] = v;
        else ((uint16_t*)P->conv_state)[base + j] = float_to_bf16(v);
      }
    }
  }

  /* Gated RMSNorm output. */
  for (int t = 0; t < T; ++t)
    kda_oracle_gated_rmsnorm(o_bf[t], P->gate + (token0 + t) * dim + (size_t)h * D, P->norm_w,
                             P->eps, P->out + (token0 + t) * dim + (size_t)h * D);

  if (taps) {
    for (int t = 0; t < T; ++t) {
      size_t ti = tap_index(P, b, h, t);
      for (int c = 0; c < D; ++c) {
        if (taps->q) taps->q[ti + c] = Y[0][t][c];
        if (taps->k) taps->k[ti + c] = Y[1][t][c];
        if (taps->v) taps->v[ti + c] = Y[2][t][c];
        if (taps->raw_g) taps->raw_g[ti + c] = raw_g[t][c];
        if (taps->decay) taps->decay[ti + c] = decay[t][c];
        if (taps->q_hat) taps->q_hat[ti + c] = q_hat[t][c];
        if (taps->k_hat) taps->k_hat[ti + c] = k_hat[t][c];
      }
      if (taps->beta) taps->beta[ti / D] = beta[t];
    }
  }
}

/* Checks of the constructor's contract; 0 = fine.  The codes match the
 * page's ValueError (tokens outside [1, 8]) and assertion (gate_mode in
 * {0, 1}; record needs tokens > 1). */
int kda_oracle_check(const kda_oracle_problem* P, int gate_mode) {
  if (P->T < 1 || P->T > MAX_T) return 1;
  if (gate_mode != 0 && gate_mode != 1) return 2;
  if (P->record && P->T == 1) return 3;
  if (P->B < 0 || P->H < 1 || P->N < 1) return 5;
  if (P->W < (P->T == 1 ? 3 : P->T + 2)) return 5;
  if (P->T > 1 && P->slot_stride < P->T) return 5;
  return 0;
}

/* Runs the items listed in `items` (item = b * H + h), or all B*H items when
 * items is NULL.  Items are independent; each touches only its own pages,
 * its own convolution channels and its own output rows. */
int kda_oracle_run(const kda_oracle_problem* P, int gate_mode, const int32_t* items,
                   int n_items, const kda_oracle_taps* taps) {
  int status = kda_oracle_check(P, gate_mode);
  if (status) return status;
  if (items == NULL) {
    for (int b = 0; b < P->B; ++b)
      for (int h = 0; h < P->H; ++h) run_item(P, b, h, taps);
  } else {
    for (int i = 0; i < n_items; ++i) {
      int it = items[i];
      if (it < 0 || it >= P->B * P->H) return 5;
      run_item(P, it / P->H, it % P->H, taps);
    }
  }
  return 0;
}

/* ---- RecoverSSM replay ------------------------------------------------- */

/* After a record-mode verify, the state after the first n accepted tokens is
 * rebuilt from the checkpoint page that verify read and its records, token by
 * token, with the step's own arithmetic:
 *   k_hat = k * (sum k^2 + 1e-6)^-1/2   (k: the recorded BF16 key, pre-norm)
 *   a     = decay(A_log[h], raw_g, dt_bias[h*128 + f], lower_bound)
 *   s     = fmaf(k_hat[key], u[v], s * a[key])   for every (v, key).
 * n = 0 copies the checkpoint.  Items whose slots fall outside [1, N) or whose
 * n falls outside [0, T] are skipped. */
typedef struct kda_oracle_replay_problem {
  int B, H, N, T;
  float lower_bound;
  const float* rec_u;      /* [B, H, T, 128] */
  const uint16_t* rec_kg;  /* [B, H, T, 256]: k | raw_g */
  const float* a_log;      /* [H] */
  const float* dt_bias;    /* [H*128] */
  const int32_t* src;      /* [B] checkpoint slot */
  const int32_t* dst;      /* [B] slot to write */
  const int32_t* n;        /* [B] tokens to apply */
  float* state;            /* [N, H, 128, 128] */
} kda_oracle_replay_problem;

int kda_oracle_replay(const kda_oracle_replay_problem* P) {
  if (P->T < 1 || P->T > MAX_T || P->B < 0 || P->H < 1 || P->N < 1) return 5;
  for (int b = 0; b < P->B; ++b) {
    const int src = P->src[b], dst = P->dst[b], n = P->n[b];
    if (src <= 0 || src >= P->N || dst <= 0 || dst >= P->N || n < 0 || n > P->T) continue;
    for (int h = 0; h < P->H; ++h) {
      float S[D][D];
      memcpy(S, P->state + (((size_t)src * P->H + h) * D) * D, sizeof(S));
      for (int t = 0; t < n; ++t) {
        const size_t rec = ((size_t)b * P->H + h) * P->T + t;
        const uint16_t* kg = P->rec_kg + rec * 2 * D;
        const float* u = P->rec_u + rec * D;
        double sk = 0.0;
        for (int c = 0; c < D; ++c) sk += (double)bf16_to_float(kg[c]) * (double)bf16_to_float(kg[c]);
        const float fk = rsqrt_f32((float)sk + 1.0e-6f);
        float k_hat[D], a[D];
        for (int c = 0; c < D; ++c) {
          k_hat[c] = bf16_to_float(kg[c]) * fk;
          a[c] = kda_oracle_decay(P->a_log[h], bf16_to_float(kg[D + c]),
                                  P->dt_bias[(size_t)h * D + c], P->lower_bound);
        }
        for (int v = 0; v < D; ++v)
          for (int k = 0; k < D; ++k) S[v][k] = fmaf(k_hat[k], u[v], S[v][k] * a[k]);
      }
      memcpy(P->state + (((size_t)dst * P->H + h) * D) * D, S, sizeof(S));
    }
  }
  return 0;
}
