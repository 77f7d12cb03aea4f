/*
 * dma.h -- C ABI of libdma.so, the MI355X (gfx950) forward hot path of Doge's
 * Dynamic Mask Attention (DMA).
 *
 * The operations follow the gitcode page "Transformers 中的 Doge 小语言模型完全指南：
 * 动态掩码注意力（DMA）与跨域 MoE（CDMoE）架构解析与实战" (the "Doge guide"), section
 * "动态掩码注意力（DMA）：从缓存 value states 生成稀疏掩码", forward chain steps 3
 * (dt from the value states, the broadcast dynamic mask and its top-k
 * sparsification) and 4 (attention with head_dim**-0.5 scaling and an fp32
 * softmax), with keep_window_size and num_key_value_heads from the DogeConfig
 * table of the same page (section "DogeConfig 全参数详解").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers to caller-owned memory, dense
 *    row-major in the layout stated per argument.  The library never
 *    allocates, frees, or keeps a pointer after the call returns.
 *  - Layouts: Q [B][S][Hq][d], K/V [B][S][Hkv][d] (token-major, heads
 *    interleaved, as a projection writes them); dt, tau, tie [B][Hkv][S].
 *  - dtype is DMA_F32 or DMA_BF16 and applies to Q, K, V, O, W and bias; A,
 *    dt and tau are always float32, tie and lengths int32.
 *  - Query head hq reads kv head hq / (Hq / Hkv) (contiguous GQA groups).
 *  - Causal: query row i sees keys j <= i.  Right padding: with a lengths
 *    array, batch b has L_b valid positions (1 <= L_b <= S); keys j >= L_b are
 *    masked and query rows i >= L_b produce zeros.  A NULL lengths array
 *    means L_b = S for every batch.  A length outside [0, S] breaks this
 *    contract; the kernels clamp it into [0, S], so it never makes them read
 *    or write past the rows it bounds (the same holds for cache lengths
 *    against Lmax).
 *  - Top-w selection order: larger dt first; among equal dt the lower key
 *    index first.  dt values of valid keys must not be NaN (the method's
 *    exp(.) never produces one); -0.0 and +0.0 compare equal.
 *  - Every call validates its arguments on the host before any HIP call and
 *    returns a dma_status; on error nothing is enqueued.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL is the default stream) and the call returns
 *    without synchronising; kernel faults surface at the caller's next
 *    synchronisation.  The library has no global mutable state; calls are
 *    thread-safe.
 */
#ifndef DMA_H_
#define DMA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dma_status {
    DMA_OK = 0,
    DMA_ERR_NULL = -1,        /* a required pointer is NULL */
    DMA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    DMA_ERR_DTYPE = -3,       /* dtype is not DMA_F32 / DMA_BF16 */
    DMA_ERR_UNSUPPORTED = -4, /* valid request outside what the kernels implement */
    DMA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
    DMA_ERR_HIP = -6          /* the HIP runtime reported an error at launch */
} dma_status;

typedef enum dma_dtype { DMA_F32 = 0, DMA_BF16 = 1 } dma_dtype;

/* Operations, for dma_workspace_bytes. */
typedef enum dma_op {
    DMA_OP_DT = 0,          /* dma_dt: no workspace */
    DMA_OP_SELECT = 1,      /* dma_select: no workspace */
    DMA_OP_ATTN_FWD = 2,    /* dma_attn_fwd: no workspace */
    DMA_OP_DECODE = 3,      /* dma_decode (S is the cache length Lmax) */
    DMA_OP_DECODE_STEP = 4, /* dma_decode_step and dma_decode_state_init (S unused) */
    DMA_OP_ATTN_BWD = 5,    /* dma_attn_bwd */
    DMA_OP_DT_BWD = 6       /* dma_dt_bwd (Hq and w unused) */
} dma_op;

/* Version of this ABI (major * 100 + minor). */
int dma_version(void);

/* Static text for a status code. */
const char *dma_status_str(int status);

/*
 * dma_workspace_bytes -- bytes of caller-provided device workspace that
 * operation `op` (a dma_op) needs for these sizes: 0 for the operations that
 * need none (dma_dt, dma_select, dma_attn_fwd, which therefore take no
 * workspace argument), the figure of the per-operation query otherwise
 * (dma_decode_workspace_bytes, dma_decode_step_workspace_bytes,
 * dma_attn_bwd_workspace_bytes, dma_dt_bwd_workspace_bytes).  Returns
 * (size_t)-1 for an unknown op or sizes the operation rejects.
 */
size_t dma_workspace_bytes(int op, int B, int S, int Hq, int Hkv, int d, int w);

/*
 * dma_dt -- Doge guide, DMA forward step 3, first two bullets: dt_proj maps
 * the value states to num_key_value_heads scores per token, then
 * dt = exp(A * softplus(.)).  dt_proj reads all kv heads of one token,
 * concatenated head-major (input width Hkv*d).
 *
 *   V       [B][S][Hkv][d]  dtype   value states
 *   W       [Hkv][Hkv*d]    dtype   dt_proj weight (row h -> kv head h)
 *   bias    [Hkv] dtype, or NULL (no bias)
 *   A       [Hkv]           float32 per-kv-head scale
 *   dt_out  float32; the result for (b, h, s) is written to
 *           dt_out[(b*Hkv + h)*ld_out + (out_pos ? out_pos[b] : 0) + s]
 *   ld_out  row stride of dt_out in elements (>= S; >= out_pos[b] + S)
 *   out_pos [B] int32 device array or NULL: first column written per batch.
 *           A decode step appends the new token's dt to a [B][Hkv][Lmax]
 *           dt cache with S = 1, ld_out = Lmax, out_pos[b] = L_b - 1.
 * Accumulation, softplus and exp are float32.  Supports Hkv <= 16,
 * d in {64, 128}.
 */
int dma_dt(const void *V, const void *W, const void *bias, const float *A, int dtype,
           int B, int S, int Hkv, int d, float *dt_out, int64_t ld_out,
           const int32_t *out_pos, void *stream);

/*
 * dma_select -- Doge guide, DMA forward step 3, third bullet: every query row
 * keeps the keep_window_size (= w) keys of largest dt among its valid keys and
 * masks the rest; rows with at most w valid keys keep them all.
 *
 * The kept set of row i is encoded by a threshold pair: (tau[i], tie[i]) is
 * the dt and index of the last (w-th) kept key, and key j is kept exactly when
 * j is valid and (dt[j] > tau[i] or (dt[j] == tau[i] and j <= tie[i])).
 * Canonical forms: (-inf, -1) when row i has at most w valid keys; (+inf, -1)
 * for a padded row (i >= L_b).  The pair is exact: no floating-point
 * arithmetic is done on dt, only comparisons.
 *
 *   dt      [B][Hkv][S] float32
 *   seqlens [B] int32 or NULL
 *   tau     [B][Hkv][S] float32 (out), tie [B][Hkv][S] int32 (out)
 * Needs no workspace.  B * Hkv * ceil(S / 64) must stay below 2^31 (else
 * DMA_ERR_UNSUPPORTED).
 */
int dma_select(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w,
               float *tau, int32_t *tie, void *stream);

/*
 * dma_attn_fwd -- Doge guide, DMA forward step 4 with the mask of step 3:
 * for query head hq of batch b at row i < L_b, with g = hq / (Hq/Hkv),
 *   s_j = d**-0.5 * (q_i . k_j) + dt[b][g][j]    over the kept keys j of row i
 *   o_i = sum_j softmax(s)_j v_j                 (softmax in float32)
 * Rows i >= L_b are written as zeros.  The kept set comes from (tau, tie) as
 * produced by dma_select for the same dt, seqlens and w.
 *
 *   Q [B][S][Hq][d], K/V [B][S][Hkv][d] dtype; dt/tau/tie [B][Hkv][S]
 *   O [B][S][Hq][d] dtype (out)
 *   w  keep_window_size used to produce (tau, tie)
 * bf16 runs on matrix cores with float32 accumulation; the softmax weights
 * are rounded once to bf16 for the weighted sum of V and the output is
 * rounded to nearest-even.  Supports d in {64, 128}, Hq/Hkv <= 128.
 * Needs no workspace.
 */
int dma_attn_fwd(const void *Q, const void *K, const void *V, int dtype, const float *dt,
                 const float *tau, const int32_t *tie, const int32_t *seqlens, int B,
                 int S, int Hq, int Hkv, int d, int w, void *O, void *stream);

/*
 * dma_decode_workspace_bytes -- bytes of device workspace dma_decode needs
 * for these sizes (0 on invalid sizes).
 */
size_t dma_decode_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int d, int w);

/*
 * dma_decode -- one decode step per batch: the query of batch b sits at
 * position L_b - 1 (L_b = cache_lens[b]) and attends over the cached keys
 * j < L_b that the top-w rule keeps (all of them when L_b <= w), using the
 * per-position dt cache.  The dt of a position depends only on that
 * position's cached value state (Doge guide, DMA forward step 3, remark that
 * dt is projected from the cached value states), so the cache holds exactly
 * what re-projecting every cached value each step would give.
 *
 *   q          [B][Hq][d] dtype
 *   Kc, Vc     [B][Lmax][Hkv][d] dtype
 *   dt_cache   [B][Hkv][Lmax] float32
 *   cache_lens [B] int32, each in [1, Lmax]
 *   out        [B][Hq][d] dtype (out)
 *   kept_idx   [B][Hkv][w] int32 (out) or NULL: kept positions ascending,
 *              padded with -1 when L_b < w
 *   ws, ws_bytes  device workspace of at least dma_decode_workspace_bytes()
 * Supports d in {64, 128}, Hq/Hkv <= 16, min(Lmax, w) <= 131072.
 */
int dma_decode(const void *q, const void *Kc, const void *Vc, int dtype,
               const float *dt_cache, const int32_t *cache_lens, int B, int Lmax, int Hq,
               int Hkv, int d, int w, void *out, int32_t *kept_idx, void *ws,
               size_t ws_bytes, void *stream);

/*
 * dma_decode_noalloc -- dma_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments without ws / ws_bytes, the same
 * kernels and results.  Its workspace is a static device array of 16 MiB
 * per device, part of the library's code object and held until the process
 * ends; sizes whose dma_decode_workspace_bytes() exceeds 16 MiB are rejected
 * with DMA_ERR_WORKSPACE before anything is enqueued (the decode workload
 * of B = 64, Lmax = 16384, Hq = 8, Hkv = 2, d = 128, w = 2048 needs about
 * 10 MiB).  The call itself allocates nothing: its first call on a device
 * looks up that device's copy of the array.  All calls on one device share
 * the array, so calls that overlap in time on one device (on different
 * streams, or from different threads without ordering) race and must not
 * be issued; calls ordered on one stream are safe, and each call writes
 * every part of the array it reads.
 */
int dma_decode_noalloc(const void *q, const void *Kc, const void *Vc, int dtype,
                       const float *dt_cache, const int32_t *cache_lens, int B, int Lmax, int Hq,
                       int Hkv, int d, int w, void *out, int32_t *kept_idx, void *stream);

/*
 * Incremental decode -- Doge guide, DMA section, forward steps 3 and 4 at
 * inference, one token at a time.  The kept sets nest (under dt desc, index
 * asc, the kept set of position p is a subset of that of p-1 plus {p}), so
 * a state that holds each (batch, kv head)'s kept keys -- their selection
 * keys, positions and K/V rows, compacted into w slots -- is enough to
 * decode the next token exactly: the new key enters iff fewer than w keys
 * are kept or it beats the worst kept key (a tie in dt loses), and then
 * replaces it.  A step reads the w kept rows per kv head, not the cache.
 * bf16 only (DMA_BF16); d in {64, 128}; Hq/Hkv <= 16.
 *
 * dma_decode_state_bytes -- bytes of the state for these sizes (0 on
 * invalid sizes).  The state is caller-owned device memory, 16-byte aligned,
 * written only by dma_decode_state_init and dma_decode_step.
 */
size_t dma_decode_state_bytes(int B, int Hkv, int d, int w);

/*
 * dma_decode_step_workspace_bytes -- device workspace of dma_decode_step and
 * dma_decode_state_init (0 on invalid sizes).
 */
size_t dma_decode_step_workspace_bytes(int B, int Hq, int Hkv, int d, int w);

/*
 * dma_decode_state_init -- the state of a cache of cache_lens[b] positions
 * (0 <= cache_lens[b] <= Lmax): the kept set of its last position, found
 * exactly as dma_decode does, with the K/V rows copied into the slots.
 *   Kc, Vc [B][Lmax][Hkv][d] bf16, dt_cache [B][Hkv][Lmax] float32,
 *   cache_lens [B] int32; state/ws of at least the sizes above.
 */
int dma_decode_state_init(const void *Kc, const void *Vc, int dtype, const float *dt_cache,
                          const int32_t *cache_lens, int B, int Lmax, int Hkv, int d, int w,
                          void *state, size_t state_bytes, void *ws, size_t ws_bytes, void *stream);

/*
 * dma_decode_step -- appends one token per batch at position L_b (the
 * state's length) and decodes it: out[b] = the attention of q[b] over the
 * kept keys of positions <= L_b, exactly what dma_decode returns for the
 * cache extended by that token with cache_lens = L_b + 1.  The state then
 * describes the extended cache.
 *   q [B][Hq][d], k_new / v_new [B][Hkv][d] bf16 (the new token's rows),
 *   dt_new [B][Hkv] float32 (its dt, e.g. from dma_dt on its value row),
 *   out [B][Hq][d] bf16.
 */
int dma_decode_step(const void *q, const void *k_new, const void *v_new, int dtype, const float *dt_new,
                    int B, int Hq, int Hkv, int d, int w, void *state, size_t state_bytes, void *out,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * dma_decode_state_kept -- the kept positions of every (batch, kv head) in
 * slot order (not sorted), padded with -1: kept_idx [B][Hkv][w] int32; and
 * the cache length of each (batch, kv head) into lens [B][Hkv] (nullable).
 */
int dma_decode_state_kept(const void *state, size_t state_bytes, int B, int Hkv, int d, int w,
                          int32_t *kept_idx, int32_t *lens, void *stream);

/*
 * dma_qk_norm_rope -- Doge guide, DMA section, forward step 1: q_norm /
 * k_norm (an RMSNorm over head_dim with one weight per element) and then the
 * rotary position embedding that Doge takes from Llama (section on the
 * modular file's imports).  For every head row x of Q and of K (weight wq for
 * Q rows, wk for K rows) at position p:
 *   y_e = w_e * x_e / sqrt(mean_e(x_e^2) + eps)
 *   a_e = p * rope_theta^(-2e/d)                       for e < d/2
 *   out_e       = y_e cos a_e - y_{e+d/2} sin a_e
 *   out_{e+d/2} = y_{e+d/2} cos a_e + y_e sin a_e
 *
 *   Q [B][S][Hq][d], K [B][S][Hkv][d] dtype
 *   q_norm_w, k_norm_w [d] dtype
 *   eps        rms_norm_eps (>= 0; the DogeConfig default is 1e-6)
 *   rope_theta rope base (> 1; Llama's default is 10000)
 *   positions  [B][S] int32 device array, or NULL for p = s
 *   Q_out, K_out  same shapes and dtype (out); they may be Q and K
 *                 themselves (in place), but must not overlap them otherwise
 * Arithmetic is float32 with the angle reduced modulo a turn in float64;
 * the output is rounded once.  Supports d in {64, 128}.
 */
int dma_qk_norm_rope(const void *Q, const void *K, int dtype, const void *q_norm_w, const void *k_norm_w, float eps,
                     double rope_theta, const int32_t *positions, int B, int S, int Hq, int Hkv, int d, void *Q_out,
                     void *K_out, void *stream);

/*
 * dma_prologue -- the per-token work upstream of the selection, from the
 * projected Q, K and V of B*S tokens: dma_qk_norm_rope on Q and K, then dt
 * from V exactly as dma_dt with ld_out = S and no out_pos (dt_out
 * [B][Hkv][S] float32).  Both are validated before either is launched.
 */
int dma_prologue(const void *Q, const void *K, const void *V, int dtype, const void *q_norm_w, const void *k_norm_w,
                 float eps, double rope_theta, const int32_t *positions, const void *W, const void *bias,
                 const float *A, int B, int S, int Hq, int Hkv, int d, void *Q_out, void *K_out, float *dt_out,
                 void *stream);

/*
 * dma_attn_bwd_workspace_bytes -- device workspace of dma_attn_bwd (0 on
 * invalid sizes): two float32 values per (batch, query head, row).
 */
size_t dma_attn_bwd_workspace_bytes(int B, int S, int Hq, int Hkv, int d, int w);

/*
 * dma_attn_bwd -- gradients of dma_attn_fwd.  Doge guide, DMA section: the
 * same masked attention runs in training, and dt is learnt end to end through
 * it (forward step 3's remark on learning what to mask).  The kept sets are
 * those of (tau, tie); the selection itself has no gradient.  With
 * p = softmax over the kept keys of s = d**-0.5 q.k + dt, dp_j = dO.v_j and
 * D = sum_j p_j dp_j (= dO.o):  ds_j = p_j (dp_j - D),
 * dq = d**-0.5 sum_j ds_j k_j,  dk_j = d**-0.5 sum ds_j q,  dv_j = sum p_j dO,
 * ddt_j = sum ds_j, the last three summed over every row and query head that
 * keeps key j.  D is recomputed in float32 from the kept keys, so the forward
 * output is not an argument.
 *
 *   Q, K, V, dt, tau, tie, seqlens, w: as given to dma_attn_fwd
 *   dO  [B][S][Hq][d]  upstream gradient of the output
 *   dQ [B][S][Hq][d], dK/dV [B][S][Hkv][d] (dtype, out); ddt [B][Hkv][S]
 *   float32 (out).  Padded rows and keys get zeros.
 *   ws, ws_bytes: device workspace of at least dma_attn_bwd_workspace_bytes()
 * bf16 only; d in {64, 128}; Hq/Hkv in {1, 2, 4, 8}.  Products on matrix
 * cores with float32 accumulation (p and ds rounded to bf16 as operands);
 * deterministic (no atomics).  The query side walks about w + 128/(Hq/Hkv)
 * candidate keys per tile of rows; the key side walks, for each tile of keys
 * (64 at d = 64, 128 at d = 128), the rows from its first key to the last
 * row that keeps any of them (with dt drawn independently per key that is
 * often most of the causal range).
 */
int dma_attn_bwd(const void *Q, const void *K, const void *V, int dtype, const float *dt, const float *tau,
                 const int32_t *tie, const int32_t *seqlens, const void *dO, int B, int S, int Hq, int Hkv, int d,
                 int w, void *dQ, void *dK, void *dV, float *ddt, void *ws, size_t ws_bytes, void *stream);

/*
 * dma_dt_bwd_workspace_bytes -- device workspace of dma_dt_bwd (0 on invalid
 * sizes): one partial sum of dW, dbias and dA per 16 tokens.
 */
size_t dma_dt_bwd_workspace_bytes(int B, int S, int Hkv, int d);

/*
 * dma_dt_bwd -- gradients of dma_dt for an upstream gradient ddt (Doge guide,
 * DMA forward step 3: dt_proj and the learnt per-head A).  With x the
 * projection of a token for kv head h and dt = exp(A softplus(x)):
 *   dx = ddt dt A sigmoid(x);  dA[h] = sum ddt dt softplus(x);
 *   dbias[h] = sum dx;  dW[h][c] = sum dx V[c];  dV[c] += sum_h dx W[h][c]
 * (sums over every batch and position).
 *
 *   V, W, bias (nullable), A, dtype: as given to dma_dt
 *   ddt  [B][Hkv][S] float32, e.g. dma_attn_bwd's
 *   dV   [B][S][Hkv][d] dtype, or NULL: the dt path's part of the value
 *        gradient is ADDED in place (pass dma_attn_bwd's dV to get the total)
 *   dW [Hkv][Hkv*d], dbias [Hkv] (nullable), dA [Hkv]: float32 (out)
 *   ws, ws_bytes: device workspace of at least dma_dt_bwd_workspace_bytes()
 * float32 arithmetic; dW, dbias and dA are summed in a fixed order
 * (deterministic).  Supports d in {64, 128}, Hkv <= 16, Hkv*Hkv*d <= 16384 -
 * 128*Hkv.
 */
int dma_dt_bwd(const void *V, const void *W, const void *bias, const float *A, int dtype, const float *ddt, int B,
               int S, int Hkv, int d, void *dV, float *dW, float *dbias, float *dA, void *ws, size_t ws_bytes,
               void *stream);

/*
 * Sliding-window variant -- Doge guide, DogeConfig table (sliding_window: with
 * a value, the attention mask is the sliding-window causal mask) and DMA
 * forward step 3 (the dynamic mask keeps the top keep_window_size of the
 * visible keys; masked keys hold min_dtype and never outrank valid ones).
 * Row i sees the keys i - win < j <= i with j < L_b.  The kept sets no longer
 * nest from row to row, so these entry points select and attend per row.
 *
 * dma_select_window -- the threshold pair of every row over its window, with
 * the conventions of dma_select: (tau, tie) is the w-th kept key under (dt
 * desc, index asc); (-inf, -1) when the row sees at most w keys; (+inf, -1)
 * for a padded row.  Exact (comparisons only).  win >= 1; B * Hkv *
 * ceil(S / 64) below 2^31 as for dma_select.
 */
int dma_select_window(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, int win, float *tau,
                      int32_t *tie, void *stream);

/*
 * dma_attn_window_fwd -- dma_attn_fwd's computation over the kept keys of
 * each row's window, (tau, tie) from dma_select_window with the same w and
 * win.  Every key of the window is tested; work grows with win, not w.
 * bf16 only; d in {64, 128}; Hq/Hkv in {1, 2, 4, 8}.  P is rounded once to
 * bf16 for the product with V and the softmax sum is taken over the rounded
 * weights; float32 accumulation; output rounded to nearest even.
 */
int dma_attn_window_fwd(const void *Q, const void *K, const void *V, int dtype, const float *dt, const float *tau,
                        const int32_t *tie, const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d, int w,
                        int win, void *O, void *stream);

/*
 * CDMoE routed experts -- Doge guide, section on Cross Domain MoE, and the
 * DogeConfig table (num_experts = nk*nk, num_experts_per_tok = k,
 * hidden_act = silu).  Tokens are rows of hidden states h [T][H].
 *
 * dma_cdmoe_logits -- router_gate: logits[t][n] = sum_c router[n][c] h[t][c]
 * for the 2*nk outputs (the first nk are the x domain, the last nk the y
 * domain).  h [T][H], router [2*nk][H] bf16; logits [T][2*nk] float32 (out).
 * Matrix cores, float32 accumulation.  H a multiple of 32, nk <= 256.
 */
int dma_cdmoe_logits(const void *h, const void *router, int dtype, int T, int H, int nk, float *logits,
                     void *stream);

/*
 * dma_cdmoe_route -- product-key routing: the top k of each domain (larger
 * first, lower index first among equal), the k best of the pairs of the two
 * lists by score x logit + y logit (a float32 sum; equal scores in the order
 * of the two domains' own rankings, x first), each naming expert
 * x index * nk + y index, and the softmax of the k best scores.
 *   logits [T][2*nk] float32; idx [T][k] int32 (out, best first);
 *   weights [T][k] float32 (out).  Exact selection.  k <= min(nk, 128),
 *   nk <= 256.
 */
int dma_cdmoe_route(const float *logits, int T, int nk, int k, int32_t *idx, float *weights, void *stream);

/*
 * dma_cdmoe_experts -- the kept experts of each token as embedding rows:
 *   out[t] = sum_e weights[t][e] * silu(down[idx[t][e]] . h[t]) * up[idx[t][e]]
 *   h [T][H], down/up [nk*nk][H] bf16; idx, weights as from dma_cdmoe_route;
 *   out [T][H] bf16 (out).  float32 arithmetic, one rounding at the end.
 *   H a multiple of 512, k <= 128.  The expert indices must be below nk*nk.
 */
int dma_cdmoe_experts(const void *h, const void *down, const void *up, int dtype, const int32_t *idx,
                      const float *weights, int T, int H, int nk, int k, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DMA_H_ */
