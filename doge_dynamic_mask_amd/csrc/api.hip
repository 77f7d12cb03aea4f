// C ABI of libdma.so: host-side validation, then one or more kernel launches
// on the caller's stream.  Nothing here allocates, synchronises or keeps
// state; every check happens before the first HIP call.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dma.h"
#include "launch.hpp"

namespace {

constexpr int kAbiVersion = 100;

bool aligned16(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }
bool dtype_ok(int t) { return t == DMA_F32 || t == DMA_BF16; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }

int from_hip(hipError_t e) { return e == hipSuccess ? DMA_OK : DMA_ERR_HIP; }

int qk_norm_rope_check(const void *Q, const void *K, int dtype, const void *q_norm_w, const void *k_norm_w, float eps,
                       double rope_theta, int B, int S, int Hq, int Hkv, int d, const void *Q_out, const void *K_out) {
    if (!Q || !K || !q_norm_w || !k_norm_w || !Q_out || !K_out) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || d < 1) return DMA_ERR_SHAPE;
    if (!(eps >= 0.f) || !(rope_theta > 1.0) || (int64_t)B * S > 0x7fffffff) return DMA_ERR_SHAPE;
    if (!head_dim_ok(d)) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(q_norm_w) || !aligned16(k_norm_w) || !aligned16(Q_out) ||
        !aligned16(K_out))
        return DMA_ERR_UNSUPPORTED;
    return DMA_OK;
}

}  // namespace

extern "C" {

int dma_version(void) { return kAbiVersion; }

const char *dma_status_str(int status) {
    switch (status) {
        case DMA_OK: return "ok";
        case DMA_ERR_NULL: return "a required pointer is NULL";
        case DMA_ERR_SHAPE: return "a size is out of range or inconsistent";
        case DMA_ERR_DTYPE: return "dtype must be DMA_F32 or DMA_BF16";
        case DMA_ERR_UNSUPPORTED: return "request outside the implemented kernels (head_dim, heads, alignment)";
        case DMA_ERR_WORKSPACE: return "workspace missing or too small";
        case DMA_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

int dma_dt(const void *V, const void *W, const void *bias, const float *A, int dtype, int B, int S,
           int Hkv, int d, float *dt_out, int64_t ld_out, const int32_t *out_pos, void *stream) {
    if (!V || !W || !A || !dt_out) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || S < 1 || Hkv < 1 || d < 1 || ld_out < S) return DMA_ERR_SHAPE;
    if (!head_dim_ok(d) || Hkv > dma::kMaxHkvDt) return DMA_ERR_UNSUPPORTED;
    const size_t esize = dtype == DMA_BF16 ? 2 : 4;
    if ((size_t)Hkv * Hkv * d * esize > dma::kDtLdsBytes) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(V) || !aligned16(W)) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_dt(V, W, bias, A, dtype, B, S, Hkv, d, dt_out, ld_out, out_pos,
                                   (hipStream_t)stream));
}

int dma_select(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, float *tau,
               int32_t *tie, void *stream) {
    if (!dt || !tau || !tie) return DMA_ERR_NULL;
    if (B < 1 || Hkv < 1 || S < 1 || w < 1) return DMA_ERR_SHAPE;
    if ((int64_t)B * Hkv * ((S + 63) / 64) >= ((int64_t)1 << 31) - 8) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_select(dt, seqlens, B, Hkv, S, w, 0, tau, tie, (hipStream_t)stream));
}

int dma_attn_fwd(const void *Q, const void *K, const void *V, int dtype, const float *dt,
                 const float *tau, const int32_t *tie, const int32_t *seqlens, int B, int S, int Hq,
                 int Hkv, int d, int w, void *O, void *stream) {
    if (!Q || !K || !V || !dt || !tau || !tie || !O) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || Hq % Hkv != 0) return DMA_ERR_SHAPE;
    if (!head_dim_ok(d) || Hq / Hkv > dma::kMaxGroupAttn) return DMA_ERR_UNSUPPORTED;
    if (B > 65535 || Hkv > 65535) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_attn(Q, K, V, dtype, dt, tau, tie, seqlens, B, S, Hq, Hkv, d, w, O,
                                     (hipStream_t)stream));
}

size_t dma_workspace_bytes(int op, int B, int S, int Hq, int Hkv, int d, int w) {
    const size_t bad = (size_t)-1;
    if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || Hq % Hkv != 0) return bad;
    size_t n = 0;
    switch (op) {
        case DMA_OP_DT:
        case DMA_OP_SELECT:
        case DMA_OP_ATTN_FWD:
            return 0;
        case DMA_OP_DECODE: n = dma_decode_workspace_bytes(B, S, Hq, Hkv, d, w); break;
        case DMA_OP_DECODE_STEP: n = dma_decode_step_workspace_bytes(B, Hq, Hkv, d, w); break;
        case DMA_OP_ATTN_BWD: n = dma_attn_bwd_workspace_bytes(B, S, Hq, Hkv, d, w); break;
        case DMA_OP_DT_BWD: n = dma_dt_bwd_workspace_bytes(B, S, Hkv, d); break;
        default: return bad;
    }
    return n == 0 ? bad : n;
}

size_t dma_decode_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int d, int w) {
    if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || Hq % Hkv != 0) return 0;
    return dma::decode_ws_bytes(B, Lmax, Hq, Hkv, d, w);
}

int dma_decode(const void *q, const void *Kc, const void *Vc, int dtype, const float *dt_cache,
               const int32_t *cache_lens, int B, int Lmax, int Hq, int Hkv, int d, int w, void *out,
               int32_t *kept_idx, void *ws, size_t ws_bytes, void *stream) {
    if (!q || !Kc || !Vc || !dt_cache || !cache_lens || !out) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || Hq % Hkv != 0) return DMA_ERR_SHAPE;
    if (!head_dim_ok(d) || Hq / Hkv > dma::kMaxGroupDecode) return DMA_ERR_UNSUPPORTED;
    if (B > 65535 || Hkv > 65535) return DMA_ERR_UNSUPPORTED;
    if ((Lmax < w ? Lmax : w) > dma::kMaxKeptDecode) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(Kc) || !aligned16(Vc)) return DMA_ERR_UNSUPPORTED;
    if (!ws) return DMA_ERR_WORKSPACE;
    if (ws_bytes < dma::decode_ws_bytes(B, Lmax, Hq, Hkv, d, w)) return DMA_ERR_WORKSPACE;
    return from_hip(dma::launch_decode(q, Kc, Vc, dtype, dt_cache, cache_lens, B, Lmax, Hq, Hkv, d, w,
                                       out, kept_idx, ws, (hipStream_t)stream));
}

int dma_decode_noalloc(const void *q, const void *Kc, const void *Vc, int dtype, const float *dt_cache,
                       const int32_t *cache_lens, int B, int Lmax, int Hq, int Hkv, int d, int w, void *out,
                       int32_t *kept_idx, void *stream) {
    if (!q || !Kc || !Vc || !dt_cache || !cache_lens || !out) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || Hq % Hkv != 0) return DMA_ERR_SHAPE;
    if (!head_dim_ok(d) || Hq / Hkv > dma::kMaxGroupDecode) return DMA_ERR_UNSUPPORTED;
    if (B > 65535 || Hkv > 65535) return DMA_ERR_UNSUPPORTED;
    if ((Lmax < w ? Lmax : w) > dma::kMaxKeptDecode) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(Kc) || !aligned16(Vc)) return DMA_ERR_UNSUPPORTED;
    if (dma::decode_ws_bytes(B, Lmax, Hq, Hkv, d, w) > dma::kDecodeNoAllocScratchBytes) return DMA_ERR_WORKSPACE;
    return from_hip(dma::launch_decode_noalloc(q, Kc, Vc, dtype, dt_cache, cache_lens, B, Lmax, Hq, Hkv, d, w, out,
                                               kept_idx, (hipStream_t)stream));
}

size_t dma_decode_state_bytes(int B, int Hkv, int d, int w) {
    if (B < 1 || Hkv < 1 || w < 1 || !head_dim_ok(d)) return 0;
    return dma::decode_state_bytes(B, Hkv, d, w);
}

size_t dma_decode_step_workspace_bytes(int B, int Hq, int Hkv, int d, int w) {
    if (B < 1 || Hq < 1 || Hkv < 1 || w < 1 || Hq % Hkv != 0 || !head_dim_ok(d)) return 0;
    return dma::decode_step_ws_bytes(B, Hq, Hkv, d, w);
}

int dma_decode_state_init(const void *Kc, const void *Vc, int dtype, const float *dt_cache,
                          const int32_t *cache_lens, int B, int Lmax, int Hkv, int d, int w, void *state,
                          size_t state_bytes, void *ws, size_t ws_bytes, void *stream) {
    if (!Kc || !Vc || !dt_cache || !cache_lens || !state) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || Lmax < 1 || Hkv < 1 || d < 1 || w < 1) return DMA_ERR_SHAPE;
    if (dtype != DMA_BF16 || !head_dim_ok(d)) return DMA_ERR_UNSUPPORTED;
    if (B > 65535 || Hkv > 65535 || w > dma::kMaxKeptDecode) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(Kc) || !aligned16(Vc) || !aligned16(state)) return DMA_ERR_UNSUPPORTED;
    if (state_bytes < dma::decode_state_bytes(B, Hkv, d, w)) return DMA_ERR_WORKSPACE;
    if (!ws || ws_bytes < dma::decode_step_ws_bytes(B, Hkv, Hkv, d, w)) return DMA_ERR_WORKSPACE;
    return from_hip(dma::launch_decode_state_init(Kc, Vc, dt_cache, cache_lens, B, Lmax, Hkv, d, w, state, ws,
                                                  (hipStream_t)stream));
}

int dma_decode_step(const void *q, const void *k_new, const void *v_new, int dtype, const float *dt_new,
                    int B, int Hq, int Hkv, int d, int w, void *state, size_t state_bytes, void *out, void *ws,
                    size_t ws_bytes, void *stream) {
    if (!q || !k_new || !v_new || !dt_new || !state || !out) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || Hq % Hkv != 0) return DMA_ERR_SHAPE;
    if (dtype != DMA_BF16 || !head_dim_ok(d) || Hq / Hkv > dma::kMaxGroupDecode) return DMA_ERR_UNSUPPORTED;
    if (B > 65535 || Hkv > 65535 || w > dma::kMaxKeptDecode) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(state)) return DMA_ERR_UNSUPPORTED;
    if (state_bytes < dma::decode_state_bytes(B, Hkv, d, w)) return DMA_ERR_WORKSPACE;
    if (!ws || ws_bytes < dma::decode_step_ws_bytes(B, Hq, Hkv, d, w)) return DMA_ERR_WORKSPACE;
    return from_hip(dma::launch_decode_step(q, k_new, v_new, dt_new, B, Hq, Hkv, d, w, state, out, ws,
                                            (hipStream_t)stream));
}

int dma_decode_state_kept(const void *state, size_t state_bytes, int B, int Hkv, int d, int w, int32_t *kept_idx,
                          int32_t *lens, void *stream) {
    if (!state || !kept_idx) return DMA_ERR_NULL;
    if (B < 1 || Hkv < 1 || d < 1 || w < 1) return DMA_ERR_SHAPE;
    if (!head_dim_ok(d) || B > 65535 || Hkv > 65535) return DMA_ERR_UNSUPPORTED;
    if (state_bytes < dma::decode_state_bytes(B, Hkv, d, w)) return DMA_ERR_WORKSPACE;
    return from_hip(dma::launch_decode_state_kept(state, B, Hkv, d, w, kept_idx, lens, (hipStream_t)stream));
}

int dma_qk_norm_rope(const void *Q, const void *K, int dtype, const void *q_norm_w, const void *k_norm_w, float eps,
                     double rope_theta, const int32_t *positions, int B, int S, int Hq, int Hkv, int d, void *Q_out,
                     void *K_out, void *stream) {
    const int st = qk_norm_rope_check(Q, K, dtype, q_norm_w, k_norm_w, eps, rope_theta, B, S, Hq, Hkv, d, Q_out,
                                      K_out);
    if (st != DMA_OK) return st;
    return from_hip(dma::launch_qk_norm_rope(Q, K, dtype, q_norm_w, k_norm_w, eps, rope_theta, positions, B, S, Hq,
                                             Hkv, d, Q_out, K_out, (hipStream_t)stream));
}

int dma_prologue(const void *Q, const void *K, const void *V, int dtype, const void *q_norm_w, const void *k_norm_w,
                 float eps, double rope_theta, const int32_t *positions, const void *W, const void *bias,
                 const float *A, int B, int S, int Hq, int Hkv, int d, void *Q_out, void *K_out, float *dt_out,
                 void *stream) {
    if (!V || !W || !A || !dt_out) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B >= 1 && S >= 1 && Hkv >= 1 && d >= 1) {
        const size_t esize = dtype == DMA_BF16 ? 2 : 4;
        if (Hkv > dma::kMaxHkvDt || (size_t)Hkv * Hkv * d * esize > dma::kDtLdsBytes) return DMA_ERR_UNSUPPORTED;
        if (!aligned16(V) || !aligned16(W)) return DMA_ERR_UNSUPPORTED;
    }
    // every argument is checked before the first launch
    const int st = qk_norm_rope_check(Q, K, dtype, q_norm_w, k_norm_w, eps, rope_theta, B, S, Hq, Hkv, d, Q_out,
                                      K_out);
    if (st != DMA_OK) return st;
    if (dtype == DMA_BF16)  // one launch: dt's tiles and the Q/K rows side by side
        return from_hip(dma::launch_prologue_bf16(Q, K, q_norm_w, k_norm_w, eps, rope_theta, positions, B, S, Hq, Hkv,
                                                  d, Q_out, K_out, V, W, bias, A, dt_out, (hipStream_t)stream));
    const hipError_t e = dma::launch_qk_norm_rope(Q, K, dtype, q_norm_w, k_norm_w, eps, rope_theta, positions, B, S,
                                                  Hq, Hkv, d, Q_out, K_out, (hipStream_t)stream);
    if (e != hipSuccess) return DMA_ERR_HIP;
    return from_hip(dma::launch_dt(V, W, bias, A, dtype, B, S, Hkv, d, dt_out, S, nullptr, (hipStream_t)stream));
}

size_t dma_attn_bwd_workspace_bytes(int B, int S, int Hq, int Hkv, int d, int w) {
    if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || w < 1 || Hq % Hkv != 0 || !head_dim_ok(d)) return 0;
    return dma::attn_bwd_ws_bytes(B, S, Hq);
}

int dma_attn_bwd(const void *Q, const void *K, const void *V, int dtype, const float *dt, const float *tau,
                 const int32_t *tie, const int32_t *seqlens, const void *dO, int B, int S, int Hq, int Hkv, int d,
                 int w, void *dQ, void *dK, void *dV, float *ddt, void *ws, size_t ws_bytes, void *stream) {
    if (!Q || !K || !V || !dt || !tau || !tie || !dO || !dQ || !dK || !dV || !ddt) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || Hq % Hkv != 0) return DMA_ERR_SHAPE;
    const int G = Hq / Hkv;
    if (dtype != DMA_BF16 || !head_dim_ok(d) || G > dma::kMaxGroupBwd || 64 % G != 0) return DMA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv * S > 0x7fffffff) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dQ) || !aligned16(dK) ||
        !aligned16(dV))
        return DMA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < dma::attn_bwd_ws_bytes(B, S, Hq)) return DMA_ERR_WORKSPACE;
    return from_hip(dma::launch_attn_bwd(Q, K, V, dt, tau, tie, seqlens, dO, B, S, Hq, Hkv, d, dQ, dK, dV, ddt, ws,
                                         (hipStream_t)stream));
}

size_t dma_dt_bwd_workspace_bytes(int B, int S, int Hkv, int d) {
    if (B < 1 || S < 1 || Hkv < 1 || !head_dim_ok(d)) return 0;
    return dma::dt_bwd_ws_bytes(B, S, Hkv, d);
}

int dma_dt_bwd(const void *V, const void *W, const void *bias, const float *A, int dtype, const float *ddt, int B,
               int S, int Hkv, int d, void *dV, float *dW, float *dbias, float *dA, void *ws, size_t ws_bytes,
               void *stream) {
    if (!V || !W || !A || !ddt || !dW || !dA) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || S < 1 || Hkv < 1 || d < 1) return DMA_ERR_SHAPE;
    if (!head_dim_ok(d) || Hkv > dma::kMaxHkvDt) return DMA_ERR_UNSUPPORTED;
    if ((int64_t)B * S > 0x7fffffff || dma::dt_bwd_lds_bytes(Hkv, d) > 65536) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(V) || !aligned16(dV)) return DMA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < dma::dt_bwd_ws_bytes(B, S, Hkv, d)) return DMA_ERR_WORKSPACE;
    return from_hip(dma::launch_dt_bwd(V, W, bias, A, dtype, ddt, B, S, Hkv, d, dV, dW, dbias, dA, ws,
                                       (hipStream_t)stream));
}

int dma_select_window(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, int win, float *tau,
                      int32_t *tie, void *stream) {
    if (!dt || !tau || !tie) return DMA_ERR_NULL;
    if (B < 1 || Hkv < 1 || S < 1 || w < 1 || win < 1) return DMA_ERR_SHAPE;
    if ((int64_t)B * Hkv * S > ((int64_t)1 << 40)) return DMA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv * ((S + 63) / 64) >= ((int64_t)1 << 31) - 8) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_select_window(dt, seqlens, B, Hkv, S, w, win, tau, tie, (hipStream_t)stream));
}

int dma_attn_window_fwd(const void *Q, const void *K, const void *V, int dtype, const float *dt, const float *tau,
                        const int32_t *tie, const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d, int w,
                        int win, void *O, void *stream) {
    if (!Q || !K || !V || !dt || !tau || !tie || !O) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || d < 1 || w < 1 || win < 1 || Hq % Hkv != 0) return DMA_ERR_SHAPE;
    const int G = Hq / Hkv;
    if (dtype != DMA_BF16 || !head_dim_ok(d) || G > dma::kMaxGroupBwd || 64 % G != 0) return DMA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv * S > 0x7fffffff) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_attn_window(Q, K, V, dt, tau, tie, seqlens, B, S, Hq, Hkv, d, win, O,
                                            (hipStream_t)stream));
}

int dma_cdmoe_logits(const void *h, const void *router, int dtype, int T, int H, int nk, float *logits,
                     void *stream) {
    if (!h || !router || !logits) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (T < 1 || H < 1 || nk < 1) return DMA_ERR_SHAPE;
    if (dtype != DMA_BF16 || H % 32 != 0 || nk > dma::kMaxCdmoeKeys) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(h) || !aligned16(router)) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_cdmoe_logits(h, router, T, H, nk, logits, (hipStream_t)stream));
}

int dma_cdmoe_route(const float *logits, int T, int nk, int k, int32_t *idx, float *weights, void *stream) {
    if (!logits || !idx || !weights) return DMA_ERR_NULL;
    if (T < 1 || nk < 1 || k < 1 || k > nk) return DMA_ERR_SHAPE;
    if (nk > dma::kMaxCdmoeKeys || k > dma::kMaxCdmoeTopk) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_cdmoe_route(logits, T, nk, k, idx, weights, (hipStream_t)stream));
}

int dma_cdmoe_experts(const void *h, const void *down, const void *up, int dtype, const int32_t *idx,
                      const float *weights, int T, int H, int nk, int k, void *out, void *stream) {
    if (!h || !down || !up || !idx || !weights || !out) return DMA_ERR_NULL;
    if (!dtype_ok(dtype)) return DMA_ERR_DTYPE;
    if (T < 1 || H < 1 || nk < 1 || nk > 46340 || k < 1 || k > nk * nk) return DMA_ERR_SHAPE;
    if (dtype != DMA_BF16 || H % 512 != 0 || k > dma::kMaxCdmoeTopk || T > 0x7fffffff) return DMA_ERR_UNSUPPORTED;
    if (!aligned16(h) || !aligned16(down) || !aligned16(up) || !aligned16(out)) return DMA_ERR_UNSUPPORTED;
    return from_hip(dma::launch_cdmoe_experts(h, down, up, idx, weights, T, H, nk, k, out, (hipStream_t)stream));
}

}  // extern "C"
