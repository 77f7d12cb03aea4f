// Host-side launchers of the DMA kernels; called only from api.hip after the
// arguments have been validated.  Each returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dma {

hipError_t launch_dt(const void *V, const void *W, const void *bias, const float *A, int dtype,
                     int B, int S, int Hkv, int d, float *dt_out, int64_t ld_out,
                     const int32_t *out_pos, hipStream_t stream);

// win = 0: the full causal range; win >= 64: a sliding window of win positions
hipError_t launch_select(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, int win,
                         float *tau, int32_t *tie, hipStream_t stream);

hipError_t launch_attn(const void *Q, const void *K, const void *V, int dtype, const float *dt,
                       const float *tau, const int32_t *tie, const int32_t *seqlens, int B, int S,
                       int Hq, int Hkv, int d, int w, void *O, hipStream_t stream);

size_t decode_ws_bytes(int B, int Lmax, int Hq, int Hkv, int d, int w);

hipError_t launch_decode(const void *q, const void *Kc, const void *Vc, int dtype,
                         const float *dt_cache, const int32_t *cache_lens, int B, int Lmax,
                         int Hq, int Hkv, int d, int w, void *out, int32_t *kept_idx, void *ws,
                         hipStream_t stream);

// dma_decode with its workspace in a static device array of
// kDecodeNoAllocScratchBytes per device (no allocation).
constexpr size_t kDecodeNoAllocScratchBytes = (size_t)16 << 20;
hipError_t launch_decode_noalloc(const void *q, const void *Kc, const void *Vc, int dtype, const float *dt_cache,
                                 const int32_t *cache_lens, int B, int Lmax, int Hq, int Hkv, int d, int w,
                                 void *out, int32_t *kept_idx, hipStream_t stream);

// The selection key of the w-th kept position of each (batch, kv head) of a
// decode cache (0 when every position is kept), as dma_decode's first step.
hipError_t launch_decode_thresholds(const float *dt_cache, const int32_t *cache_lens, int B, int Lmax, int Hkv,
                                    int w, uint64_t *thr, hipStream_t stream);

// Incremental decode state (decode_state.hip).
size_t decode_state_bytes(int B, int Hkv, int d, int w);
size_t decode_step_ws_bytes(int B, int Hq, int Hkv, int d, int w);
hipError_t launch_decode_state_init(const void *Kc, const void *Vc, const float *dt_cache, const int32_t *cache_lens,
                                    int B, int Lmax, int Hkv, int d, int w, void *state, void *ws,
                                    hipStream_t stream);
hipError_t launch_decode_step(const void *q, const void *k_new, const void *v_new, const float *dt_new, int B,
                              int Hq, int Hkv, int d, int w, void *state, void *out, void *ws, hipStream_t stream);
hipError_t launch_decode_state_kept(const void *state, int B, int Hkv, int d, int w, int32_t *kept_idx,
                                    int32_t *lens, hipStream_t stream);

// Q/K RMSNorm over head_dim and rotary embedding (prologue.hip).
hipError_t launch_qk_norm_rope(const void *Q, const void *K, int dtype, const void *wq, const void *wk, float eps,
                               double rope_theta, const int32_t *positions, int B, int S, int Hq, int Hkv, int d,
                               void *Qo, void *Ko, hipStream_t stream);

// The bf16 prologue in one launch: Q/K RMSNorm + rotary and dt from V
// (dt_out [B][Hkv][S], no out_pos), prologue.hip.
hipError_t launch_prologue_bf16(const void *Q, const void *K, const void *wq, const void *wk, float eps,
                                double rope_theta, const int32_t *positions, int B, int S, int Hq, int Hkv, int d,
                                void *Qo, void *Ko, const void *V, const void *W, const void *bias, const float *A,
                                float *dt_out, hipStream_t stream);

// Backward of the prefill attention (bwd.hip), bf16.
size_t attn_bwd_ws_bytes(int B, int S, int Hq);
hipError_t launch_attn_bwd(const void *Q, const void *K, const void *V, const float *dt, const float *tau,
                           const int32_t *tie, const int32_t *seqlens, const void *dO, int B, int S, int Hq,
                           int Hkv, int d, void *dQ, void *dK, void *dV, float *ddt, void *ws, hipStream_t stream);

// Backward of dt (dt_bwd.hip).
size_t dt_bwd_ws_bytes(int B, int S, int Hkv, int d);
size_t dt_bwd_lds_bytes(int Hkv, int d);
hipError_t launch_dt_bwd(const void *V, const void *W, const void *bias, const float *A, int dtype, const float *ddt,
                         int B, int S, int Hkv, int d, void *dV, float *dW, float *dbias, float *dA, void *ws,
                         hipStream_t stream);

// Sliding-window variant (window.hip).
hipError_t launch_select_window(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, int win,
                                float *tau, int32_t *tie, hipStream_t stream);
hipError_t launch_attn_window(const void *Q, const void *K, const void *V, const float *dt, const float *tau,
                              const int32_t *tie, const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                              int win, void *O, hipStream_t stream);

// CDMoE routed experts (cdmoe.hip), bf16.
hipError_t launch_cdmoe_logits(const void *h, const void *router, int T, int H, int nk, float *logits,
                               hipStream_t stream);
hipError_t launch_cdmoe_route(const float *logits, int T, int nk, int k, int32_t *idx, float *wts,
                              hipStream_t stream);
hipError_t launch_cdmoe_experts(const void *h, const void *down, const void *up, const int32_t *idx, const float *wts,
                                int T, int H, int nk, int k, void *out, hipStream_t stream);

// Limits the launchers rely on (checked by the ABI layer).
constexpr int kMaxHkvDt = 16;          // dt kernel: heads accumulated in registers
constexpr int kMaxGroupAttn = 128;     // prefill: query heads per kv head
constexpr int kMaxGroupDecode = 16;    // decode: query heads per kv head
constexpr int kMaxKeptDecode = 131072; // decode: kept positions per (batch, kv head)
constexpr size_t kDtLdsBytes = 65536;  // dt kernel: W staged in LDS
constexpr int kMaxGroupBwd = 8;        // backward: query heads per kv head (a divisor of 64)
constexpr int kMaxCdmoeKeys = 256;     // CDMoE routing: keys per domain
constexpr int kMaxCdmoeTopk = 128;     // CDMoE routing: experts kept per token

}  // namespace dma
