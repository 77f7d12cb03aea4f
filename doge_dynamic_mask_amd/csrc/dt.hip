// dt kernel: dt[b][h][s] = exp(A[h] * softplus(bias[h] + sum_c W[h][c] * V[b][s][c]))
// Doge guide (gitcode), DMA section, forward step 3: dt_proj over the value
// states of all kv heads of a token (input width Hkv*d, head-major), then
// exp(A * softplus(.)).
//
// A skinny matrix product X[tokens][Hkv] = V[tokens][Hkv*d] * W^T that must
// stream V once from HBM.  bf16 runs on matrix cores: one wave takes 16
// tokens, v_mfma_f32_16x16x32_bf16 with the tokens as M, the (zero-padded)
// kv heads as N and the channels as K, so V and W are fed to the MFMA
// straight from their 16-byte loads with no conversion.  The contraction
// order over channels is free, so each lane owns 32 consecutive channels per
// 128-channel chunk (64 contiguous bytes of its token row) and W uses the
// same order.
// float32 uses VALU: eight lanes per token, 16-byte vectors, xor-shuffle
// reduction.  A bf16 call with few tokens (a decode step's append of one
// token per batch) takes a VALU kernel with one wave per (token, kv head)
// and a single round of loads.  softplus and exp run in float32 in all.
#include "common.hpp"
#include "dt_mfma.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerToken = 8;
constexpr int kTokensPerBlock = kThreads / kLanesPerToken;
constexpr int kBatch = 8;  // 16-byte vectors per lane loaded together

template <typename T>
__device__ __forceinline__ void unpack16(const uint4 &v, float *x);
template <>
__device__ __forceinline__ void unpack16<float>(const uint4 &v, float *x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
}

__device__ __forceinline__ float softplus_f32(float x) {
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dt_kernel(const T *__restrict__ V, const T *__restrict__ W,
                                                      const T *__restrict__ bias,
                                                      const float *__restrict__ A, int S, int Hkv,
                                                      int d, int64_t ntok, float *__restrict__ out,
                                                      int64_t ld, const int32_t *__restrict__ out_pos) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float As[kMaxHkvDt], bs[kMaxHkvDt];
    constexpr int EV = 16 / (int)sizeof(T);  // elements per 16-byte vector
    const int width = Hkv * d;
    const int nvec = width / EV;             // vectors per token row
    uint4 *Ws = reinterpret_cast<uint4 *>(smem);
    // W, A and bias are staged together so that their load latencies overlap
    for (int v = threadIdx.x; v < Hkv * nvec; v += kThreads) Ws[v] = reinterpret_cast<const uint4 *>(W)[v];
    if (threadIdx.x < (unsigned)Hkv) {
        As[threadIdx.x] = A[threadIdx.x];
        bs[threadIdx.x] = bias ? Elem<T>::load(bias, threadIdx.x) : 0.f;
    }
    __syncthreads();

    const int q = threadIdx.x % kLanesPerToken;
    for (int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + threadIdx.x / kLanesPerToken; t < ntok;
         t += (int64_t)gridDim.x * kTokensPerBlock) {
        const uint4 *vrow = reinterpret_cast<const uint4 *>(V + t * width);
        const int b = (int)(t / S);
        const int s = (int)(t - (int64_t)b * S);
        const int64_t col = (out_pos ? (int64_t)out_pos[b] : 0) + s;  // loaded with the rows
        float acc[kMaxHkvDt];
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h) acc[h] = 0.f;
        // this lane's vectors of the token, kBatch at a time, all loaded
        // before any is used so that their latencies overlap
        for (int v0 = q; v0 < nvec; v0 += kBatch * kLanesPerToken) {
            uint4 vb[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int v = v0 + k * kLanesPerToken;
                if (v < nvec) vb[k] = vrow[v];
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int v = v0 + k * kLanesPerToken;
                if (v >= nvec) break;
                float x[EV];
                unpack16<T>(vb[k], x);
#pragma unroll
                for (int h = 0; h < kMaxHkvDt; ++h) {
                    if (h < Hkv) {
                        float wv[EV];
                        unpack16<T>(Ws[h * nvec + v], wv);
                        float a = acc[h];
#pragma unroll
                        for (int e = 0; e < EV; ++e) a = fmaf(wv[e], x[e], a);
                        acc[h] = a;
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h) {
            if (h < Hkv) {
#pragma unroll
                for (int o = 1; o < kLanesPerToken; o <<= 1) acc[h] += __shfl_xor(acc[h], o, kLanesPerToken);
            }
        }
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h) {
            if (h < Hkv && (h % kLanesPerToken) == q && (uint64_t)col < (uint64_t)ld) {
                const float x = acc[h] + bs[h];
                out[((int64_t)b * Hkv + h) * ld + col] = expf(As[h] * softplus_f32(x));
            }
        }
    }
}

constexpr int kMfmaThreads = 128;     // two waves, one 16-token tile each

__global__ __launch_bounds__(kMfmaThreads) void dt_mfma_kernel(
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ W, const uint16_t *__restrict__ bias,
    const float *__restrict__ A, int S, int Hkv, int width, int64_t ntok,
    float *__restrict__ out, int64_t ld, const int32_t *__restrict__ out_pos) {
    // one 128-channel chunk per batch of loads: fewer registers, so more
    // waves in flight, beat fewer rounds (padded 26 -> 22 us, c2 6.0 -> 5.5 us
    // against four chunks per batch)
    constexpr int kWavesPerBlock = kMfmaThreads / 64;
    dt_mfma_tiles<1>((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6), (int64_t)gridDim.x * kWavesPerBlock,
                  V, W, bias, A, S, Hkv, width, ntok, out, ld, out_pos);
}

// A few tokens (a decode step's append form): one wave per (token, kv head)
// with a single round of loads (dt_pair); a launch over a handful of 16-token
// tiles would be bound by their latency chain.
__global__ __launch_bounds__(kThreads) void dt_small_kernel(
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ W, const uint16_t *__restrict__ bias,
    const float *__restrict__ A, int S, int Hkv, int width, int64_t ntok,
    float *__restrict__ out, int64_t ld, const int32_t *__restrict__ out_pos) {
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= ntok * Hkv) return;  // whole waves
    dt_pair(wid, V, W, bias, A, S, Hkv, width, out, ld, out_pos);
}

}  // namespace

hipError_t launch_dt(const void *V, const void *W, const void *bias, const float *A, int dtype,
                     int B, int S, int Hkv, int d, float *dt_out, int64_t ld_out,
                     const int32_t *out_pos, hipStream_t stream) {
    const int64_t ntok = (int64_t)B * S;
    if (dtype == 1 && ntok <= kDtSmallTokens) {
        const int64_t waves = ntok * Hkv;
        hipLaunchKernelGGL(dt_small_kernel, dim3((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64))),
                           dim3(kThreads), 0, stream, (const uint16_t *)V, (const uint16_t *)W,
                           (const uint16_t *)bias, A, S, Hkv, Hkv * d, ntok, dt_out, ld_out, out_pos);
    } else if (dtype == 1) {
        const int width = Hkv * d;
        const int64_t ntiles = (ntok + 15) / 16;
        const int64_t want = (ntiles + kMfmaThreads / 64 - 1) / (kMfmaThreads / 64);
        const int grid = (int)(want < 4096 ? want : 4096);
        hipLaunchKernelGGL(dt_mfma_kernel, dim3(grid), dim3(kMfmaThreads), 0, stream,
                           (const uint16_t *)V, (const uint16_t *)W, (const uint16_t *)bias, A, S, Hkv,
                           width, ntok, dt_out, ld_out, out_pos);
    } else {
        const int64_t want = (ntok + kTokensPerBlock - 1) / kTokensPerBlock;
        const int grid = (int)(want < 2048 ? want : 2048);
        const size_t lds = (size_t)Hkv * Hkv * d * sizeof(float);
        hipLaunchKernelGGL(dt_kernel<float>, dim3(grid), dim3(kThreads), lds, stream, (const float *)V,
                           (const float *)W, (const float *)bias, A, S, Hkv, d, ntok, dt_out, ld_out,
                           out_pos);
    }
    return hipGetLastError();
}

}  // namespace dma
