// Backward of dt = exp(A * softplus(bias + W . concat_h V)).
// Doge guide (gitcode), DMA section, forward step 3 (dt_proj over the value
// states of all kv heads of a token, then exp(A * softplus(.)); A is learnt,
// one scalar per kv head).  With x the projection of token t for kv head h:
//   dx = ddt dt A sigmoid(x),   dA[h] += ddt dt softplus(x),   dbias[h] += dx,
//   dW[h][c] += dx V[t][c],     dV[t][c] += sum_h dx W[h][c].
//
// dt_bwd_token_kernel: one workgroup per run of kTok tokens.  W is staged in
// LDS; each wave takes a token at a time, its lanes splitting the Hkv*d
// channels: x by a wave reduction per head, then dx and the dA term, and the
// token's dV contribution added in place.  Then the workgroup's partial sums
// of dW (each thread a (head, channel) entry at a time, channel fastest, so
// the V reads are coalesced), dbias and dA go to the workspace.
// dt_bwd_reduce_kernel sums the partials of every workgroup in a fixed order:
// the result does not depend on scheduling.
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 64;  // tokens per workgroup

__device__ __forceinline__ float softplus_acc(float x) {
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dt_bwd_token_kernel(
    const T *__restrict__ V, const T *__restrict__ W, const T *__restrict__ bias, const float *__restrict__ A,
    const float *__restrict__ ddt, int S, int Hkv, int width, int ntok, T *__restrict__ dV, float *__restrict__ part) {
    extern __shared__ __align__(16) float smem[];
    float *Ws = smem;                          // [Hkv][width] as float
    float *dxs = Ws + (size_t)Hkv * width;     // [kTok][Hkv]
    float *gas = dxs + kTok * Hkv;             // [kTok][Hkv]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t0 = blockIdx.x * kTok;
    const int nt = min(kTok, ntok - t0);
    for (int e = tid; e < Hkv * width; e += kThreads) Ws[e] = Elem<T>::load(W, e);
    __syncthreads();

    const int nc = width / 64;  // channels per lane (width is a multiple of 64)
    for (int tt = wave; tt < nt; tt += kThreads / 64) {
        const int t = t0 + tt;
        const int b = t / S, s = t - b * S;
        const T *vrow = V + (size_t)t * width;
        float xs[kMaxHkvDt];
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h) xs[h] = 0.f;
        for (int k = 0; k < nc; ++k) {
            const int c = lane + 64 * k;
            const float v = Elem<T>::load(vrow, c);
#pragma unroll
            for (int h = 0; h < kMaxHkvDt; ++h)
                if (h < Hkv) xs[h] = fmaf(Ws[h * width + c], v, xs[h]);
        }
        float dx[kMaxHkvDt];
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h) {
            dx[h] = 0.f;
            if (h < Hkv) {
                const float x = wave_sum(xs[h]) + (bias ? Elem<T>::load(bias, h) : 0.f);
                const float a = A[h];
                const float sp = softplus_acc(x);
                const float dtv = expf(a * sp);
                const float g = ddt[((size_t)b * Hkv + h) * S + s];
                dx[h] = g * dtv * a / (1.f + expf(-x));
                if (lane == 0) {
                    dxs[tt * Hkv + h] = dx[h];
                    gas[tt * Hkv + h] = g * dtv * sp;
                }
            }
        }
        if (dV) {
            T *drow = dV + (size_t)t * width;
            for (int k = 0; k < nc; ++k) {
                const int c = lane + 64 * k;
                float acc = Elem<T>::load(drow, c);
#pragma unroll
                for (int h = 0; h < kMaxHkvDt; ++h)
                    if (h < Hkv) acc = fmaf(dx[h], Ws[h * width + c], acc);
                Elem<T>::store(drow, c, acc);
            }
        }
    }
    __syncthreads();

    // partial sums of this workgroup's tokens
    const size_t stride = (size_t)Hkv * width + 2 * Hkv;
    float *out = part + (size_t)blockIdx.x * stride;
    for (int e = tid; e < Hkv * width; e += kThreads) {
        const int h = e / width, c = e - h * width;
        float acc = 0.f;
        for (int tt = 0; tt < nt; ++tt) acc = fmaf(dxs[tt * Hkv + h], Elem<T>::load(V, (size_t)(t0 + tt) * width + c), acc);
        out[e] = acc;
    }
    if (tid < Hkv) {
        float sb = 0.f, sa = 0.f;
        for (int tt = 0; tt < nt; ++tt) {
            sb += dxs[tt * Hkv + tid];
            sa += gas[tt * Hkv + tid];
        }
        out[(size_t)Hkv * width + tid] = sb;
        out[(size_t)Hkv * width + Hkv + tid] = sa;
    }
}

__global__ __launch_bounds__(kThreads) void dt_bwd_reduce_kernel(const float *__restrict__ part, int nparts, int Hkv,
                                                                 int width, float *__restrict__ dW,
                                                                 float *__restrict__ dbias, float *__restrict__ dA) {
    const size_t stride = (size_t)Hkv * width + 2 * Hkv;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= (int)stride) return;
    float acc = 0.f;
    for (int p = 0; p < nparts; ++p) acc += part[(size_t)p * stride + e];
    if (e < Hkv * width) {
        dW[e] = acc;
    } else if (e < Hkv * width + Hkv) {
        if (dbias) dbias[e - Hkv * width] = acc;
    } else {
        dA[e - Hkv * width - Hkv] = acc;
    }
}

}  // namespace

size_t dt_bwd_ws_bytes(int B, int S, int Hkv, int d) {
    const size_t ntok = (size_t)B * S;
    const size_t nparts = (ntok + kTok - 1) / kTok;
    return nparts * ((size_t)Hkv * Hkv * d + 2 * Hkv) * sizeof(float);
}

size_t dt_bwd_lds_bytes(int Hkv, int d) { return ((size_t)Hkv * Hkv * d + 2 * kTok * Hkv) * sizeof(float); }

hipError_t launch_dt_bwd(const void *V, const void *W, const void *bias, const float *A, int dtype, const float *ddt,
                         int B, int S, int Hkv, int d, void *dV, float *dW, float *dbias, float *dA, void *ws,
                         hipStream_t stream) {
    const int ntok = B * S, width = Hkv * d;
    const int nparts = (ntok + kTok - 1) / kTok;
    const size_t lds = dt_bwd_lds_bytes(Hkv, d);
    float *part = (float *)ws;
    if (dtype == 1)
        hipLaunchKernelGGL(dt_bwd_token_kernel<uint16_t>, dim3(nparts), dim3(kThreads), lds, stream,
                           (const uint16_t *)V, (const uint16_t *)W, (const uint16_t *)bias, A, ddt, S, Hkv, width,
                           ntok, (uint16_t *)dV, part);
    else
        hipLaunchKernelGGL(dt_bwd_token_kernel<float>, dim3(nparts), dim3(kThreads), lds, stream, (const float *)V,
                           (const float *)W, (const float *)bias, A, ddt, S, Hkv, width, ntok, (float *)dV, part);
    const int nout = width * Hkv + 2 * Hkv;
    hipLaunchKernelGGL(dt_bwd_reduce_kernel, dim3((nout + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                       (const float *)part, nparts, Hkv, width, dW, dbias, dA);
    return hipGetLastError();
}

}  // namespace dma
