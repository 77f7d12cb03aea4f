// Backward of dt = exp(A * softplus(bias + W . concat_h V)).
// Doge guide (gitcode), DMA section, forward step 3 (dt_proj over the value
// states of all kv heads of a token, then exp(A * softplus(.)); A is learnt,
// one scalar per kv head).  With x the projection of token t for kv head h:
//   dx = ddt dt A sigmoid(x),   dA[h] += ddt dt softplus(x),   dbias[h] += dx,
//   dW[h][c] += dx V[t][c],     dV[t][c] += sum_h dx W[h][c].
//
// dt_bwd_token_kernel: one workgroup per run of 16 tokens.  W is staged in
// LDS; each 16-lane group takes one token, its lanes splitting the token's
// Hkv*d channels in 16-byte vectors: x by a group reduction per head, then dx
// and the dA term, and the token's dV contribution added in place.  Then the workgroup's partial sums
// of dW (each thread a channel and every head, the loads of all the
// workgroup's tokens for that channel issued together and coalesced across
// threads), dbias and dA go to the workspace.
// The partials are summed in fixed-order levels (dt_bwd_sum_kernel): slices
// of kSlice partials, all of a slice's loads in flight at once, until at
// most kFinalRows are left, which dt_bwd_final_kernel sums (four waves take
// a quarter of the rows each, then add their sums in wave order); the
// result does not depend on scheduling.
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 16;  // tokens per workgroup

__device__ __forceinline__ float softplus_acc(float x) {
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

template <typename T> __device__ __forceinline__ void unpack_vec(const u32x4 &u, float *v);
template <> __device__ __forceinline__ void unpack_vec<uint16_t>(const u32x4 &u, float *v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
template <> __device__ __forceinline__ void unpack_vec<float>(const u32x4 &u, float *v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(u[i]);
}
template <typename T> __device__ __forceinline__ u32x4 pack_vec(const float *v);
template <> __device__ __forceinline__ u32x4 pack_vec<uint16_t>(const float *v) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    return u;
}
template <> __device__ __forceinline__ u32x4 pack_vec<float>(const float *v) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __float_as_uint(v[i]);
    return u;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dt_bwd_token_kernel(
    const T *__restrict__ V, const T *__restrict__ W, const T *__restrict__ bias, const float *__restrict__ A,
    const float *__restrict__ ddt, int S, int Hkv, int width, int ntok, T *__restrict__ dV, float *__restrict__ part) {
    extern __shared__ __align__(16) float smem[];
    float *Ws = smem;                          // [Hkv][width] as float
    float *dxs = Ws + (size_t)Hkv * width;     // [kTok][Hkv]
    float *gas = dxs + kTok * Hkv;             // [kTok][Hkv]
    static_assert(kTok == 4 * (kThreads / 64), "one token per 16-lane group");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t0 = blockIdx.x * kTok;
    const int nt = min(kTok, ntok - t0);
    for (int e = tid; e < Hkv * width; e += kThreads) Ws[e] = Elem<T>::load(W, e);
    __syncthreads();

    // Every 16-lane group of a wave takes one token (so a workgroup's 16
    // tokens are all in flight at once); its lanes split the token's 16-byte
    // vectors of Hkv*d channels.
    constexpr int EV = 16 / (int)sizeof(T);
    const int nvec = width / EV;
    const int grp = lane >> 4, l16 = lane & 15;
    const int tt = 4 * wave + grp;
    const bool tok_ok = tt < nt;
    const int t = t0 + (tok_ok ? tt : nt - 1);
    const int b = t / S, s = t - b * S;
    const T *vrow = V + (size_t)t * width;
    float xs[kMaxHkvDt];
#pragma unroll
    for (int h = 0; h < kMaxHkvDt; ++h) xs[h] = 0.f;
    for (int j = l16; j < nvec; j += 16) {
        float v[EV];
        unpack_vec<T>(*reinterpret_cast<const u32x4 *>(vrow + EV * j), v);
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h) {
            if (h < Hkv) {
                const float *wr = Ws + h * width + EV * j;
#pragma unroll
                for (int e = 0; e < EV; ++e) xs[h] = fmaf(wr[e], v[e], xs[h]);
            }
        }
    }
    float dx[kMaxHkvDt];
#pragma unroll
    for (int h = 0; h < kMaxHkvDt; ++h) {
        dx[h] = 0.f;
        if (h < Hkv) {
            float xh = xs[h];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) xh += __shfl_xor(xh, o, 64);
            const float x = xh + (bias ? Elem<T>::load(bias, h) : 0.f);
            const float a = A[h];
            const float sp = softplus_acc(x);
            const float dtv = expf(a * sp);
            const float g = ddt[((size_t)b * Hkv + h) * S + s];
            dx[h] = g * dtv * a / (1.f + expf(-x));
            if (l16 == 0 && tok_ok) {
                dxs[tt * Hkv + h] = dx[h];
                gas[tt * Hkv + h] = g * dtv * sp;
            }
        }
    }
    if (dV && tok_ok) {
        T *drow = dV + (size_t)t * width;
        for (int j = l16; j < nvec; j += 16) {
            float v[EV];
            unpack_vec<T>(*reinterpret_cast<const u32x4 *>(drow + EV * j), v);
#pragma unroll
            for (int h = 0; h < kMaxHkvDt; ++h) {
                if (h < Hkv) {
                    const float *wr = Ws + h * width + EV * j;
#pragma unroll
                    for (int e = 0; e < EV; ++e) v[e] = fmaf(dx[h], wr[e], v[e]);
                }
            }
            *reinterpret_cast<u32x4 *>(drow + EV * j) = pack_vec<T>(v);
        }
    }
    __syncthreads();

    // partial sums of this workgroup's tokens
    const size_t stride = (size_t)Hkv * width + 2 * Hkv;
    float *out = part + (size_t)blockIdx.x * stride;
    for (int c = tid; c < width; c += kThreads) {
        float v[kTok];
#pragma unroll
        for (int tt = 0; tt < kTok; ++tt) v[tt] = Elem<T>::load(V, (size_t)(t0 + min(tt, nt - 1)) * width + c);
        float acc[kMaxHkvDt];
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h) acc[h] = 0.f;
#pragma unroll
        for (int tt = 0; tt < kTok; ++tt) {
            if (tt < nt) {
#pragma unroll
                for (int h = 0; h < kMaxHkvDt; ++h)
                    if (h < Hkv) acc[h] = fmaf(dxs[tt * Hkv + h], v[tt], acc[h]);
            }
        }
#pragma unroll
        for (int h = 0; h < kMaxHkvDt; ++h)
            if (h < Hkv) out[(size_t)h * width + c] = acc[h];
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

constexpr int kSlice = 16;  // partials summed per thread and level

// out[y][e] = sum of in[p][e] over the y-th slice of kSlice rows p (rows of
// nout floats).
__global__ __launch_bounds__(kThreads) void dt_bwd_sum_kernel(const float *__restrict__ in, int nrows, int nout,
                                                              float *__restrict__ out) {
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= nout) return;
    const int p0 = blockIdx.y * kSlice;
    float v[kSlice];
#pragma unroll
    for (int k = 0; k < kSlice; ++k) v[k] = p0 + k < nrows ? in[(size_t)(p0 + k) * nout + e] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kSlice; ++k) acc += v[k];
    out[(size_t)blockIdx.y * nout + e] = acc;
}

constexpr int kFinalRows = 4 * kSlice;  // rows the last level sums

// The last level: column e = 64 blockIdx.x + lane of the n <= kFinalRows
// rows of in, summed into dW, dbias and dA.
__global__ __launch_bounds__(kThreads) void dt_bwd_final_kernel(const float *__restrict__ in, int nrows, int nout,
                                                                int Hkv, int width, float *__restrict__ dW,
                                                                float *__restrict__ dbias, float *__restrict__ dA) {
    __shared__ float part[kThreads / 64][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int ec = min(e, nout - 1);
    const int per = (nrows + 3) / 4;
    const int p0 = wave * per;
    float v[kSlice];
#pragma unroll
    for (int k = 0; k < kSlice; ++k) {
        const int p = min(p0 + k, nrows - 1);  // past the wave's rows: a repeat, not added
        v[k] = in[(size_t)p * nout + ec];
    }
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kSlice; ++k)
        if (k < per && p0 + k < nrows) acc += v[k];
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0 || e >= nout) return;
    acc = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    if (e < Hkv * width) {
        dW[e] = acc;
    } else if (e < Hkv * width + Hkv) {
        if (dbias) dbias[e - Hkv * width] = acc;
    } else {
        dA[e - Hkv * width - Hkv] = acc;
    }
}

}  // namespace

// rows of partial sums left after each level: ceil(n / kSlice) until at most
// kFinalRows
static size_t sum_levels_rows(size_t nparts) {
    size_t tot = 0;
    for (size_t n = nparts; n > (size_t)kFinalRows;) {
        n = (n + kSlice - 1) / kSlice;
        tot += n;
    }
    return tot;
}

size_t dt_bwd_ws_bytes(int B, int S, int Hkv, int d) {
    const size_t ntok = (size_t)B * S;
    const size_t nparts = (ntok + kTok - 1) / kTok;
    return (nparts + sum_levels_rows(nparts)) * ((size_t)Hkv * Hkv * d + 2 * Hkv) * sizeof(float);
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
    const unsigned gx = (unsigned)((nout + kThreads - 1) / kThreads);
    const float *in = part;
    float *next = part + (size_t)nparts * nout;
    int n = nparts;
    while (n > kFinalRows) {
        const int m = (n + kSlice - 1) / kSlice;
        hipLaunchKernelGGL(dt_bwd_sum_kernel, dim3(gx, (unsigned)m), dim3(kThreads), 0, stream, in, n, nout, next);
        in = next;
        next += (size_t)m * nout;
        n = m;
    }
    hipLaunchKernelGGL(dt_bwd_final_kernel, dim3((unsigned)((nout + 63) / 64)), dim3(kThreads), 0, stream, in, n, nout,
                       Hkv, width, dW, dbias, dA);
    return hipGetLastError();
}

}  // namespace dma
