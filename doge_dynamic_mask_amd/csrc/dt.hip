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
// reduction.  softplus and exp run in float32 in both.
#include "common.hpp"
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
            if (h < Hkv && (h % kLanesPerToken) == q) {
                const float x = acc[h] + bs[h];
                out[((int64_t)b * Hkv + h) * ld + col] = expf(As[h] * softplus_f32(x));
            }
        }
    }
}

constexpr int kMfmaThreads = 128;     // two waves, one 16-token tile each
constexpr int kChunk = 128;           // channels per lane group pass (4 lanes x 32)
constexpr int kChunksPerBatch = 4;    // chunks loaded before the first multiply

// softplus and exp on the hardware exp2 / log2: softplus(x) = max(x, 0) +
// ln(1 + e^-|x|) and e^y, with an absolute error in softplus of a few 1e-8
// and a relative error in e^y of about |y| * 2^-23, far inside the float32
// tolerance of dt (which is relative to exp of their product).
__device__ __forceinline__ float dt_from_x(float a, float x) {
    constexpr float kLn2 = 0.6931471805599453f;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    const float sp = fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * kLn2;
    return __builtin_amdgcn_exp2f(a * sp * kLog2e);
}

// bf16 dt on matrix cores.  16x16x32 bf16 operand layouts (l = lane):
//   A[m = l%16][k = 8*(l/16) + j], B[k = 8*(l/16) + j][n = l%16],
//   C[m = 4*(l/16) + i][n = l%16], i = 0..3.
// Channel of k-slot (kg = l/16, j) in step s of chunk c: c*128 + 32*kg + 8*s + j.
// Both operands come straight from global memory (W is small and stays in
// the caches), so no LDS and no barrier stand between the loads and the math.
__global__ __launch_bounds__(kMfmaThreads) void dt_mfma_kernel(
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ W, const uint16_t *__restrict__ bias,
    const float *__restrict__ A, int S, int Hkv, int width, int64_t ntok,
    float *__restrict__ out, int64_t ld, const int32_t *__restrict__ out_pos) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mr = lane & 15, kg = lane >> 4;
    const int nchunk = (width + kChunk - 1) / kChunk;
    const bool head_ok = mr < Hkv;
    const int hc = head_ok ? mr : 0;  // clamped head for the (unused) W loads
    const int64_t ntiles = (ntok + 15) / 16;
    const int64_t stride = (int64_t)gridDim.x * (kMfmaThreads / 64);
    const float a_h = A[hc];
    const float b_h = bias ? bf16_to_f32(bias[hc]) : 0.f;

    // this lane's 16-byte vectors of chunks c0 .. c0 + kChunksPerBatch - 1 of
    // its token row and of W's row for head l%16 (zeros past the row, the last
    // token or the last head).  Requests are unconditional from clamped, valid
    // addresses: a conditional load would be a branch of its own.
    uint4 va[kChunksPerBatch][4], wa[kChunksPerBatch][4];
    auto load_batch = [&](int64_t tile, int c0) __attribute__((always_inline)) {
        const int64_t t = tile * 16 + mr;
        const bool tok_ok = t < ntok;
        const uint16_t *vrow = V + (tok_ok ? t : ntok - 1) * (int64_t)width;
        const uint16_t *wrow = W + (size_t)hc * width;
#pragma unroll
        for (int cc = 0; cc < kChunksPerBatch; ++cc) {
            const int base = (c0 + cc) * kChunk + 32 * kg;
            const bool in = base < width;
            const int cb = in ? base : width - 32;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint4 x = *reinterpret_cast<const uint4 *>(vrow + cb + 8 * st);
                const uint4 y = *reinterpret_cast<const uint4 *>(wrow + cb + 8 * st);
                va[cc][st] = (tok_ok && in) ? x : make_uint4(0, 0, 0, 0);
                wa[cc][st] = (head_ok && in) ? y : make_uint4(0, 0, 0, 0);
            }
        }
    };

    int64_t tile = (int64_t)blockIdx.x * (kMfmaThreads / 64) + wave;
    if (tile < ntiles) load_batch(tile, 0);
    for (; tile < ntiles; tile += stride) {
        // batch and column of this lane's four output tokens, out_pos loaded
        // now so that its latency hides behind the products
        int ob[4], os[4];
        int64_t ocol[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t tok = tile * 16 + 4 * kg + i;
            const int64_t tc = tok < ntok ? tok : ntok - 1;
            ob[i] = ntok <= 0x7fffffff ? (int)((uint32_t)tc / (uint32_t)S) : (int)(tc / S);
            os[i] = (int)(tc - (int64_t)ob[i] * S);
            ocol[i] = out_pos ? (int64_t)out_pos[ob[i]] : 0;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nchunk; c0 += kChunksPerBatch) {
            if (c0 > 0) load_batch(tile, c0);  // the first batch is already in flight
#pragma unroll
            for (int cc = 0; cc < kChunksPerBatch; ++cc) {
                if (c0 + cc >= nchunk) break;
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va[cc][st]),
                                                                  __builtin_bit_cast(bf16x8, wa[cc][st]), acc, 0, 0, 0);
            }
        }
        if (tile + stride < ntiles) load_batch(tile + stride, 0);  // next tile's rows in flight
        if (head_ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tok = tile * 16 + 4 * kg + i;
                if (tok < ntok)
                    out[((int64_t)ob[i] * Hkv + mr) * ld + ocol[i] + os[i]] = dt_from_x(a_h, acc[i] + b_h);
            }
        }
    }
}

}  // namespace

hipError_t launch_dt(const void *V, const void *W, const void *bias, const float *A, int dtype,
                     int B, int S, int Hkv, int d, float *dt_out, int64_t ld_out,
                     const int32_t *out_pos, hipStream_t stream) {
    const int64_t ntok = (int64_t)B * S;
    if (dtype == 1) {
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
