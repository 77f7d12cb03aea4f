// Q/K normalisation and rotary position embedding: one pass over each
// token's Q and K head rows.
// Doge guide (gitcode), DMA section, forward step 1: after q_proj / k_proj,
// Q and K go through q_norm / k_norm -- an RMSNorm over head_dim with one
// learnable weight per element (eps = rms_norm_eps) -- and then the rotary
// position embedding of the Llama code: element e < d/2 pairs with e + d/2
// and the pair turns by pos * theta^(-2e/d), towards +e_{e+d/2}.
//
// One wave per token.  A lane holds 16 bytes of a head row (8 bf16 or 4
// float32 elements); the lanes of a row reduce its sum of squares with
// shuffles, and the rotation partner of a lane's elements sits in the lane
// half a row away.  A token has d/2 distinct angles, the same for all of its
// Hq + Hkv rows: lane l works out the sine and cosine of angle l % (d/2) once
// and the wave shares them through LDS.  The angle is reduced modulo one turn
// in float64 (pos * theta^(-2e/d) reaches 10^4 radians and more, where a
// float32 angle is off by 10^-3), so the sine and cosine come from a float32
// argument in [-pi, pi].  Every Q and K element is read once and written once;
// the outputs may alias the inputs (each lane writes only the 16 bytes it
// read, after reading them).
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <typename T> struct Lanes;
template <> struct Lanes<uint16_t> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void unpack(const u32x4 &v, float (&x)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(v[i] << 16);
            x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static u32x4 pack(const float (&y)[8]) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = (uint32_t)f32_to_bf16(y[2 * i]) | ((uint32_t)f32_to_bf16(y[2 * i + 1]) << 16);
        return v;
    }
};
template <> struct Lanes<float> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void unpack(const u32x4 &v, float (&x)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
    }
    __device__ __forceinline__ static u32x4 pack(const float (&y)[4]) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(y[i]);
        return v;
    }
};

// D: head_dim; NS: row steps whose loads are issued together (a step covers
// 64 / (lanes per row) rows of the token).
template <int D, typename T, int NS>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    const T *Q, const T *K, const T *__restrict__ wq, const T *__restrict__ wk, float eps, double log2_theta,
    const int32_t *__restrict__ positions, int S, int Hq, int Hkv, int ntok, T *Qo, T *Ko) {
    using L = Lanes<T>;
    constexpr int E = L::kElems;   // elements per lane
    constexpr int LR = D / E;      // lanes per row
    constexpr int RW = 64 / LR;    // rows per step
    constexpr int H = D / 2;       // distinct angles per token
    static_assert(LR >= 2 && LR <= 64 && 64 % LR == 0 && H <= 64 && H % E == 0, "row split");
    // turns per position of frequency e: theta^(-2e/d) / (2 pi)
    __shared__ double turns[H];
    // per wave: cosines then sines of the token's d/2 angles
    __shared__ __align__(16) float trig[kWaves][2][H];

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int tok_raw = blockIdx.x * kWaves + wv;
    const int tok = min(tok_raw, ntok - 1);
    const int li = lane % LR, ri = lane / LR;
    const int e0 = E * li;         // this lane's first element
    const bool low = e0 < H;       // first half: out = y cos - partner sin
    const int nrows = Hq + Hkv;

    // the loads of NS row steps are issued together; rows past the last
    // repeat it and are not stored
    u32x4 xr[NS];
    size_t off[NS];
    bool isq[NS];
    auto load_rows = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int r = min(r0 + st * RW + ri, nrows - 1);
            isq[st] = r < Hq;
            off[st] = isq[st] ? ((size_t)tok * Hq + r) * D + e0 : ((size_t)tok * Hkv + (r - Hq)) * D + e0;
            xr[st] = *reinterpret_cast<const u32x4 *>((isq[st] ? Q : K) + off[st]);
        }
    };
    // the first rows are requested before anything else, so that their
    // latency overlaps the position load and the angle work
    load_rows(0);
    const int pos = positions ? positions[tok] : tok % S;
    const u32x4 wqr = *reinterpret_cast<const u32x4 *>(wq + e0);
    const u32x4 wkr = *reinterpret_cast<const u32x4 *>(wk + e0);
    if (threadIdx.x < H) turns[threadIdx.x] = exp2(-(2.0 * threadIdx.x / D) * log2_theta) * 0.15915494309189535;
    __syncthreads();
    if (tok_raw >= ntok) return;  // uniform per wave, after the only block barrier

    {
        const int e = lane % H;   // lanes past d/2 repeat the first d/2 (same values, same slots)
        const double a = (double)pos * turns[e];
        const float r = (float)(a - rint(a)) * 6.283185307179586f;  // in [-pi, pi]
        float s, c;
        sincosf(r, &s, &c);
        trig[wv][0][e] = c;
        trig[wv][1][e] = s;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float cs[E], sn[E], wqv[E], wkv[E];
#pragma unroll
    for (int i = 0; i < E; i += 4) {
        const float4 c4 = *reinterpret_cast<const float4 *>(&trig[wv][0][e0 % H + i]);
        const float4 s4 = *reinterpret_cast<const float4 *>(&trig[wv][1][e0 % H + i]);
        cs[i] = c4.x; cs[i + 1] = c4.y; cs[i + 2] = c4.z; cs[i + 3] = c4.w;
        sn[i] = s4.x; sn[i + 1] = s4.y; sn[i + 2] = s4.z; sn[i + 3] = s4.w;
    }
    L::unpack(wqr, wqv);
    L::unpack(wkr, wkv);

    for (int r0 = 0;;) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            float x[E];
            L::unpack(xr[st], x);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < E; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
            for (int o = 1; o < LR; o <<= 1) ss += __shfl_xor(ss, o, 64);
            const float inv = rsqrtf(ss / (float)D + eps);
            float y[E], out[E];
#pragma unroll
            for (int i = 0; i < E; ++i) y[i] = x[i] * inv * (isq[st] ? wqv[i] : wkv[i]);
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float p = __shfl_xor(y[i], LR / 2, 64);  // element e + d/2 (or e - d/2)
                out[i] = fmaf(y[i], cs[i], (low ? -p : p) * sn[i]);
            }
            if (r0 + st * RW + ri < nrows) *reinterpret_cast<u32x4 *>((isq[st] ? Qo : Ko) + off[st]) = L::pack(out);
        }
        r0 += NS * RW;
        if (r0 >= nrows) break;
        load_rows(r0);
    }
}

template <int D, typename T>
void launch_t(const void *Q, const void *K, const void *wq, const void *wk, float eps, double log2_theta,
              const int32_t *positions, int S, int Hq, int Hkv, int ntok, void *Qo, void *Ko, hipStream_t stream) {
    constexpr int RW = 64 / (D / Lanes<T>::kElems);
    const int steps = (Hq + Hkv + RW - 1) / RW;
    const unsigned grid = (unsigned)((ntok + kWaves - 1) / kWaves);
#define DMA_QKNR(NS)                                                                                         \
    hipLaunchKernelGGL((qk_norm_rope_kernel<D, T, NS>), dim3(grid), dim3(kThreads), 0, stream, (const T *)Q, \
                       (const T *)K, (const T *)wq, (const T *)wk, eps, log2_theta, positions, S, Hq, Hkv, ntok, \
                       (T *)Qo, (T *)Ko)
    if (steps <= 1)
        DMA_QKNR(1);
    else if (steps <= 2)
        DMA_QKNR(2);
    else if (steps <= 4)
        DMA_QKNR(4);
    else
        DMA_QKNR(8);
#undef DMA_QKNR
}

}  // namespace

hipError_t launch_qk_norm_rope(const void *Q, const void *K, int dtype, const void *wq, const void *wk, float eps,
                               double rope_theta, const int32_t *positions, int B, int S, int Hq, int Hkv, int d,
                               void *Qo, void *Ko, hipStream_t stream) {
    const int ntok = B * S;
    const double log2_theta = __builtin_log2(rope_theta);
    if (dtype == 1) {
        if (d == 128)
            launch_t<128, uint16_t>(Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv, ntok, Qo, Ko, stream);
        else
            launch_t<64, uint16_t>(Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv, ntok, Qo, Ko, stream);
    } else {
        if (d == 128)
            launch_t<128, float>(Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv, ntok, Qo, Ko, stream);
        else
            launch_t<64, float>(Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv, ntok, Qo, Ko, stream);
    }
    return hipGetLastError();
}

}  // namespace dma
