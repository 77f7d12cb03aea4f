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
#include "dt_mfma.hpp"
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

// Cross-lane moves inside a row's group of LR lanes (LR in {8, 16, 32},
// groups aligned to LR): DPP where the pattern exists, else ds_swizzle.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int PATTERN> __device__ __forceinline__ float swz(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), PATTERN));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowMirror = 0x140, kRowHalfMirror = 0x141;
constexpr int kSwzXor16 = (0x10 << 10) | 0x1F, kSwzXor31 = (0x1F << 10) | 0x1F;

// sum over the LR lanes of the group, in every lane
template <int LR> __device__ __forceinline__ float group_sum(float v) {
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kRowHalfMirror>(v);                     // lane i <-> 7 - i: the other quad
    if constexpr (LR >= 16) v += dpp<kRowMirror>(v);  // lane i <-> 15 - i: the other half row
    if constexpr (LR >= 32) v += swz<kSwzXor16>(v);
    return v;
}
// the value of the mirror lane LR - 1 - i of the group
template <int LR> __device__ __forceinline__ float group_mirror(float v) {
    if constexpr (LR == 8) return dpp<kRowHalfMirror>(v);
    else if constexpr (LR == 16) return dpp<kRowMirror>(v);
    else return swz<kSwzXor31>(v);
}

// D: head_dim; NS: row steps per chunk (a step covers 64 / (lanes per row)
// rows of a token); MULTI: the token's Hq + Hkv rows take more than one chunk.
//
// Lane i of a row's group holds 16-byte chunk i of the row's first half if
// i < LR/2, else chunk LR/2 + (LR - 1 - i) of its second half: the rotation
// partner of every element then sits in the mirror lane LR - 1 - i, one DPP
// move away.
template <int D, typename T, int NS, bool MULTI>
__device__ __forceinline__ void qk_norm_rope_block(
    int blk, const T *Q, const T *K, const T *__restrict__ wq, const T *__restrict__ wk, float eps,
    double log2_theta, const int32_t *__restrict__ positions, int S, int Hq, int Hkv, int ntok, T *Qo, T *Ko) {
    using L = Lanes<T>;
    constexpr int E = L::kElems;   // elements per lane
    constexpr int LR = D / E;      // lanes per row
    constexpr int RW = 64 / LR;    // rows per step
    constexpr int H = D / 2;       // distinct angles per token
    static_assert(LR == 8 || LR == 16 || LR == 32, "row split");
    static_assert(H <= 64 && H % E == 0, "angles");
    // turns per position of frequency e: theta^(-2e/d) / (2 pi)
    __shared__ double turns[H];
    // per wave: cosines then sines of the current token's d/2 angles
    __shared__ __align__(16) float trig[kWaves][2][H];

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int li = lane % LR, ri = lane / LR;
    const bool low = li < LR / 2;  // first half: out = y cos - partner sin
    const int e0 = E * (low ? li : LR / 2 + (LR - 1 - li));  // this lane's first element
    const int nrows = Hq + Hkv;
    const int nch = (nrows + NS * RW - 1) / (NS * RW);  // chunks per token
    const int t_raw = __builtin_amdgcn_readfirstlane(blk * kWaves + wv);
    const int t = min(t_raw, ntok - 1);  // the wave's token

    // Element offset of this lane's 16 bytes of row r of token t in Q (r < Hq)
    // or K.  Rows past the last are clamped to it: such lanes load and store
    // the last row with the very values its own lanes hold.
    auto row_off = [&](int t, int r) __attribute__((always_inline)) {
        const bool q = r < Hq;
        const int64_t row = (int64_t)t * (q ? Hq : Hkv) + (q ? r : r - Hq);
        return row * D + e0;
    };
    auto load = [&](u32x4 (&x)[NS], int t, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int r = min(c * NS * RW + st * RW + ri, nrows - 1);
            x[st] = *reinterpret_cast<const u32x4 *>((r < Hq ? Q : K) + row_off(t, r));
        }
    };

    const u32x4 wqr = *reinterpret_cast<const u32x4 *>(wq + e0);
    const u32x4 wkr = *reinterpret_cast<const u32x4 *>(wk + e0);
    u32x4 xa[NS], xb[NS];
    load(xa, t, 0);
    const int pos = positions ? positions[t] : t % S;
    if (threadIdx.x < H) turns[threadIdx.x] = exp2(-(2.0 * threadIdx.x / D) * log2_theta) * 0.15915494309189535;
    __syncthreads();
    if (t_raw >= ntok) return;      // uniform per wave, after the only block barrier

    float wqv[E], wkv[E], cs[E], sn[E];
    L::unpack(wqr, wqv);
    L::unpack(wkr, wkv);

    // the sine and cosine of this lane's elements at position p: lane l
    // works out angle l % (d/2), the wave exchanges them through LDS
    auto angles = [&](int p) __attribute__((always_inline)) {
        const int e = lane % H;     // lanes past d/2 repeat the first d/2 (same values, same slots)
        const double a = (double)p * turns[e];
        const float r = (float)(a - rint(a)) * 6.283185307179586f;  // in [-pi, pi]
        float sv, cv;
        sincosf(r, &sv, &cv);
        trig[wv][0][e] = cv;
        trig[wv][1][e] = sv;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < E; i += 4) {
            const float4 c4 = *reinterpret_cast<const float4 *>(&trig[wv][0][e0 % H + i]);
            const float4 s4 = *reinterpret_cast<const float4 *>(&trig[wv][1][e0 % H + i]);
            cs[i] = c4.x; cs[i + 1] = c4.y; cs[i + 2] = c4.z; cs[i + 3] = c4.w;
            sn[i] = s4.x; sn[i + 1] = s4.y; sn[i + 2] = s4.z; sn[i + 3] = s4.w;
        }
    };

    auto compute = [&](const u32x4 (&x)[NS], int t, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int r = min(c * NS * RW + st * RW + ri, nrows - 1);
            const bool q = r < Hq;
            float xv[E];
            L::unpack(x[st], xv);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < E; ++i) ss = fmaf(xv[i], xv[i], ss);
            ss = group_sum<LR>(ss);
            const float inv = rsqrtf(ss / (float)D + eps);
            float y[E], out[E];
#pragma unroll
            for (int i = 0; i < E; ++i) y[i] = xv[i] * inv * (q ? wqv[i] : wkv[i]);
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float pv = group_mirror<LR>(y[i]);  // element e + d/2 (or e - d/2)
                out[i] = fmaf(y[i], cs[i], (low ? -pv : pv) * sn[i]);
            }
            *reinterpret_cast<u32x4 *>((q ? Qo : Ko) + row_off(t, r)) = L::pack(out);
        }
    };

    angles(pos);
    if constexpr (!MULTI) {
        compute(xa, t, 0);
    } else {
        // chunk c is worked on while chunk c + 1 is in flight; past the last
        // chunk the request repeats it, so that requests and stores are
        // unconditional and the wait for a chunk counts exactly the memory
        // operations issued after it
        for (int c = 0;;) {
            load(xb, t, min(c + 1, nch - 1));
            compute(xa, t, c);
            if (++c >= nch) break;
            load(xa, t, min(c + 1, nch - 1));
            compute(xb, t, c);
            if (++c >= nch) break;
        }
    }
}

template <int D, typename T, int NS, bool MULTI>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    const T *Q, const T *K, const T *__restrict__ wq, const T *__restrict__ wk, float eps, double log2_theta,
    const int32_t *__restrict__ positions, int S, int Hq, int Hkv, int ntok, T *Qo, T *Ko) {
    qk_norm_rope_block<D, T, NS, MULTI>(blockIdx.x, Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv, ntok,
                                        Qo, Ko);
}

// The whole prologue of bf16 projections in one launch: the first ndt
// workgroups run dt over V — matrix-core tiles (four waves, a 16-token tile
// each, striding over the tiles, one 128-channel chunk of loads in flight so
// that the kernel's register count stays that of the Q/K part), or for calls
// of at most kDtSmallTokens tokens one wave per (token, kv head), exactly as
// dma_dt does, so both give the same dt — and the rest normalise and rotate
// Q and K one token per wave.  The two streams read disjoint inputs and write
// disjoint outputs, so they run side by side instead of one after the other.
template <int D, int NS, bool MULTI>
__global__ __launch_bounds__(kThreads) void prologue_kernel(
    const uint16_t *Q, const uint16_t *K, const uint16_t *__restrict__ wq, const uint16_t *__restrict__ wk,
    float eps, double log2_theta, const int32_t *__restrict__ positions, int S, int Hq, int Hkv, int ntok,
    uint16_t *Qo, uint16_t *Ko, const uint16_t *__restrict__ V, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, const float *__restrict__ A, float *__restrict__ dt_out, int ndt) {
    if ((int)blockIdx.x < ndt) {
        const int64_t first = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
        if (ntok <= kDtSmallTokens) {
            if (first < (int64_t)ntok * Hkv) dt_pair(first, V, W, bias, A, S, Hkv, Hkv * D, dt_out, S, nullptr);
        } else {
            dt_mfma_tiles<1>(first, (int64_t)ndt * kWaves, V, W, bias, A, S, Hkv, Hkv * D, ntok, dt_out, S,
                             nullptr);
        }
        return;  // uniform per workgroup
    }
    qk_norm_rope_block<D, uint16_t, NS, MULTI>(blockIdx.x - ndt, Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv,
                                               ntok, Qo, Ko);
}

// rows per chunk step and chunk layout of a token's Q and K rows: as few
// chunks of at most 4 steps as possible, each of equal size
template <int D, typename T>
inline void qk_chunks(int Hq, int Hkv, int &nchunk, int &ns) {
    constexpr int RW = 64 / (D / Lanes<T>::kElems);
    const int steps = (Hq + Hkv + RW - 1) / RW;
    nchunk = (steps + 3) / 4;
    ns = (steps + nchunk - 1) / nchunk;
}

template <int D>
void launch_prologue_t(const void *Q, const void *K, const void *wq, const void *wk, float eps, double log2_theta,
                       const int32_t *positions, int S, int Hq, int Hkv, int ntok, void *Qo, void *Ko,
                       const void *V, const void *W, const void *bias, const float *A, float *dt_out,
                       hipStream_t stream) {
    int nchunk, ns;
    qk_chunks<D, uint16_t>(Hq, Hkv, nchunk, ns);
    const int nqk = (ntok + kWaves - 1) / kWaves;
    const int64_t ntiles = (ntok + 15) / 16;
    const int64_t want = ntok <= kDtSmallTokens ? ((int64_t)ntok * Hkv + kWaves - 1) / kWaves  // a wave per pair
                                                : (ntiles + kWaves - 1) / kWaves;                 // a wave per tile
    const int ndt = (int)(want < 2048 ? want : 2048);
    const dim3 grid((unsigned)(ndt + nqk));
#define DMA_PRO(NS, MULTI)                                                                                          \
    hipLaunchKernelGGL((prologue_kernel<D, NS, MULTI>), grid, dim3(kThreads), 0, stream, (const uint16_t *)Q,          \
                       (const uint16_t *)K, (const uint16_t *)wq, (const uint16_t *)wk, eps, log2_theta, positions, S, \
                       Hq, Hkv, ntok, (uint16_t *)Qo, (uint16_t *)Ko, (const uint16_t *)V, (const uint16_t *)W,        \
                       (const uint16_t *)bias, A, dt_out, ndt)
    if (nchunk == 1) {
        switch (ns) {
            case 1: DMA_PRO(1, false); break;
            case 2: DMA_PRO(2, false); break;
            case 3: DMA_PRO(3, false); break;
            default: DMA_PRO(4, false); break;
        }
    } else {
        switch (ns) {
            case 2: DMA_PRO(2, true); break;
            case 3: DMA_PRO(3, true); break;
            default: DMA_PRO(4, true); break;
        }
    }
#undef DMA_PRO
}

template <int D, typename T>
void launch_t(const void *Q, const void *K, const void *wq, const void *wk, float eps, double log2_theta,
              const int32_t *positions, int S, int Hq, int Hkv, int ntok, void *Qo, void *Ko, hipStream_t stream) {
    int nchunk, ns;
    qk_chunks<D, T>(Hq, Hkv, nchunk, ns);
    const unsigned grid = (unsigned)((ntok + kWaves - 1) / kWaves);
#define DMA_QKNR(NS, MULTI)                                                                                   \
    hipLaunchKernelGGL((qk_norm_rope_kernel<D, T, NS, MULTI>), dim3(grid), dim3(kThreads), 0, stream,         \
                       (const T *)Q, (const T *)K, (const T *)wq, (const T *)wk, eps, log2_theta, positions, S, Hq, \
                       Hkv, ntok, (T *)Qo, (T *)Ko)
    if (nchunk == 1) {
        switch (ns) {
            case 1: DMA_QKNR(1, false); break;
            case 2: DMA_QKNR(2, false); break;
            case 3: DMA_QKNR(3, false); break;
            default: DMA_QKNR(4, false); break;
        }
    } else {
        switch (ns) {
            case 2: DMA_QKNR(2, true); break;
            case 3: DMA_QKNR(3, true); break;
            default: DMA_QKNR(4, true); break;
        }
    }
#undef DMA_QKNR
}

}  // namespace

hipError_t launch_prologue_bf16(const void *Q, const void *K, const void *wq, const void *wk, float eps,
                                double rope_theta, const int32_t *positions, int B, int S, int Hq, int Hkv, int d,
                                void *Qo, void *Ko, const void *V, const void *W, const void *bias, const float *A,
                                float *dt_out, hipStream_t stream) {
    const int ntok = B * S;
    const double log2_theta = __builtin_log2(rope_theta);
    if (d == 128)
        launch_prologue_t<128>(Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv, ntok, Qo, Ko, V, W, bias, A,
                               dt_out, stream);
    else
        launch_prologue_t<64>(Q, K, wq, wk, eps, log2_theta, positions, S, Hq, Hkv, ntok, Qo, Ko, V, W, bias, A,
                              dt_out, stream);
    return hipGetLastError();
}

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
