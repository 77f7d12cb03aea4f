// Cross Domain MoE (CDMoE) routed experts: product-key routing and the
// embedding experts.
// Doge guide (gitcode), CDMoE section and the DogeConfig table
// (num_experts, num_experts_per_tok, hidden_act): router_gate maps a hidden
// state to 2 * nk logits (nk = floor(sqrt(num_experts))), a top-k is taken in
// each of the two domains, their Cartesian product names the experts
// (x index * nk + y index, score = x logit + y logit), and the kept experts
// are embedding rows: down_embed row . h, the activation, and up_embed rows
// weighted by the routing weights.
//
// cdmoe_logits_kernel: the router product on matrix cores: 16x16x32 bf16
// MFMA, tokens as M, router outputs as N, hidden as K; both operands straight
// from their 16-byte loads (the router weight stays in L2).
//
// cdmoe_route_kernel: one wave per token.  Each domain's top k by rank
// (larger first, lower index first among equal; a rank is a count of better
// keys, so ranks are unique).  A pair (a, b) of domain ranks is preceded by
// every (a', b') with a' <= a and b' <= b (their scores are at least as large,
// and equal scores go in the order of the domain ranks), so only the pairs
// with (a + 1)(b + 1) <= k can be among the k best: about k (1 + ln k) of them
// instead of k^2.  These are ranked among themselves the same way; the
// softmax of the k best scores gives the weights.  Pair scores are float32
// sums of the two logits.
//
// cdmoe_experts_kernel: one workgroup per token.  Its waves take the kept
// experts in turn for z = down_e . h (lanes split the hidden size), each
// expert's act = silu(z) * weight goes to LDS, then every thread owns a slice
// of the hidden size and sums act_e * up_e over the experts, all of a slice's
// expert rows requested before they are summed.
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- logits
constexpr int kNT = 4;     // 16-output tiles per wave
constexpr int kBatch = 4;  // k-steps of 32 whose loads are issued together

__global__ __launch_bounds__(kThreads) void cdmoe_logits_kernel(const uint16_t *__restrict__ h,
                                                                const uint16_t *__restrict__ Wr, int T, int H, int N,
                                                                float *__restrict__ logits) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, q = lane >> 4;
    const int t0 = blockIdx.x * 64 + 16 * wave;
    const int n0 = blockIdx.y * 16 * kNT;
    const uint16_t *arow = h + (size_t)min(t0 + m, T - 1) * H + 8 * q;
    const uint16_t *brow[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) brow[j] = Wr + (size_t)min(n0 + 16 * j + m, N - 1) * H + 8 * q;
    f32x4 acc[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nsteps = H / 32;
    for (int s0 = 0; s0 < nsteps; s0 += kBatch) {
        bf16x8 a[kBatch], b[kBatch][kNT];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int s = min(s0 + u, nsteps - 1);
            a[u] = ld8(arow + 32 * s);
#pragma unroll
            for (int j = 0; j < kNT; ++j) b[u][j] = ld8(brow[j] + 32 * s);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (s0 + u < nsteps) {
#pragma unroll
                for (int j = 0; j < kNT; ++j) acc[j] = mfma16(a[u], b[u][j], acc[j]);
            }
        }
    }
    // C[m = token 4q + i][n = output l % 16]
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int n = n0 + 16 * j + m;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 4 * q + i;
            if (t < T && n < N) logits[(size_t)t * N + n] = acc[j][i];
        }
    }
}

// ---------------------------------------------------------------- routing
constexpr int kMaxNk = 256;
constexpr int kMaxK = 128;
constexpr int kMaxCand = 768;  // sum over a < k of floor(k / (a + 1)) for k <= 128 is 695

struct RouteLds {
    float lv[2][kMaxNk];   // logits of the two domains
    float sv[2][kMaxK];    // top-k values in rank order
    int si[2][kMaxK];      // and their indices
    int pref[kMaxK + 1];   // first candidate of each x rank
    float cs[kMaxCand];    // candidate scores
    int ct[kMaxCand];      // candidate tie order a * k + b
    int ce[kMaxCand];      // candidate expert index
};

__global__ __launch_bounds__(kThreads) void cdmoe_route_kernel(const float *__restrict__ logits, int T, int nk, int k,
                                                               int32_t *__restrict__ idx, float *__restrict__ wts) {
    __shared__ RouteLds lds[kWaves];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * kWaves + wave;
    if (t >= T) return;  // uniform per wave; no block barrier below
    RouteLds &L = lds[wave];
    const float *lrow = logits + (size_t)t * 2 * nk;
    for (int n = lane; n < 2 * nk; n += 64) L.lv[n >= nk][n >= nk ? n - nk : n] = lrow[n];
    wave_lds_sync();
    // rank of each key in its domain; the k best go to (sv, si) in rank order
    for (int d = 0; d < 2; ++d) {
        for (int n = lane; n < nk; n += 64) {
            const float v = L.lv[d][n];
            int rank = 0;
            for (int m2 = 0; m2 < nk; ++m2) {
                const float u = L.lv[d][m2];
                rank += (u > v) | ((u == v) & (m2 < n));
            }
            if (rank < k) {
                L.sv[d][rank] = v;
                L.si[d][rank] = n;
            }
        }
    }
    // candidates: x rank a takes y ranks b < min(k, k / (a + 1))
    {
        int cnt[2], s = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int a = 2 * lane + u;
            cnt[u] = a < k ? min(k, k / (a + 1)) : 0;
            s += cnt[u];
        }
        int incl = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const int ex = incl - s;
        if (2 * lane < k) L.pref[2 * lane] = ex;
        if (2 * lane + 1 < k) L.pref[2 * lane + 1] = ex + cnt[0];
        if (lane == 63) L.pref[k] = incl;
    }
    wave_lds_sync();
    const int ncand = L.pref[k];
    for (int c = lane; c < ncand; c += 64) {
        int lo = 0, hi = k - 1;  // the last a with pref[a] <= c
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (L.pref[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int a = lo, b = c - L.pref[a];
        L.cs[c] = L.sv[0][a] + L.sv[1][b];
        L.ct[c] = a * k + b;
        L.ce[c] = L.si[0][a] * nk + L.si[1][b];
    }
    wave_lds_sync();
    // rank the candidates; the best score is the softmax's offset
    const float top = L.sv[0][0] + L.sv[1][0];
    float mysum = 0.f;
    int myrank[kMaxCand / 64];
    float myscore[kMaxCand / 64];
    for (int u = 0; u < kMaxCand / 64; ++u) {
        const int c = lane + 64 * u;
        myrank[u] = k;
        myscore[u] = 0.f;
        if (c < ncand) {
            const float v = L.cs[c];
            const int tb = L.ct[c];
            int rank = 0;
            for (int c2 = 0; c2 < ncand; ++c2) {
                const float v2 = L.cs[c2];
                rank += (v2 > v) | ((v2 == v) & (L.ct[c2] < tb));
            }
            myrank[u] = rank;
            myscore[u] = v;
            if (rank < k) mysum += __expf(v - top);
        }
    }
    const float denom = wave_sum(mysum);
    for (int u = 0; u < kMaxCand / 64; ++u) {
        const int c = lane + 64 * u;
        if (c < ncand && myrank[u] < k) {
            idx[(size_t)t * k + myrank[u]] = L.ce[c];
            wts[(size_t)t * k + myrank[u]] = __expf(myscore[u] - top) / denom;
        }
    }
}

// ---------------------------------------------------------------- experts
constexpr int kMaxExperts = 128;

__global__ __launch_bounds__(kThreads) void cdmoe_experts_kernel(const uint16_t *__restrict__ h,
                                                                 const uint16_t *__restrict__ down,
                                                                 const uint16_t *__restrict__ up,
                                                                 const int32_t *__restrict__ idx,
                                                                 const float *__restrict__ wts, int H, int k,
                                                                 uint16_t *__restrict__ out) {
    __shared__ float act[kMaxExperts];
    __shared__ int eid[kMaxExperts];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = blockIdx.x;
    const uint16_t *hrow = h + (size_t)t * H;
    if (tid < k) eid[tid] = idx[(size_t)t * k + tid];
    __syncthreads();
    // z_e = down_e . h: wave w takes experts w, w + 4, ...; lanes split H in
    // 16-byte vectors (H is a multiple of 512)
    const int nv = H / 512;
    for (int e = wave; e < k; e += kWaves) {
        const uint16_t *drow = down + (size_t)eid[e] * H;
        float z = 0.f;
        for (int v = 0; v < nv; ++v) {
            const int c = 8 * (lane + 64 * v);
            const bf16x8 dv = ld8(drow + c), hv = ld8(hrow + c);
#pragma unroll
            for (int j = 0; j < 8; ++j) z = fmaf((float)dv[j], (float)hv[j], z);
        }
        z = wave_sum(z);
        if (lane == 0) act[e] = z / (1.f + __expf(-z)) * wts[(size_t)t * k + e];
    }
    __syncthreads();
    // out[c] = sum_e act_e up_e[c]: each thread a run of 4 channels per 1024
    constexpr int kEB = 8;  // expert rows requested together
    for (int c0 = 4 * tid; c0 < H; c0 += 4 * kThreads) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int e0 = 0; e0 < k; e0 += kEB) {
            uint2 u[kEB];
#pragma unroll
            for (int j = 0; j < kEB; ++j)
                u[j] = *reinterpret_cast<const uint2 *>(up + (size_t)eid[min(e0 + j, k - 1)] * H + c0);
#pragma unroll
            for (int j = 0; j < kEB; ++j) {
                if (e0 + j < k) {
                    const float a = act[e0 + j];
                    acc[0] = fmaf(a, __uint_as_float(u[j].x << 16), acc[0]);
                    acc[1] = fmaf(a, __uint_as_float(u[j].x & 0xffff0000u), acc[1]);
                    acc[2] = fmaf(a, __uint_as_float(u[j].y << 16), acc[2]);
                    acc[3] = fmaf(a, __uint_as_float(u[j].y & 0xffff0000u), acc[3]);
                }
            }
        }
        *reinterpret_cast<uint2 *>(out + (size_t)t * H + c0) =
            make_uint2((uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16),
                       (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16));
    }
}

}  // namespace

hipError_t launch_cdmoe_logits(const void *h, const void *router, int T, int H, int nk, float *logits,
                               hipStream_t stream) {
    const int N = 2 * nk;
    const dim3 grid((unsigned)((T + 63) / 64), (unsigned)((N + 16 * kNT - 1) / (16 * kNT)));
    hipLaunchKernelGGL(cdmoe_logits_kernel, grid, dim3(kThreads), 0, stream, (const uint16_t *)h,
                       (const uint16_t *)router, T, H, N, logits);
    return hipGetLastError();
}

hipError_t launch_cdmoe_route(const float *logits, int T, int nk, int k, int32_t *idx, float *wts,
                              hipStream_t stream) {
    hipLaunchKernelGGL(cdmoe_route_kernel, dim3((unsigned)((T + kWaves - 1) / kWaves)), dim3(kThreads), 0, stream,
                       logits, T, nk, k, idx, wts);
    return hipGetLastError();
}

hipError_t launch_cdmoe_experts(const void *h, const void *down, const void *up, const int32_t *idx, const float *wts,
                                int T, int H, int k, void *out, hipStream_t stream) {
    hipLaunchKernelGGL(cdmoe_experts_kernel, dim3((unsigned)T), dim3(kThreads), 0, stream, (const uint16_t *)h,
                       (const uint16_t *)down, (const uint16_t *)up, idx, wts, H, k, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace dma
