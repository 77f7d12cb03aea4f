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
// instead of k^2.  For k <= 64 the k-th best of them is found one bit of its
// 64-bit key at a time and the k winners are sorted across the lanes; larger
// k ranks every candidate against every other.  The softmax of the k best
// scores gives the weights.  Pair scores are float32 sums of the two logits.
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
// candidates for k <= 64 (sum over a < k of floor(k / (a + 1)) is at most
// 303) and for k <= 128 (695); SMALL kernels hold the smaller LDS layout, so
// that more of them are resident
constexpr int kMaxCandSmall = 320;
constexpr int kMaxCandLarge = 768;

template <int MAXC, int MAXK>
struct RouteLds {
    __align__(16) float cs[MAXC];        // candidate scores
    __align__(16) int ct[MAXC];          // candidate tie order a * k + b
    __align__(16) int ce[MAXC];          // candidate expert index
    __align__(16) float lv[2][kMaxNk];   // logits of the two domains
    __align__(16) float sv[2][MAXK];     // top-k values in rank order
    __align__(16) int si[2][MAXK];       // and their indices
    __align__(16) int pref[MAXK + 4];    // first candidate of each x rank
};

template <bool SMALL>
__global__ __launch_bounds__(kThreads) void cdmoe_route_kernel(const float *__restrict__ logits, int T, int nk, int k,
                                                               int32_t *__restrict__ idx, float *__restrict__ wts) {
    constexpr int kMaxCand = SMALL ? kMaxCandSmall : kMaxCandLarge;
    using Lds = RouteLds<kMaxCand, SMALL ? 64 : kMaxK>;
    __shared__ Lds lds[kWaves];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * kWaves + wave;
    if (t >= T) return;  // uniform per wave; no block barrier below
    Lds &L = lds[wave];
    const float *lrow = logits + (size_t)t * 2 * nk;
    const int nk4 = (nk + 3) & ~3;  // domains padded to 4 with -inf (never better)
    for (int n = lane; n < 2 * nk4; n += 64) {
        const int d = n >= nk4, m2 = n - d * nk4;
        L.lv[d][m2] = m2 < nk ? lrow[d * nk + m2] : -INFINITY;
    }
    wave_lds_sync();
    // rank of each key in its domain (4 keys per LDS read); the k best go to
    // (sv, si) in rank order
    for (int d = 0; d < 2; ++d) {
        for (int n = lane; n < nk; n += 64) {
            const float v = L.lv[d][n];
            int rank = 0;
#pragma unroll 8
            for (int m2 = 0; m2 < nk4; m2 += 4) {
                const float4 u = *reinterpret_cast<const float4 *>(&L.lv[d][m2]);
                rank += (u.x > v) | ((u.x == v) & (m2 < n));
                rank += (u.y > v) | ((u.y == v) & (m2 + 1 < n));
                rank += (u.z > v) | ((u.z == v) & (m2 + 2 < n));
                rank += (u.w > v) | ((u.w == v) & (m2 + 3 < n));
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
    const int ncand4 = (ncand + 3) & ~3;  // padded with candidates that lose to all
    for (int c = ncand + lane; c < ncand4; c += 64) {
        L.cs[c] = -INFINITY;
        L.ct[c] = 0x7fffffff;
    }
    {
        // x rank a pairs with y ranks b < k / (a + 1): lane b writes (a, b)
        const int b = lane;
        const float yv = b < k ? L.sv[1][b] : 0.f;
        const int yi = b < k ? L.si[1][b] : 0;
        for (int a = 0; a < k; ++a) {
            if (b < min(k, k / (a + 1))) {
                const int c = L.pref[a] + b;
                L.cs[c] = L.sv[0][a] + yv;
                L.ct[c] = a * k + b;
                L.ce[c] = L.si[0][a] * nk + yi;
            }
        }
        // y ranks 64 .. k-1 (k > 64) pair only with x rank 0
        for (int b2 = 64 + lane; b2 < k; b2 += 64) {
            L.cs[b2] = L.sv[0][0] + L.sv[1][b2];
            L.ct[b2] = b2;
            L.ce[b2] = L.si[0][0] * nk + L.si[1][b2];
        }
    }
    wave_lds_sync();
    // the best score is the softmax's offset
    const float top = L.sv[0][0] + L.sv[1][0];
    if constexpr (SMALL) {
        // A candidate's 44-bit selection key: its score's order bits, then the
        // lower tie order first; keys are unique.  The k-th largest key by one
        // bit at a time (a count over all candidates per bit), the k winners
        // compacted one per lane, then sorted across the lanes.
        constexpr int NC = 5;  // for k <= 64 there are at most 303 candidates
        uint64_t key[NC];
        int cid[NC];
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int c = lane + 64 * u;
            cid[u] = c;
            // tie orders a * k + b are below 64 * 64 = 2^12
            key[u] = c < ncand ? ((uint64_t)ordkey(L.cs[c]) << 12) | (uint64_t)(4095u - (uint32_t)L.ct[c]) : 0ull;
        }
        // the wave's count of keys >= probe: each lane counts at most NC < 8,
        // summed over the lanes bit by bit with ballots (no lane shuffles)
        uint64_t thr = 0;
        for (int bit = 43; bit >= 0; --bit) {
            const uint64_t probe = thr | (1ull << bit);
            int c1 = 0;
#pragma unroll
            for (int u = 0; u < NC; ++u) c1 += key[u] >= probe;
            const int cnt = __popcll(__ballot(c1 & 1)) + 2 * __popcll(__ballot(c1 & 2)) +
                            4 * __popcll(__ballot(c1 & 4));
            if (cnt >= k) thr = probe;
        }
        // winners (exactly k keys are >= thr) to LDS, one slot each
        uint64_t *wk = reinterpret_cast<uint64_t *>(&L.lv[0][0]);  // the logits are no longer needed
        int *we = reinterpret_cast<int *>(&L.lv[1][0]);
        int base = 0;
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const bool win = key[u] >= thr && key[u] != 0ull;
            const uint64_t m = __ballot(win);
            if (win) {
                const int pos = base + __popcll(m & ((1ull << lane) - 1));
                wk[pos] = key[u];
                we[pos] = L.ce[cid[u]];
            }
            base += __popcll(m);
        }
        wave_lds_sync();
        uint64_t kk = lane < k ? wk[lane] : 0ull;
        int ee = lane < k ? we[lane] : 0;
        // bitonic sort across the 64 lanes, largest key first
        for (int size = 2; size <= 64; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const uint32_t lo32 = (uint32_t)__shfl_xor((int)(uint32_t)kk, stride, 64);
                const uint32_t hi32 = (uint32_t)__shfl_xor((int)(uint32_t)(kk >> 32), stride, 64);
                const uint64_t pk = ((uint64_t)hi32 << 32) | lo32;
                const int pe = __shfl_xor(ee, stride, 64);
                const bool up = (lane & size) == 0, lower = (lane & stride) == 0;
                const bool take_max = up == lower;
                const bool mine = take_max ? kk >= pk : kk <= pk;
                if (!mine) {
                    kk = pk;
                    ee = pe;
                }
            }
        }
        // the winner's score from its order bits (ordkey is invertible up to
        // the sign of zero)
        const uint32_t ob = (uint32_t)(kk >> 12);
        const float sc = __uint_as_float((ob & 0x80000000u) ? (ob & 0x7fffffffu) : ~ob);
        const float e = lane < k ? __expf(sc - top) : 0.f;
        const float den = wave_sum(e);
        if (lane < k) {
            idx[(size_t)t * k + lane] = ee;
            wts[(size_t)t * k + lane] = e / den;
        }
        return;
    } else {
    // k > 64: every candidate ranked against every other
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
#pragma unroll 8
            for (int c2 = 0; c2 < ncand4; c2 += 4) {
                const float4 v2 = *reinterpret_cast<const float4 *>(&L.cs[c2]);
                const int4 t2 = *reinterpret_cast<const int4 *>(&L.ct[c2]);
                rank += (v2.x > v) | ((v2.x == v) & (t2.x < tb));
                rank += (v2.y > v) | ((v2.y == v) & (t2.y < tb));
                rank += (v2.z > v) | ((v2.z == v) & (t2.z < tb));
                rank += (v2.w > v) | ((v2.w == v) & (t2.w < tb));
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
}

// ---------------------------------------------------------------- experts
constexpr int kMaxExperts = 128;

__global__ __launch_bounds__(kThreads) void cdmoe_experts_kernel(const uint16_t *__restrict__ h,
                                                                 const uint16_t *__restrict__ down,
                                                                 const uint16_t *__restrict__ up,
                                                                 const int32_t *__restrict__ idx,
                                                                 const float *__restrict__ wts, int H, int k,
                                                                 int E, uint16_t *__restrict__ out) {
    __shared__ float act[kMaxExperts];
    __shared__ int eid[kMaxExperts];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = blockIdx.x;
    const uint16_t *hrow = h + (size_t)t * H;
    // an index outside [0, E) is outside the contract; it reads row 0 and
    // gets weight zero rather than a row past the tables
    if (tid < k) {
        const int v = idx[(size_t)t * k + tid];
        eid[tid] = (unsigned)v < (unsigned)E ? v : -1;
    }
    __syncthreads();
    // z_e = down_e . h: wave w takes experts w, w + 4, ...; lanes split H in
    // 16-byte vectors (H is a multiple of 512)
    const int nv = H / 512;
    for (int e = wave; e < k; e += kWaves) {
        const int ee = eid[e];
        const uint16_t *drow = down + (size_t)max(ee, 0) * H;
        float z = 0.f;
        for (int v = 0; v < nv; ++v) {
            const int c = 8 * (lane + 64 * v);
            const bf16x8 dv = ld8(drow + c), hv = ld8(hrow + c);
#pragma unroll
            for (int j = 0; j < 8; ++j) z = fmaf((float)dv[j], (float)hv[j], z);
        }
        z = wave_sum(z);
        if (lane == 0) act[e] = ee < 0 ? 0.f : z / (1.f + __expf(-z)) * wts[(size_t)t * k + e];
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
                u[j] = *reinterpret_cast<const uint2 *>(up + (size_t)max(eid[min(e0 + j, k - 1)], 0) * H + c0);
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
    const dim3 grid((unsigned)((T + kWaves - 1) / kWaves));
    if (k <= 64)
        hipLaunchKernelGGL(cdmoe_route_kernel<true>, grid, dim3(kThreads), 0, stream, logits, T, nk, k, idx, wts);
    else
        hipLaunchKernelGGL(cdmoe_route_kernel<false>, grid, dim3(kThreads), 0, stream, logits, T, nk, k, idx, wts);
    return hipGetLastError();
}

hipError_t launch_cdmoe_experts(const void *h, const void *down, const void *up, const int32_t *idx, const float *wts,
                                int T, int H, int nk, int k, void *out, hipStream_t stream) {
    hipLaunchKernelGGL(cdmoe_experts_kernel, dim3((unsigned)T), dim3(kThreads), 0, stream, (const uint16_t *)h,
                       (const uint16_t *)down, (const uint16_t *)up, idx, wts, H, k, nk * nk, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace dma
