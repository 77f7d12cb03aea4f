// Sliding-window variant of the dynamic mask.
// Doge guide (gitcode), DogeConfig table: with sliding_window set, the
// attention mask is the sliding-window causal mask, so row i sees the keys
// i - win < j <= i (and j < L); DMA forward step 3 then keeps the top
// keep_window_size (= w) of them by dt, masked keys (min_dtype) never
// outranking valid ones.  The kept sets no longer nest from row to row (keys
// leave the window).  Windows of at least 64 are selected by the chunked band
// selector (select_kernel with a window); shorter ones here:
//
// select_window_kernel: one wave per row.  The w-th key of the row's window
// under (dt desc, index asc) by a range-adapted radix select on the
// order-preserving dt keys: the min and max of the window's keys, then a
// 256-bin histogram (LDS) of the keys in the current range and the bin that
// holds the wanted rank, until the range is one value; the tie among keys of
// that value goes to the lower index, found by a ballot scan in index order.
// Exact: comparisons and integer arithmetic only.
//
// attn_window_kernel: one workgroup per (batch, kv head, tile of 128 / G
// rows), eight waves of 16 (row, head) pairs in lane columns.  The candidate keys of the
// tile's window range [i0 - win + 1, last row] (those at or above the
// smallest threshold of its rows; no other key is kept by any of them) are
// compacted into an LDS list, and blocks of 64 candidates are gathered into
// LDS, every (pair, key) tested (j in the row's window, selkey(dt_j, j) >= selkey(tau_i, tie_i)),
// S^T = K Q^T and O^T += V^T P^T on 16x16x32 bf16 MFMA with an online softmax
// in base 2 (the running max shared by the four lanes of a pair; P rounded
// once to bf16 and the softmax sum taken over the same rounded weights).
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 256;
// window attention: eight waves of 16 (row, head) pairs, 128 pairs a tile
// (the K/V tiles in LDS serve twice the pairs of four waves: 0.34 -> 0.24 ms
// on the long workload with a 4096-key window)
constexpr int kAttnThreads = 512;
constexpr int kPairs = kAttnThreads / 4;
constexpr int kBlk = 64;
constexpr int kWinCap = 4224;            // candidate keys of a query tile held in LDS
constexpr int kScanKeys = 4 * kAttnThreads;  // keys the attention classifies per scan step

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o, 64));
    return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, 64));
    return x;
}

__global__ __launch_bounds__(kThreads) void select_window_kernel(const float *__restrict__ dt,
                                                                 const int32_t *__restrict__ seqlens, int Hkv, int S,
                                                                 int w, int win, int64_t nrows,
                                                                 float *__restrict__ tau, int32_t *__restrict__ tie) {
    __shared__ uint32_t hist[kWaves][kBins];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * kWaves + wave;
    if (r >= nrows) return;  // uniform per wave; no block barrier below
    const int i = (int)(r % S);
    const int64_t bg = r / S;
    const int b = (int)(bg / Hkv);
    const int L = clamp_len(seqlens, b, S);
    if (i >= L) {
        if (lane == 0) {
            tau[r] = INFINITY;
            tie[r] = -1;
        }
        return;
    }
    const int lo = max(0, i - win + 1);
    const int n = i - lo + 1;
    if (n <= w) {
        if (lane == 0) {
            tau[r] = -INFINITY;
            tie[r] = -1;
        }
        return;
    }
    const float *drow = dt + bg * S;
    uint32_t *h = hist[wave];

    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int j = lo + lane; j <= i; j += 64) {
        const uint32_t k = ordkey(drow[j]);
        mn = min(mn, k);
        mx = max(mx, k);
    }
    uint32_t rlo = wave_min_u32(mn), rhi = wave_max_u32(mx);
    int need = w;  // rank, from the top, of the wanted key among the keys in [rlo, rhi]
    while (rlo < rhi) {
        const uint64_t span = (uint64_t)(rhi - rlo) + 1;
#pragma unroll
        for (int k = 0; k < kBins / 64; ++k) h[lane + 64 * k] = 0u;
        wave_lds_sync();
        for (int j = lo + lane; j <= i; j += 64) {
            const uint32_t k = ordkey(drow[j]);
            if (k >= rlo && k <= rhi) atomicAdd(&h[(uint32_t)(((uint64_t)(k - rlo) * kBins) / span)], 1u);
        }
        wave_lds_sync();
        // lane l holds bins 4l .. 4l+3; keys in bins above lane l's
        uint32_t c[4], s = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c[k] = h[4 * lane + k];
            s += c[k];
        }
        uint32_t above = 0;  // exclusive suffix sum over higher lanes
        {
            uint32_t incl = s;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = (uint32_t)__shfl_down((int)incl, o, 64);
                if (lane + o < 64) incl += y;
            }
            above = incl - s;
        }
        const bool mine = above < (uint32_t)need && (uint32_t)need <= above + s;
        const uint64_t sel = __ballot(mine);
        const int owner = __ffsll((unsigned long long)sel) - 1;
        int bin = 0;
        uint32_t before = 0;
        if (mine) {
            uint32_t acc = above;
            for (int k = 3; k >= 0; --k) {
                if ((uint32_t)need <= acc + c[k]) {
                    bin = 4 * lane + k;
                    before = acc;
                    break;
                }
                acc += c[k];
            }
        }
        bin = __shfl(bin, owner, 64);
        before = (uint32_t)__shfl((int)before, owner, 64);
        need -= (int)before;
        // ordkeys of bin b: k - rlo in [ceil(b span / 256), ceil((b + 1) span / 256) - 1]
        const uint64_t a0 = ((uint64_t)bin * span + kBins - 1) / kBins;
        const uint64_t a1 = ((uint64_t)(bin + 1) * span + kBins - 1) / kBins - 1;
        rhi = rlo + (uint32_t)a1;
        rlo = rlo + (uint32_t)a0;
    }
    // the need-th key (lowest index first) among those of order key rlo
    int cum = 0, found = -1;
    for (int j0 = lo; j0 <= i && found < 0; j0 += 64) {
        const int j = j0 + lane;
        const bool eq = j <= i && ordkey(drow[min(j, i)]) == rlo;
        const uint64_t m = __ballot(eq);
        const int cnt = __popcll(m);
        if (cum + cnt >= need) {
            const int rank = cum + __popcll(m & ((1ull << lane) - 1)) + 1;
            const uint64_t hit = __ballot(eq && rank == need);
            found = j0 + __ffsll((unsigned long long)hit) - 1;
        }
        cum += cnt;
    }
    if (lane == 0) {
        tau[r] = drow[found];
        tie[r] = found;
    }
}

// ------------------------------------------------------------- attention
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4 lds_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// A operand over rows base .. base+31 of an LDS tile (pitch P), column
// c0 + l%16, k-slot (q, j) -> row base + 16 (j / 4) + 4q + j % 4; the B operand
// in the same order is the pair of accumulator tiles (lo, hi) a lane holds.
template <int P>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *T, int base, int c0, int lane) {
    const int q = lane >> 4, k = lane & 15;
    const uint16_t *p = T + (base + 4 * q + (k >> 2)) * P + c0 + 4 * (k & 3);
    const i16x4 lo = lds_tr16(p);
    const i16x4 hi = lds_tr16(p + 16 * P);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_window_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, int S, int Hq, int Hkv, int G, int ntq, int win, float qscale,
    uint16_t *__restrict__ O) {
    constexpr int P = D + 32;
    constexpr int NS = D / 32;
    constexpr int NV = kBlk * D / 8 / kAttnThreads;
    __shared__ __align__(16) uint16_t Ks[kBlk * P];
    __shared__ __align__(16) uint16_t Vs[kBlk * P];
    __shared__ float dtl_s[kBlk];
    __shared__ uint64_t skey_s[kBlk];
    __shared__ int jk_s[kBlk];
    __shared__ int c_idx[kWinCap];
    __shared__ uint32_t wcnt[kAttnThreads / 64];
    __shared__ uint64_t tmin[kAttnThreads / 64];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, pq = lane & 15;
    // tiles of one (batch, kv head) on one XCD (shared K/V in its L2)
    const int nwg = gridDim.x, per_xcd = nwg >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int item = (slot < per_xcd && (nwg & 7) == 0) ? xcd * per_xcd + slot : blockIdx.x;
    const int tq = item % ntq;
    const int g = (item / ntq) % Hkv;
    const int b = item / (ntq * Hkv);
    const int L = clamp_len(seqlens, b, S);
    const int RB = kPairs / G;
    const int i0 = tq * RB;
    const int pr = 16 * wave + pq;
    const int i = i0 + pr / G, hq = g * G + pr % G;
    const bool live = i < L;
    const size_t orow = (((size_t)b * S + min(i, S - 1)) * Hq + hq) * D;
    if (i0 >= L) {
        if (i < S) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) *reinterpret_cast<uint2 *>(O + orow + 16 * t + 4 * q) = make_uint2(0, 0);
        }
        return;
    }
    const size_t urow = ((size_t)b * Hkv + g) * S;
    const int kmax = min(i0 + RB, L) - 1;
    const int kmin = max(0, i0 - win + 1);
    const int lo_i = max(0, i - win + 1);
    const uint64_t thr = live ? selkey(tau[urow + i], (uint32_t)tie[urow + i]) : ~0ull;
    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = ld8(Q + orow + 32 * s + 8 * q);

    const uint32_t kvs = (uint32_t)(Hkv * D);
    const uint16_t *Kb = K + (size_t)b * S * kvs + (size_t)g * D;
    const uint16_t *Vb = V + (size_t)b * S * kvs + (size_t)g * D;
    const float *drow = dt + urow;

    // ---- candidate keys: a key of the tile's window range that no row of
    // the tile keeps lies below every row's threshold, so only the keys at or
    // above the smallest threshold of the tile's valid rows are walked
    // (about w / win of the range), compacted into LDS in index order within
    // each scan step's wave and register; past kWinCap candidates the whole
    // range is walked instead
    int n;
    {
        uint64_t tm = ~0ull;
        for (int r = tid; r < kmax - i0 + 1; r += kAttnThreads) {
            const uint64_t t = selkey(tau[urow + i0 + r], (uint32_t)tie[urow + i0 + r]);
            tm = t < tm ? t : tm;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const uint64_t y = __shfl_xor(tm, o, 64);
            tm = y < tm ? y : tm;
        }
        if (lane == 0) tmin[wave] = tm;
        __syncthreads();
        tm = tmin[0];
#pragma unroll
        for (int w2 = 1; w2 < kAttnThreads / 64; ++w2) tm = tmin[w2] < tm ? tmin[w2] : tm;
        const uint64_t lt_mask = (1ull << lane) - 1ull;
        int base = 0;
        for (int c0 = kmin; c0 <= kmax; c0 += kScanKeys) {
            float dv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) dv[e] = drow[min(c0 + tid + kAttnThreads * e, kmax)];
            bool pr[4];
            uint32_t nw = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = c0 + tid + kAttnThreads * e;
                pr[e] = j <= kmax && selkey(dv[e], (uint32_t)j) >= tm;
                nw += (uint32_t)__popcll(__ballot(pr[e]));
            }
            if (lane == 0) wcnt[wave] = nw;
            __syncthreads();
            int off = base, tot = 0;
#pragma unroll
            for (int w2 = 0; w2 < kAttnThreads / 64; ++w2) {
                const int cw = (int)wcnt[w2];
                off += w2 < wave ? cw : 0;
                tot += cw;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint64_t bl = __ballot(pr[e]);
                const int pos = off + (int)__popcll(bl & lt_mask);
                if (pr[e] && pos < kWinCap) c_idx[pos] = c0 + tid + kAttnThreads * e;
                off += (int)__popcll(bl);
            }
            base += tot;
            __syncthreads();  // wcnt is rewritten by the next step
        }
        n = base;
    }
    const bool gathered = n <= kWinCap;
    if (!gathered) n = kmax - kmin + 1;
    // key at list position x (x < n)
    auto key_at = [&](int x) __attribute__((always_inline)) { return gathered ? c_idx[x] : kmin + x; };

    // A key block's K and V rows and dt are requested into registers one
    // block ahead and written to LDS after the barrier that ends the block
    // before.  Positions past the list's end repeat its last key and are
    // marked never kept.
    u32x4 rk[NV], rv[NV];
    float rdt;
    int rj;
    auto fetch = [&](int x0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = tid + u * kAttnThreads;
            const size_t off = (size_t)(uint32_t)key_at(min(x0 + v / (D / 8), n - 1)) * kvs + 8 * (v % (D / 8));
            rk[u] = *reinterpret_cast<const u32x4 *>(Kb + off);
            rv[u] = *reinterpret_cast<const u32x4 *>(Vb + off);
        }
        rj = key_at(min(x0 + (tid & (kBlk - 1)), n - 1));
        rdt = drow[rj];
    };
    auto put = [&](int x0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = tid + u * kAttnThreads;
            const int kk = v / (D / 8), cv = v % (D / 8);
            *reinterpret_cast<u32x4 *>(&Ks[kk * P + 8 * cv]) = rk[u];
            *reinterpret_cast<u32x4 *>(&Vs[kk * P + 8 * cv]) = rv[u];
        }
        if (tid < kBlk) {
            dtl_s[tid] = rdt * kLog2e;
            skey_s[tid] = selkey(rdt, (uint32_t)rj);
            jk_s[tid] = x0 + tid < n ? rj : 0x7fffffff;
        }
    };

    float m = -INFINITY, l = 0.f;
    f32x4 oacc[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    if (n > 0) fetch(0);
    for (int x0 = 0; x0 < n; x0 += kBlk) {
        put(x0);
        __syncthreads();
        if (x0 + kBlk < n) fetch(x0 + kBlk);
        float z[4][4];
        float mb = -INFINITY;
        // wave priority 3 while forming scores, 1 for the weighted sum of V,
        // 0 in the softmax (the waves of a SIMD then interleave their phases)
        __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) sacc = mfma16(ld8(&Ks[(16 * mt + pq) * P + 32 * s + 8 * q]), qf[s], sacc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kk = 16 * mt + 4 * q + r, j = jk_s[kk];
                const bool kept = live & (j >= lo_i) & (j <= i) & (skey_s[kk] >= thr);
                const float zz = fmaf(sacc[r], qscale, dtl_s[kk]);
                z[mt][r] = kept ? zz : -INFINITY;
                mb = fmaxf(mb, z[mt][r]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // the running max is shared by the four lanes of a pair, so that
        // every weight of the pair's row has the same scale
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        if (mb > m) {
            const float a = __builtin_amdgcn_exp2f(m - mb);  // 0 when m = -inf
            l *= a;
#pragma unroll
            for (int t = 0; t < D / 16; ++t) oacc[t] *= a;
            m = mb;
        }
        const float msub = m == -INFINITY ? 0.f : m;
        f32x4 pm[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) pm[mt][r] = __builtin_amdgcn_exp2f(z[mt][r] - msub);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pb[e] = (__bf16)pm[2 * s2][e];
                pb[4 + e] = (__bf16)pm[2 * s2 + 1][e];
            }
            // the softmax sum over the same rounded weights that multiply V
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one2, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one2, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one2, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one2, l, false);
#pragma unroll
            for (int t = 0; t < D / 16; ++t) oacc[t] = mfma16(tr_operand<P>(Vs, 32 * s2, 16 * t, lane), pb, oacc[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = (live && l > 0.f) ? 1.f / l : 0.f;
    if (i < S) {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const uint32_t w0 = (uint32_t)f32_to_bf16(oacc[t][0] * inv) | ((uint32_t)f32_to_bf16(oacc[t][1] * inv) << 16);
            const uint32_t w1 = (uint32_t)f32_to_bf16(oacc[t][2] * inv) | ((uint32_t)f32_to_bf16(oacc[t][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(O + orow + 16 * t + 4 * q) = make_uint2(w0, w1);
        }
    }
}

}  // namespace

hipError_t launch_select_window(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, int win,
                                float *tau, int32_t *tie, hipStream_t stream) {
    // windows of at least one selector chunk: the chunked band selector
    if (win >= 64)
        return launch_select(dt, seqlens, B, Hkv, S, w, win, tau, tie, stream);
    const int64_t nrows = (int64_t)B * Hkv * S;
    const unsigned grid = (unsigned)((nrows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(select_window_kernel, dim3(grid), dim3(kThreads), 0, stream, dt, seqlens, Hkv, S, w, win,
                       nrows, tau, tie);
    return hipGetLastError();
}

hipError_t launch_attn_window(const void *Q, const void *K, const void *V, const float *dt, const float *tau,
                              const int32_t *tie, const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                              int win, void *O, hipStream_t stream) {
    const int G = Hq / Hkv;
    const int RB = kPairs / G;
    const int ntq = (S + RB - 1) / RB;
    const unsigned grid = (unsigned)(B * Hkv * ntq);
    const float qscale = (1.0f / sqrtf((float)d)) * kLog2e;
    if (d == 128)
        hipLaunchKernelGGL((attn_window_kernel<128>), dim3(grid), dim3(kAttnThreads), 0, stream, (const uint16_t *)Q,
                           (const uint16_t *)K, (const uint16_t *)V, dt, tau, tie, seqlens, S, Hq, Hkv, G, ntq, win,
                           qscale, (uint16_t *)O);
    else
        hipLaunchKernelGGL((attn_window_kernel<64>), dim3(grid), dim3(kAttnThreads), 0, stream, (const uint16_t *)Q,
                           (const uint16_t *)K, (const uint16_t *)V, dt, tau, tie, seqlens, S, Hq, Hkv, G, ntq, win,
                           qscale, (uint16_t *)O);
    return hipGetLastError();
}

}  // namespace dma
