// Decode step over a long KV cache under the dynamic top-w mask.
// Doge guide (gitcode), DMA section, forward step 3 (top-w of the per-position
// dt, computed from the cached value states) and step 4 (scaled, dt-biased
// fp32 softmax attention); the query of batch b sits at position L_b - 1.
//
// Three launches on the caller's stream:
//  1. select:  one workgroup per (batch, kv head) finds the w-th best cached
//     position with an exact radix select over the dt cache row (order: dt
//     desc, index asc) and stores the threshold pair; optionally writes the
//     kept positions in ascending order.
//  2. attend:  split over the cache: one workgroup per (batch, kv head, 1024
//     positions) re-reads its dt slice, keeps positions that pass the
//     threshold test, gathers only their K/V rows and produces, for each of
//     the G query heads, a partial (max, sum, unnormalised output) in base 2.
//  3. combine: merges the partials of each (batch, query head).
// HBM traffic is the dt cache plus the K/V rows of the w kept positions per
// kv head, not the whole cache.
#include "common.hpp"
#include "launch.hpp"
#include "radix_select.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kSplit = 1024;  // cache positions per attend workgroup
constexpr int kHeadSlots = kMaxGroupDecode / (kThreads / 64);  // heads per wave, max

inline int nsplit_of(int Lmax) { return (Lmax + kSplit - 1) / kSplit; }

struct WsLayout {
    size_t thr_tau, thr_tie, pm, pl, po, total;
};

inline WsLayout ws_layout(int B, int Lmax, int Hq, int Hkv, int d) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t ns = (size_t)nsplit_of(Lmax);
    WsLayout l;
    l.thr_tau = 0;
    l.thr_tie = up(l.thr_tau + sizeof(float) * B * Hkv);
    l.pm = up(l.thr_tie + sizeof(int32_t) * B * Hkv);
    l.pl = up(l.pm + sizeof(float) * B * Hq * ns);
    l.po = up(l.pl + sizeof(float) * B * Hq * ns);
    l.total = up(l.po + sizeof(float) * B * Hq * ns * d);
    return l;
}

__global__ __launch_bounds__(kThreads) void decode_select_kernel(
    const float *__restrict__ dt_cache, const int32_t *__restrict__ cache_lens, int Hkv, int Lmax,
    int w, float *__restrict__ thr_tau, int32_t *__restrict__ thr_tie, int32_t *__restrict__ kept_idx) {
    __shared__ RadixShared<kThreads> rs;
    __shared__ int wsum[kThreads / 64];
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = cache_lens[b];
    const float *row = dt_cache + ((size_t)b * Hkv + g) * Lmax;
    float t_tau = -INFINITY;
    int t_tie = -1;
    if (L > w) {
        const uint32_t ranks[2] = {(uint32_t)(w - 1), 0u};
        uint64_t keys[2];
        radix_select<kThreads>(row, L, 1, ranks, keys, rs);
        t_tie = (int)selkey_idx(keys[0]);
        t_tau = row[t_tie];
    }
    if (tid == 0) {
        thr_tau[b * Hkv + g] = t_tau;
        thr_tie[b * Hkv + g] = t_tie;
    }
    if (!kept_idx) return;
    // kept positions in ascending order: contiguous ranges per thread,
    // counted, prefix-summed across the workgroup, then written.
    const int per = (L + kThreads - 1) / kThreads;
    const int j0 = min(tid * per, L), j1 = min(j0 + per, L);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += kept_test(row[j], j, t_tau, t_tie) ? 1 : 0;
    const int lane = tid & 63, wave = tid >> 6;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int off = incl - cnt;
    for (int w2 = 0; w2 < wave; ++w2) off += wsum[w2];
    int32_t *out = kept_idx + ((size_t)b * Hkv + g) * w;
    for (int j = j0; j < j1; ++j)
        if (kept_test(row[j], j, t_tau, t_tie)) {
            if (off < w) out[off] = j;  // at most w positions pass the test
            ++off;
        }
    const int total = min(L, w);
    for (int k = total + tid; k < w; k += kThreads) out[k] = -1;
}

template <typename T, int D>
struct DecTile {
    static constexpr int BK = sizeof(T) == 2 ? 64 : 32;  // keys per block (= lanes used)
    static constexpr int P = D + 16 / (int)sizeof(T);    // LDS row pitch (elements)
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_attend_kernel(
    const T *__restrict__ q, const T *__restrict__ Kc, const T *__restrict__ Vc,
    const float *__restrict__ dt_cache, const int32_t *__restrict__ cache_lens, int Lmax, int Hq,
    int Hkv, const float *__restrict__ thr_tau, const int32_t *__restrict__ thr_tie,
    float *__restrict__ pm, float *__restrict__ pl, float *__restrict__ po, float qscale) {
    using C = DecTile<T, D>;
    constexpr int BK = C::BK;
    constexpr int PER = D / 64;  // output columns per lane
    __shared__ int c_idx[kSplit];
    __shared__ float c_dt[kSplit];
    __shared__ float qs[kMaxGroupDecode][D];
    __shared__ __align__(16) T Ks[BK * C::P];
    __shared__ __align__(16) T Vs[BK * C::P];
    __shared__ int wcnt[kThreads / 64];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int G = Hq / Hkv;
    const int nsplit = gridDim.x;
    const int L = cache_lens[b];
    const int s0 = split * kSplit;
    const int s1 = min(s0 + kSplit, L);
    const float t_tau = thr_tau[b * Hkv + g];
    const int t_tie = thr_tie[b * Hkv + g];
    const float *row = dt_cache + ((size_t)b * Hkv + g) * Lmax;

    for (int x = tid; x < G * D; x += kThreads) {
        const int hh = x / D, e = x % D;
        qs[hh][e] = Elem<T>::load(q, ((size_t)b * Hq + g * G + hh) * D + e);
    }
    // candidates of this slice
    int n = 0;
    for (int base = s0; base < s1; base += kThreads) {
        const int j = base + tid;
        bool take = false;
        float dj = 0.f;
        if (j < s1) {
            dj = row[j];
            take = kept_test(dj, j, t_tau, t_tie);
        }
        const uint64_t bal = __ballot(take);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wcnt[wave] = __popcll(bal);
        __syncthreads();
        int off = n, tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kThreads / 64; ++w2) {
            const int c = wcnt[w2];
            off += (w2 < wave) ? c : 0;
            tot += c;
        }
        if (take) {
            c_idx[off + pre] = j;
            c_dt[off + pre] = dj;
        }
        n += tot;
        __syncthreads();
    }

    float mh[kHeadSlots], lh[kHeadSlots], acc[kHeadSlots][PER];
#pragma unroll
    for (int s = 0; s < kHeadSlots; ++s) {
        mh[s] = -INFINITY;
        lh[s] = 0.f;
#pragma unroll
        for (int u = 0; u < PER; ++u) acc[s][u] = 0.f;
    }
    const size_t kvs = (size_t)Hkv * D;
    const T *Kb = Kc + (size_t)b * Lmax * kvs + (size_t)g * D;
    const T *Vb = Vc + (size_t)b * Lmax * kvs + (size_t)g * D;
    constexpr int EV = 16 / (int)sizeof(T);
    for (int blk = 0; blk < n; blk += BK) {
        for (int v = tid; v < BK * D / EV; v += kThreads) {
            const int kk = v / (D / EV), cv = v % (D / EV);
            const int pos = blk + kk;
            uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
            if (pos < n) {
                const size_t off = (size_t)c_idx[pos] * kvs + cv * EV;
                a = *reinterpret_cast<const uint4 *>(Kb + off);
                c = *reinterpret_cast<const uint4 *>(Vb + off);
            }
            *reinterpret_cast<uint4 *>(&Ks[kk * C::P + cv * EV]) = a;
            *reinterpret_cast<uint4 *>(&Vs[kk * C::P + cv * EV]) = c;
        }
        __syncthreads();
        const int kk = lane;  // this lane's key for the scores
        const bool kval = (kk < BK) && (blk + kk < n);
        const float dkk = kval ? c_dt[blk + kk] : 0.f;
#pragma unroll
        for (int s = 0; s < kHeadSlots; ++s) {
            const int hh = wave + (kThreads / 64) * s;
            if (hh >= G) continue;  // wave-uniform
            float sc = 0.f;
            if (kk < BK) {
                for (int e = 0; e < D; ++e) sc = fmaf(qs[hh][e], Elem<T>::load(Ks, (size_t)kk * C::P + e), sc);
            }
            const float z = kval ? fmaf(sc, qscale, dkk * kLog2e) : -INFINITY;
            const float mnew = fmaxf(mh[s], wave_max(z));
            const bool none = (mnew == -INFINITY);
            const float alpha = none ? 1.f : exp2f(mh[s] - mnew);
            const float p = none ? 0.f : exp2f(z - mnew);
            lh[s] = lh[s] * alpha + p;  // per-lane partial, summed at the end
            mh[s] = mnew;
#pragma unroll
            for (int u = 0; u < PER; ++u) acc[s][u] *= alpha;
            for (int k2 = 0; k2 < BK; ++k2) {
                const float pk = __shfl(p, k2, 64);
#pragma unroll
                for (int u = 0; u < PER; ++u)
                    acc[s][u] = fmaf(pk, Elem<T>::load(Vs, (size_t)k2 * C::P + lane + 64 * u), acc[s][u]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < kHeadSlots; ++s) {
        const int hh = wave + (kThreads / 64) * s;
        if (hh >= G) continue;
        const float lt = wave_sum(lh[s]);
        const size_t pidx = ((size_t)b * Hq + g * G + hh) * nsplit + split;
        if (lane == 0) {
            pm[pidx] = mh[s];
            pl[pidx] = lt;
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) po[pidx * D + lane + 64 * u] = acc[s][u];
    }
}

template <typename T>
__global__ void decode_combine_kernel(const float *__restrict__ pm, const float *__restrict__ pl,
                                      const float *__restrict__ po, int nsplit, int d,
                                      T *__restrict__ out) {
    const int bh = blockIdx.x;  // b * Hq + hq
    const float *m = pm + (size_t)bh * nsplit;
    const float *l = pl + (size_t)bh * nsplit;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, m[s]);
    for (int e = threadIdx.x; e < d; e += blockDim.x) {
        float num = 0.f, den = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            if (m[s] == -INFINITY) continue;
            const float f = exp2f(m[s] - M);
            den = fmaf(l[s], f, den);
            num = fmaf(po[((size_t)bh * nsplit + s) * d + e], f, num);
        }
        Elem<T>::store(out, (size_t)bh * d + e, den > 0.f ? num / den : 0.f);
    }
}

template <typename T>
hipError_t launch_decode_t(const T *q, const T *Kc, const T *Vc, const float *dt_cache,
                           const int32_t *cache_lens, int B, int Lmax, int Hq, int Hkv, int d, int w,
                           T *out, int32_t *kept_idx, void *ws, hipStream_t stream) {
    const WsLayout lay = ws_layout(B, Lmax, Hq, Hkv, d);
    char *base = (char *)ws;
    float *thr_tau = (float *)(base + lay.thr_tau);
    int32_t *thr_tie = (int32_t *)(base + lay.thr_tie);
    float *pm = (float *)(base + lay.pm);
    float *pl = (float *)(base + lay.pl);
    float *po = (float *)(base + lay.po);
    const int ns = nsplit_of(Lmax);
    const float qscale = (float)(1.0 / __builtin_sqrt((double)d) * 1.4426950408889634);
    hipLaunchKernelGGL(decode_select_kernel, dim3(Hkv, B), dim3(kThreads), 0, stream, dt_cache,
                       cache_lens, Hkv, Lmax, w, thr_tau, thr_tie, kept_idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d == 128)
        hipLaunchKernelGGL((decode_attend_kernel<T, 128>), dim3(ns, Hkv, B), dim3(kThreads), 0, stream,
                           q, Kc, Vc, dt_cache, cache_lens, Lmax, Hq, Hkv, thr_tau, thr_tie, pm, pl,
                           po, qscale);
    else
        hipLaunchKernelGGL((decode_attend_kernel<T, 64>), dim3(ns, Hkv, B), dim3(kThreads), 0, stream,
                           q, Kc, Vc, dt_cache, cache_lens, Lmax, Hq, Hkv, thr_tau, thr_tie, pm, pl,
                           po, qscale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3(B * Hq), dim3(d), 0, stream, pm, pl, po, ns, d,
                       out);
    return hipGetLastError();
}

}  // namespace

size_t decode_ws_bytes(int B, int Lmax, int Hq, int Hkv, int d, int w) {
    (void)w;
    return ws_layout(B, Lmax, Hq, Hkv, d).total;
}

hipError_t launch_decode(const void *q, const void *Kc, const void *Vc, int dtype,
                         const float *dt_cache, const int32_t *cache_lens, int B, int Lmax,
                         int Hq, int Hkv, int d, int w, void *out, int32_t *kept_idx, void *ws,
                         hipStream_t stream) {
    if (dtype == 1)
        return launch_decode_t<uint16_t>((const uint16_t *)q, (const uint16_t *)Kc,
                                         (const uint16_t *)Vc, dt_cache, cache_lens, B, Lmax, Hq, Hkv,
                                         d, w, (uint16_t *)out, kept_idx, ws, stream);
    return launch_decode_t<float>((const float *)q, (const float *)Kc, (const float *)Vc, dt_cache,
                                  cache_lens, B, Lmax, Hq, Hkv, d, w, (float *)out, kept_idx, ws,
                                  stream);
}

}  // namespace dma
