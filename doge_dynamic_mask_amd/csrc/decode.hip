// Decode step over a long KV cache under the dynamic top-w mask.
// Doge guide (gitcode), DMA section, forward step 3 (top-w of the per-position
// dt, computed from the cached value states) and step 4 (scaled, dt-biased
// fp32 softmax attention); the query of batch b sits at position L_b - 1.
//
// Three launches on the caller's stream:
//  1. select: one workgroup per (batch, kv head) finds the w-th best cached
//     position exactly (order: dt desc, index asc) and stores the threshold
//     pair; optionally writes the kept positions in ascending order.  Rows of
//     up to 32768 positions are held in registers (1024 threads) and resolved
//     with one range-adapted 4096-bin histogram plus an exact rank of the few
//     keys in the threshold bin; longer rows use the multi-pass radix select.
//  2. attend: split over the cache: one workgroup per (batch, kv head, 1024
//     positions) re-reads its dt slice, keeps the positions that pass the
//     threshold test and gathers only their K/V rows, 64 at a time, into LDS
//     with coalesced 16-byte loads (the next block's loads are issued before
//     the current block's math).  Scores use 4 lanes per key; the weighted V
//     sum uses lanes over head_dim.  It writes a partial (max, sum, output)
//     per query head.
//  3. combine: merges the partials of each (batch, kv head) into the output.
//     (A separate launch: merging inside the last attend workgroup would need
//     device-scope fences, which on a multi-XCD part write back and
//     invalidate L2 in every workgroup.)
// HBM traffic is the dt cache plus the K/V rows of the w kept positions per
// kv head, not the whole cache.
#include "common.hpp"
#include "launch.hpp"
#include "radix_select.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kSplit = 1024;       // cache positions per attend workgroup
constexpr int kSelThreads = 1024;  // select workgroup (register-resident rows)
constexpr int kBins = 4096;
constexpr int kCandCap = 1024;

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

// ---------------------------------------------------------------- select --

struct SelShared {
    uint32_t hist[kBins];
    uint64_t cand[kCandCap];
    uint32_t red[kSelThreads / 64];
    uint32_t red2[kSelThreads / 64];
    uint32_t ncand;
    uint32_t bin, above, cnt;
    uint64_t result;
};

// Exclusive prefix count of `flag` over threads (thread order), and the total.
__device__ __forceinline__ uint32_t block_excl_count(bool flag, uint32_t &total, SelShared &sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const uint32_t pre = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) sh.red2[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kSelThreads / 64; ++k) {
        const uint32_t c = sh.red2[k];
        off += (k < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return off + pre;
}

// Histogram of bin(key) for the keys with filter(key) true, then the bin that
// holds descending rank rr; sets sh.bin / sh.above / sh.cnt.
template <int ITEMS, typename BinF, typename FiltF>
__device__ void hist_find(const uint32_t *k, int L, uint32_t rr, BinF binf, FiltF filt, SelShared &sh) {
    const int tid = threadIdx.x;
    for (int x = tid; x < kBins; x += kSelThreads) sh.hist[x] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int j = it * kSelThreads + tid;
        if (j < L && filt(k[it])) atomicAdd(&sh.hist[binf(k[it])], 1u);
    }
    __syncthreads();
    // bins in descending order, 4 per thread
    constexpr int PER = kBins / kSelThreads;
    uint32_t c[PER], s = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        c[q] = sh.hist[kBins - 1 - (PER * tid + q)];
        s += c[q];
    }
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) sh.red[wave] = incl;
    __syncthreads();
    uint32_t woff = 0;
    for (int q = 0; q < wave; ++q) woff += sh.red[q];
    const uint32_t excl = woff + incl - s;
    if (excl <= rr && rr < excl + s) {
        uint32_t run = excl;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (rr < run + c[q]) {
                sh.bin = (uint32_t)(kBins - 1 - (PER * tid + q));
                sh.above = run;
                sh.cnt = c[q];
                break;
            }
            run += c[q];
        }
    }
    __syncthreads();
}

template <int ITEMS>
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(
    const float *__restrict__ dt_cache, const int32_t *__restrict__ cache_lens, int Hkv, int Lmax,
    int w, float *__restrict__ thr_tau, int32_t *__restrict__ thr_tie, int32_t *__restrict__ kept_idx) {
    __shared__ SelShared sh;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = cache_lens[b];
    const float *row = dt_cache + ((size_t)b * Hkv + g) * Lmax;

    uint32_t k[ITEMS];
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int j = it * kSelThreads + tid;
        k[it] = j < L ? ordkey(row[j]) : 0u;
        if (j < L) {
            kmin = min(kmin, k[it]);
            kmax = max(kmax, k[it]);
        }
    }
    uint64_t result = 0;  // (ordkey << 32) | ~index of the w-th kept position
    float t_tau = -INFINITY;
    int t_tie = -1;
    if (L > w) {
        // block min / max of the keys
        const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor(kmin, o, 64));
            kmax = max(kmax, (uint32_t)__shfl_xor(kmax, o, 64));
        }
        if (lane == 0) {
            sh.red[wave] = kmin;
            sh.red2[wave] = kmax;
        }
        __syncthreads();
        kmin = 0xffffffffu;
        kmax = 0u;
        for (int q = 0; q < kSelThreads / 64; ++q) {
            kmin = min(kmin, sh.red[q]);
            kmax = max(kmax, sh.red2[q]);
        }
        __syncthreads();

        // Range-adapted digits: the current bin is [base, base + 2^bw); each
        // level splits it into <= 4096 sub-bins of width 2^shift and keeps the
        // one holding rank rr, until it holds <= kCandCap keys or one value.
        const uint32_t range = kmax - kmin;
        int bw = range == 0u ? 0 : 32 - __clz(range);
        uint32_t base = kmin;
        uint32_t rr = (uint32_t)(w - 1);
        uint32_t cnt;
        for (;;) {
            const int shift = bw > 12 ? bw - 12 : 0;
            const uint32_t b0 = base;
            const int bw0 = bw;
            hist_find<ITEMS>(
                k, L, rr, [=](uint32_t x) { return (x - b0) >> shift; },
                [=](uint32_t x) { return x >= b0 && (bw0 >= 32 || ((x - b0) >> bw0) == 0u); }, sh);
            rr -= sh.above;
            cnt = sh.cnt;
            base = b0 + (sh.bin << shift);
            bw = shift;
            if (cnt <= (uint32_t)kCandCap || bw == 0) break;
        }
        // keys of the chosen bin: [base, base + 2^bw)
        const int s = bw;
        const uint32_t bsel = base;
        auto in_bin = [=](uint32_t x) { return x >= bsel && ((x - bsel) >> s) == 0u; };
        if (cnt <= (uint32_t)kCandCap) {
            if (tid == 0) sh.ncand = 0;
            __syncthreads();
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) {
                const int j = it * kSelThreads + tid;
                if (j < L && in_bin(k[it])) {
                    const uint32_t at = atomicAdd(&sh.ncand, 1u);
                    sh.cand[at] = ((uint64_t)k[it] << 32) | (uint64_t)(~(uint32_t)j);
                }
            }
            __syncthreads();
            if (tid < (int)cnt) {
                const uint64_t me = sh.cand[tid];
                uint32_t rank = 0;
                for (uint32_t u = 0; u < cnt; ++u) rank += sh.cand[u] > me ? 1u : 0u;
                if (rank == rr) sh.result = me;
            }
            __syncthreads();
            result = sh.result;
        } else {
            // a single key value shared by more than kCandCap positions: the
            // rr-th of them in index order.  Index order is item-major here.
            const uint32_t kv = bsel;
            uint32_t seen = 0;
            for (int it = 0; it < ITEMS; ++it) {
                const int j = it * kSelThreads + tid;
                const bool m = j < L && k[it] == kv;
                uint32_t tot;
                const uint32_t pre = block_excl_count(m, tot, sh);
                if (seen + tot > rr) {
                    if (m && seen + pre == rr) sh.result = ((uint64_t)kv << 32) | (uint64_t)(~(uint32_t)j);
                    __syncthreads();
                    break;
                }
                seen += tot;
            }
            result = sh.result;
        }
        t_tie = (int)selkey_idx(result);
        t_tau = row[t_tie];
    }
    if (tid == 0) {
        thr_tau[b * Hkv + g] = t_tau;
        thr_tie[b * Hkv + g] = t_tie;
    }
    if (!kept_idx) return;
    // kept positions in ascending order (item-major = index order)
    int32_t *out = kept_idx + ((size_t)b * Hkv + g) * w;
    const uint64_t thr = (L > w) ? result : 0ull;
    uint32_t offset = 0;
    for (int it = 0; it < ITEMS; ++it) {
        const int j = it * kSelThreads + tid;
        const bool keep = j < L && ((((uint64_t)k[it] << 32) | (uint64_t)(~(uint32_t)j)) >= thr);
        uint32_t tot;
        const uint32_t pre = block_excl_count(keep, tot, sh);
        if (keep && offset + pre < (uint32_t)w) out[offset + pre] = j;
        offset += tot;
    }
    for (int q = min(L, w) + tid; q < w; q += kSelThreads) out[q] = -1;
}

// Rows longer than the register-resident path: multi-pass radix select.
__global__ __launch_bounds__(kThreads) void decode_select_long_kernel(
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
            if (off < w) out[off] = j;
            ++off;
        }
    for (int q = min(L, w) + tid; q < w; q += kThreads) out[q] = -1;
}

// ---------------------------------------------------------------- attend --

template <typename T, int D, int GM>
__global__ __launch_bounds__(kThreads) void decode_attend_kernel(
    const T *__restrict__ q, const T *__restrict__ Kc, const T *__restrict__ Vc,
    const float *__restrict__ dt_cache, const int32_t *__restrict__ cache_lens, int Lmax, int Hq,
    int Hkv, const float *__restrict__ thr_tau, const int32_t *__restrict__ thr_tie,
    float *__restrict__ pm, float *__restrict__ pl, float *__restrict__ po, float qscale) {
    constexpr int NW = kThreads / 64;
    constexpr int BK = 64;                      // kept keys per block
    constexpr int EV = 16 / (int)sizeof(T);     // elements per 16-byte vector
    constexpr int RV = D / EV;                  // vectors per K/V row
    constexpr int P = D + EV;                   // LDS row pitch (elements), 16-byte pad
    constexpr int NL = BK * RV / kThreads;      // row vectors per thread per block
    constexpr int QD = D / 4;                   // head_dim quarter per lane (scores)
    constexpr int PER = D / 64;                 // output columns per lane (weighted sum)
    static_assert(BK * RV % kThreads == 0, "block staging split");
    __shared__ __align__(16) float qs[GM][D];
    __shared__ __align__(16) T Ks[BK * P];
    __shared__ __align__(16) T Vs[BK * P];
    __shared__ int c_idx[kSplit];
    __shared__ float c_dtl[kSplit];
    __shared__ float zs[GM][BK];
    __shared__ float hm[GM], halpha[GM], hl[GM];
    __shared__ float ored[GM][D];
    __shared__ int wcnt[NW];

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
        ored[hh][e] = 0.f;
    }
    if (tid < GM) {
        hm[tid] = -INFINITY;
        hl[tid] = 0.f;
    }
    // kept positions of this slice, in index order
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
        for (int w2 = 0; w2 < NW; ++w2) {
            const int c = wcnt[w2];
            off += (w2 < wave) ? c : 0;
            tot += c;
        }
        if (take) {
            c_idx[off + pre] = j;
            c_dtl[off + pre] = dj * kLog2e;
        }
        n += tot;
        __syncthreads();
    }
    __syncthreads();

    const size_t kvs = (size_t)Hkv * D;
    const T *Kb = Kc + (size_t)b * Lmax * kvs + (size_t)g * D;
    const T *Vb = Vc + (size_t)b * Lmax * kvs + (size_t)g * D;

    // coalesced staging: 16-byte vector v of the block is (row v / RV, column v % RV)
    uint4 rk[NL], rv[NL];
    auto load_block = [&](int blk) {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int v = tid + u * kThreads;
            const int kk = v / RV, cv = v % RV;
            const int pos = blk + kk;
            if (pos < n) {
                const size_t off = (size_t)c_idx[pos] * kvs + (size_t)cv * EV;
                rk[u] = *reinterpret_cast<const uint4 *>(Kb + off);
                rv[u] = *reinterpret_cast<const uint4 *>(Vb + off);
            } else {
                rk[u] = make_uint4(0, 0, 0, 0);
                rv[u] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    float acc[GM][PER];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
        for (int u = 0; u < PER; ++u) acc[hh][u] = 0.f;

    if (n > 0) load_block(0);
    for (int blk = 0; blk < n; blk += BK) {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int v = tid + u * kThreads;
            const int kk = v / RV, cv = v % RV;
            *reinterpret_cast<uint4 *>(&Ks[kk * P + cv * EV]) = rk[u];
            *reinterpret_cast<uint4 *>(&Vs[kk * P + cv * EV]) = rv[u];
        }
        __syncthreads();
        if (blk + BK < n) load_block(blk + BK);

        // scores: wave takes 16 keys, 4 lanes per key split head_dim in quarters
        {
            const int kk = wave * 16 + (lane >> 2);
            const int qq = lane & 3;
            float sc[GM];
#pragma unroll
            for (int hh = 0; hh < GM; ++hh) sc[hh] = 0.f;
#pragma unroll
            for (int e0 = 0; e0 < QD; e0 += 8) {
                const int e = qq * QD + e0;
                float x[8];
                if constexpr (sizeof(T) == 2) {
                    const uint4 kv = *reinterpret_cast<const uint4 *>(&Ks[kk * P + e]);
                    const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        x[2 * r] = __uint_as_float(w4[r] << 16);
                        x[2 * r + 1] = __uint_as_float(w4[r] & 0xffff0000u);
                    }
                } else {
                    const float4 a4 = *reinterpret_cast<const float4 *>(&Ks[kk * P + e]);
                    const float4 b4 = *reinterpret_cast<const float4 *>(&Ks[kk * P + e + 4]);
                    x[0] = a4.x; x[1] = a4.y; x[2] = a4.z; x[3] = a4.w;
                    x[4] = b4.x; x[5] = b4.y; x[6] = b4.z; x[7] = b4.w;
                }
#pragma unroll
                for (int hh = 0; hh < GM; ++hh) {
                    if (hh < G) {
                        const float4 qa = *reinterpret_cast<const float4 *>(&qs[hh][e]);
                        const float4 qb = *reinterpret_cast<const float4 *>(&qs[hh][e + 4]);
                        float a = sc[hh];
                        a = fmaf(qa.x, x[0], a); a = fmaf(qa.y, x[1], a);
                        a = fmaf(qa.z, x[2], a); a = fmaf(qa.w, x[3], a);
                        a = fmaf(qb.x, x[4], a); a = fmaf(qb.y, x[5], a);
                        a = fmaf(qb.z, x[6], a); a = fmaf(qb.w, x[7], a);
                        sc[hh] = a;
                    }
                }
            }
            const bool kval = blk + kk < n;
            const float dl = kval ? c_dtl[blk + kk] : 0.f;
#pragma unroll
            for (int hh = 0; hh < GM; ++hh) {
                if (hh < G) {
                    float a = sc[hh];
                    a += __shfl_xor(a, 1, 64);
                    a += __shfl_xor(a, 2, 64);
                    if (qq == 0) zs[hh][kk] = kval ? fmaf(a, qscale, dl) : -INFINITY;
                }
            }
        }
        __syncthreads();
        // per head: block max, running max and rescale, probabilities
        for (int hh = wave; hh < G; hh += NW) {
            const float z = zs[hh][lane];
            const float mo = hm[hh];
            const float mn = fmaxf(mo, wave_max(z));
            const float p = (mn == -INFINITY) ? 0.f : exp2f(z - mn);
            zs[hh][lane] = p;
            const float ps = wave_sum(p);
            if (lane == 0) {
                const float al = (mn == -INFINITY) ? 1.f : exp2f(mo - mn);
                halpha[hh] = al;
                hm[hh] = mn;
                hl[hh] = hl[hh] * al + ps;
            }
        }
        __syncthreads();
        // weighted V rows: wave takes every NW-th key, lanes cover head_dim
#pragma unroll
        for (int hh = 0; hh < GM; ++hh)
            if (hh < G) {
                const float al = halpha[hh];
#pragma unroll
                for (int u = 0; u < PER; ++u) acc[hh][u] *= al;
            }
        for (int kk = wave; kk < BK; kk += NW) {
            float v[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u) v[u] = Elem<T>::load(Vs, (size_t)kk * P + lane * PER + u);
#pragma unroll
            for (int hh = 0; hh < GM; ++hh) {
                if (hh < G) {
                    const float p = zs[hh][kk];
#pragma unroll
                    for (int u = 0; u < PER; ++u) acc[hh][u] = fmaf(p, v[u], acc[hh][u]);
                }
            }
        }
        __syncthreads();
    }
    // reduce over the waves and write this split's partials
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
        if (hh < G) {
#pragma unroll
            for (int u = 0; u < PER; ++u) atomicAdd(&ored[hh][lane * PER + u], acc[hh][u]);
        }
    }
    __syncthreads();
    for (int x = tid; x < G * D; x += kThreads) {
        const int hh = x / D, e = x % D;
        const size_t pidx = ((size_t)b * Hq + g * G + hh) * nsplit + split;
        po[pidx * D + e] = ored[hh][e];
        if (e == 0) {
            pm[pidx] = hm[hh];
            pl[pidx] = hl[hh];
        }
    }
}

// Merge the split partials of one (batch, kv head): one thread per (head, column).
template <typename T>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(const float *__restrict__ pm,
                                                                  const float *__restrict__ pl,
                                                                  const float *__restrict__ po, int Hq,
                                                                  int Hkv, int nsplit, int d,
                                                                  T *__restrict__ out) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int G = Hq / Hkv;
    for (int x = threadIdx.x; x < G * d; x += kThreads) {
        const int hh = x / d, e = x % d;
        const size_t pbase = ((size_t)b * Hq + g * G + hh) * nsplit;
        float M = -INFINITY;
        for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pm[pbase + s]);
        float num = 0.f, den = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float ms = pm[pbase + s];
            if (ms == -INFINITY) continue;
            const float f = exp2f(ms - M);
            den = fmaf(pl[pbase + s], f, den);
            num = fmaf(po[(pbase + s) * d + e], f, num);
        }
        Elem<T>::store(out, ((size_t)b * Hq + g * G + hh) * d + e, den > 0.f ? num / den : 0.f);
    }
}

template <typename T, int D>
hipError_t launch_attend(int gm, dim3 grid, hipStream_t stream, const T *q, const T *Kc, const T *Vc,
                         const float *dt_cache, const int32_t *cache_lens, int Lmax, int Hq, int Hkv,
                         const float *thr_tau, const int32_t *thr_tie, float *pm, float *pl, float *po,
                         float qscale) {
#define DMA_ATTEND(GMV)                                                                                  \
    hipLaunchKernelGGL((decode_attend_kernel<T, D, GMV>), grid, dim3(kThreads), 0, stream, q, Kc, Vc,    \
                       dt_cache, cache_lens, Lmax, Hq, Hkv, thr_tau, thr_tie, pm, pl, po, qscale)
    if (gm <= 4) DMA_ATTEND(4);
    else if (gm <= 8) DMA_ATTEND(8);
    else DMA_ATTEND(16);
#undef DMA_ATTEND
    return hipGetLastError();
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
    const dim3 sgrid(Hkv, B);
    if (Lmax <= 16 * kSelThreads)
        hipLaunchKernelGGL(decode_select_kernel<16>, sgrid, dim3(kSelThreads), 0, stream, dt_cache,
                           cache_lens, Hkv, Lmax, w, thr_tau, thr_tie, kept_idx);
    else if (Lmax <= 32 * kSelThreads)
        hipLaunchKernelGGL(decode_select_kernel<32>, sgrid, dim3(kSelThreads), 0, stream, dt_cache,
                           cache_lens, Hkv, Lmax, w, thr_tau, thr_tie, kept_idx);
    else
        hipLaunchKernelGGL(decode_select_long_kernel, sgrid, dim3(kThreads), 0, stream, dt_cache,
                           cache_lens, Hkv, Lmax, w, thr_tau, thr_tie, kept_idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 agrid(ns, Hkv, B);
    const int G = Hq / Hkv;
    e = d == 128 ? launch_attend<T, 128>(G, agrid, stream, q, Kc, Vc, dt_cache, cache_lens, Lmax, Hq, Hkv,
                                         thr_tau, thr_tie, pm, pl, po, qscale)
                 : launch_attend<T, 64>(G, agrid, stream, q, Kc, Vc, dt_cache, cache_lens, Lmax, Hq, Hkv,
                                        thr_tau, thr_tie, pm, pl, po, qscale);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3(Hkv, B), dim3(kThreads), 0, stream, pm, pl, po, Hq,
                       Hkv, ns, d, out);
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
