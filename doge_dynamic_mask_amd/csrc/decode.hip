// Decode step over a long KV cache under the dynamic top-w mask.
// Doge guide (gitcode), DMA section, forward step 3 (top-w of the per-position
// dt, computed from the cached value states) and step 4 (scaled, dt-biased
// fp32 softmax attention); the query of batch b sits at position L_b - 1.
//
// Three launches on the caller's stream:
//  1. select: one workgroup per (batch, kv head) finds the w-th best cached
//     position exactly (order: dt desc, index asc) and writes its selection
//     key to the workspace (and, when asked or for the float32 path, the kept
//     positions in ascending order).  Rows of up to 32768 positions are held
//     in registers (1024 threads, each owning consecutive positions) and
//     resolved with a range-adapted 4096-bin histogram plus an exact rank of
//     the few keys in the threshold bin; longer rows use the multi-pass radix
//     select.
//  2. attend: bf16 takes one workgroup per (contiguous range of positions,
//     kv head, batch), compacts the range's kept positions in LDS from the
//     threshold and walks them 64 at a time (non-temporal 16-byte gathers of
//     the K/V rows, the next block in flight, scores and P V on 16x16x32 MFMA
//     with the G query heads as the N dimension, online softmax across
//     blocks); float32 takes one workgroup per 64 kept positions of the list
//     and uses VALU.  Each writes a partial (max, sum, output) per query head.
//  3. combine: merges the partials of each (batch, query head).
//     (A separate launch: merging inside the last attend workgroup would need
//     device-scope fences, which on a multi-XCD part write back and
//     invalidate L2 in every workgroup.)
// HBM traffic is the dt cache plus the K/V rows of the w kept positions per
// kv head, not the whole cache.
#include "common.hpp"
#include "launch.hpp"
#include "radix_select.hpp"

#include <mutex>

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kKPC = 64;           // kept positions per attend workgroup
constexpr int kSelThreads = 1024;  // select workgroup (register-resident rows)
constexpr int kBins = 4096;
constexpr int kCandCap = 1024;

inline int nchunk_of(int Lmax, int w) {
    const int n = Lmax < w ? Lmax : w;
    return (n + kKPC - 1) / kKPC;
}

struct WsLayout {
    size_t thr, kept, kdt, pm, pl, po, total;
};

inline WsLayout ws_layout(int B, int Lmax, int Hq, int Hkv, int d, int w) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t nc = (size_t)nchunk_of(Lmax, w);
    WsLayout l;
    l.thr = 0;
    l.kept = up(l.thr + sizeof(uint64_t) * B * Hkv);
    l.kdt = up(l.kept + sizeof(int32_t) * B * Hkv * w);
    l.pm = up(l.kdt + sizeof(float) * B * Hkv * w);
    l.pl = up(l.pm + sizeof(float) * B * Hq * nc);
    l.po = up(l.pl + sizeof(float) * B * Hq * nc);
    l.total = up(l.po + sizeof(float) * B * Hq * nc * d);
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

// Exclusive prefix sum of v over the threads (thread order), and the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total, SelShared &sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) sh.red2[wave] = incl;
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
    return off + incl - v;
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
        const int j = tid * ITEMS + it;
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

// Kept positions (ascending) and their dt*log2(e) into the workspace lists;
// also into kept_idx (padded with -1 up to w) when it is given.
__device__ __forceinline__ void write_kept(int32_t *kl, float *kd, int32_t *kept_idx, uint32_t pos, int j,
                                           float dtv, int w) {
    if (pos < (uint32_t)w) {
        if (kl) {
            kl[pos] = j;
            kd[pos] = dtv * kLog2e;
        }
        if (kept_idx) kept_idx[pos] = j;
    }
}

template <int ITEMS>
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(
    const float *__restrict__ dt_cache, const int32_t *__restrict__ cache_lens, int Hkv, int Lmax,
    int w, uint64_t *__restrict__ thr_ws, int32_t *__restrict__ kept_ws, float *__restrict__ kdt_ws,
    int32_t *__restrict__ kept_idx) {
    static_assert(ITEMS % 4 == 0, "float4 loads");
    __shared__ SelShared sh;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = clamp_len(cache_lens, b, Lmax);
    const float *row = dt_cache + ((size_t)b * Hkv + g) * Lmax;
    const int j0 = tid * ITEMS;  // this thread owns positions j0 .. j0 + ITEMS - 1

    float dv[ITEMS];
    uint32_t k[ITEMS];
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int q4 = 0; q4 < ITEMS / 4; ++q4) {
        const int jj = j0 + 4 * q4;
        if (jj + 3 < L && (((uintptr_t)(row + jj)) & 15u) == 0) {
            const float4 v = *reinterpret_cast<const float4 *>(row + jj);
            dv[4 * q4] = v.x; dv[4 * q4 + 1] = v.y; dv[4 * q4 + 2] = v.z; dv[4 * q4 + 3] = v.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) dv[4 * q4 + u] = jj + u < L ? row[jj + u] : 0.f;
        }
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool valid = j0 + it < L;
        k[it] = valid ? ordkey(dv[it]) : 0u;
        if (valid) {
            kmin = min(kmin, k[it]);
            kmax = max(kmax, k[it]);
        }
    }
    uint64_t result = 0;  // (ordkey << 32) | ~index of the w-th kept position
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
                const int j = j0 + it;
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
        } else {
            // a single key value shared by more than kCandCap positions: the
            // rr-th of them in index order (threads own consecutive positions)
            const uint32_t kv = bsel;
            uint32_t c = 0;
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) c += (j0 + it < L && k[it] == kv) ? 1u : 0u;
            uint32_t tot;
            const uint32_t before = block_excl_scan(c, tot, sh);
            if (before <= rr && rr < before + c) {
                uint32_t seen = before;
#pragma unroll
                for (int it = 0; it < ITEMS; ++it) {
                    if (j0 + it < L && k[it] == kv) {
                        if (seen == rr) sh.result = ((uint64_t)kv << 32) | (uint64_t)(~(uint32_t)(j0 + it));
                        ++seen;
                    }
                }
            }
            __syncthreads();
        }
        result = sh.result;
    }
    // the w-th kept key (0, below every key, when all positions are kept)
    if (tid == 0) thr_ws[(size_t)b * Hkv + g] = result;
    if (!kept_ws && !kept_idx) return;  // uniform: no list asked for
    // kept positions, ascending: per-thread counts, one block scan
    uint32_t c = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it)
        c += (j0 + it < L && ((((uint64_t)k[it] << 32) | (uint64_t)(~(uint32_t)(j0 + it))) >= result)) ? 1u : 0u;
    uint32_t tot;
    uint32_t pos = block_excl_scan(c, tot, sh);
    int32_t *kl = kept_ws ? kept_ws + ((size_t)b * Hkv + g) * w : nullptr;
    float *kd = kept_ws ? kdt_ws + ((size_t)b * Hkv + g) * w : nullptr;
    int32_t *ki = kept_idx ? kept_idx + ((size_t)b * Hkv + g) * w : nullptr;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int j = j0 + it;
        if (j < L && ((((uint64_t)k[it] << 32) | (uint64_t)(~(uint32_t)j)) >= result)) {
            write_kept(kl, kd, ki, pos, j, dv[it], w);
            ++pos;
        }
    }
    if (ki)
        for (int q = min(L, w) + tid; q < w; q += kSelThreads) ki[q] = -1;
}

// Rows longer than the register-resident path: multi-pass radix select.
__global__ __launch_bounds__(kThreads) void decode_select_long_kernel(
    const float *__restrict__ dt_cache, const int32_t *__restrict__ cache_lens, int Hkv, int Lmax,
    int w, uint64_t *__restrict__ thr_ws, int32_t *__restrict__ kept_ws, float *__restrict__ kdt_ws,
    int32_t *__restrict__ kept_idx) {
    __shared__ RadixShared<kThreads> rs;
    __shared__ int wsum[kThreads / 64];
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = clamp_len(cache_lens, b, Lmax);
    const float *row = dt_cache + ((size_t)b * Hkv + g) * Lmax;
    float t_tau = -INFINITY;
    int t_tie = -1;
    uint64_t result = 0;  // selection key of the w-th kept position (0: all kept)
    if (L > w) {
        const uint32_t ranks[2] = {(uint32_t)(w - 1), 0u};
        uint64_t keys[2];
        radix_select<kThreads>(row, L, 1, ranks, keys, rs);
        result = keys[0];
        t_tie = (int)selkey_idx(keys[0]);
        t_tau = row[t_tie];
    }
    if (tid == 0) thr_ws[(size_t)b * Hkv + g] = result;
    if (!kept_ws && !kept_idx) return;  // uniform: no list asked for
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
    int32_t *kl = kept_ws ? kept_ws + ((size_t)b * Hkv + g) * w : nullptr;
    float *kd = kept_ws ? kdt_ws + ((size_t)b * Hkv + g) * w : nullptr;
    int32_t *ki = kept_idx ? kept_idx + ((size_t)b * Hkv + g) * w : nullptr;
    for (int j = j0; j < j1; ++j) {
        const float dj = row[j];
        if (kept_test(dj, j, t_tau, t_tie)) {
            write_kept(kl, kd, ki, (uint32_t)off, j, dj, w);
            ++off;
        }
    }
    if (ki)
        for (int q = min(L, w) + tid; q < w; q += kThreads) ki[q] = -1;
}

// ---------------------------------------------------------------- attend --

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streamed-once rows: non-temporal 16-byte loads, so the gather neither
// allocates in nor evicts from the caches.
__device__ __forceinline__ uint4 load_nt16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename T, int D, int GM>
__global__ __launch_bounds__(kThreads) void decode_attend_kernel(
    const T *__restrict__ q, const T *__restrict__ Kc, const T *__restrict__ Vc,
    const int32_t *__restrict__ cache_lens, int Lmax, int Hq, int Hkv, int w,
    const int32_t *__restrict__ kept_ws, const float *__restrict__ kdt_ws, float *__restrict__ pm,
    float *__restrict__ pl, float *__restrict__ po, float qscale) {
    constexpr int NW = kThreads / 64;
    constexpr int BK = kKPC;                    // kept keys per workgroup (one block)
    constexpr int EV = 16 / (int)sizeof(T);     // elements per 16-byte vector
    constexpr int RV = D / EV;                  // vectors per K/V row
    constexpr int P = D + EV;                   // LDS row pitch (elements), 16-byte pad
    constexpr int NL = BK * RV / kThreads;      // row vectors per thread
    constexpr int QD = D / 4;                   // head_dim quarter per lane (scores)
    constexpr int PER = D / 64;                 // output columns per lane (weighted sum)
    static_assert(BK * RV % kThreads == 0 && BK == 64, "one 64-key block per workgroup");
    __shared__ __align__(16) float qs[GM][D];
    __shared__ __align__(16) T Ks[BK * P];
    __shared__ __align__(16) T Vs[BK * P];
    __shared__ float c_dtl[BK];
    __shared__ float zs[GM][BK];
    __shared__ float hm[GM], hl[GM];
    __shared__ float ored[GM][D];

    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int G = Hq / Hkv;
    const int nchunk = gridDim.x;
    const int L = clamp_len(cache_lens, b, Lmax);
    const int c0 = chunk * BK;
    const int n = max(0, min(min(L, w) - c0, BK));  // kept positions of this chunk
    const size_t lbase = ((size_t)b * Hkv + g) * w + c0;

    // Issue every global load before anything waits on one: the query and
    // the chunk's dt first, then all kept indices (16 lanes share each
    // entry), then all K/V row loads.  Stores to LDS come after the issue.
    constexpr int QPT = (GM * D + kThreads - 1) / kThreads;  // query values per thread
    float qv[QPT];
#pragma unroll
    for (int u = 0; u < QPT; ++u) {  // clamped, unconditional loads: nothing waits yet
        const int x = min(tid + u * kThreads, G * D - 1);
        qv[u] = Elem<T>::load(q, ((size_t)b * Hq + g * G) * D + x);
    }
    const float dlv = kdt_ws[lbase + min(tid, BK - 1)];
    const size_t kvs = (size_t)Hkv * D;
    const T *Kb = Kc + (size_t)b * Lmax * kvs + (size_t)g * D;
    const T *Vb = Vc + (size_t)b * Lmax * kvs + (size_t)g * D;
    uint4 rk[NL], rv[NL];
    if (n > 0) {
        int jr[NL];
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int kk = (tid + u * kThreads) / RV;
            jr[u] = kept_ws[lbase + min(kk, n - 1)];
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const size_t off = (size_t)jr[u] * kvs + (size_t)((tid + u * kThreads) % RV) * EV;
            rk[u] = load_nt16(Kb + off);
            rv[u] = load_nt16(Vb + off);
        }
    }
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
        const int x = tid + u * kThreads;
        if (x < G * D) {
            qs[x / D][x % D] = qv[u];
            ored[x / D][x % D] = 0.f;
        }
    }
    if (tid < BK) c_dtl[tid] = tid < n ? dlv : 0.f;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int v = tid + u * kThreads;
        const int kk = v / RV, cv = v % RV;
        const bool ok = kk < n;
        *reinterpret_cast<uint4 *>(&Ks[kk * P + cv * EV]) = ok ? rk[u] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(&Vs[kk * P + cv * EV]) = ok ? rv[u] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();

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
        const bool kval = kk < n;
        const float dl = c_dtl[kk];
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
    // per head: max, probabilities, sum (wave hh % NW owns head hh)
    for (int hh = wave; hh < G; hh += NW) {
        const float z = zs[hh][lane];
        const float mx = wave_max(z);
        const float p = (mx == -INFINITY) ? 0.f : exp2f(z - mx);
        zs[hh][lane] = p;
        const float ps = wave_sum(p);
        if (lane == 0) {
            hm[hh] = mx;
            hl[hh] = ps;
        }
    }
    __syncthreads();
    // weighted V rows: wave takes every NW-th key, lanes cover head_dim
    float acc[GM][PER];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
        for (int u = 0; u < PER; ++u) acc[hh][u] = 0.f;
    for (int kk = wave; kk < n; kk += NW) {
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
        const size_t pidx = ((size_t)b * Hq + g * G + hh) * nchunk + chunk;
        po[pidx * D + e] = ored[hh][e];
        if (e == 0) {
            pm[pidx] = hm[hh];
            pl[pidx] = hl[hh];
        }
    }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives
// element (i % 4) of the 4 x 16-bit values at the address of lane (i/4 + 4s),
// s = 0..3; lane k pointing at row r0 + k/4, columns c0 + 4*(k%4) of a
// row-major tile gives lane i the column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

constexpr int kRange = 4096;            // positions compacted per pass
constexpr int kTargetSplitWGs = 512;   // attend workgroups a launch aims for

// bf16 attend, wave-independent: one workgroup per (range of positions, kv
// head, batch) compacts the range's kept positions into LDS (one barrier per
// pass); then each wave takes every fourth block of 32 kept keys with no
// further barrier until the end.  A block's K and V rows are gathered with
// whole-row, non-temporal 16-byte loads (16 lanes per row) into the wave's own
// LDS region; scores S^T = K Q^T on 16x16x32 MFMA leave each lane the 8 keys
// kappa(g, j) = 16*(j/4) + 4g + j%4 of head l%16 (g = l/16), which are exactly
// the k-slots of the P operand of O = P V, so P never leaves registers; V
// comes back as the B operand by transpose reads.  The next block's rows are
// in flight while a block is computed.  Each wave keeps its own online
// softmax state; the four are merged in LDS into one partial per query head.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_attend_wave_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ Kc, const uint16_t *__restrict__ Vc,
    const float *__restrict__ dt_cache, const int32_t *__restrict__ cache_lens, int Lmax, int Hq,
    int Hkv, const uint64_t *__restrict__ thr_ws, float *__restrict__ pm, float *__restrict__ pl,
    float *__restrict__ po, float qscale) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    constexpr int NW = kThreads / 64;
    constexpr int KB = 32;                   // kept keys per wave block
    constexpr int NS = D / 32;               // 32-wide head_dim slices
    constexpr int KP = D + 8;                // K and V row pitch in LDS (bf16): 16-byte pad
    constexpr int RV = D / 8;                // 16-byte vectors per row
    constexpr int NU = KB * RV / 64;         // row vectors per lane per block
    constexpr int PER = kRange / kThreads;   // positions per thread per compaction pass
    constexpr int NT = D / 16;               // output column tiles
    static_assert(NW * KB * KP * 2 >= NW * 16 * D * 4, "the merge buffer fits in the row regions");
    __shared__ int l_idx[kRange];
    __shared__ float l_dtl[kRange];
    __shared__ uint32_t wcnt[NW];
    __shared__ __align__(16) uint16_t KVw[NW][KB * KP];  // per-wave V rows; reused for the merge
    __shared__ float mw[NW][16], lw[NW][16];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int nsplit = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int G = Hq / Hkv;
    const int col = lane & 15, grp = lane >> 4;
    const int L = clamp_len(cache_lens, b, Lmax);
    const int len = (L + nsplit - 1) / nsplit;
    const int jbeg = min(split * len, L), jend = min(jbeg + len, L);
    const uint64_t thr = thr_ws[(size_t)b * Hkv + g];
    const float *drow = dt_cache + ((size_t)b * Hkv + g) * Lmax;
    const size_t kvs = (size_t)Hkv * D;
    const uint16_t *Kb = Kc + (size_t)b * Lmax * kvs + (size_t)g * D;
    const uint16_t *Vb = Vc + (size_t)b * Lmax * kvs + (size_t)g * D;
    uint16_t *vw = KVw[wave];

    bf16x8 qf[NS];
    {
        const int hq = g * G + min(col, G - 1);
        const uint16_t *qp = q + ((size_t)b * Hq + hq) * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 32 * s);
            if (col >= G) qf[s] = bf16x8{};
        }
    }

    float m_run = -INFINITY, l_run = 0.f;  // head `col`
    f32x4 oacc[NT];                        // rows: heads 4*grp + i; columns 16t + col
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[t] = f32x4{};

    // K of a block goes straight to registers in the layout of the score
    // MFMA's A operand: lane (col, grp) takes key 16c + col, columns
    // 32s + 8grp .. +7 (NK = 2 * NS pieces).  V rows go through LDS for the
    // transpose reads: vector v = lane + 64u is row v / RV, 16-byte column v % RV.
    constexpr int NK = 2 * NS;
    u32x4 kr[NK], vr[NU], kn[NK], vn[NU];
    auto load_rows = [&](u32x4 (&kx)[NK], u32x4 (&vx)[NU], int kb, int n) __attribute__((always_inline)) {
        int jk[2], jr[NU];
#pragma unroll
        for (int c = 0; c < 2; ++c) jk[c] = l_idx[min(kb + 16 * c + col, n - 1)];
#pragma unroll
        for (int u = 0; u < NU; ++u) jr[u] = l_idx[min(kb + (lane + 64 * u) / RV, n - 1)];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2)
                kx[c * NS + s2] = *reinterpret_cast<const u32x4 *>(Kb + (size_t)(uint32_t)jk[c] * kvs + 32 * s2 + 8 * grp);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const size_t off = (size_t)(uint32_t)jr[u] * kvs + (size_t)((lane + 64 * u) % RV) * 8;
            vx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(Vb + off));
        }
    };
    // one block: S, online softmax, O += P V
    auto block = [&](const u32x4 (&kx)[NK], const u32x4 (&vx)[NU], int kb, int n) __attribute__((always_inline)) {
        const int nb = min(KB, n - kb);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int v = lane + 64 * u;
            *reinterpret_cast<u32x4 *>(&vw[(v / RV) * KP + (v % RV) * 8]) = vx[u];
        }
        float z[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f32x4 sacc = f32x4{};
#pragma unroll
            for (int s = 0; s < NS; ++s)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kx[c * NS + s]), qf[s], sacc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 16 * c + 4 * grp + i;
                z[c][i] = (kk < nb && col < G) ? fmaf(sacc[i], qscale, l_dtl[kb + kk]) : -INFINITY;
                mx = fmaxf(mx, z[c][i]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float msub = m_new == -INFINITY ? 0.f : m_new;
        bf16x8 pa;
        float ps = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(z[c][i] - msub);
                pa[4 * c + i] = pb;
                ps += (float)pb;  // the denominator sums the same rounded weights
            }
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l_run = l_run * alpha + ps;
        m_run = m_new;
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * grp + i, 64);
        const int tr_k = lane & 15;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[t][i] *= ar[i];
            const uint16_t *vp = &vw[(4 * grp + (tr_k >> 2)) * KP + 16 * t + 4 * (tr_k & 3)];
            const i16x4 lo = lds_read_tr16(vp);
            const i16x4 hi = lds_read_tr16(vp + 16 * KP);
            const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, oacc[t], 0, 0, 0);
        }
    };

    // dt of a pass's positions; positions past the range load the range's
    // last one (never kept there), so no load is conditional.  The next
    // pass's loads are issued before this pass's blocks.
    float dv[PER], dnx[PER];
    auto load_dt = [&](float (&x)[PER], int jb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < PER; ++u) x[u] = drow[min(jb + PER * tid + u, jend - 1)];
    };
    if (jbeg < jend) load_dt(dv, jbeg);
    for (int jb = jbeg; jb < jend; jb += kRange) {
        // ---- compaction: this thread's PER consecutive positions, block scan
        const int je = min(jb + kRange, jend);
        bool kp[PER];
        uint32_t cnt = 0;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int j = jb + PER * tid + u;
            kp[u] = j < je && selkey(dv[u], (uint32_t)j) >= thr;
            cnt += kp[u] ? 1u : 0u;
        }
        uint32_t incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        __syncthreads();  // the previous pass's readers of the list are done
        if (lane == 63) wcnt[wave] = incl;
        __syncthreads();
        uint32_t off = incl - cnt;
        int n = 0;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            off += w2 < wave ? wcnt[w2] : 0u;
            n += (int)wcnt[w2];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            if (kp[u]) {
                l_idx[off] = jb + PER * tid + u;
                l_dtl[off] = dv[u] * kLog2e;
                ++off;
            }
        }
        __syncthreads();
        if (jb + kRange < jend) load_dt(dnx, jb + kRange);

        // ---- this wave's blocks: kb = (wave + NW*k) * KB, two at a time so
        // that the register sets alternate without copies.  The next block's
        // rows are requested unconditionally (indices clamp to the last kept
        // position, so past the end they repeat cached rows): a conditional
        // request would make the compiler wait for it before the current
        // block's math.
        int kb = wave * KB;
        if (kb < n) {
            load_rows(kr, vr, kb, n);
            for (;;) {
                load_rows(kn, vn, kb + NW * KB, n);
                block(kr, vr, kb, n);
                kb += NW * KB;
                if (kb >= n) break;
                load_rows(kr, vr, kb + NW * KB, n);
                block(kn, vn, kb, n);
                kb += NW * KB;
                if (kb >= n) break;
            }
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) dv[u] = dnx[u];
    }

    // ---- merge the four waves' states into one partial per query head
    __syncthreads();  // the V regions are reused below
    float *om = reinterpret_cast<float *>(&KVw[0][0]);  // [NW][16][D]
    if (grp == 0) {
        mw[wave][col] = m_run;
        lw[wave][col] = l_run;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) om[(wave * 16 + 4 * grp + i) * D + 16 * t + col] = oacc[t][i];
    }
    __syncthreads();
    for (int x = tid; x < G * D; x += kThreads) {
        const int hh = x / D, e = x - hh * D;
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, mw[w2][hh]);
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            const float f = mw[w2][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w2][hh] - M);
            lsum = fmaf(lw[w2][hh], f, lsum);
            osum = fmaf(om[(w2 * 16 + hh) * D + e], f, osum);
        }
        const size_t pidx = ((size_t)b * Hq + g * G + hh) * nsplit + split;
        po[pidx * D + e] = osum;
        if (e == 0) {
            pm[pidx] = M;
            pl[pidx] = lsum;
        }
    }
}

// Merge the chunk partials of one (batch, query head): one thread per column.
template <typename T>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float *__restrict__ pm,
                                                            const float *__restrict__ pl,
                                                            const float *__restrict__ po, int nchunk,
                                                            int d, T *__restrict__ out) {
    // Thread e merges column e of the partials of one (batch, query head),
    // kGroup partials at a time with all of their loads in flight together;
    // every thread forms the same weights.  Slots past the last partial
    // repeat it with weight zero, so no load is conditional.
    constexpr int kGroup = 8;
    const int bh = blockIdx.x;  // b * Hq + hq
    const int e = min((int)threadIdx.x, d - 1);
    const float *m = pm + (size_t)bh * nchunk;
    const float *l = pl + (size_t)bh * nchunk;
    const float *o = po + (size_t)bh * nchunk * d + e;
    float M = -INFINITY, den = 0.f, num = 0.f;
    for (int s0 = 0; s0 < nchunk; s0 += kGroup) {
        float mv[kGroup], lv[kGroup], ov[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const int s = min(s0 + u, nchunk - 1);
            mv[u] = m[s];
            lv[u] = l[s];
            ov[u] = o[(size_t)s * d];
        }
#pragma unroll
        for (int u = 0; u < kGroup; ++u)
            if (s0 + u >= nchunk) mv[u] = -INFINITY;
        float Mn = M;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) Mn = fmaxf(Mn, mv[u]);
        if (Mn == -INFINITY) continue;  // nothing kept so far
        const float c = M == -INFINITY ? 0.f : exp2f(M - Mn);
        den *= c;
        num *= c;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const float f = mv[u] == -INFINITY ? 0.f : exp2f(mv[u] - Mn);
            den = fmaf(lv[u], f, den);
            num = fmaf(ov[u], f, num);
        }
        M = Mn;
    }
    if ((int)threadIdx.x < d) Elem<T>::store(out, (size_t)bh * d + threadIdx.x, den > 0.f ? num / den : 0.f);
}

template <typename T, int D>
hipError_t launch_attend(int gm, dim3 grid, hipStream_t stream, const T *q, const T *Kc, const T *Vc,
                         const int32_t *cache_lens, int Lmax, int Hq, int Hkv, int w,
                         const int32_t *kept_ws, const float *kdt_ws, float *pm, float *pl, float *po,
                         float qscale) {
#define DMA_ATTEND(GMV)                                                                                  \
    hipLaunchKernelGGL((decode_attend_kernel<T, D, GMV>), grid, dim3(kThreads), 0, stream, q, Kc, Vc,    \
                       cache_lens, Lmax, Hq, Hkv, w, kept_ws, kdt_ws, pm, pl, po, qscale)
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
    const WsLayout lay = ws_layout(B, Lmax, Hq, Hkv, d, w);
    char *base = (char *)ws;
    int32_t *kept_ws = (int32_t *)(base + lay.kept);
    float *kdt_ws = (float *)(base + lay.kdt);
    float *pm = (float *)(base + lay.pm);
    float *pl = (float *)(base + lay.pl);
    float *po = (float *)(base + lay.po);
    const int nc = nchunk_of(Lmax, w);
    const float qscale = (float)(1.0 / __builtin_sqrt((double)d) * 1.4426950408889634);
    uint64_t *thr_ws = (uint64_t *)(base + lay.thr);
    constexpr bool kRangeAttend = sizeof(T) == 2;  // bf16: attend scans ranges, no lists
    int32_t *lists = kRangeAttend ? nullptr : kept_ws;
    const dim3 sgrid(Hkv, B);
    if (Lmax <= 16 * kSelThreads)
        hipLaunchKernelGGL(decode_select_kernel<16>, sgrid, dim3(kSelThreads), 0, stream, dt_cache,
                           cache_lens, Hkv, Lmax, w, thr_ws, lists, kdt_ws, kept_idx);
    else if (Lmax <= 32 * kSelThreads)
        hipLaunchKernelGGL(decode_select_kernel<32>, sgrid, dim3(kSelThreads), 0, stream, dt_cache,
                           cache_lens, Hkv, Lmax, w, thr_ws, lists, kdt_ws, kept_idx);
    else
        hipLaunchKernelGGL(decode_select_long_kernel, sgrid, dim3(kThreads), 0, stream, dt_cache,
                           cache_lens, Hkv, Lmax, w, thr_ws, lists, kdt_ws, kept_idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int nparts = nc;  // partials per (batch, query head)
    if constexpr (kRangeAttend) {
        // ranges per (batch, kv head): about kTargetSplitWGs workgroups in
        // all, never more partials than the workspace holds
        const int want = (kTargetSplitWGs + B * Hkv - 1) / (B * Hkv);
        nparts = want < 1 ? 1 : (want > nc ? nc : want);
        const dim3 rgrid(nparts, Hkv, B);
        if (d == 128)
            hipLaunchKernelGGL(decode_attend_wave_kernel<128>, rgrid, dim3(kThreads), 0, stream, q, Kc, Vc,
                               dt_cache, cache_lens, Lmax, Hq, Hkv, thr_ws, pm, pl, po, qscale);
        else
            hipLaunchKernelGGL(decode_attend_wave_kernel<64>, rgrid, dim3(kThreads), 0, stream, q, Kc, Vc,
                               dt_cache, cache_lens, Lmax, Hq, Hkv, thr_ws, pm, pl, po, qscale);
        e = hipGetLastError();
    } else {
        const dim3 agrid(nc, Hkv, B);
        const int G = Hq / Hkv;
        e = d == 128 ? launch_attend<T, 128>(G, agrid, stream, q, Kc, Vc, cache_lens, Lmax, Hq, Hkv, w,
                                             kept_ws, kdt_ws, pm, pl, po, qscale)
                     : launch_attend<T, 64>(G, agrid, stream, q, Kc, Vc, cache_lens, Lmax, Hq, Hkv, w,
                                            kept_ws, kdt_ws, pm, pl, po, qscale);
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3(B * Hq), dim3(d), 0, stream, pm, pl, po, nparts, d,
                       out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_thresholds(const float *dt_cache, const int32_t *cache_lens, int B, int Lmax, int Hkv,
                                    int w, uint64_t *thr, hipStream_t stream) {
    const dim3 sgrid(Hkv, B);
    if (Lmax <= 16 * kSelThreads)
        hipLaunchKernelGGL(decode_select_kernel<16>, sgrid, dim3(kSelThreads), 0, stream, dt_cache, cache_lens, Hkv,
                           Lmax, w, thr, (int32_t *)nullptr, (float *)nullptr, (int32_t *)nullptr);
    else if (Lmax <= 32 * kSelThreads)
        hipLaunchKernelGGL(decode_select_kernel<32>, sgrid, dim3(kSelThreads), 0, stream, dt_cache, cache_lens, Hkv,
                           Lmax, w, thr, (int32_t *)nullptr, (float *)nullptr, (int32_t *)nullptr);
    else
        hipLaunchKernelGGL(decode_select_long_kernel, sgrid, dim3(kThreads), 0, stream, dt_cache, cache_lens, Hkv,
                           Lmax, w, thr, (int32_t *)nullptr, (float *)nullptr, (int32_t *)nullptr);
    return hipGetLastError();
}

size_t decode_ws_bytes(int B, int Lmax, int Hq, int Hkv, int d, int w) {
    return ws_layout(B, Lmax, Hq, Hkv, d, w).total;
}

// ---------------------------------------------------- allocation-free decode --
// dma_decode_noalloc's workspace: a file-scope device array, one copy per
// device the library runs on, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (in host code the name is a host-side
// stand-in, not a device address): the device address of each device's copy
// is looked up once, with that device current, and kept per device.
namespace {
static __device__ __align__(256) unsigned char scratch[kDecodeNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void *g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
}  // namespace

hipError_t launch_decode_noalloc(const void *q, const void *Kc, const void *Vc, int dtype, const float *dt_cache,
                                 const int32_t *cache_lens, int B, int Lmax, int Hq, int Hkv, int d, int w,
                                 void *out, int32_t *kept_idx, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    // every part of the workspace that the kernels read is written first by
    // the same call (thresholds by the select, one partial per attend
    // workgroup), so nothing needs clearing between calls
    return launch_decode(q, Kc, Vc, dtype, dt_cache, cache_lens, B, Lmax, Hq, Hkv, d, w, out, kept_idx,
                         g_scratch_ptr[dev], stream);
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
