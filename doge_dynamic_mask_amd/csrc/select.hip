// Per-row threshold selector for the top-w dynamic mask.
// Doge guide (gitcode), DMA section, forward step 3: each query row keeps the
// keep_window_size (w) keys of largest dt among its valid keys.
//
// The selection is made exact and row-parallel through two facts about the
// kept sets K_i = top_w({0..i} \ padding) under the order (dt desc, index asc):
//   (1) nesting: K_{i+1} is a subset of K_i plus {i+1}, so the w-th best key
//       only moves towards better keys as i grows; and
//   (2) for a chunk of C rows starting at r0, every row's kept set is the top
//       w of (prefix [0, r0)) plus at most C new keys.  A prefix key of
//       prefix rank k has between k and k + C better keys in a row's set, so
//       the best A0 = w-C-1 prefix keys are kept by every row of the chunk and
//       are never its w-th key, prefix keys of rank >= w are kept by none, and
//       each row's threshold key lies in the "band" of prefix ranks [A0, w)
//       plus the chunk's own keys: at most 2C+1 candidates.
// One workgroup per (batch, kv head, chunk of C rows), C = 32 for rows up to
// 4096 keys, 64 beyond (128 for a sliding window over rows longer than 4096
// with win >= 128):
//   a. finds the band: the key range of the prefix (of all of it when it is
//      staged in LDS, else of 1024 keys sampled in blocks spread over it,
//      keys outside the sampled range counting in the end bins), one
//      histogram pass with 1024 bins (4096 for the 128-row chunks) spanning
//      that range, the bins holding ranks A0 and w-1, and
//      an exact rank of the keys gathered from those bins (a multi-pass radix
//      select over the prefix when those bins hold too many keys, e.g. under
//      heavy ties);
//   b. lets each candidate find the rows it is the threshold of: at row i
//      the threshold is the candidate with exactly w-A0-1 better candidates
//      that row already sees (band keys always; new key j from row j on).
// Output per row: (tau, tie) = (dt, index) of the w-th kept key, or the
// canonical (-inf, -1) / (+inf, -1).  Only comparisons touch dt.
//
// Sliding window of win >= C positions (row i sees [i - win + 1, i]): the
// keys every valid row of the chunk sees form the "prefix" [pl, r0) with
// pl = hi - win (hi: end of the chunk's valid rows), and row i sees besides
// them the chunk's keys up to i and the "leaving" keys [i - win + 1, pl),
// at most C keys in all, so the same band argument holds; the leaving keys
// join the candidates (at most C - 1 more), and a candidate counts the
// leaving keys a row still sees with a ballot and a shifted bit count.
// Without a window the kernel is the full causal one (WIN = false).
#include "common.hpp"
#include "launch.hpp"
#include "radix_select.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kCollectCap = 512;    // boundary-bin keys ranked exactly in LDS
constexpr int kUnroll = 16;         // prefix keys per thread per pass step (loads in flight)
constexpr int kUnroll4 = 8;         // float4 loads per thread per pass step
constexpr int kSampleKeys = 1024;   // keys whose range bins a prefix too long to stage

// STAGE: prefixes up to this many keys are kept in LDS for the second and
// third passes (longer ones are read again from memory).  The workgroups are
// latency-bound, so a small LDS footprint (more workgroups per CU) beats
// keeping long prefixes: measured on rows of 8192 and 32768 keys, 1024-key
// staging is 18-30 % faster than 8192.
template <int C, int NB, int STAGE, bool WIN>
struct SelectShared {
    RadixShared<kThreads> rs;       // fallback radix select
    uint32_t hist[NB];
    uint64_t col[kCollectCap];
    uint64_t cand[(WIN ? 3 : 2) * C + 1];  // band (by rank), the chunk's own keys, the keys leaving its windows
    uint32_t red[2][kThreads / 64];
    uint32_t ncol, nfound;
    uint32_t binA, binB, aboveA;
    uint32_t keys[STAGE];           // prefix order keys, when P <= STAGE
};

// The float of order bits o = ordkey(f): f itself, except that -0.0 comes
// back as +0.0.
__device__ __forceinline__ float order_value(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// f(j, dt[j]) for every prefix position j < P.  A 16-byte aligned row is read
// in float4 loads, kUnroll4 of them per thread per step (32 positions), all
// issued before any is used; the last P % 4 positions, and rows that are not
// 16-byte aligned, go key by key, kUnroll per thread per step.  The passes
// are bound by the latency of these reads, so the fewer steps the better.
template <typename F>
__device__ __forceinline__ void for_prefix(const float *__restrict__ row, int P, F f) {
    int jt = 0;  // first position left to the key-by-key loop
    if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
        const int P4 = P & ~3;
        for (int j0 = 0; j0 < P4; j0 += 4 * kUnroll4 * kThreads) {
            float4 v[kUnroll4];
#pragma unroll
            for (int u = 0; u < kUnroll4; ++u) {
                const int j = j0 + 4 * (u * kThreads + (int)threadIdx.x);
                v[u] = j < P4 ? *reinterpret_cast<const float4 *>(row + j) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < kUnroll4; ++u) {
                const int j = j0 + 4 * (u * kThreads + (int)threadIdx.x);
                if (j < P4) {
                    f(j, v[u].x);
                    f(j + 1, v[u].y);
                    f(j + 2, v[u].z);
                    f(j + 3, v[u].w);
                }
            }
        }
        jt = P4;
    }
    for (int j0 = jt; j0 < P; j0 += kUnroll * kThreads) {
        float v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = j0 + u * kThreads + (int)threadIdx.x;
            v[u] = j < P ? row[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = j0 + u * kThreads + (int)threadIdx.x;
            if (j < P) f(j, v[u]);
        }
    }
}

// f(j, key_j) over the prefix from the LDS copy of its order keys.
template <typename F>
__device__ __forceinline__ void for_staged(const uint32_t *keys, int P, F f) {
    for (int j = threadIdx.x; j < P; j += kThreads) f(j, keys[j]);
}

// C: rows per chunk (the band holds C+1 prefix keys); NB: histogram bins;
// STAGE: prefix keys kept in LDS; WIN: rows see a sliding window of win >= C
// positions (else the full causal range, win unused)
template <int C, int NB, int STAGE, bool WIN>
__global__ __launch_bounds__(kThreads) void select_kernel(const float *__restrict__ dt,
                                                          const int32_t *__restrict__ seqlens,
                                                          int Hkv, int S, int w, int win, int nb_total,
                                                          float *__restrict__ tau,
                                                          int32_t *__restrict__ tie) {
    constexpr int kChunk = C;
    __shared__ SelectShared<C, NB, STAGE, WIN> sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Work item of this workgroup, items ordered by (batch, kv head, chunk).
    // Workgroup ids go round-robin over the 8 XCDs (XCD x = id mod 8).  Rows
    // of one length (no seqlens): XCD x takes items x*per_xcd ..
    // (x+1)*per_xcd - 1, so the chunks of one row run on one XCD, whose L2
    // then holds that row's dt for all of them.  Rows of different lengths
    // carry different work (it grows with the square of the length): with at
    // least four rows, row u goes to the XCD pair u mod 4 and its chunks
    // alternate between the pair's two XCDs, so each row is read into two L2s
    // and the two XCDs of a pair carry the same work; with fewer rows the
    // items stay in id order, spread over all the XCDs.  Slots past an XCD's
    // items return at once (select_grid sizes the grid for the fullest XCD).
    const uint32_t per_xcd = gridDim.x >> 3;
    const uint32_t nchunks = (uint32_t)((S + kChunk - 1) / kChunk);
    const uint32_t nunits = (uint32_t)(nb_total * Hkv);
    uint32_t item;
    if (seqlens && nunits >= 4u) {
        const uint32_t x = blockIdx.x & 7u, slot = blockIdx.x >> 3, par = x & 1u;
        const uint32_t per_row = (nchunks + 1u - par) >> 1;  // chunks par, par + 2, ... of a row
        if (per_row == 0u) return;
        const uint32_t m = slot / per_row, u = (x >> 1) + 4u * m;
        if (u >= nunits) return;
        item = u * nchunks + par + 2u * (slot - m * per_row);
    } else {
        item = seqlens ? blockIdx.x : (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
    }
    const uint32_t unit = item / nchunks;  // b * Hkv + g
    if (unit >= (uint32_t)(nb_total * Hkv)) return;  // uniform across the workgroup
    const int g = (int)(unit % (uint32_t)Hkv), b = (int)(unit / (uint32_t)Hkv);
    const int r0 = (int)(item - unit * nchunks) * kChunk;
    const int L = clamp_len(seqlens, b, S);
    const size_t base = ((size_t)b * Hkv + g) * S;
    const float *row = dt + base;
    const int rend = min(r0 + kChunk, S);
    const bool all_kept = WIN && win <= w;  // every window holds at most w keys
    const int lo = max(r0, w);    // first row holding more than w valid keys
    const int hi = min(rend, L);  // end of the valid rows of this chunk
    // With a sliding window (win >= C) the keys every valid row of the chunk
    // sees are [pl, r0); row i also sees the chunk's keys up to i and the
    // "leaving" keys [max(0, i - win + 1), pl), together at most C keys.
    const int pl = WIN ? min(r0, max(0, hi - win)) : 0;
    const int jl0 = WIN ? min(pl, max(0, lo - win + 1)) : 0;  // first leaving key
    // this thread's key of the chunk (C <= kThreads) and leaving key,
    // requested before the prefix work so that their latency is hidden there
    const float own = row[min(r0 + tid, S - 1)];
    const float lvk = WIN ? row[min(jl0 + tid, S - 1)] : 0.f;

    for (int t = tid; t < rend - r0; t += kThreads) {
        const int i = r0 + t;
        if (i >= L) {
            tau[base + i] = INFINITY;
            tie[base + i] = -1;
        } else if (i < w || all_kept) {
            tau[base + i] = -INFINITY;
            tie[base + i] = -1;
        }
    }
    if (lo >= hi || all_kept) return;  // uniform across the workgroup

    const int P = r0 - pl;  // prefix [pl, r0): all valid, as r0 < hi <= L
    row += pl;              // prefix positions below are relative to pl
    // a selection key with a prefix-relative index, made absolute (the order
    // of equal values is kept: both indices count from the same end)
    auto absolute = [&](uint64_t k) {
        return (k & 0xffffffff00000000ull) | (uint64_t)(~(uint32_t)(pl + (int)~(uint32_t)k));
    };
    const int A0 = max(0, min(P, w - kChunk - 1));
    const int nb = min(P, w) - A0;  // band size, 0 when the prefix is empty
    if (nb > 0) {
        const uint32_t rankA = (uint32_t)A0, rankB = (uint32_t)(A0 + nb - 1);
        // ---- a1: key range of the prefix.  A staged prefix is read whole
        // (into LDS).  A longer one takes its range from kSampleKeys keys in
        // blocks of 64 consecutive positions spread evenly over it; keys
        // outside that range go to the end bins, so the histogram is still a
        // monotone bucketing of the keys and the ranks it gives are exact.
        // Only when a rank of the band falls in a clamped end bin (which the
        // spread sample makes unlikely: the band sits w keys below the top)
        // does the collect step overflow and take the exact fallback.
        const bool staged = P <= STAGE;
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        if (staged) {
            for_prefix(row, P, [&](int j, float x) {
                const uint32_t k = ordkey(x);
                kmin = min(kmin, k);
                kmax = max(kmax, k);
                sh.keys[j] = k;
            });
        } else {
            static_assert(STAGE >= kSampleKeys, "a sampled prefix holds every sample block");
            constexpr int kBlocks = kSampleKeys / 64;
            float v[kSampleKeys / kThreads];
#pragma unroll
            for (int u = 0; u < kSampleKeys / kThreads; ++u) {
                const int x = tid + u * kThreads, blk = x >> 6;
                v[u] = row[(int)((int64_t)blk * (P - 64) / (kBlocks - 1)) + (x & 63)];
            }
#pragma unroll
            for (int u = 0; u < kSampleKeys / kThreads; ++u) {
                const uint32_t k = ordkey(v[u]);
                kmin = min(kmin, k);
                kmax = max(kmax, k);
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor(kmin, o, 64));
            kmax = max(kmax, (uint32_t)__shfl_xor(kmax, o, 64));
        }
        if (lane == 0) {
            sh.red[0][wave] = kmin;
            sh.red[1][wave] = kmax;
        }
        for (int x = tid; x < NB; x += kThreads) sh.hist[x] = 0u;
        if (tid == 0) {
            sh.ncol = 0u;
            sh.nfound = 0u;
        }
        __syncthreads();
        kmin = 0xffffffffu;
        kmax = 0u;
#pragma unroll
        for (int q = 0; q < kThreads / 64; ++q) {
            kmin = min(kmin, sh.red[0][q]);
            kmax = max(kmax, sh.red[1][q]);
        }
        const uint32_t range = kmax - kmin;
        const int bw = range == 0u ? 0 : 32 - __clz(range);
        constexpr int kLogBins = __builtin_ctz(NB);
        const int shift = bw > kLogBins ? bw - kLogBins : 0;
        // bin of a key: keys outside [kmin, kmax] (only a sampled range has
        // them) go to the end bins
        auto bin_of = [=](uint32_t k) -> uint32_t {
            return k < kmin ? 0u : min((k - kmin) >> shift, (uint32_t)(NB - 1));
        };
        // ---- a2: histogram, then the bins of ranks A0 and w-1 (descending)
        if (staged)
            for_staged(sh.keys, P, [&](int, uint32_t k) { atomicAdd(&sh.hist[(k - kmin) >> shift], 1u); });
        else
            for_prefix(row, P, [&](int, float x) { atomicAdd(&sh.hist[bin_of(ordkey(x))], 1u); });
        __syncthreads();
        {
            constexpr int PER = NB / kThreads;  // bins per thread, descending
            uint32_t c[PER], s = 0;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                c[q] = sh.hist[NB - 1 - (PER * tid + q)];
                s += c[q];
            }
            uint32_t incl = s;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o, 64);
                if (lane >= o) incl += y;
            }
            if (lane == 63) sh.red[0][wave] = incl;
            __syncthreads();
            uint32_t excl = incl - s;
            for (int q = 0; q < wave; ++q) excl += sh.red[0][q];
            uint32_t run = excl;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const uint32_t bin = (uint32_t)(NB - 1 - (PER * tid + q));
                if (run <= rankA && rankA < run + c[q]) {
                    sh.binA = bin;
                    sh.aboveA = run;
                }
                if (run <= rankB && rankB < run + c[q]) sh.binB = bin;
                run += c[q];
            }
        }
        __syncthreads();
        const uint32_t binA = sh.binA, binB = sh.binB, aboveA = sh.aboveA;
        // ---- a3: keys of bins [binB, binA] into LDS, ranked exactly
        auto collect = [&](int j, uint32_t k) {
            const uint32_t bin = bin_of(k);
            if (bin >= binB && bin <= binA) {
                const uint32_t at = atomicAdd(&sh.ncol, 1u);
                if (at < (uint32_t)kCollectCap) sh.col[at] = ((uint64_t)k << 32) | (uint64_t)(~(uint32_t)j);
            }
        };
        if (staged)
            for_staged(sh.keys, P, collect);
        else
            for_prefix(row, P, [&](int j, float x) { collect(j, ordkey(x)); });
        __syncthreads();
        const uint32_t m = sh.ncol;
        if (m <= (uint32_t)kCollectCap) {
            for (uint32_t x = tid; x < m; x += kThreads) {
                const uint64_t me = sh.col[x];
                uint32_t r = aboveA;
                for (uint32_t u = 0; u < m; ++u) r += sh.col[u] > me ? 1u : 0u;
                if (r >= rankA && r <= rankB) sh.cand[r - rankA] = absolute(me);
            }
        } else {
            // fallback: exact two-target radix select, then the keys between
            const uint32_t ranks[2] = {rankA, rankB};
            uint64_t keys[2];
            const int nt = nb > 1 ? 2 : 1;
            radix_select<kThreads>(row, P, nt, ranks, keys, sh.rs);
            const uint64_t khi = keys[0];
            const uint64_t klo = nt > 1 ? keys[1] : keys[0];
            for_prefix(row, P, [&](int j, float x) {
                const uint64_t k = selkey(x, (uint32_t)j);
                if (k <= khi && k >= klo) {
                    const uint32_t at = atomicAdd(&sh.nfound, 1u);
                    if (at < (uint32_t)kCollectCap) sh.col[at] = k;
                }
            });
            __syncthreads();
            const uint32_t f = min(sh.nfound, (uint32_t)kCollectCap);  // == nb
            for (uint32_t x = tid; x < f; x += kThreads) {
                const uint64_t me = sh.col[x];
                uint32_t r = 0;
                for (uint32_t u = 0; u < f; ++u) r += sh.col[u] > me ? 1u : 0u;
                if (r < (uint32_t)nb) sh.cand[r] = absolute(me);
            }
        }
    }
    row -= pl;
    // the chunk's own keys after the band, then the leaving keys
    const int nnew = hi - r0;
    const int nleave = pl - jl0;  // < C
    if (tid < nnew) sh.cand[nb + tid] = selkey(own, (uint32_t)(r0 + tid));
    if (WIN && tid < nleave) sh.cand[nb + nnew + tid] = selkey(lvk, (uint32_t)(jl0 + tid));
    __syncthreads();

    // ---- b: each candidate finds the rows it is the threshold of.  The
    // chunk's new keys sit one per lane (rows t = lane and t = lane + 64), so
    // "new keys of rows <= t better than the candidate" is a ballot and a
    // masked bit count per lane.  Band keys are distinct and held by rank, so
    // the band ballots count x keys above the band key of rank x, and its
    // position lies before the chunk: one formula serves both kinds.  A wave
    // takes kUnrollB candidates per step with no branch between them, so
    // their dependency chains overlap; each lane keeps the position found for
    // its rows in registers and stores the pair once at the end.
    constexpr int kWaves = kThreads / 64;
    constexpr int kUnrollB = 4;
    const int need = w - A0 - 1;  // better candidates a row's w-th key has
    const int ncand = nb + nnew + nleave;
    const uint64_t nk0 = lane < nnew ? sh.cand[nb + lane] : 0ull;  // 0: below every key
    const uint64_t nk1 = (C > 64 && lane + 64 < nnew) ? sh.cand[nb + 64 + lane] : 0ull;
    // leaving key jl0 + x in lane x (of two registers); row i sees those from
    // position i - win + 1 on, i.e. from lane s = i - win + 1 - jl0
    const uint64_t lk0 = WIN && lane < nleave ? sh.cand[nb + nnew + lane] : 0ull;
    const uint64_t lk1 = (WIN && C > 64 && lane + 64 < nleave) ? sh.cand[nb + nnew + 64 + lane] : 0ull;
    uint64_t bk[(C + 1 + 63) / 64];  // the band holds at most C + 1 keys
#pragma unroll
    for (int q = 0; q < (int)(sizeof(bk) / sizeof(bk[0])); ++q)
        bk[q] = 64 * q + lane < nb ? sh.cand[64 * q + lane] : 0ull;
    const int t0 = lane, t1 = lane + 64;  // this lane's rows (chunk offsets)
    const bool v0 = r0 + t0 >= lo && r0 + t0 < hi;
    const bool v1 = C > 64 && r0 + t1 >= lo && r0 + t1 < hi;
    // first position each row sees (0 without a window), and its first
    // leaving lane
    const int f0 = WIN ? max(0, r0 + t0 - win + 1) : 0, f1 = WIN ? max(0, r0 + t1 - win + 1) : 0;
    const int s0 = max(0, f0 - jl0), s1 = max(0, f1 - jl0);
    // set bits of the 128-bit mask (hi:lo) at positions >= s
    auto count_from = [](uint64_t lo64, uint64_t hi64, int s) {
        return s >= 128 ? 0 : s >= 64 ? __popcll(hi64 >> (s - 64)) : __popcll(lo64 >> s) + __popcll(hi64);
    };
    int h0 = -1, h1 = -1;  // threshold position of rows t0, t1 if this wave has it
    uint32_t o0 = 0, o1 = 0;  // and its dt order bits
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    for (int xb = wv; xb < ncand; xb += kWaves * kUnrollB) {
        uint64_t kx[kUnrollB];
#pragma unroll
        for (int u = 0; u < kUnrollB; ++u) {
            // past the end the read repeats the last candidate, whose second
            // pass sets the same positions again
            kx[u] = sh.cand[min(xb + kWaves * u, ncand - 1)];
        }
#pragma unroll
        for (int u = 0; u < kUnrollB; ++u) {
            const int jx = (int)selkey_idx(kx[u]);
            int better = 0;
#pragma unroll
            for (int q = 0; q < (int)(sizeof(bk) / sizeof(bk[0])); ++q) better += __popcll(__ballot(bk[q] > kx[u]));
            const int need_x = need - better;  // better new keys the row must see
            const uint64_t m0 = __ballot(nk0 > kx[u]);
            const uint64_t m1 = C > 64 ? __ballot(nk1 > kx[u]) : 0ull;
            // set bits of m at lanes 0..lane: those of m >> 1 below the lane,
            // plus bit 0
            const int c0 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m0 >> 33),
                                 __builtin_amdgcn_mbcnt_lo((uint32_t)(m0 >> 1), 0u)) + (int)(m0 & 1);
            int c1 = C > 64 ? __popcll(m0) + (int)(m1 & 1) +
                                  (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m1 >> 33),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)(m1 >> 1), 0u))
                            : 0;
            int cl0 = 0;
            if (WIN && nleave > 0) {  // uniform
                const uint64_t l0 = __ballot(lk0 > kx[u]);
                const uint64_t l1 = C > 64 ? __ballot(lk1 > kx[u]) : 0ull;
                cl0 = count_from(l0, l1, s0);
                if (C > 64) c1 += count_from(l0, l1, s1);
            }
            // the candidate is visible to rows at or after its own position
            // (and, with a window, to those whose window still holds it)
            const bool g0 = v0 & (c0 + cl0 == need_x) & (r0 + t0 >= jx) & (jx >= f0);
            h0 = g0 ? jx : h0;
            o0 = g0 ? (uint32_t)(kx[u] >> 32) : o0;
            if (C > 64) {
                const bool g1 = v1 & (c1 == need_x) & (r0 + t1 >= jx) & (jx >= f1);
                h1 = g1 ? jx : h1;
                o1 = g1 ? (uint32_t)(kx[u] >> 32) : o1;
            }
        }
    }
    // every row in [lo, hi) has exactly one threshold, found by one wave;
    // its value comes back from the order bits (only a zero, whose sign the
    // order folds, is read again)
    if (h0 >= 0) {
        tau[base + r0 + t0] = o0 == 0x80000000u ? row[h0] : order_value(o0);
        tie[base + r0 + t0] = h0;
    }
    if (C > 64 && h1 >= 0) {
        tau[base + r0 + t1] = o1 == 0x80000000u ? row[h1] : order_value(o1);
        tie[base + r0 + t1] = h1;
    }
}

}  // namespace

// The 1-D grid of select_kernel, a multiple of 8 (one share per XCD): at
// least nchunks * Hkv * B workgroups, and with seqlens and four or more rows
// the fullest XCD's share (ceil(rows / 4) rows of ceil(nchunks / 2) chunks).
// 0 when it would not fit a grid dimension.
static unsigned select_grid(int nchunks, int Hkv, int B, bool pairs) {
    const int64_t units = (int64_t)Hkv * B;
    const int64_t per_xcd = pairs && units >= 4 ? ((units + 3) / 4) * ((nchunks + 1) / 2)
                                                 : (units * nchunks + 7) / 8;
    return 8 * per_xcd > 0x7fffffff ? 0u : (unsigned)(8 * per_xcd);
}

hipError_t launch_select(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, int win,
                         float *tau, int32_t *tie, hipStream_t stream) {
    // Full causal range: chunks of 32 rows for rows up to 4096 keys, staged
    // whole in LDS (more, shorter workgroups: 7 % faster at S = 2048 than 64
    // rows), chunks of 64 rows with 1024-key staging beyond (the prefix passes
    // then dominate, and 32-row chunks would double them), 128 rows past
    // 16384 keys (half the prefix passes again: 55.0 -> 51.5 us at the
    // padded size).  Sliding window: short windows take 64-row chunks,
    // longer rows and windows 128-row chunks (a window needs win >= C).
#define DMA_SEL(C, NB, STAGE, WIN)                                                                                \
    do {                                                                                                          \
        const unsigned grid = select_grid((S + C - 1) / C, Hkv, B, seqlens != nullptr);                           \
        if (grid == 0u) return hipErrorInvalidValue;                                                              \
        hipLaunchKernelGGL((select_kernel<C, NB, STAGE, WIN>), dim3(grid), dim3(kThreads), 0, stream, dt, seqlens, \
                           Hkv, S, w, win, B, tau, tie);                                                          \
    } while (0)
    if (win > 0) {
        if (S <= 4096 || win < 128) DMA_SEL(64, 1024, 8192, true);
        else DMA_SEL(128, 4096, 8192, true);
    } else {
        if (S <= 4096) DMA_SEL(32, 1024, 4096, false);
        else if (S <= 16384) DMA_SEL(64, 1024, 1024, false);
        else DMA_SEL(128, 1024, 1024, false);
    }
#undef DMA_SEL
    return hipGetLastError();
}

}  // namespace dma
