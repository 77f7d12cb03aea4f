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
//       the best w-C-1 prefix keys are kept by every row of the chunk and are
//       never its w-th key, prefix keys of rank >= w are kept by none, and
//       each row's threshold key lies in the "band" of prefix ranks
//       [w-C-1, w) plus the chunk's own keys: at most 2C+1 keys.
// One workgroup per (batch, kv head, chunk of 64 rows) finds the two band
// limits with a two-target radix select over the prefix, gathers the band and
// the chunk's keys into LDS, sorts them, and lets each row walk the sorted
// list to its threshold.  Output per row: (tau, tie) = (dt, index) of the
// w-th kept key, or the canonical (-inf, -1) / (+inf, -1).
#include "common.hpp"
#include "launch.hpp"
#include "radix_select.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;
constexpr int kBand = kChunk + 1;  // band width: prefix ranks [w - kChunk - 1, w)
constexpr int kSortN = 256;        // power of two >= kBand + kChunk

__global__ __launch_bounds__(kThreads) void select_kernel(const float *__restrict__ dt,
                                                          const int32_t *__restrict__ seqlens,
                                                          int Hkv, int S, int w,
                                                          float *__restrict__ tau,
                                                          int32_t *__restrict__ tie) {
    __shared__ RadixShared<kThreads> rs;
    __shared__ uint64_t cand[kSortN];
    __shared__ int ncand;

    const int tid = threadIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    const int r0 = blockIdx.x * kChunk;
    const int L = seqlens ? seqlens[b] : S;
    const size_t base = ((size_t)b * Hkv + g) * S;
    const float *row = dt + base;
    const int rend = min(r0 + kChunk, S);
    const int lo = max(r0, w);       // first row holding more than w valid keys
    const int hi = min(rend, L);     // end of the valid rows of this chunk

    for (int t = tid; t < rend - r0; t += kThreads) {
        const int i = r0 + t;
        if (i >= L) {
            tau[base + i] = INFINITY;
            tie[base + i] = -1;
        } else if (i < w) {
            tau[base + i] = -INFINITY;
            tie[base + i] = -1;
        }
    }
    if (lo >= hi) return;  // uniform across the workgroup

    const int P = r0;  // prefix [0, r0): all valid, as r0 < hi <= L
    const int A0 = max(0, min(P, w - kChunk - 1));
    const int nb = min(P, w) - A0;
    if (tid == 0) ncand = 0;
    __syncthreads();
    if (nb > 0) {
        const uint32_t ranks[2] = {(uint32_t)A0, (uint32_t)(A0 + nb - 1)};
        uint64_t keys[2];
        const int nt = nb > 1 ? 2 : 1;
        radix_select<kThreads>(row, P, nt, ranks, keys, rs);
        const uint64_t khi = keys[0];
        const uint64_t klo = nt > 1 ? keys[1] : keys[0];
        for (int j = tid; j < P; j += kThreads) {
            const uint64_t k = selkey(row[j], (uint32_t)j);
            if (k <= khi && k >= klo) {
                const int at = atomicAdd(&ncand, 1);
                if (at < kBand) cand[at] = k;  // exactly nb <= kBand keys match
            }
        }
    }
    __syncthreads();
    const int nband = min(ncand, kBand);
    const int nnew = hi - r0;
    for (int t = tid; t < kSortN; t += kThreads) {
        if (t >= nband && t < nband + nnew) {
            const int j = r0 + (t - nband);
            cand[t] = selkey(row[j], (uint32_t)j);
        } else if (t >= nband + nnew) {
            cand[t] = 0ull;  // sorts last; never counted (see below)
        }
    }
    __syncthreads();
    // bitonic sort, descending
    for (int k = 2; k <= kSortN; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            if (tid < kSortN / 2) {
                const int i = (tid / jj) * 2 * jj + (tid % jj);
                const int p = i + jj;
                const uint64_t a = cand[i], c = cand[p];
                const bool desc = (i & k) == 0;
                if (desc ? (a < c) : (a > c)) {
                    cand[i] = c;
                    cand[p] = a;
                }
            }
            __syncthreads();
        }
    }
    const int total = nband + nnew;
    for (int t = tid; t < kChunk; t += kThreads) {
        const int i = r0 + t;
        if (i < lo || i >= hi) continue;
        const int need = w - A0;  // rank of the threshold inside band + new keys
        int cnt = 0;
        for (int e = 0; e < total; ++e) {
            const uint32_t j = selkey_idx(cand[e]);
            if ((int)j <= i && ++cnt == need) {
                tau[base + i] = row[j];
                tie[base + i] = (int32_t)j;
                break;
            }
        }
    }
}

}  // namespace

hipError_t launch_select(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w,
                         float *tau, int32_t *tie, hipStream_t stream) {
    const dim3 grid((S + kChunk - 1) / kChunk, Hkv, B);
    hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), 0, stream, dt, seqlens, Hkv, S, w, tau,
                       tie);
    return hipGetLastError();
}

}  // namespace dma
