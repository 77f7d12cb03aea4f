// Exact order-statistic selection over one row of dt values, done by a whole
// workgroup: find the key of descending rank r (0 = best) among positions
// [0, P) under the selection order "larger dt first, lower index first".
//
// MSB-first radix select on the 64-bit selection key (ordkey(dt) << 32 | ~j):
// four 8-bit passes over the dt word, each an LDS histogram of the elements
// that still match the chosen prefix, then -- only when the chosen dt value is
// shared by several positions and the rank inside that tie is not the first --
// 8-bit passes over the index bits.  Up to two target ranks are resolved in
// the same passes (one read of the row per pass); while both targets share a
// prefix they share a histogram.
#pragma once

#include "common.hpp"

namespace dma {

template <int NT>
struct RadixShared {
    static constexpr int NW = NT / 64;
    uint32_t hist[2][NW][256];
    uint32_t minidx[2][256];
    uint32_t res_digit[2], res_above[2], res_cnt[2], res_min[2];
};

// One histogram pass.  word 1 = dt order key, word 0 = complemented index.
template <int NT>
__device__ __forceinline__ void radix_pass(const float *__restrict__ row, int P, int nt, bool same,
                                           int word, int shift, uint32_t hmask,
                                           const uint32_t *hval, uint32_t lmask,
                                           const uint32_t *lval, RadixShared<NT> &sh) {
    const int tid = threadIdx.x, wave = tid >> 6;
    for (int x = tid; x < 2 * RadixShared<NT>::NW * 256; x += NT) (&sh.hist[0][0][0])[x] = 0u;
    for (int x = tid; x < 2 * 256; x += NT) (&sh.minidx[0][0])[x] = 0xffffffffu;
    __syncthreads();
    const int ntl = (nt == 2 && !same) ? 2 : 1;
    // the minimum index per bin is only read after the last dt digit
    const bool track_min = (word == 1 && shift == 0);
    for (int j = tid; j < P; j += NT) {
        const uint32_t hi = ordkey(row[j]);
        const uint32_t lo = ~(uint32_t)j;
        const uint32_t dg = ((word ? hi : lo) >> shift) & 255u;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (t < ntl && (hi & hmask) == hval[t] && (lo & lmask) == lval[t]) {
                atomicAdd(&sh.hist[t][wave][dg], 1u);
                if (track_min) atomicMin(&sh.minidx[t][dg], (uint32_t)j);
            }
        }
    }
    __syncthreads();
}

// Wave `t` finds the digit of target t: the bin holding descending rank rr.
template <int NT>
__device__ __forceinline__ void radix_find_digit(int t, bool same, uint32_t rr, RadixShared<NT> &sh) {
    const int lane = threadIdx.x & 63;
    const int src = (t == 1 && same) ? 0 : t;
    uint32_t c[4];
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int bin = 255 - (4 * lane + k);
        uint32_t v = 0;
#pragma unroll
        for (int w = 0; w < RadixShared<NT>::NW; ++w) v += sh.hist[src][w][bin];
        c[k] = v;
        s += v;
    }
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    const uint32_t excl = incl - s;
    if (excl <= rr && rr < incl) {
        uint32_t run = excl;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (rr < run + c[k]) {
                const int bin = 255 - (4 * lane + k);
                sh.res_digit[t] = (uint32_t)bin;
                sh.res_above[t] = run;
                sh.res_cnt[t] = c[k];
                sh.res_min[t] = sh.minidx[src][bin];
                break;
            }
            run += c[k];
        }
    }
}

// Select up to two descending ranks (ranks[0] <= ranks[1] < P) among row[0..P).
// Must be called by all NT threads of the workgroup with uniform arguments.
// Returns the 64-bit selection keys in keys[0..nt).
template <int NT>
__device__ void radix_select(const float *__restrict__ row, int P, int nt, const uint32_t *ranks,
                             uint64_t *keys, RadixShared<NT> &sh) {
    static_assert(NT >= 128, "two targets need two waves");
    const int wave = threadIdx.x >> 6;
    uint32_t hval[2] = {0u, 0u}, lval[2] = {0u, 0u};
    uint32_t rrem[2] = {ranks[0], nt > 1 ? ranks[1] : 0u};
    uint32_t minj[2] = {0u, 0u};
    uint32_t hmask = 0u, lmask = 0u;
    bool same = true;

    // dt word, four 8-bit digits
    for (int shift = 24; shift >= 0; shift -= 8) {
        radix_pass<NT>(row, P, nt, same, 1, shift, hmask, hval, lmask, lval, sh);
        if (wave < nt) radix_find_digit<NT>(wave, same, wave == 0 ? rrem[0] : rrem[1], sh);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (t < nt) {
                hval[t] |= sh.res_digit[t] << shift;
                rrem[t] -= sh.res_above[t];
                minj[t] = sh.res_min[t];
            }
        }
        hmask |= 255u << shift;
        same = (nt == 1) || (hval[0] == hval[1]);
        __syncthreads();
    }

    // ties on the dt value: rank rrem inside the tie, by ascending index
    const bool need = (rrem[0] != 0u) || (nt > 1 && rrem[1] != 0u);
    if (need) {
        const uint32_t top = (P > 1) ? 32u - (uint32_t)__clz((unsigned)(P - 1)) : 1u;
        const int first = (int)(((top + 7u) / 8u) * 8u) - 8;
        // bits of ~j above `top` are all ones for every j < P
        lmask = (top >= 32u) ? 0u : ~((1u << top) - 1u);
        lval[0] = lval[1] = lmask;
        same = (nt == 1) || (hval[0] == hval[1]);
        for (int shift = first; shift >= 0; shift -= 8) {
            radix_pass<NT>(row, P, nt, same, 0, shift, hmask, hval, lmask, lval, sh);
            if (wave < nt) radix_find_digit<NT>(wave, same, wave == 0 ? rrem[0] : rrem[1], sh);
            __syncthreads();
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (t < nt) {
                    lval[t] |= sh.res_digit[t] << shift;
                    rrem[t] -= sh.res_above[t];
                }
            }
            lmask |= 255u << shift;
            same = (nt == 1) || (hval[0] == hval[1] && lval[0] == lval[1]);
            __syncthreads();
        }
        minj[0] = ~lval[0];
        minj[1] = ~lval[1];
    }
    keys[0] = ((uint64_t)hval[0] << 32) | (uint64_t)(~minj[0]);
    if (nt > 1) keys[1] = ((uint64_t)hval[1] << 32) | (uint64_t)(~minj[1]);
}

}  // namespace dma
