// Backward of the prefill attention under the dynamic top-w mask.
// Doge guide (gitcode), DMA section, forward steps 3 and 4: training runs the
// same masked attention, s_ij = d^-0.5 q_i.k_j + dt_j over the kept keys j of
// row i, p = softmax(s), o_i = sum_j p_ij v_j, and learns end to end through
// dt what to mask.  The kept sets are the forward's (the top-w selection is
// piecewise constant in dt); with dp_ij = dO_i.v_j and D_i = dO_i.o_i =
// sum_j p_ij dp_ij:
//   ds_ij = p_ij (dp_ij - D_i)
//   dq_i = c sum_j ds_ij k_j,  dk_j = c sum_i ds_ij q_i,  dv_j = sum_i p_ij dO_i,
//   ddt_j = sum_i ds_ij        (c = d^-0.5; sums over rows and query heads).
//
// Two kernels, neither with atomics, so every result is deterministic.
//
// Query side (attn_bwd_q_kernel): one workgroup per (batch, kv head, tile of
// 128 / G query rows), its eight waves holding 16 (row, head) pairs each, one
// pair per lane column.  Only candidate keys are walked: by nesting, those
// kept by row i0 (the tile's first row) and the tile's own keys, about
// w + 128/G of them, compacted into an LDS list (the causal range when they
// overflow it).  Key blocks of 64 candidates are gathered into LDS and every
// kept test is evaluated (key j is kept by row i when j <= i < L and
// selkey(dt_j, j) >= selkey(tau_i, tie_i)).  Pass 1 finds
// each pair's log-sum-exp; pass 2 recomputes the scores and forms dS^T and
// dQ^T += K^T dS^T.  D_i is accumulated in pass 1 as sum_j p_ij dp_ij (with
// the same online rescaling as the softmax sum), in float32 from the very
// weights the gradients use, rather than from a rounded output: the dt
// gradient of a key kept with weight near 1 by many rows is a sum of nearly
// cancelling terms, and an output rounded to bf16 would leave its rounding in
// every one of them.  It also writes each pair's log-sum-exp and D_i for the
// key side.
//
// Key side (attn_bwd_kv_kernel): one workgroup per (batch, kv head, tile of
// 16 KW keys), NG row groups of KW waves (three groups of four at d = 64; one
// group of eight at d = 128, so each staged row block serves 128 keys: long
// backward 1.37 -> 1.26 ms); every wave holds 16 keys, one key per lane
// column, with their K and V rows as MFMA operands in registers.  By nesting
// the rows that keep key j form a run [j, e_j), and the thresholds grow with
// the row, so the workgroup walks row blocks of 64 pairs from its first key
// on (the groups take the blocks in turn) and stops at the first row whose
// threshold passes all of its keys.  The tile's keys are ordered by selection
// key into rank blocks of 16 (a wave whose keys have all dropped out skips
// the block), each row group holding the blocks on rotated waves so that the
// long-lived ones run on different SIMDs.  Per block each lane finds its
// key's run of rows (two threshold compares, a binary search in the block
// where the key drops out), so the element test is one unsigned compare.
// dV^T += dO^T P and dK^T += Q^T dS accumulate in registers, ddt is the
// column sum of dS; the other groups hand their sums to the first through
// LDS, in group order (in passes of as many rank blocks as the free row
// tiles hold).
//
// The key side touches every (pair, key) of the row range it walks, not only
// the kept ones: its work grows like the dense causal attention rather than
// like the kept count.
//
// Layout facts of v_mfma_f32_16x16x32_bf16 (l = lane, q = l / 16):
//   A[m = l%16][k = 8q + j], B[k = 8q + j][n = l%16], C[m = 4q + i][n = l%16].
// A product over a 32-long k range whose operand comes from accumulators uses
// the k-slot order (q, j) -> 16 (j / 4) + 4q + j % 4: then the B operand of
// lane l is exactly the four values of each of two 16-row accumulator tiles
// that lane l holds, and the A operand is two LDS transpose reads of four rows
// each.
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kPairs = 64;   // (row, head) pairs per query tile and per row block
constexpr int kBlk = 64;     // keys per block on the query side
constexpr int kCandCap = 3072;  // candidate keys of a query tile held in LDS
// The query side runs eight waves of 16 pairs (128 pairs a tile): each
// gathered key block in LDS serves twice the pairs of four waves, and half
// as many tiles scan the prefix for candidates (c2 backward 139 -> 132 us).
constexpr int kQThreads = 512;
constexpr int kQPairs = kQThreads / 4;
constexpr int kQScanKeys = 4 * kQThreads;  // prefix keys classified per scan step

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4 lds_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS row pitch (bf16 elements) of every staged tile: a 16- or 48-word step
// between rows, so that row reads and transpose reads spread over the banks.
template <int D> constexpr int pitch() { return D + 32; }

// A operand of a product over the 32 rows base .. base+31 of the row-major
// LDS tile T (pitch P), column c0 + l%16, in the permuted k-slot order.
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the four 16-bit values at the addresses of lanes i/4 + 4s (s = 0..3);
// with lane k of group q pointing at row r0 + k/4, column c0 + 4 (k%4), lane i
// gets column c0 + i of rows r0 .. r0+3.
template <int P>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *T, int base, int c0, int lane) {
    const int q = lane >> 4, k = lane & 15;
    const uint16_t *p = T + (base + 4 * q + (k >> 2)) * P + c0 + 4 * (k & 3);
    const i16x4 lo = lds_tr16(p);
    const i16x4 hi = lds_tr16(p + 16 * P);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B operand in the same permuted order from two accumulator tiles.
__device__ __forceinline__ bf16x8 acc_operand(const f32x4 &lo, const f32x4 &hi) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b[i] = (__bf16)lo[i];
        b[4 + i] = (__bf16)hi[i];
    }
    return b;
}

// eight bf16 at p (16-byte aligned), from global memory or LDS
__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// ---------------------------------------------------------------- query side
template <int D>
__global__ __launch_bounds__(kQThreads, D == 64 ? 2 : 1) void attn_bwd_q_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, const uint16_t *__restrict__ dO, int S, int Hq, int Hkv, int G, int ntq,
    float qscale, float c, uint16_t *__restrict__ dQ, float *__restrict__ lse_ws,
    float *__restrict__ dd_ws) {
    constexpr int P = pitch<D>();
    constexpr int NS = D / 32;          // k-steps of 32 over head_dim
    constexpr int NV = kBlk * D / 8 / kQThreads;  // 16-byte vectors per thread per tile
    __shared__ __align__(16) uint16_t Ks[kBlk * P];
    __shared__ __align__(16) uint16_t Vs[kBlk * P];
    __shared__ float dtl_s[kBlk];
    __shared__ uint64_t skey_s[kBlk];
    __shared__ int jk_s[kBlk];
    __shared__ int c_idx[kCandCap];
    __shared__ uint32_t wcnt[kQThreads / 64];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, pq = lane & 15;
    // Work item = (batch, kv head, query tile).  Workgroup ids go round-robin
    // over the 8 XCDs: hand each XCD a contiguous run of items, so that the
    // tiles of one (batch, kv head), which all read the same K and V rows,
    // share that XCD's L2; within a run the tiles with the most keys first.
    const int nwg = gridDim.x, per_xcd = nwg >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int item = (slot < per_xcd && (nwg & 7) == 0) ? xcd * per_xcd + slot : blockIdx.x;
    const int tq = ntq - 1 - item % ntq;
    const int g = (item / ntq) % Hkv;
    const int b = item / (ntq * Hkv);
    const int L = clamp_len(seqlens, b, S);
    const int RB = kQPairs / G;
    const int i0 = tq * RB;
    const int pr = 16 * wave + pq;      // this lane's pair
    const int i = i0 + pr / G, hq = g * G + pr % G;
    const bool live = i < L;
    const int ic = min(i, S - 1);
    const size_t qrow = (((size_t)b * S + ic) * Hq + hq) * D;
    const size_t urow = ((size_t)b * Hkv + g) * S;

    if (i0 >= L) {  // every row of the tile is padding (uniform)
        if (i < S) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t)
                *reinterpret_cast<uint2 *>(dQ + qrow + 16 * t + 4 * q) = make_uint2(0, 0);
            if (q == 0) {
                lse_ws[((size_t)b * Hq + hq) * S + i] = 0.f;
                dd_ws[((size_t)b * Hq + hq) * S + i] = 0.f;
            }
        }
        return;
    }
    const int kmax = min(i0 + RB, L) - 1;  // last key any row of the tile can keep
    const uint64_t thr = live ? selkey(tau[urow + i], (uint32_t)tie[urow + i]) : ~0ull;

    // Q and dO of this lane's pair (elements 32s + 8q .. +7)
    bf16x8 qf[NS], of[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        qf[s] = ld8(Q + qrow + 32 * s + 8 * q);
        of[s] = ld8(dO + qrow + 32 * s + 8 * q);
    }

    const uint32_t kvs = (uint32_t)(Hkv * D);
    const uint16_t *Kb = K + (size_t)b * S * kvs + (size_t)g * D;
    const uint16_t *Vb = V + (size_t)b * S * kvs + (size_t)g * D;
    const float *drow = dt + urow;

    // ---- candidate keys.  By nesting, a key j <= i0 that some row of the
    // tile keeps is kept by row i0, and the keys (i0, kmax] are the tile's
    // own: only those are walked, about w + 64/G keys instead of the causal
    // range.  They are compacted into LDS in two classes: "full" keys, kept
    // by every row of the tile (a key j <= i0 kept by the last row kmax, as
    // thresholds grow with the row), from the front, and the rest from the
    // back (each class in index order within a scan step's wave and register;
    // the order changes only the summation order).  Blocks of full keys need
    // no kept test.  Past kCandCap candidates the whole causal range is
    // walked instead.
    int n, nF;
    {
        const uint64_t thr0 = selkey(tau[urow + i0], (uint32_t)tie[urow + i0]);
        const uint64_t thrl = selkey(tau[urow + kmax], (uint32_t)tie[urow + kmax]);
        const uint64_t lt_mask = (1ull << lane) - 1ull;
        int baseF = 0, baseP = 0;
        for (int c0 = 0; c0 <= i0; c0 += kQScanKeys) {
            float dv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) dv[e] = drow[min(c0 + tid + kQThreads * e, i0)];
            bool pf[4], pp[4];
            uint32_t nfw = 0, npw = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = c0 + tid + kQThreads * e;
                const uint64_t sk = selkey(dv[e], (uint32_t)j);
                const bool cand = j <= i0 && sk >= thr0;
                pf[e] = cand && sk >= thrl;
                pp[e] = cand && !pf[e];
                nfw += (uint32_t)__popcll(__ballot(pf[e]));
                npw += (uint32_t)__popcll(__ballot(pp[e]));
            }
            if (lane == 0) wcnt[wave] = nfw | (npw << 16);  // at most 1024 each
            __syncthreads();
            int offF = baseF, offP = baseP, totF = 0, totP = 0;
#pragma unroll
            for (int w2 = 0; w2 < kQThreads / 64; ++w2) {
                const int cf = (int)(wcnt[w2] & 0xffffu), cp = (int)(wcnt[w2] >> 16);
                offF += w2 < wave ? cf : 0;
                offP += w2 < wave ? cp : 0;
                totF += cf;
                totP += cp;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = c0 + tid + kQThreads * e;
                const uint64_t bf = __ballot(pf[e]), bp = __ballot(pp[e]);
                const int posF = offF + (int)__popcll(bf & lt_mask);
                const int posP = offP + (int)__popcll(bp & lt_mask);
                if (pf[e] && posF < kCandCap) c_idx[posF] = j;
                if (pp[e] && posP < kCandCap) c_idx[kCandCap - 1 - posP] = j;
                offF += (int)__popcll(bf);
                offP += (int)__popcll(bp);
            }
            baseF += totF;
            baseP += totP;
            __syncthreads();  // wcnt is rewritten by the next step
        }
        for (int x = tid; x < kmax - i0; x += kQThreads)
            if (baseP + x < kCandCap) c_idx[kCandCap - 1 - (baseP + x)] = i0 + 1 + x;
        nF = baseF;
        n = baseF + baseP + (kmax - i0);
    }
    const bool gathered = n <= kCandCap;  // then the two classes do not overlap
    if (!gathered) {
        n = kmax + 1;
        nF = 0;
    }
    __syncthreads();  // c_idx visible

    // key at list position x (x < n)
    auto key_at = [&](int x) __attribute__((always_inline)) {
        return gathered ? c_idx[x < nF ? x : kCandCap - 1 - (x - nF)] : x;
    };
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
            const int v = tid + u * kQThreads;
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
            const int v = tid + u * kQThreads;
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
    // base-2 scores of the block's 64 keys against this lane's pair and
    // dp = dO . v: z[mt][r] and dp[mt][r] are key 16 mt + 4 q + r, z = -inf
    // where not kept; a block of full keys (full) is kept by every row of
    // the tile, so only the rows past the length need masking, which the
    // caller does
    auto scores = [&](bool full, float (&z)[4][4], f32x4 (&dp)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                sacc = mfma16(ld8(&Ks[(16 * mt + pq) * P + 32 * s + 8 * q]), qf[s], sacc);
                dp[mt] = mfma16(ld8(&Vs[(16 * mt + pq) * P + 32 * s + 8 * q]), of[s], dp[mt]);
            }
            const float4 d4 = *reinterpret_cast<const float4 *>(&dtl_s[16 * mt + 4 * q]);
            const float dls[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) z[mt][r] = fmaf(sacc[r], qscale, dls[r]);
        }
        if (!full) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kk = 16 * mt + 4 * q + r;
                    const bool kept = live & (jk_s[kk] <= i) & (skey_s[kk] >= thr);
                    z[mt][r] = kept ? z[mt][r] : -INFINITY;
                }
            }
        }
    };

    // ---- pass 1: log-sum-exp (base 2) of each pair over its kept keys, and
    // D = sum_j p_j dp_j, both with the online rescaling
    float m = -INFINITY, l = 0.f, u = 0.f;
    fetch(0);
    for (int x0 = 0; x0 < n; x0 += kBlk) {
        put(x0);
        __syncthreads();
        fetch(x0 + kBlk < n ? x0 + kBlk : 0);  // the next block, or pass 2's first
        float z[4][4];
        f32x4 dp[4];
        // wave priority 3 while forming scores, 1 for the gradient products,
        // 0 in the vector work between them (the waves of a SIMD then
        // interleave their phases)
        __builtin_amdgcn_s_setprio(3);
        scores(x0 + kBlk <= nF, z, dp);  // rows past the length: results unused
        __builtin_amdgcn_s_setprio(0);
        float mb = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mb = fmaxf(mb, z[mt][r]);
        if (mb > m) {
            const float a = __builtin_amdgcn_exp2f(m - mb);  // 0 when m = -inf
            l *= a;
            u *= a;
            m = mb;
        }
        if (m > -INFINITY) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = __builtin_amdgcn_exp2f(z[mt][r] - m);
                    l += e;
                    u = fmaf(e, dp[mt][r], u);
                }
        }
        __syncthreads();
    }
    float dd;
    {
        float mo = fmaxf(m, __shfl_xor(m, 16, 64));
        mo = fmaxf(mo, __shfl_xor(mo, 32, 64));
        const float a = m > -INFINITY ? __builtin_amdgcn_exp2f(m - mo) : 0.f;
        float lo = l * a, uo = u * a;
        lo += __shfl_xor(lo, 16, 64);
        lo += __shfl_xor(lo, 32, 64);
        uo += __shfl_xor(uo, 16, 64);
        uo += __shfl_xor(uo, 32, 64);
        m = mo;
        l = lo;
        dd = live ? uo / lo : 0.f;
    }
    const float lse2 = live ? m + log2f(l) : 0.f;
    const float lse_p = live ? lse2 : INFINITY;  // p = 0 for rows past the length

    // ---- pass 2: dS^T and dQ^T += K^T dS^T
    f32x4 dq[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) dq[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int x0 = 0; x0 < n; x0 += kBlk) {
        put(x0);
        __syncthreads();
        if (x0 + kBlk < n) fetch(x0 + kBlk);
        float z[4][4];
        f32x4 dp[4], ds[4];
        __builtin_amdgcn_s_setprio(3);
        scores(x0 + kBlk <= nF, z, dp);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(z[mt][r] - lse_p);  // 0 where not kept
                ds[mt][r] = p * (dp[mt][r] - dd);
            }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8 bop = acc_operand(ds[2 * s2], ds[2 * s2 + 1]);
#pragma unroll
            for (int t = 0; t < D / 16; ++t) dq[t] = mfma16(tr_operand<P>(Ks, 32 * s2, 16 * t, lane), bop, dq[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    }

    if (i < S) {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const uint32_t w0 = (uint32_t)f32_to_bf16(dq[t][0] * c) | ((uint32_t)f32_to_bf16(dq[t][1] * c) << 16);
            const uint32_t w1 = (uint32_t)f32_to_bf16(dq[t][2] * c) | ((uint32_t)f32_to_bf16(dq[t][3] * c) << 16);
            *reinterpret_cast<uint2 *>(dQ + qrow + 16 * t + 4 * q) = make_uint2(w0, w1);
        }
        if (q == 0) {
            lse_ws[((size_t)b * Hq + hq) * S + i] = lse2;
            dd_ws[((size_t)b * Hq + hq) * S + i] = dd;
        }
    }
}

// ------------------------------------------------------------------ key side
// NG row groups of KW waves (64 KW threads each)
template <int D, int NG, int KW>
__global__ __launch_bounds__(NG * KW * 64) void attn_bwd_kv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, const uint16_t *__restrict__ dO, const float *__restrict__ lse_ws,
    const float *__restrict__ dd_ws, int S, int Hq, int Hkv, int G, int nkt, float qscale, float c,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, float *__restrict__ ddt) {
    constexpr int P = pitch<D>();
    constexpr int NS = D / 32;
    constexpr int NT = D / 16;
    constexpr int GT = KW * 64;                   // threads per row group
    constexpr int KT = 16 * KW;                   // keys per tile
    constexpr int NV = kPairs * D / 8 / GT;       // 16-byte vectors per group thread per tile
    static_assert(NV >= 1 && kPairs * D / 8 % GT == 0, "row block staging split");
    // rank blocks whose sums the row tiles hold at once for the exchange
    constexpr int XB = (2 * NG * kPairs * P * 2) / ((2 * NT + 1) * 4 * 64 * 4);
    static_assert(XB >= 1, "the exchange fits in the row tiles");
    constexpr int NPASS = (KW + XB - 1) / XB;
    // Q of each group's row block, then dO of each ([NG + h])
    __shared__ __align__(16) uint16_t tiles[2 * NG][kPairs * P];
    __shared__ __align__(16) float lse_s[NG][kPairs], dd_s[NG][kPairs];
    __shared__ uint64_t thr_s[NG][kPairs];
    __shared__ uint64_t kmax_s[KW];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hg = wave / KW, kw = wave % KW;  // row group; key wave within it
    const int gt = tid % GT;                   // thread index within the row group
    const int q = lane >> 4, kk = lane & 15;
    // Early key tiles (the longest row ranges) are dispatched first.  Ids go
    // round-robin over the 8 XCDs, so with a multiple of 8 (batch, kv head)
    // units each unit stays on one XCD, whose L2 then holds its Q and dO rows.
    const int nbg = gridDim.x / nkt;
    const int kt = blockIdx.x / nbg, bg = blockIdx.x % nbg;
    const int g = bg % Hkv, b = bg / Hkv;
    const int L = clamp_len(seqlens, b, S);
    const int j0 = kt * KT;
    const uint32_t kvs = (uint32_t)(Hkv * D);
    const size_t urow = ((size_t)b * Hkv + g) * S;

    // The tile's keys ordered by selection key, best first, in KW rank
    // blocks of 16: the waves holding the lower keys, which leave the rows'
    // kept sets first, stop working early (a wave skips the blocks where none
    // of its keys is kept).  Every row group holds the same 16 KW keys, group
    // h key wave kw the rank block (kw + h) mod KW, so that the long-lived blocks
    // of the groups sit on different SIMDs (wave i of a workgroup runs on
    // SIMD i mod 4).
    __shared__ uint64_t tsk[KT];
    __shared__ int perm[KT];
    if (tid < KT) {
        const int j = j0 + tid;
        tsk[tid] = j < L ? selkey(dt[urow + min(j, S - 1)], (uint32_t)j) : 0ull;
    }
    __syncthreads();
    if (tid < KT) {
        const uint64_t mine = tsk[tid];
        int r = 0;
        for (int u = 0; u < KT; ++u) {
            const uint64_t o = tsk[u];
            r += (int)((o > mine) | ((o == mine) & (u < tid)));
        }
        perm[r] = tid;
    }
    __syncthreads();
    const int rb = (kw + hg) % KW;  // rank block of this wave's keys
    const int jk = j0 + perm[16 * rb + kk];
    const bool kvalid = jk < L;
    const int jc = min(jk, S - 1);
    bf16x8 kb[NS], vb[NS];
    float dtl;
    uint64_t skey;
    {
        const float dv = dt[urow + jc];
        dtl = dv * kLog2e;
        skey = kvalid ? selkey(dv, (uint32_t)jc) : 0ull;
        const uint16_t *kr = K + ((size_t)b * S + jc) * kvs + (size_t)g * D;
        const uint16_t *vr = V + ((size_t)b * S + jc) * kvs + (size_t)g * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kb[s] = ld8(kr + 32 * s + 8 * q);
            vb[s] = ld8(vr + 32 * s + 8 * q);
        }
    }
    // largest selection key of the workgroup's valid keys
    uint64_t kmax = skey;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t y = __shfl_xor(kmax, o, 64);
        kmax = y > kmax ? y : kmax;
    }
    if (lane == 0 && hg == 0) kmax_s[kw] = kmax;
    __syncthreads();
    kmax = kmax_s[0];
#pragma unroll
    for (int w2 = 1; w2 < KW; ++w2) kmax = kmax_s[w2] > kmax ? kmax_s[w2] : kmax;

    f32x4 dka[NT], dva[NT];
    float dsum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        dka[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        dva[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int RB = kPairs / G;
    uint16_t *Qg = tiles[hg], *Og = tiles[NG + hg];
    float *lse_g = lse_s[hg], *dd_g = dd_s[hg];
    uint64_t *thr_g = thr_s[hg];
    // A row block (Q and dO of its 64 pairs, their log-sum-exp and D, the
    // row thresholds) is requested into registers one block ahead and written
    // to LDS after the barrier that ends the block before.  Rows past the end
    // repeat the last one; rows past the valid length keep nothing.
    u32x4 rq[NV], ro[NV];
    float rlse, rdd;
    uint64_t rthr;
    auto fetch = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = gt + u * GT;
            const int p = v / (D / 8), cv = v % (D / 8);
            const int row = min(r0 + p / G, S - 1), hq = g * G + p % G;
            const size_t off = (((size_t)b * S + row) * Hq + hq) * D + 8 * cv;
            rq[u] = *reinterpret_cast<const u32x4 *>(Q + off);
            ro[u] = *reinterpret_cast<const u32x4 *>(dO + off);
        }
        const int pp = gt & (kPairs - 1);
        const int row = min(r0 + pp / G, S - 1), hq = g * G + pp % G;
        rlse = lse_ws[((size_t)b * Hq + hq) * S + row];
        rdd = dd_ws[((size_t)b * Hq + hq) * S + row];
        const int rr = r0 + pp, rc = min(rr, S - 1);
        const uint64_t t = selkey(tau[urow + rc], (uint32_t)tie[urow + rc]);
        rthr = (pp < RB && rr < L) ? t : ~0ull;
    };
    auto put = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = gt + u * GT;
            const int p = v / (D / 8), cv = v % (D / 8);
            *reinterpret_cast<u32x4 *>(&Qg[p * P + 8 * cv]) = rq[u];
            *reinterpret_cast<u32x4 *>(&Og[p * P + 8 * cv]) = ro[u];
        }
        if (gt < kPairs) {
            lse_g[gt] = rlse;
            dd_g[gt] = rdd;
            thr_g[gt] = rthr;
        }
    };
    // This lane's key against the group's row block: S and dP on the matrix
    // cores, P and dS in registers, dV^T += dO^T P and dK^T += Q^T dS.  The
    // pairs keeping the key form the run [plo, phi) of the block (the rows
    // keeping a key are a run, and pair p holds row p / G); elsewhere the
    // bias is -inf.
    auto subtile = [&](int plo, int phi) __attribute__((always_inline)) {
        const uint32_t span = (uint32_t)(phi - plo);
        const int pb = 4 * q - plo;
        // two halves of 32 pairs: the second half's scores are formed while
        // the first half's products run
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            f32x4 pm[2], dsm[2];
#pragma unroll
            for (int th = 0; th < 2; ++th) {
                const int t = 2 * s2 + th;
                f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
                __builtin_amdgcn_s_setprio(3);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    sacc = mfma16(ld8(&Qg[(16 * t + kk) * P + 32 * s + 8 * q]), kb[s], sacc);
                    dp = mfma16(ld8(&Og[(16 * t + kk) * P + 32 * s + 8 * q]), vb[s], dp);
                }
                __builtin_amdgcn_s_setprio(0);
                const float4 l4 = *reinterpret_cast<const float4 *>(&lse_g[16 * t + 4 * q]);
                const float4 d4 = *reinterpret_cast<const float4 *>(&dd_g[16 * t + 4 * q]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float bb = (uint32_t)(pb + 16 * t + r) < span ? dtl : -INFINITY;
                    const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], qscale, bb) - lv[r]);  // 0 where not kept
                    pm[th][r] = pv;
                    dsm[th][r] = pv * (dp[r] - dv[r]);
                    dsum += dsm[th][r];
                }
            }
            const bf16x8 pbf = acc_operand(pm[0], pm[1]);
            const bf16x8 sbf = acc_operand(dsm[0], dsm[1]);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                dva[t] = mfma16(tr_operand<P>(Og, 32 * s2, 16 * t, lane), pbf, dva[t]);
                dka[t] = mfma16(tr_operand<P>(Qg, 32 * s2, 16 * t, lane), sbf, dka[t]);
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };

    // The row groups take turns over the row blocks: group h the blocks
    // base + h RB for base = j0, j0 + NG RB, ...
    if (j0 < L) {
        if (j0 + hg * RB < L) fetch(j0 + hg * RB);
        for (int base = j0; base < L; base += NG * RB) {
            const int r0 = base + hg * RB;
            const bool act = r0 < L;
            if (act) put();
            __syncthreads();
            // the first row of group 0's block and every later row keep none
            // of the keys (thresholds grow with the row): done
            if (thr_s[0][0] > kmax) break;
            if (r0 + NG * RB < L) fetch(r0 + NG * RB);
            if (act && thr_g[0] <= kmax) {
                const int rl = min(RB, L - r0);  // rows of the block inside the sequence
                // the block rows keeping key jk: from row jk on (j <= i), while
                // the row's threshold is at most its key (a key once dropped
                // stays dropped)
                const int lo = min(max(jk - r0, 0), RB);
                int hi = 0;
                if (kvalid && thr_g[0] <= skey) {
                    if (thr_g[rl - 1] <= skey) {
                        hi = rl;
                    } else {  // first row in (0, rl - 1] whose threshold passes the key
                        int a = 1, e = rl - 1;
                        while (a < e) {
                            const int mid = (a + e) >> 1;
                            if (thr_g[mid] > skey) e = mid; else a = mid + 1;
                        }
                        hi = a;
                    }
                }
                const int plo = lo * G, phi = max(hi, lo) * G;
                if (__any(phi > plo)) subtile(plo, phi);
            }
            __syncthreads();
        }
    }

    // the other groups hand their sums to group 0 through LDS (the row tiles
    // are free now), one group at a time in group order, and group 0 writes
    // the key's gradients
    // in passes of XB rank blocks when the row tiles cannot hold all of them
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const bool mine = rb / XB == pass;
        float *xw = reinterpret_cast<float *>(&tiles[0][0]) + (rb - pass * XB) * (2 * NT + 1) * 4 * 64;
#pragma unroll
        for (int h2 = 1; h2 < NG; ++h2) {
            __syncthreads();
            if (hg == h2 && mine) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xw[((2 * t) * 4 + i) * 64 + lane] = dka[t][i];
                        xw[((2 * t + 1) * 4 + i) * 64 + lane] = dva[t][i];
                    }
                }
                xw[(2 * NT * 4) * 64 + lane] = dsum;
            }
            __syncthreads();
            if (hg == 0 && mine) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        dka[t][i] += xw[((2 * t) * 4 + i) * 64 + lane];
                        dva[t][i] += xw[((2 * t + 1) * 4 + i) * 64 + lane];
                    }
                }
                dsum += xw[(2 * NT * 4) * 64 + lane];
            }
        }
    }
    if (hg > 0) return;

    float sdt = dsum;
    sdt += __shfl_xor(sdt, 16, 64);
    sdt += __shfl_xor(sdt, 32, 64);
    if (jk < S) {
        if (q == 0) ddt[urow + jk] = sdt;
        const size_t off = ((size_t)b * S + jk) * kvs + (size_t)g * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t k0w = (uint32_t)f32_to_bf16(dka[t][0] * c) | ((uint32_t)f32_to_bf16(dka[t][1] * c) << 16);
            const uint32_t k1w = (uint32_t)f32_to_bf16(dka[t][2] * c) | ((uint32_t)f32_to_bf16(dka[t][3] * c) << 16);
            const uint32_t v0w = (uint32_t)f32_to_bf16(dva[t][0]) | ((uint32_t)f32_to_bf16(dva[t][1]) << 16);
            const uint32_t v1w = (uint32_t)f32_to_bf16(dva[t][2]) | ((uint32_t)f32_to_bf16(dva[t][3]) << 16);
            *reinterpret_cast<uint2 *>(dK + off + 16 * t + 4 * q) = make_uint2(k0w, k1w);
            *reinterpret_cast<uint2 *>(dV + off + 16 * t + 4 * q) = make_uint2(v0w, v1w);
        }
    }
}

template <int D>
hipError_t launch_bwd_d(const void *Q, const void *K, const void *V, const float *dt, const float *tau,
                        const int32_t *tie, const int32_t *seqlens, const void *dO, int B, int S,
                        int Hq, int Hkv, void *dQ, void *dK, void *dV, float *ddt, void *ws, hipStream_t stream) {
    const int G = Hq / Hkv;
    const int RB = kQPairs / G;
    const int ntq = (S + RB - 1) / RB;
    const float c = 1.0f / sqrtf((float)D);
    const float qscale = c * kLog2e;
    float *lse_ws = (float *)ws;
    float *dd_ws = lse_ws + (size_t)B * Hq * S;
    hipLaunchKernelGGL((attn_bwd_q_kernel<D>), dim3((unsigned)(B * Hkv * ntq)), dim3(kQThreads), 0, stream,
                       (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, dt, tau, tie, seqlens,
                       (const uint16_t *)dO, S, Hq, Hkv, G, ntq, qscale, c, (uint16_t *)dQ, lse_ws, dd_ws);
    constexpr int KW = D == 64 ? 4 : 8;  // key waves per row group (16 keys each)
    constexpr int NG = D == 64 ? 3 : 1;  // row groups the registers and LDS allow
    const int nkt = (S + 16 * KW - 1) / (16 * KW);
    hipLaunchKernelGGL((attn_bwd_kv_kernel<D, NG, KW>), dim3((unsigned)(B * Hkv * nkt)), dim3(NG * KW * 64), 0, stream,
                       (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, dt, tau, tie, seqlens,
                       (const uint16_t *)dO, lse_ws, dd_ws, S, Hq, Hkv, G, nkt, qscale, c, (uint16_t *)dK,
                       (uint16_t *)dV, ddt);
    return hipGetLastError();
}

}  // namespace

size_t attn_bwd_ws_bytes(int B, int S, int Hq) { return (size_t)2 * B * Hq * S * sizeof(float); }

hipError_t launch_attn_bwd(const void *Q, const void *K, const void *V, const float *dt, const float *tau,
                           const int32_t *tie, const int32_t *seqlens, const void *dO, int B, int S, int Hq,
                           int Hkv, int d, void *dQ, void *dK, void *dV, float *ddt, void *ws, hipStream_t stream) {
    if (d == 128)
        return launch_bwd_d<128>(Q, K, V, dt, tau, tie, seqlens, dO, B, S, Hq, Hkv, dQ, dK, dV, ddt, ws, stream);
    return launch_bwd_d<64>(Q, K, V, dt, tau, tie, seqlens, dO, B, S, Hq, Hkv, dQ, dK, dV, ddt, ws, stream);
}

}  // namespace dma
