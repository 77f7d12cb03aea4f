// Prefill attention under the dynamic top-w mask.
// Doge guide (gitcode), DMA section, forward step 4 with the mask of step 3:
// s_ij = d^-0.5 * q_i.k_j + dt_j over the kept keys j of row i, softmax in
// float32, o_i = sum_j p_ij v_j; query head hq reads kv head hq / G.
//
// bf16 kernel (matrix cores).  One workgroup = one (batch, kv head, tile of
// Bq query rows); its NW waves (8 at d = 128, 4 at d = 64) hold the
// G*Bq <= 32*NW stacked (row, head) pairs, 32 per wave, so the G query heads
// of a kv head share every K/V tile and the mask (which depends only on the
// kv head and the row).
//
// Gathered keys instead of dense key tiles: by nesting, the union of the kept
// sets of rows [i0, i_last] lies inside K_{i0} plus the keys (i0, i_last].
// The workgroup scans dt[0..i_last] and compacts those candidate keys into
// LDS in two passes (count per wave and step of four keys a thread, with the
// loads of eight steps in flight, one scan, then write with ballot offsets),
// in index order and split
// in two groups: "full" keys, kept by every row of the tile (a key j <= i0
// kept by i_last is kept by every row in between, by nesting), first, and the
// "partial" rest after them (at most 2*Bq keys: each row drops at most one
// key, plus the tile's own keys), each with the run of tile rows that keeps
// it.  It then walks the candidates in blocks of 64 keys: gather the K and V
// rows (row-major, plain 16-byte copies) into LDS, S^T = K Q^T on 32x32x16
// bf16 MFMA, the dt bias (plus, in blocks holding partial keys only, the
// row-run test) in registers, an online softmax in base 2, and O^T += V^T P^T
// on MFMA with P rounded once to bf16.  The V^T operand is read straight from the row-major
// V tile with the gfx950 LDS transpose read (ds_read_b64_tr_b16).  Only
// ~w + Bq keys are touched per tile instead of the dense causal prefix.
//
// Accumulator layout facts used below (32x32x16 bf16, wave64, l = lane):
//   A operand: A[m = l%32][k = 8*(l/32) + 0..7]
//   B operand: B[k = 8*(l/32) + 0..7][n = l%32]
//   C/D:       C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15
// S^T = K Q^T puts one query per lane (n) and 32 keys per lane, so row max /
// sum need only a swap between the two lane halves.  O^T = V^T P^T keeps one
// query per lane, so the online-softmax rescale is lane-local.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kBK = 64;          // keys per block
constexpr int kCap = 2560;       // candidate slots in LDS (multiple of kBK)
constexpr int kFillKeys = 4;     // consecutive keys per thread per fill step
constexpr int kBatchSteps = 8;   // fill steps whose loads are issued together
constexpr int kRowThreads = 256; // the float32 row kernel's workgroup

// Workgroup shape: NW waves of 32 stacked (row, head) pairs each.  d = 128
// runs eight waves, one workgroup per CU (256 pairs a tile: half the K/V
// staging per flop and half the candidate fills per row of the four-wave
// shape; measured 4.4 % faster at the padded and 3.3 % at the long
// workload), d = 64 four, two workgroups per CU (eight were 4 % slower on the
// small c2 workload).
template <int NW>
struct Shape {
    static constexpr int kThreads = 64 * NW;
    static constexpr int kRowsPerWG = 32 * NW;                 // stacked (row, head) pairs per workgroup
    static constexpr int kStepKeys = kThreads * kFillKeys;     // keys per fill step
    static constexpr int kMaxSteps = 128 / NW;                 // fill steps counted per round (two scan entries a lane)
    static constexpr int kPartCap = 2 * kRowsPerWG + 2 * kBK;  // slots of the masked region
    static constexpr int kCarrySlots = kCap / kThreads;        // carried candidates per thread
    // work items a launch aims for: enough for balance, few enough that
    // each group's one full candidate scan serves several tiles
    static constexpr int kTargetItems = NW == 4 ? 2048 : 1024;
};
template <int D> constexpr int waves_for() { return D == 128 ? 8 : 4; }

template <int D>
struct Tiles {
    // K tile pitch: D + 8 bf16 (a 4-word bank step per row, so the 32 rows a
    // score MFMA reads spread over all banks).  V tile pitch: D + 32 bf16 (a
    // 16- or 48-word step, so the 4 rows x 32 bytes each 16-lane group of a
    // transpose read touches fall in disjoint banks).
    static constexpr int KP = D + 8;
    static constexpr int VP = D + 32;
};

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives
// element (i % 4) of the 4 x 16-bit values at the address of lane (i/4 + 4s),
// for s = 0..3.  With lane k of the group pointing at row (r0 + k/4), columns
// c0 + 4*(k%4) .. +3 of a row-major tile, lane i gets the column c0 + i of
// rows r0 .. r0+3: a 4 x 16 tile transposed across the lanes.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
}

// Valid tile groups of batch b (those holding a row below L_b).
__device__ __forceinline__ int valid_groups(const int32_t *seqlens, int b, int S, int Bq, int tpw) {
    const int Lb = clamp_len(seqlens, b, S);
    return ((Lb + Bq - 1) / Bq + tpw - 1) / tpw;
}

// Wave 0: the batch holding item k when batch b holds cnt(b) * Hkv items
// (items ordered by batch, then kv head, then group), and k's place in it.
template <typename F>
__device__ __forceinline__ void locate_item(long long k, int B, int Hkv, int lane, F cnt, int &b_out,
                                            long long &off_out) {
    long long base = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int bb = b0 + lane;
        long long c = bb < B ? (long long)cnt(bb) * Hkv : 0;
        long long incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const long long y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const long long tot = __shfl(incl, 63, 64);
        if (k < base + tot) {
            // the first lane whose inclusive count passes k
            const unsigned long long m = __ballot(bb < B && base + incl > k);
            const int src = __ffsll((long long)m) - 1;
            const long long excl = __shfl(incl - c, src, 64);
            b_out = b0 + src;
            off_out = k - base - excl;
            return;
        }
        base += tot;
    }
    b_out = -1;
    off_out = 0;
}

// Upper bound: first t in [lo, n) with thr[t] > key (thr nondecreasing), else n.
__device__ __forceinline__ int first_row_above(const uint64_t *thr, int lo, int n, uint64_t key) {
    int a = lo, b = n;
    while (a < b) {
        const int mid = (a + b) >> 1;
        if (thr[mid] > key) b = mid; else a = mid + 1;
    }
    return a;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, int S, int Hq, int Hkv, int G, int Bq, int ntiles, int tpw,
    int B, uint16_t *__restrict__ O, float qscale) {
    using T = Tiles<D>;
    using SH = Shape<NW>;
    constexpr int kThreads = SH::kThreads, kRowsPerWG = SH::kRowsPerWG, kStepKeys = SH::kStepKeys,
                  kMaxSteps = SH::kMaxSteps, kPartCap = SH::kPartCap, kCarrySlots = SH::kCarrySlots;
    constexpr int RV = D / 8;                    // 16-byte vectors per K/V row
    constexpr int NL = kBK * RV / kThreads;      // K (and V) vectors per thread per block
    static_assert(kBK * RV % kThreads == 0, "block staging split");
    static_assert(NW * (kCarrySlots + 1) <= 64 && kCarrySlots + 1 <= kMaxSteps, "carry scan");
    static_assert(NW * kMaxSteps == 128, "two (step, wave) entries per lane in the fill scan");
    __shared__ __align__(16) int c_idx[kCap];
    __shared__ __align__(16) float c_dtl[kCap];     // (dt - dref) * log2(e); raw dt while filling
    __shared__ __align__(16) int c_lo[kPartCap];    // masked region: first tile row keeping the key
    __shared__ __align__(16) int c_span[kPartCap];  // masked region: rows keeping it
    __shared__ uint64_t thr[kRowsPerWG];            // threshold key of each tile row
    __shared__ uint32_t cnt[kMaxSteps * NW];        // per (fill step, wave): full | partial << 16
    __shared__ int fill_info[3];                    // steps used, full count, partial count
    __shared__ float red_max[kThreads / 64];        // per-wave maxima of the candidates' dt
    __shared__ __align__(16) uint16_t Ks[kBK * T::KP];
    __shared__ __align__(16) uint16_t Vs[kBK * T::VP];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane >> 5, ql = lane & 31;
    // Work items: the tile groups (tpw consecutive query tiles of one
    // (batch, kv head)) that hold a valid row, ordered by batch, kv head and
    // row.  XCD x (workgroup ids go round-robin over the 8 XCDs) takes the
    // x-th eighth of that list, in row order, on its own workgroup slots: the
    // work is balanced over the XCDs whatever the lengths, and each XCD works
    // on one or two kv heads at a time, whose candidate K/V rows stay in its
    // L2.  Each workgroup finds its item from the lengths; slots past the
    // XCD's share write the zeros of the groups that hold only padded rows.
    const int ngroups = (ntiles + tpw - 1) / tpw;
    __shared__ int wmap[4];  // batch, kv head, first group, group count (-1: none)
    if (wave == 0) {
        long long T = 0;  // valid items
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int bb = b0 + lane;
            long long c = bb < B ? (long long)valid_groups(seqlens, bb, S, Bq, tpw) * Hkv : 0;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
            T += c;
        }
        const long long qx = (T + 7) / 8;  // items per XCD
        const long long per_xcd = gridDim.x >> 3;
        const long long slot = blockIdx.x >> 3, xcd = blockIdx.x & 7;
        int bsel = -1, gsel = 0, gfirst = 0, gcount = 0;
        long long off = 0;
        if (slot < qx) {
            const long long k = xcd * qx + slot;
            if (k < T) {
                locate_item(k, B, Hkv, lane, [&](int bb) { return valid_groups(seqlens, bb, S, Bq, tpw); }, bsel, off);
                const int vg = valid_groups(seqlens, bsel, S, Bq, tpw);
                gsel = (int)(off / vg);
                gfirst = (int)(off % vg);
                gcount = 1;
            }
        } else {
            // padded groups, one per spare slot (spare slots: 8 (per_xcd - qx)
            // >= all groups - T + 1)
            const long long e = xcd * (per_xcd - qx) + (slot - qx);
            const long long P = (long long)B * Hkv * ngroups - T;
            if (e < P) {
                // one padded item: (batch, kv head, group) past the valid groups
                locate_item(e, B, Hkv, lane, [&](int bb) { return ngroups - valid_groups(seqlens, bb, S, Bq, tpw); },
                            bsel, off);
                const int pg = ngroups - valid_groups(seqlens, bsel, S, Bq, tpw);
                gsel = (int)(off / pg);
                gfirst = valid_groups(seqlens, bsel, S, Bq, tpw) + (int)(off % pg);
                gcount = 1;
            }
        }
        if (lane == 0) {
            wmap[0] = bsel;
            wmap[1] = gsel;
            wmap[2] = gfirst;
            wmap[3] = gcount;
        }
    }
    __syncthreads();
    if (wmap[0] < 0) return;
    const int b = wmap[0], g = wmap[1], grp = wmap[2];
    const int L = clamp_len(seqlens, b, S);

    const int m = wave * 32 + ql;  // stacked (row, head) pair of this lane
    const int r = m / G, hh = m - r * G;
    const int hq = g * G + hh;
    const size_t urow = ((size_t)b * Hkv + g) * S;
    const float *dtrow = dt + urow;
    const uint32_t kvs = (uint32_t)(Hkv * D);
    const uint16_t *Kb = K + (size_t)b * S * kvs + (size_t)g * D;
    const uint16_t *Vb = V + (size_t)b * S * kvs + (size_t)g * D;

    // the current tile: first and last valid row, and their thresholds
    int i0 = 0, i_last = 0, nrows = 0;
    float tau0 = 0.f, taul = 0.f;
    int tie0 = 0, tiel = 0;

    // candidate class of key j: 0 not a candidate, 1 kept by every tile row,
    // 2 kept by some tile rows
    auto cls_of = [&](float dv, int j) __attribute__((always_inline)) -> int {
        if (j > i_last) return 0;
        if (j > i0) return 2;
        if (!kept_test(dv, j, tau0, tie0)) return 0;
        return kept_test(dv, j, taul, tiel) ? 1 : 2;
    };
    // the fill step's keys of this thread: scan + step*kStepKeys + 4*tid + e
    auto load_step_keys = [&](float (&dv)[kBatchSteps][kFillKeys], int scan, int s0, int nsteps)
        __attribute__((always_inline)) {
#pragma unroll
        for (int bb = 0; bb < kBatchSteps; ++bb) {
#pragma unroll
            for (int e = 0; e < kFillKeys; ++e) {
                const int j = scan + (s0 + bb) * kStepKeys + kFillKeys * tid + e;
                dv[bb][e] = (s0 + bb < nsteps && j <= i_last) ? dtrow[j] : 0.f;
            }
        }
    };

    // next block, staged in registers: vector v = tid + u*256 is row v / RV,
    // 16-byte column v % RV of both the K and the V tile.  Positions past the
    // last candidate repeat it (a real row; its weight is masked to zero).
    u32x4 pk[NL], pv[NL];
    auto load_block = [&](int blk, int n) __attribute__((always_inline)) {
        int idx[NL];
#pragma unroll
        for (int u = 0; u < NL; ++u) idx[u] = c_idx[min(blk + (tid + u * kThreads) / RV, n - 1)];
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const size_t off = (size_t)(uint32_t)idx[u] * kvs + ((tid + u * kThreads) % RV) * 8;
            pk[u] = *reinterpret_cast<const u32x4 *>(Kb + off);
            pv[u] = *reinterpret_cast<const u32x4 *>(Vb + off);
        }
    };
    auto store_block = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int v = tid + u * kThreads;
            const int kk = v / RV, cv = v % RV;
            *reinterpret_cast<u32x4 *>(&Ks[kk * T::KP + cv * 8]) = pk[u];
            *reinterpret_cast<u32x4 *>(&Vs[kk * T::VP + cv * 8]) = pv[u];
        }
    };

    // Per-lane LDS addresses for the transpose reads of the PV operand: lane
    // l (group (l>>4), index k = l & 15) points at row 4h + k/4 (+16c + 8rr),
    // column 16*((l>>4)&1) + 4*(k&3) (+32t).
    const int tr_k = lane & 15;
    const int tr_off = (4 * h + (tr_k >> 2)) * T::VP + 16 * ((lane >> 4) & 1) + 4 * (tr_k & 3);
    const uint64_t lt_mask = (1ull << lane) - 1ull;

    int n = 0, nF = 0;    // candidates in LDS: nF full ones, then the partial ones
    bool carry = false;   // LDS holds the whole candidate list of the previous tile

    const int t_end = min(ntiles, (grp + 1) * tpw);
    for (int tile = grp * tpw; tile < t_end; ++tile) {
        i0 = tile * Bq;
        const int i = i0 + r;
        const bool active = (r < Bq) && (i < S);
        uint16_t *orow = O + (((size_t)b * S + (active ? i : 0)) * Hq + hq) * D;
        if (i0 >= L) {  // the whole tile is padding (so are the later ones): zero rows
            if (active) {
                for (int c = h * (D / 2); c < (h + 1) * (D / 2); c += 8)
                    *reinterpret_cast<uint4 *>(orow + c) = make_uint4(0, 0, 0, 0);
            }
            continue;
        }
        const bool live = active && i < L;
        i_last = min(i0 + Bq, L) - 1;
        nrows = i_last - i0 + 1;
        tau0 = tau[urow + i0];
        taul = tau[urow + i_last];
        tie0 = tie[urow + i0];
        tiel = tie[urow + i_last];
        // (the previous tile's readers of thr have all passed a barrier since)
        for (int t = tid; t < nrows; t += kThreads) thr[t] = selkey(tau[urow + i0 + t], (uint32_t)tie[urow + i0 + t]);

        float mrow = -INFINITY, lrow = 0.f;
        float dref = 0.f;  // reference dt of the tile (set with its first round of candidates)
        f32x16 oacc[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
        bf16x8 qf[D / 16];

        int scan = 0, rounds = 0;
        while (scan <= i_last) {
            if (rounds == 0 && carry) {
                // ---- carried list: by nesting, this tile's candidates are the
                // previous tile's candidates plus this tile's own keys,
                // re-classified against this tile's first and last rows
                int jc[kCarrySlots + 1];
                float dc[kCarrySlots + 1];
#pragma unroll
                for (int q = 0; q < kCarrySlots; ++q) {
                    const int k = tid + q * kThreads;
                    jc[q] = k < n ? c_idx[k] : -1;
                }
                jc[kCarrySlots] = tid < nrows ? i0 + tid : -1;
#pragma unroll
                for (int q = 0; q <= kCarrySlots; ++q) dc[q] = jc[q] >= 0 ? dtrow[jc[q]] : 0.f;
                int cc[kCarrySlots + 1];
#pragma unroll
                for (int q = 0; q <= kCarrySlots; ++q) {
                    cc[q] = jc[q] >= 0 ? cls_of(dc[q], jc[q]) : 0;
                    const uint32_t nf = (uint32_t)__popcll(__ballot(cc[q] == 1));
                    const uint32_t np = (uint32_t)__popcll(__ballot(cc[q] == 2));
                    if (lane == 0) cnt[q * NW + wave] = nf | (np << 16);
                }
                __syncthreads();  // counts visible; every read of the old list done
                if (wave == 0) {
                    constexpr int ne = NW * (kCarrySlots + 1);
                    const uint32_t v = lane < ne ? cnt[lane] : 0u;
                    uint32_t incl = v;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const uint32_t y = __shfl_up(incl, o, 64);
                        if (lane >= o) incl += y;
                    }
                    if (lane < ne) cnt[lane] = incl - v;
                    const uint32_t tot = __shfl(incl, 63, 64);
                    if (lane == 0) {
                        fill_info[1] = (int)(tot & 0xffffu);
                        fill_info[2] = (int)(tot >> 16);
                    }
                }
                __syncthreads();
                nF = fill_info[1];
                n = nF + fill_info[2];
#pragma unroll
                for (int q = 0; q <= kCarrySlots; ++q) {
                    const uint32_t base = cnt[q * NW + wave];
                    const int of = (int)(base & 0xffffu) + (int)__popcll(__ballot(cc[q] == 1) & lt_mask);
                    const int op = nF + (int)(base >> 16) + (int)__popcll(__ballot(cc[q] == 2) & lt_mask);
                    if (cc[q] == 1) {
                        c_idx[of] = jc[q];
                        c_dtl[of] = dc[q];
                    } else if (cc[q] == 2) {
                        c_idx[op] = jc[q];
                        c_dtl[op] = dc[q];
                    }
                }
                scan = i_last + 1;
            } else {
            // ---- fill pass 1: candidates per (step, wave), loads of kBatchSteps
            // steps in flight
            const int nsteps = min((i_last - scan) / kStepKeys + 1, kMaxSteps);
            // with d = 64 the keys of a round of at most kBatchSteps steps stay
            // in registers for pass 2 (with d = 128 there is no room for them)
            constexpr bool kKeepKeys = D <= 64;
            float dv[kBatchSteps][kFillKeys];
            for (int s0 = 0; s0 < nsteps; s0 += kBatchSteps) {
                load_step_keys(dv, scan, s0, nsteps);
#pragma unroll
                for (int bb = 0; bb < kBatchSteps; ++bb) {
                    if (s0 + bb >= nsteps) break;
                    uint32_t nf = 0, np = 0;
#pragma unroll
                    for (int e = 0; e < kFillKeys; ++e) {
                        const int c = cls_of(dv[bb][e], scan + (s0 + bb) * kStepKeys + kFillKeys * tid + e);
                        nf += (uint32_t)__popcll(__ballot(c == 1));
                        np += (uint32_t)__popcll(__ballot(c == 2));
                    }
                    if (lane == 0) cnt[(s0 + bb) * NW + wave] = nf | (np << 16);
                }
            }
            __syncthreads();
            // ---- exclusive scan over (step, wave) in key order; the steps whose
            // candidates fit in kCap are used this round
            if (wave == 0) {
                const int e0 = 2 * lane, ne = NW * nsteps;
                const uint32_t v0 = e0 < ne ? cnt[e0] : 0u, v1 = e0 + 1 < ne ? cnt[e0 + 1] : 0u;
                uint32_t incl = v0 + v1;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t y = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += y;
                }
                if (e0 < ne) cnt[e0] = incl - v0 - v1;
                if (e0 + 1 < ne) cnt[e0 + 1] = incl - v1;
                // the last of step s's LPS lanes holds the running total
                // through the end of step s
                constexpr int LPS = NW / 2;  // lanes per step
                const bool fits = (lane % LPS) == LPS - 1 && (lane / LPS) < nsteps &&
                                  (incl & 0xffffu) + (incl >> 16) <= (uint32_t)kCap;
                const int used = __popcll(__ballot(fits));  // >= 1: one step never exceeds kCap
                const uint32_t tot = __shfl(incl, LPS * used - 1, 64);
                if (lane == 0) {
                    fill_info[0] = used;
                    fill_info[1] = (int)(tot & 0xffffu);
                    fill_info[2] = (int)(tot >> 16);
                }
            }
            __syncthreads();
                const int used = fill_info[0];
                nF = fill_info[1];
                n = nF + fill_info[2];
            // ---- fill pass 2: write the candidates (full first, partial after)
            for (int s0 = 0; s0 < used; s0 += kBatchSteps) {
                if (!kKeepKeys || nsteps > kBatchSteps) load_step_keys(dv, scan, s0, used);
#pragma unroll
                for (int bb = 0; bb < kBatchSteps; ++bb) {
                    if (s0 + bb >= used) break;
                    const uint32_t base = cnt[(s0 + bb) * NW + wave];
                    int of = (int)(base & 0xffffu), op = nF + (int)(base >> 16);
                    const int jb = scan + (s0 + bb) * kStepKeys + kFillKeys * tid;
                    int c[kFillKeys];
#pragma unroll
                    for (int e = 0; e < kFillKeys; ++e) {
                        c[e] = cls_of(dv[bb][e], jb + e);
                        of += (int)__popcll(__ballot(c[e] == 1) & lt_mask);
                        op += (int)__popcll(__ballot(c[e] == 2) & lt_mask);
                    }
#pragma unroll
                    for (int e = 0; e < kFillKeys; ++e) {
                        const int j = jb + e;
                        if (c[e] == 1) {
                            c_idx[of] = j;
                            c_dtl[of] = dv[bb][e];
                            ++of;
                        } else if (c[e] == 2) {
                            c_idx[op] = j;
                            c_dtl[op] = dv[bb][e];
                            ++op;
                        }
                    }
                }
            }
                scan += used * kStepKeys;
            }
            ++rounds;
            if (rounds == 1) {  // Q of the tile, loaded while the row runs are found
                if (live) {
                    const uint16_t *qp = Q + (((size_t)b * S + i) * Hq + hq) * D + 8 * h;
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
                } else {
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = bf16x8{};
                }
            }
            const int pbase = nF / kBK * kBK;           // first block holding a partial key
            const int npad = (n + kBK - 1) / kBK * kBK;
            __syncthreads();
            // The dt bias enters each score relative to dref, the largest dt
            // among the keys kept by every row of the tile (a shift common to
            // every key of a row leaves its softmax unchanged).  Every row
            // keeps that key, so its own largest kept dt is at least dref:
            // the keys that carry a row's weight have dt - dref small (exact
            // in float32 when within a factor 2 of dref) and never larger
            // than dt itself, so a large dt shared by the kept keys does not
            // swallow the query-key term.  dref is fixed by the tile's first
            // round of candidates (every round of a row must use one shift;
            // the first round's full keys are still kept by every row).
            if (rounds == 1) {
                float mx = -INFINITY;
                for (int k = tid; k < nF; k += kThreads) mx = fmaxf(mx, c_dtl[k]);
                mx = wave_max(mx);
                if (lane == 0) red_max[wave] = mx;
                __syncthreads();
                dref = red_max[0];
#pragma unroll
                for (int w2 = 1; w2 < NW; ++w2) dref = fmaxf(dref, red_max[w2]);
                if (!(dref > -INFINITY && dref < INFINITY)) dref = 0.f;
            }
            for (int k = tid; k < n; k += kThreads) c_dtl[k] = (c_dtl[k] - dref) * kLog2e;
            // row runs of the masked region: a partial key j is kept on the tile
            // rows [lo, lo + span) (by nesting a run: from its own row, or from
            // i0, until the first row whose threshold passes it); full keys
            // sharing a block with partial ones keep every row; slots past the
            // last candidate keep none
            for (int k = pbase + tid; k < npad; k += kThreads) {
                int lo = 0, span = 0;
                if (k < nF) {
                    span = nrows;
                } else if (k < n) {
                    const int j = c_idx[k];
                    lo = j > i0 ? j - i0 : 0;
                    span = first_row_above(thr, lo, nrows, selkey(dtrow[j], (uint32_t)j)) - lo;
                } else {
                    c_dtl[k] = 0.f;
                }
                c_lo[k - pbase] = lo;
                c_span[k - pbase] = span;
            }
            __syncthreads();

            // ---- attend over the candidates, 64 keys at a time
            if (n > 0) load_block(0, n);
            for (int blk = 0; blk < n; blk += kBK) {
                store_block();
                __syncthreads();
                if (blk + kBK < n) load_block(blk + kBK, n);  // in flight during the math below

                // S^T = K Q^T for two 32-key halves of the block; the K fragments
                // of step ks+1 are read while step ks multiplies
                // Wave priorities: the two waves of a SIMD (one per resident
                // workgroup) interleave their phases best when a wave forming
                // scores wins instruction arbitration, one forming the weighted
                // sum of V comes next and one in its softmax yields; measured
                // 5-18 % faster than equal priorities.
                __builtin_amdgcn_s_setprio(3);
                f32x16 sacc[2] = {f32x16{}, f32x16{}};
                const uint16_t *kp0 = &Ks[ql * T::KP + 8 * h];
                const uint16_t *kp1 = &Ks[(32 + ql) * T::KP + 8 * h];
                bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(kp0);
                bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(kp1);
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    bf16x8 n0 = a0, n1 = a1;
                    if (ks + 1 < D / 16) {
                        n0 = *reinterpret_cast<const bf16x8 *>(kp0 + 16 * (ks + 1));
                        n1 = *reinterpret_cast<const bf16x8 *>(kp1 + 16 * (ks + 1));
                    }
                    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], sacc[0], 0, 0, 0);
                    sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], sacc[1], 0, 0, 0);
                    a0 = n0;
                    a1 = n1;
                }

                __builtin_amdgcn_s_setprio(0);
                // dt bias (and, where partial keys are, the row-run test), then
                // the online softmax in base 2
                float z[2][16];
                float mloc = -INFINITY;
                if (blk < pbase) {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const int pos = blk + 32 * kt + 8 * r4 + 4 * h;
                            const float4 dl4 = *reinterpret_cast<const float4 *>(&c_dtl[pos]);
                            const float dls[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float zz = fmaf(sacc[kt][4 * r4 + e], qscale, dls[e]);
                                z[kt][4 * r4 + e] = zz;
                                mloc = fmaxf(mloc, zz);
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const int pos = blk + 32 * kt + 8 * r4 + 4 * h;
                            const int4 lo4 = *reinterpret_cast<const int4 *>(&c_lo[pos - pbase]);
                            const int4 sp4 = *reinterpret_cast<const int4 *>(&c_span[pos - pbase]);
                            const float4 dl4 = *reinterpret_cast<const float4 *>(&c_dtl[pos]);
                            const int los[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
                            const int sps[4] = {sp4.x, sp4.y, sp4.z, sp4.w};
                            const float dls[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const bool ok = (unsigned)(r - los[e]) < (unsigned)sps[e];
                                const float zz = fmaf(sacc[kt][4 * r4 + e], qscale, ok ? dls[e] : -INFINITY);
                                z[kt][4 * r4 + e] = zz;
                                mloc = fmaxf(mloc, zz);
                            }
                        }
                    }
                }
                // Lazy rescale: the running max only moves when a block raises it
                // by more than 8 (base 2), so p stays <= 256 and most blocks skip
                // the O rescale.  The final normalisation uses the same max, so
                // the result is the softmax whatever max was used.
                const float mblk = half_swap_max(mloc);
                const bool upd = mblk > mrow + 8.f;
                if (__any(upd)) {
                    const float mnew = upd ? mblk : mrow;
                    const float alpha = upd ? __builtin_amdgcn_exp2f(mrow - mnew) : 1.f;
                    mrow = mnew;
                    lrow *= alpha;
#pragma unroll
                    for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
                }
                const float msub = (mrow == -INFINITY) ? 0.f : mrow;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) z[kt][e] = __builtin_amdgcn_exp2f(z[kt][e] - msub);
                }

                // O^T += V^T P^T.  PV call c covers keys 16c..16c+15; lane half h
                // holds, in k-slots 0..7, keys 16c + 8*(j/4) + 4h + j%4, which are
                // exactly its score registers z[c/2][8*(c%2) + j].  The V^T operand
                // comes from two transpose reads (rows 16c + 4h + {0..3} and
                // 16c + 8 + 4h + {0..3}).  The softmax denominator sums the same
                // bf16-rounded weights that multiply V, so that the rounding of P
                // perturbs the weights of a normalised average (an output
                // dominated by one key keeps that key's value).
                __builtin_amdgcn_s_setprio(1);
                float psum = 0.f;
                const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    bf16x8 pb;
#pragma unroll
                    for (int jx = 0; jx < 8; ++jx) pb[jx] = (__bf16)z[c >> 1][8 * (c & 1) + jx];
                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one2, psum, false);
                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one2, psum, false);
                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one2, psum, false);
                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one2, psum, false);
#pragma unroll
                    for (int t = 0; t < D / 32; ++t) {
                        const uint16_t *vp = &Vs[16 * c * T::VP + 32 * t + tr_off];
                        const i16x4 lo = lds_read_tr16(vp);
                        const i16x4 hi = lds_read_tr16(vp + 8 * T::VP);
                        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, oacc[t], 0, 0, 0);
                    }
                }
                lrow += psum;
                __builtin_amdgcn_s_setprio(0);
                __syncthreads();  // LDS tiles are rewritten next
            }
        }

        carry = rounds == 1 && n + Bq <= kCap;

        const float ltot = half_swap_sum(lrow);
        const float inv = (live && ltot > 0.f) ? 1.f / ltot : 0.f;
        if (active) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int col = 32 * t + 8 * r4 + 4 * h;
                    const uint32_t w0 = (uint32_t)f32_to_bf16(oacc[t][4 * r4 + 0] * inv) |
                                        ((uint32_t)f32_to_bf16(oacc[t][4 * r4 + 1] * inv) << 16);
                    const uint32_t w1 = (uint32_t)f32_to_bf16(oacc[t][4 * r4 + 2] * inv) |
                                        ((uint32_t)f32_to_bf16(oacc[t][4 * r4 + 3] * inv) << 16);
                    *reinterpret_cast<uint2 *>(orow + col) = make_uint2(w0, w1);
                }
            }
        }
    }
}

// float32 path: one wave per (batch, query head, row); lanes split head_dim.
// Scans the row's causal keys, applies the kept test and runs the online
// softmax in float32.  Serves the fp32 workloads (small shapes).
template <typename Tin>
__global__ __launch_bounds__(kRowThreads) void attn_rowwise_kernel(
    const Tin *__restrict__ Q, const Tin *__restrict__ K, const Tin *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, int B, int S, int Hq, int Hkv, int d,
    Tin *__restrict__ O, float qscale) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
    if (wid >= (int64_t)B * Hq * S) return;
    const int i = (int)(wid % S);
    const int hq = (int)((wid / S) % Hq);
    const int b = (int)(wid / ((int64_t)S * Hq));
    const int G = Hq / Hkv, g = hq / G;
    const int L = clamp_len(seqlens, b, S);
    const size_t obase = (((size_t)b * S + i) * Hq + hq) * d;
    constexpr int kMaxPer = 4;  // d <= 256
    if (i >= L) {
        for (int e = lane; e < d; e += 64) Elem<Tin>::store(O, obase + e, 0.f);
        return;
    }
    const size_t urow = ((size_t)b * Hkv + g) * S;
    const float ti = tau[urow + i];
    const int ki = tie[urow + i];
    float qv[kMaxPer], acc[kMaxPer];
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
        const int e = lane + 64 * u;
        qv[u] = e < d ? Elem<Tin>::load(Q, obase + e) : 0.f;
        acc[u] = 0.f;
    }
    // the bias enters relative to the largest kept dt of the row (a shift
    // common to all its keys leaves the softmax unchanged), so a large dt
    // shared by the kept keys does not swallow q.k in float32
    float dref = -INFINITY;
    for (int j = lane; j <= i; j += 64) {
        const float dj = dt[urow + j];
        if (kept_test(dj, j, ti, ki)) dref = fmaxf(dref, dj);
    }
    dref = wave_max(dref);
    if (!(dref > -INFINITY && dref < INFINITY)) dref = 0.f;
    float mrow = -INFINITY, lrow = 0.f;
    for (int j = 0; j <= i; ++j) {
        const float dj = dt[urow + j];
        if (!kept_test(dj, j, ti, ki)) continue;
        const size_t kb = (((size_t)b * S + j) * Hkv + g) * d;
        float part = 0.f;
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            const int e = lane + 64 * u;
            if (e < d) part = fmaf(qv[u], Elem<Tin>::load(K, kb + e), part);
        }
        const float zz = fmaf(wave_sum(part), qscale, (dj - dref) * kLog2e);
        const float mnew = fmaxf(mrow, zz);
        const float alpha = exp2f(mrow - mnew);
        const float p = exp2f(zz - mnew);
        lrow = lrow * alpha + p;
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            const int e = lane + 64 * u;
            const float vv = e < d ? Elem<Tin>::load(V, kb + e) : 0.f;
            acc[u] = fmaf(p, vv, acc[u] * alpha);
        }
        mrow = mnew;
    }
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
        const int e = lane + 64 * u;
        if (e < d) Elem<Tin>::store(O, obase + e, acc[u] * inv);
    }
}


// bf16 launch of one head_dim: the workgroup shape of that head_dim, its
// tile groups, and a grid of one slot per group plus spares.
template <int D>
void launch_attn_bf16(const void *Q, const void *K, const void *V, const float *dt, const float *tau,
                      const int32_t *tie, const int32_t *seqlens, int B, int S, int Hq, int Hkv, void *O,
                      float qscale, hipStream_t stream, hipError_t &err) {
    constexpr int NW = waves_for<D>();
    using SH = Shape<NW>;
    const int G = Hq / Hkv;
    const int Bq = SH::kRowsPerWG / G;
    const int ntiles = (S + Bq - 1) / Bq;
    // consecutive tiles per workgroup: enough work items to fill the chip's
    // workgroup slots several times over (a short last round), and the prefix
    // scan of a group's first candidate list amortised over the rest of its
    // group
    const int64_t total = (int64_t)ntiles * Hkv * B;
    const int tpw = (int)std::max<int64_t>(1, std::min<int64_t>(total / SH::kTargetItems, ntiles));
    const int64_t ngroups = (ntiles + tpw - 1) / tpw;
    const int64_t all_groups = (int64_t)B * Hkv * ngroups;
    // one slot per group, plus one spare per XCD: the slots past each XCD's
    // share of the valid groups then outnumber the padded groups
    const int64_t items = 8 * ((all_groups + 7) / 8 + 1);
    if (items > 0x7fffffff) {
        err = hipErrorInvalidValue;
        return;
    }
    hipLaunchKernelGGL((attn_bf16_kernel<D, NW>), dim3((unsigned)items), dim3(SH::kThreads), 0, stream,
                       (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, dt, tau, tie, seqlens, S,
                       Hq, Hkv, G, Bq, ntiles, tpw, B, (uint16_t *)O, qscale);
}

}  // namespace

hipError_t launch_attn(const void *Q, const void *K, const void *V, int dtype, const float *dt,
                       const float *tau, const int32_t *tie, const int32_t *seqlens, int B, int S,
                       int Hq, int Hkv, int d, int w, void *O, hipStream_t stream) {
    (void)w;
    const float qscale = (float)(1.0 / __builtin_sqrt((double)d) * 1.4426950408889634);
    if (dtype == 1) {
        hipError_t err = hipSuccess;
        if (d == 128)
            launch_attn_bf16<128>(Q, K, V, dt, tau, tie, seqlens, B, S, Hq, Hkv, O, qscale, stream, err);
        else
            launch_attn_bf16<64>(Q, K, V, dt, tau, tie, seqlens, B, S, Hq, Hkv, O, qscale, stream, err);
        if (err != hipSuccess) return err;
    } else {
        const int64_t waves = (int64_t)B * Hq * S;
        const int64_t blocks = (waves + kRowThreads / 64 - 1) / (kRowThreads / 64);
        hipLaunchKernelGGL(attn_rowwise_kernel<float>, dim3((unsigned)blocks), dim3(kRowThreads), 0,
                           stream, (const float *)Q, (const float *)K, (const float *)V, dt, tau, tie,
                           seqlens, B, S, Hq, Hkv, d, (float *)O, qscale);
    }
    return hipGetLastError();
}

}  // namespace dma
