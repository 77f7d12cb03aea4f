// Prefill attention under the dynamic top-w mask.
// Doge guide (gitcode), DMA section, forward step 4 with the mask of step 3:
// s_ij = d^-0.5 * q_i.k_j + dt_j over the kept keys j of row i, softmax in
// float32, o_i = sum_j p_ij v_j; query head hq reads kv head hq / G.
//
// bf16 kernel (matrix cores).  One workgroup = one (batch, kv head, tile of
// Bq query rows); its 4 waves hold the G*Bq <= 128 stacked (row, head) pairs,
// 32 per wave, so the G query heads of a kv head share every K/V tile and the
// mask (which depends only on the kv head and the row).
//
// Gathered keys instead of dense key tiles: by nesting, the union of the kept
// sets of rows [i0, i0+Bq) lies inside K_{i0} plus the keys (i0, i0+Bq).  The
// workgroup scans dt[0..i_last] once, keeps keys passing row i0's threshold
// test (or newer than i0) and compacts their indices into LDS (ballot +
// popcount).  It then walks that candidate list in blocks of 64 keys: gather
// the K and V rows (row-major, plain 16-byte copies) into LDS, S^T = K Q^T on
// 32x32x16 bf16 MFMA, the exact per-row kept test and the dt bias in
// registers, an online softmax in base 2, and O^T += V^T P^T on MFMA with P
// rounded once to bf16.  The V^T operand is read straight from the row-major
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
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWG = 128;  // stacked (row, head) pairs per workgroup
constexpr int kBK = 64;          // keys per block
constexpr int kCap = 2560;       // candidate slots in LDS (multiple of kBK)
constexpr int kFillPer = 2;      // consecutive keys per thread per fill step

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

// Upper bound: first t in [lo, n) with thr[t] > key (thr nondecreasing), else n.
__device__ __forceinline__ int first_row_above(const uint64_t *thr, int lo, int n, uint64_t key) {
    int a = lo, b = n;
    while (a < b) {
        const int mid = (a + b) >> 1;
        if (thr[mid] > key) b = mid; else a = mid + 1;
    }
    return a;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, int S, int Hq, int Hkv, int G, int Bq, int ntiles,
    uint16_t *__restrict__ O, float qscale) {
    using T = Tiles<D>;
    constexpr int RV = D / 8;                    // 16-byte vectors per K/V row
    constexpr int NL = kBK * RV / kThreads;      // K (and V) vectors per thread per block
    static_assert(kBK * RV % kThreads == 0, "block staging split");
    __shared__ __align__(16) int c_idx[kCap];
    __shared__ __align__(16) int c_lo[kCap];     // first tile row (offset) keeping the key
    __shared__ __align__(16) int c_span[kCap];   // number of consecutive rows keeping it
    __shared__ __align__(16) float c_dtl[kCap];  // dt * log2(e)
    __shared__ uint64_t thr[kRowsPerWG];           // threshold key of each tile row
    __shared__ __align__(16) uint16_t Ks[kBK * T::KP];
    __shared__ __align__(16) uint16_t Vs[kBK * T::VP];
    __shared__ int wcnt[2][kThreads / 64];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane >> 5, ql = lane & 31;
    // XCD-aware order: workgroup ids go round-robin over the 8 XCDs, so hand
    // each XCD a contiguous run of (batch, kv head, tile) work items; nearby
    // tiles of one kv head share most candidate K/V rows in that XCD's L2.
    const int nwg = gridDim.x;
    const int per_xcd = nwg >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int item = (slot < per_xcd && (nwg & 7) == 0) ? xcd * per_xcd + slot : blockIdx.x;
    const int tile = item % ntiles;
    const int g = (item / ntiles) % Hkv;
    const int b = item / (ntiles * Hkv);
    const int i0 = tile * Bq;
    const int L = seqlens ? seqlens[b] : S;

    const int m = wave * 32 + ql;  // stacked (row, head) pair of this lane
    const int r = m / G, hh = m - r * G;
    const int i = i0 + r;
    const bool active = (r < Bq) && (i < S);
    const int hq = g * G + hh;
    uint16_t *orow = O + (((size_t)b * S + (active ? i : 0)) * Hq + hq) * D;

    if (i0 >= L) {  // the whole tile is padding: zero rows
        if (active) {
            for (int c = h * (D / 2); c < (h + 1) * (D / 2); c += 8)
                *reinterpret_cast<uint4 *>(orow + c) = make_uint4(0, 0, 0, 0);
        }
        return;
    }

    const size_t urow = ((size_t)b * Hkv + g) * S;
    const bool live = active && i < L;
    const int i_last = min(i0 + Bq, L) - 1;
    const int nrows = i_last - i0 + 1;
    for (int t = tid; t < nrows; t += kThreads) thr[t] = selkey(tau[urow + i0 + t], (uint32_t)tie[urow + i0 + t]);

    bf16x8 qf[D / 16];
    if (live) {
        const uint16_t *qp = Q + (((size_t)b * S + i) * Hq + hq) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
    } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = bf16x8{};
    }

    const float tau0 = tau[urow + i0];
    const int tie0 = tie[urow + i0];
    const float *dtrow = dt + urow;
    const size_t kvs = (size_t)Hkv * D;
    const uint16_t *Kb = K + (size_t)b * S * kvs + (size_t)g * D;
    const uint16_t *Vb = V + (size_t)b * S * kvs + (size_t)g * D;

    float mrow = -INFINITY, lrow = 0.f;
    f32x16 oacc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};

    // next block, staged in registers: vector v = tid + u*256 is row v / RV,
    // 16-byte column v % RV of both the K and the V tile
    uint4 pk[NL], pv[NL];
    auto load_block = [&](int blk, int n) {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int v = tid + u * kThreads;
            const int pos = blk + v / RV;
            if (pos < n) {
                const size_t off = (size_t)c_idx[pos] * kvs + (v % RV) * 8;
                pk[u] = *reinterpret_cast<const uint4 *>(Kb + off);
                pv[u] = *reinterpret_cast<const uint4 *>(Vb + off);
            } else {
                pk[u] = make_uint4(0, 0, 0, 0);
                pv[u] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_block = [&]() {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int v = tid + u * kThreads;
            const int kk = v / RV, cv = v % RV;
            *reinterpret_cast<uint4 *>(&Ks[kk * T::KP + cv * 8]) = pk[u];
            *reinterpret_cast<uint4 *>(&Vs[kk * T::VP + cv * 8]) = pv[u];
        }
    };

    // Per-lane LDS addresses for the transpose reads of the PV operand: lane
    // l (group (l>>4), index k = l & 15) points at row 4h + k/4 (+16c + 8rr),
    // column 16*((l>>4)&1) + 4*(k&3) (+32t).
    const int tr_k = lane & 15;
    const int tr_off = (4 * h + (tr_k >> 2)) * T::VP + 16 * ((lane >> 4) & 1) + 4 * (tr_k & 3);

    int scan = 0;
    while (scan <= i_last) {
        // ---- fill: compact the candidate keys of this tile into LDS, two
        // consecutive keys per thread, one barrier per 512 keys
        int n = 0, par = 0;
        while (scan <= i_last && n + kFillPer * kThreads <= kCap) {
            const int j0 = scan + kFillPer * tid;
            float dj[kFillPer];
            bool take[kFillPer];
            int cnt = 0;
#pragma unroll
            for (int u = 0; u < kFillPer; ++u) {
                const int j = j0 + u;
                dj[u] = j <= i_last ? dtrow[j] : 0.f;
                take[u] = j <= i_last && ((j > i0) || kept_test(dj[u], j, tau0, tie0));
                cnt += take[u] ? 1 : 0;
            }
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o, 64);
                if (lane >= o) incl += y;
            }
            if (lane == 63) wcnt[par][wave] = incl;
            __syncthreads();
            int off = n + incl - cnt, tot = 0;
#pragma unroll
            for (int w2 = 0; w2 < kThreads / 64; ++w2) {
                const int c = wcnt[par][w2];
                off += (w2 < wave) ? c : 0;
                tot += c;
            }
#pragma unroll
            for (int u = 0; u < kFillPer; ++u) {
                if (take[u]) {
                    c_idx[off] = j0 + u;
                    c_dtl[off] = dj[u];
                    ++off;
                }
            }
            n += tot;
            scan += kFillPer * kThreads;
            par ^= 1;
        }
        __syncthreads();
        // ---- per candidate: the run of tile rows that keep it.  By nesting a
        // key kept by row r is kept by every earlier row >= its own index, so
        // it is kept exactly on rows [lo, lo + span) (offsets from i0).
        const int npad = (n + kBK - 1) / kBK * kBK;
        for (int k = tid; k < npad; k += kThreads) {
            int lo = 0, span = 0;
            float dl = 0.f;
            if (k < n) {
                const int j = c_idx[k];
                const float dv = c_dtl[k];
                lo = j > i0 ? j - i0 : 0;
                span = first_row_above(thr, lo, nrows, selkey(dv, (uint32_t)j)) - lo;
                dl = dv * kLog2e;
            }
            c_lo[k] = lo;
            c_span[k] = span;
            c_dtl[k] = dl;
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

            // mask (row runs), dt bias, online softmax in base 2
            float z[2][16];
            float mloc = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int pos = blk + 32 * kt + 8 * r4 + 4 * h;
                    const int4 lo4 = *reinterpret_cast<const int4 *>(&c_lo[pos]);
                    const int4 sp4 = *reinterpret_cast<const int4 *>(&c_span[pos]);
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
            float psum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = __builtin_amdgcn_exp2f(z[kt][e] - msub);
                    z[kt][e] = p;
                    psum += p;
                }
            }
            lrow += psum;

            // O^T += V^T P^T.  PV call c covers keys 16c..16c+15; lane half h
            // holds, in k-slots 0..7, keys 16c + 8*(j/4) + 4h + j%4, which are
            // exactly its score registers z[c/2][8*(c%2) + j].  The V^T operand
            // comes from two transpose reads (rows 16c + 4h + {0..3} and
            // 16c + 8 + 4h + {0..3}).
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bf16x8 pb;
#pragma unroll
                for (int jx = 0; jx < 8; ++jx) pb[jx] = (__bf16)z[c >> 1][8 * (c & 1) + jx];
#pragma unroll
                for (int t = 0; t < D / 32; ++t) {
                    const uint16_t *vp = &Vs[16 * c * T::VP + 32 * t + tr_off];
                    const i16x4 lo = lds_read_tr16(vp);
                    const i16x4 hi = lds_read_tr16(vp + 8 * T::VP);
                    const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, oacc[t], 0, 0, 0);
                }
            }
            __syncthreads();  // LDS tiles are rewritten next
        }
    }

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

// float32 path: one wave per (batch, query head, row); lanes split head_dim.
// Scans the row's causal keys, applies the kept test and runs the online
// softmax in float32.  Serves the fp32 workloads (small shapes).
template <typename Tin>
__global__ __launch_bounds__(kThreads) void attn_rowwise_kernel(
    const Tin *__restrict__ Q, const Tin *__restrict__ K, const Tin *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, int B, int S, int Hq, int Hkv, int d,
    Tin *__restrict__ O, float qscale) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= (int64_t)B * Hq * S) return;
    const int i = (int)(wid % S);
    const int hq = (int)((wid / S) % Hq);
    const int b = (int)(wid / ((int64_t)S * Hq));
    const int G = Hq / Hkv, g = hq / G;
    const int L = seqlens ? seqlens[b] : S;
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
        const float zz = fmaf(wave_sum(part), qscale, dj * kLog2e);
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

}  // namespace

hipError_t launch_attn(const void *Q, const void *K, const void *V, int dtype, const float *dt,
                       const float *tau, const int32_t *tie, const int32_t *seqlens, int B, int S,
                       int Hq, int Hkv, int d, int w, void *O, hipStream_t stream) {
    (void)w;
    const float qscale = (float)(1.0 / __builtin_sqrt((double)d) * 1.4426950408889634);
    if (dtype == 1) {
        const int G = Hq / Hkv;
        const int Bq = kRowsPerWG / G;
        const int ntiles = (S + Bq - 1) / Bq;
        const int64_t items = (int64_t)ntiles * Hkv * B;
        if (items > 0x7fffffff) return hipErrorInvalidValue;
        const dim3 grid((unsigned)items);
        if (d == 128)
            hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(kThreads), 0, stream,
                               (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, dt, tau,
                               tie, seqlens, S, Hq, Hkv, G, Bq, ntiles, (uint16_t *)O, qscale);
        else
            hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(kThreads), 0, stream,
                               (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, dt, tau,
                               tie, seqlens, S, Hq, Hkv, G, Bq, ntiles, (uint16_t *)O, qscale);
    } else {
        const int64_t waves = (int64_t)B * Hq * S;
        const int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
        hipLaunchKernelGGL(attn_rowwise_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, (const float *)Q, (const float *)K, (const float *)V, dt, tau, tie,
                           seqlens, B, S, Hq, Hkv, d, (float *)O, qscale);
    }
    return hipGetLastError();
}

}  // namespace dma
