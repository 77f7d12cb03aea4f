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
// the K rows (row-major) and V rows (transposed, keys permuted to match the
// score accumulator layout) into LDS, S^T = K Q^T on 32x32x16 bf16 MFMA, the
// exact per-row kept test and the dt bias in registers, an online softmax in
// base 2, and O^T += V^T P^T on MFMA with P rounded once to bf16.  Only
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
constexpr int kSeg = kThreads;   // keys scanned per fill step

template <int D>
struct Tiles {
    static constexpr int KP = D + 8;    // K tile pitch (bf16), 16-byte pad
    static constexpr int VP = kBK + 8;  // V^T tile pitch (bf16)
};

// LDS column of block-local key u inside the transposed V tile: within each
// 16-key group the order is [0..3, 8..11, 4..7, 12..15], so that lane half h
// of PV call c reads its 8 keys 16c + {4h..4h+3, 8+4h..8+4h+3} as one 16-byte
// vector at column 16c + 8h.
__device__ __forceinline__ int vt_col(int u) {
    const int grp = u >> 4, v = u & 15;
    return 16 * grp + 8 * ((v >> 2) & 1) + 4 * (v >> 3) + (v & 3);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ dt, const float *__restrict__ tau, const int32_t *__restrict__ tie,
    const int32_t *__restrict__ seqlens, int S, int Hq, int Hkv, int G, int Bq,
    uint16_t *__restrict__ O, float qscale) {
    using T = Tiles<D>;
    __shared__ __align__(16) int c_idx[kCap];
    __shared__ __align__(16) float c_dt[kCap];
    __shared__ __align__(16) uint16_t Ks[kBK * T::KP];
    __shared__ __align__(16) uint16_t Vt[D * T::VP];
    __shared__ int wcnt[kThreads / 64];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane >> 5, ql = lane & 31;
    const int g = blockIdx.y, b = blockIdx.z;
    const int i0 = blockIdx.x * Bq;
    const int L = seqlens ? seqlens[b] : S;

    const int m = wave * 32 + ql;  // stacked pair
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
    const float tau_i = live ? tau[urow + i] : INFINITY;
    const int tie_i = live ? tie[urow + i] : -1;

    bf16x8 qf[D / 16];
    if (live) {
        const uint16_t *qp = Q + (((size_t)b * S + i) * Hq + hq) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
    } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = bf16x8{};
    }

    const int i_last = min(i0 + Bq, L) - 1;
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

    int scan = 0;
    while (scan <= i_last) {
        // ---- fill: compact the candidate keys of this tile into LDS
        int n = 0;
        while (scan <= i_last && n + kSeg <= kCap) {
            const int j = scan + tid;
            bool take = false;
            float dj = 0.f;
            if (j <= i_last) {
                dj = dtrow[j];
                take = (j > i0) || kept_test(dj, j, tau0, tie0);
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
            scan += kSeg;
            __syncthreads();
        }

        // ---- attend over the candidates, 64 keys at a time
        for (int blk = 0; blk < n; blk += kBK) {
            // K rows, row-major
            for (int v = tid; v < kBK * D / 8; v += kThreads) {
                const int kk = v / (D / 8), cv = v % (D / 8);
                const int pos = blk + kk;
                uint4 val = make_uint4(0, 0, 0, 0);
                if (pos < n) val = *reinterpret_cast<const uint4 *>(Kb + (size_t)c_idx[pos] * kvs + cv * 8);
                *reinterpret_cast<uint4 *>(&Ks[kk * T::KP + cv * 8]) = val;
            }
            // V rows, transposed, two keys per 32-bit LDS store
            for (int v = tid; v < (kBK / 2) * (D / 8); v += kThreads) {
                const int pr = v / (D / 8), cv = v % (D / 8);
                const int u0 = 2 * pr;
                const int pos0 = blk + u0;
                uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
                if (pos0 < n) a = *reinterpret_cast<const uint4 *>(Vb + (size_t)c_idx[pos0] * kvs + cv * 8);
                if (pos0 + 1 < n) c = *reinterpret_cast<const uint4 *>(Vb + (size_t)c_idx[pos0 + 1] * kvs + cv * 8);
                const int col = vt_col(u0);
                const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
                const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const uint32_t lo = (aw[e2] & 0xffffu) | (cw[e2] << 16);
                    const uint32_t hi = (aw[e2] >> 16) | (cw[e2] & 0xffff0000u);
                    *reinterpret_cast<uint32_t *>(&Vt[(cv * 8 + 2 * e2) * T::VP + col]) = lo;
                    *reinterpret_cast<uint32_t *>(&Vt[(cv * 8 + 2 * e2 + 1) * T::VP + col]) = hi;
                }
            }
            __syncthreads();

            // S^T = K Q^T for two 32-key halves of the block
            f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&Ks[(32 * kt + ql) * T::KP + 16 * ks + 8 * h]);
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kt], 0, 0, 0);
                }
            }

            // mask, dt bias, online softmax (base 2)
            float z[2][16];
            float mloc = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int pos = blk + 32 * kt + 8 * r4 + 4 * h;
                    const int4 jj = *reinterpret_cast<const int4 *>(&c_idx[pos]);
                    const float4 dd = *reinterpret_cast<const float4 *>(&c_dt[pos]);
                    const int js[4] = {jj.x, jj.y, jj.z, jj.w};
                    const float ds[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = (pos + e < n) && (js[e] <= i) && kept_test(ds[e], js[e], tau_i, tie_i);
                        const float zz = ok ? fmaf(sacc[kt][4 * r4 + e], qscale, ds[e] * kLog2e) : -INFINITY;
                        z[kt][4 * r4 + e] = zz;
                        mloc = fmaxf(mloc, zz);
                    }
                }
            }
            const float mnew = fmaxf(mrow, half_swap_max(mloc));
            const bool none = (mnew == -INFINITY);
            const float msub = none ? 0.f : mnew;
            const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(mrow - mnew);
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
            lrow = lrow * alpha + psum;
            mrow = mnew;
#pragma unroll
            for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;

            // O^T += V^T P^T
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bf16x8 pb;
#pragma unroll
                for (int jx = 0; jx < 8; ++jx) pb[jx] = (__bf16)z[c >> 1][8 * (c & 1) + jx];
#pragma unroll
                for (int t = 0; t < D / 32; ++t) {
                    const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&Vt[(32 * t + ql) * T::VP + 16 * c + 8 * h]);
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, oacc[t], 0, 0, 0);
                }
            }
            __syncthreads();  // LDS tiles and candidates are rewritten next
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
        const dim3 grid((S + Bq - 1) / Bq, Hkv, B);
        if (d == 128)
            hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(kThreads), 0, stream,
                               (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, dt, tau,
                               tie, seqlens, S, Hq, Hkv, G, Bq, (uint16_t *)O, qscale);
        else
            hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(kThreads), 0, stream,
                               (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, dt, tau,
                               tie, seqlens, S, Hq, Hkv, G, Bq, (uint16_t *)O, qscale);
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
