// dt for bf16 value states: the per-wave matrix-core tile loop and the
// per-pair path of small calls, shared by dma_dt's kernels and the fused
// prologue kernel.
// Doge guide (gitcode), DMA section, forward step 3: dt_proj over the value
// states of all kv heads of a token (input width Hkv*d, head-major), then
// exp(A * softplus(.)).
#pragma once

#include "common.hpp"

namespace dma {

constexpr int kDtChunk = 128;          // channels per lane group pass (4 lanes x 32)

// softplus and exp on the hardware exp2 / log2: softplus(x) = max(x, 0) +
// ln(1 + e^-|x|) and e^y, with an absolute error in softplus of a few 1e-8
// and a relative error in e^y of about |y| * 2^-23, far inside the float32
// tolerance of dt (which is relative to exp of their product).
__device__ __forceinline__ float dt_from_x(float a, float x) {
    constexpr float kLn2 = 0.6931471805599453f;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    const float sp = fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * kLn2;
    return __builtin_amdgcn_exp2f(a * sp * kLog2e);
}

// One wave takes 16-token tiles first, first + stride, ...  16x16x32 bf16
// operand layouts (l = lane):
//   A[m = l%16][k = 8*(l/16) + j], B[k = 8*(l/16) + j][n = l%16],
//   C[m = 4*(l/16) + i][n = l%16], i = 0..3.
// Channel of k-slot (kg = l/16, j) in step s of chunk c: c*128 + 32*kg + 8*s + j.
// Both operands come straight from global memory (W is small and stays in
// the caches), so no LDS and no barrier stand between the loads and the math.
// CPB chunks of both operands are requested before the first multiply (16 *
// CPB * 2 VGPRs of loads in flight).
template <int CPB>
__device__ __forceinline__ void dt_mfma_tiles(int64_t first, int64_t stride, const uint16_t *__restrict__ V,
                                              const uint16_t *__restrict__ W, const uint16_t *__restrict__ bias,
                                              const float *__restrict__ A, int S, int Hkv, int width, int64_t ntok,
                                              float *__restrict__ out, int64_t ld,
                                              const int32_t *__restrict__ out_pos) {
    const int lane = threadIdx.x & 63;
    const int mr = lane & 15, kg = lane >> 4;
    const int nchunk = (width + kDtChunk - 1) / kDtChunk;
    const bool head_ok = mr < Hkv;
    const int hc = head_ok ? mr : 0;  // clamped head for the (unused) W loads
    const int64_t ntiles = (ntok + 15) / 16;
    const float a_h = A[hc];
    const float b_h = bias ? bf16_to_f32(bias[hc]) : 0.f;
    // this lane's 16-byte vectors of chunks c0 .. c0 + CPB - 1 of
    // its token row and of W's row for head l%16 (zeros past the row, the last
    // token or the last head).  Requests are unconditional from clamped, valid
    // addresses: a conditional load would be a branch of its own.
    uint4 va[CPB][4], wa[CPB][4];
    auto load_batch = [&](int64_t tile, int c0) __attribute__((always_inline)) {
        const int64_t t = tile * 16 + mr;
        const bool tok_ok = t < ntok;
        const uint16_t *vrow = V + (tok_ok ? t : ntok - 1) * (int64_t)width;
        const uint16_t *wrow = W + (size_t)hc * width;
#pragma unroll
        for (int cc = 0; cc < CPB; ++cc) {
            const int base = (c0 + cc) * kDtChunk + 32 * kg;
            const bool in = base < width;
            const int cb = in ? base : width - 32;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint4 x = *reinterpret_cast<const uint4 *>(vrow + cb + 8 * st);
                const uint4 y = *reinterpret_cast<const uint4 *>(wrow + cb + 8 * st);
                va[cc][st] = (tok_ok && in) ? x : make_uint4(0, 0, 0, 0);
                wa[cc][st] = (head_ok && in) ? y : make_uint4(0, 0, 0, 0);
            }
        }
    };

    int64_t tile = first;
    if (tile < ntiles) load_batch(tile, 0);
    for (; tile < ntiles; tile += stride) {
        // batch and column of this lane's four output tokens, out_pos loaded
        // now so that its latency hides behind the products
        int ob[4], os[4];
        int64_t ocol[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t tok = tile * 16 + 4 * kg + i;
            const int64_t tc = tok < ntok ? tok : ntok - 1;
            ob[i] = ntok <= 0x7fffffff ? (int)((uint32_t)tc / (uint32_t)S) : (int)(tc / S);
            os[i] = (int)(tc - (int64_t)ob[i] * S);
            ocol[i] = out_pos ? (int64_t)out_pos[ob[i]] : 0;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nchunk; c0 += CPB) {
            if (c0 > 0) load_batch(tile, c0);  // the first batch is already in flight
#pragma unroll
            for (int cc = 0; cc < CPB; ++cc) {
                if (c0 + cc >= nchunk) break;
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va[cc][st]),
                                                                  __builtin_bit_cast(bf16x8, wa[cc][st]), acc, 0, 0, 0);
            }
        }
        if (tile + stride < ntiles) load_batch(tile + stride, 0);  // next tile's rows in flight
        if (head_ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tok = tile * 16 + 4 * kg + i;
                // a column outside [0, ld) (an out_pos past the row) is not written
                if (tok < ntok && (uint64_t)(ocol[i] + os[i]) < (uint64_t)ld)
                    out[((int64_t)ob[i] * Hkv + mr) * ld + ocol[i] + os[i]] = dt_from_x(a_h, acc[i] + b_h);
            }
        }
    }
}

// A few tokens (a decode step's append form): dt of pair wid = token * Hkv +
// head by one wave, the dot product of the width-long rows of V and W split
// over the lanes in 16-byte vectors, all loaded before any is used, a
// butterfly sum, then softplus and exp as on the matrix-core path.  Calls with
// at most kDtSmallTokens tokens take this path in dma_dt and in the fused
// prologue alike, so both give the same bits.  Width <= 16 heads x 128.
constexpr int kDtSmallTokens = 256;
__device__ __forceinline__ void dt_pair(int64_t wid, const uint16_t *__restrict__ V, const uint16_t *__restrict__ W,
                                        const uint16_t *__restrict__ bias, const float *__restrict__ A, int S,
                                        int Hkv, int width, float *__restrict__ out, int64_t ld,
                                        const int32_t *__restrict__ out_pos) {
    constexpr int kMaxVec = 16 * 128 / 8 / 64;  // vectors per lane at the widest row
    const int lane = threadIdx.x & 63;
    const int64_t t = wid / Hkv;
    const int h = (int)(wid - t * Hkv);
    const int b = (int)(t / S), s = (int)(t - (int64_t)b * S);
    const int64_t col = (out_pos ? (int64_t)out_pos[b] : 0) + s;
    const float a_h = A[h];  // requested with the rows, not after the sum
    const float b_h = bias ? bf16_to_f32(bias[h]) : 0.f;
    const int nvec = width / 8;
    const uint4 *vrow = reinterpret_cast<const uint4 *>(V + t * width);
    const uint4 *wrow = reinterpret_cast<const uint4 *>(W + (size_t)h * width);
    uint4 vv[kMaxVec], wv[kMaxVec];
#pragma unroll
    for (int u = 0; u < kMaxVec; ++u) {
        const int v = lane + 64 * u;
        vv[u] = v < nvec ? vrow[v] : make_uint4(0, 0, 0, 0);
        wv[u] = v < nvec ? wrow[v] : make_uint4(0, 0, 0, 0);
    }
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kMaxVec; ++u) {
        const uint32_t a[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        const uint32_t c[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc = fmaf(__uint_as_float(a[k] << 16), __uint_as_float(c[k] << 16), acc);
            acc = fmaf(__uint_as_float(a[k] & 0xffff0000u), __uint_as_float(c[k] & 0xffff0000u), acc);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0 && (uint64_t)col < (uint64_t)ld) out[((int64_t)b * Hkv + h) * ld + col] = dt_from_x(a_h, acc + b_h);
}

}  // namespace dma
