// Incremental decode: the kept set of each (batch, kv head) carried across
// decode steps, with its K/V rows stored compactly.
// Doge guide (gitcode), DMA section: at inference the mask keeps, for the
// query at position p, the keep_window_size (w) keys of largest dt among the
// positions <= p (forward step 3), and attends over them with the dt bias
// (step 4).  Under the order (dt desc, index asc) the kept sets nest:
// kept(p) is a subset of kept(p-1) plus {p}.  So a step admits the new key
// iff fewer than w keys are kept or it beats the worst kept key (a new key
// tying that key's dt loses: its index is the largest), and then evicts that
// worst key.  The state holds, per (batch, kv head), the kept keys'
// selection keys, positions and K/V rows in w slots, and which slot holds
// the worst key; a step costs the w kept rows instead of a pass over the
// whole cache's dt.
//
// State (caller-owned device memory, decode_state_bytes(), bf16 K/V):
//   hdr  [B][Hkv] {n kept, cache length, slot of the worst kept key, its key}
//   keys [B][Hkv][w] uint64 selection key (dt order bits << 32 | ~position)
//   pos  [B][Hkv][w] int32 position
//   K, V [B][Hkv][w][d] bf16 rows
// A step (two launches):
//  1. attend: one workgroup per (range of slots, kv head, batch) reads the
//     header, decides the admission of the new key (which slot it takes,
//     if any) and attends over its slots with the new row in place of the
//     slot it takes: K straight into the score MFMA's operand registers, V
//     through LDS, 32-slot blocks per wave with the next in flight, as the
//     cache-scanning decode; one partial (max, sum, output) per query head,
//     and the smallest key of its range after the step.
//  2. combine: merges the partials of each (batch, query head) into the
//     output; the workgroup of the first query head of each kv head then
//     writes the admitted key into its slot and takes the new worst key
//     from the range minima.
#include "common.hpp"
#include "launch.hpp"

namespace dma {
namespace {

constexpr int kThreads = 256;
constexpr int kInitThreads = 1024;
constexpr int kInitItems = 8;             // consecutive positions per init thread per chunk
constexpr int kMaxSlotsPerWG = 2048;      // slots one attend workgroup covers
constexpr int kTargetWGs = 512;           // attend workgroups a step aims for

struct BgHdr {
    int32_t n;         // kept keys (slots in use)
    int32_t len;       // cache length: the next position
    int32_t min_slot;  // slot of the worst kept key (when n > 0)
    int32_t pad;
    uint64_t min_key;  // its selection key
};

struct StateLayout {
    size_t hdr, keys, pos, K, V, total;
};

inline StateLayout state_layout(int B, int Hkv, int d, int w) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t nbg = (size_t)B * Hkv;
    StateLayout l;
    l.hdr = 0;
    l.keys = up(l.hdr + sizeof(BgHdr) * nbg);
    l.pos = up(l.keys + sizeof(uint64_t) * nbg * w);
    l.K = up(l.pos + sizeof(int32_t) * nbg * w);
    l.V = up(l.K + sizeof(uint16_t) * nbg * w * d);
    l.total = up(l.V + sizeof(uint16_t) * nbg * w * d);
    return l;
}

inline int max_parts(int w) { return (w + 63) / 64; }

struct StepWs {
    size_t pm, pl, po, pk, ps, total;
};

inline StepWs step_ws_layout(int B, int Hq, int Hkv, int d, int w) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t np = (size_t)max_parts(w);
    StepWs l;
    l.pm = 0;
    l.pl = up(l.pm + sizeof(float) * B * Hq * np);
    l.po = up(l.pl + sizeof(float) * B * Hq * np);
    l.pk = up(l.po + sizeof(float) * B * Hq * np * d);
    l.ps = up(l.pk + sizeof(uint64_t) * B * Hkv * np);
    l.total = up(l.ps + sizeof(int32_t) * B * Hkv * np);
    // state initialisation borrows the start of the workspace for thresholds
    if (l.total < up(sizeof(uint64_t) * B * Hkv)) l.total = up(sizeof(uint64_t) * B * Hkv);
    return l;
}

// Attend workgroups per (batch, kv head) for n kept slots.
inline int parts_for(int B, int Hkv, int w) {
    int p = (kTargetWGs + B * Hkv - 1) / (B * Hkv);
    const int need = (w + kMaxSlotsPerWG - 1) / kMaxSlotsPerWG;  // LDS bound on slots per workgroup
    if (p < need) p = need;
    if (p > max_parts(w)) p = max_parts(w);
    return p < 1 ? 1 : p;
}

// The dt value of a selection key (exact; -0 was folded into +0).
__device__ __forceinline__ float key_dt(uint64_t key) {
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Admission of the new key at position len: the slot it takes (-1: none)
// and the number of kept keys after the step.
__device__ __forceinline__ int admit(const BgHdr &h, uint64_t key_new, int w, int &n_after) {
    if (h.n < w) {
        n_after = h.n + 1;
        return h.n;
    }
    n_after = h.n;
    return key_new > h.min_key ? h.min_slot : -1;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

// Block-wide exclusive scan of one value per thread (kInitThreads threads).
__device__ __forceinline__ uint32_t init_excl_scan(uint32_t v, uint32_t &total, uint32_t *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kInitThreads / 64; ++k) {
        const uint32_t c = red[k];
        off += k < wave ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return off + incl - v;
}

// Smallest key (and its slot) over slots [0, n) of one (batch, kv head),
// the key of slot `sub` read as `key_sub`; every thread of the block (nt
// threads, a multiple of 64) gets it.
__device__ __forceinline__ void worst_key(const uint64_t *keys, int n, int sub, uint64_t key_sub, int nt,
                                          uint64_t &kmin, int &smin, uint64_t *red_k, int *red_s) {
    constexpr int kBatch = 16;  // keys per thread whose loads are in flight together
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t mk = ~0ull;
    int ms = -1;
    for (int s0 = threadIdx.x; s0 < n; s0 += nt * kBatch) {
        uint64_t k[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) k[u] = keys[min(s0 + u * nt, n - 1)];  // past n: a repeat, skipped below
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int s = s0 + u * nt;
            const uint64_t ku = s == sub ? key_sub : k[u];
            if (s < n && ku < mk) {
                mk = ku;
                ms = s;
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)mk, o, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(mk >> 32), o, 64);
        const int os = __shfl_xor(ms, o, 64);
        const uint64_t ok = ((uint64_t)hi << 32) | lo;
        if (ok < mk) {
            mk = ok;
            ms = os;
        }
    }
    if (lane == 0) {
        red_k[wave] = mk;
        red_s[wave] = ms;
    }
    __syncthreads();
    kmin = ~0ull;
    smin = -1;
    for (int q = 0; q < nt / 64; ++q) {
        if (red_k[q] < kmin) {
            kmin = red_k[q];
            smin = red_s[q];
        }
    }
}

// ---------------------------------------------------------------- init ----
// One workgroup per (kv head, batch): the kept positions of the cache (those
// at or above the threshold key from the exact selector) into slots 0..n-1 in
// ascending order, with their K/V rows, then the worst kept key.
__global__ __launch_bounds__(kInitThreads) void state_init_kernel(
    const uint16_t *__restrict__ Kc, const uint16_t *__restrict__ Vc, const float *__restrict__ dt_cache,
    const int32_t *__restrict__ cache_lens, int Lmax, int Hkv, int d, int w, const uint64_t *__restrict__ thr_ws,
    BgHdr *__restrict__ hdr, uint64_t *__restrict__ keys, int32_t *__restrict__ pos, uint16_t *__restrict__ Ks,
    uint16_t *__restrict__ Vs) {
    constexpr int kChunk = kInitThreads * kInitItems;
    __shared__ int list[kChunk];
    __shared__ uint32_t red[kInitThreads / 64];
    __shared__ uint64_t red_k[kInitThreads / 64];
    __shared__ int red_s[kInitThreads / 64];
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const size_t bg = (size_t)b * Hkv + g;
    const int L = clamp_len(cache_lens, b, Lmax);
    const uint64_t thr = thr_ws[bg];
    const float *row = dt_cache + bg * Lmax;
    uint64_t *kb = keys + bg * w;
    int32_t *pb = pos + bg * w;
    uint16_t *Kb = Ks + bg * w * d;
    uint16_t *Vb = Vs + bg * w * d;
    const int RV = d / 8;
    int running = 0;
    for (int j0 = 0; j0 < L; j0 += kChunk) {
        uint64_t k[kInitItems];
        uint32_t c = 0;
#pragma unroll
        for (int u = 0; u < kInitItems; ++u) {
            const int j = j0 + tid * kInitItems + u;
            k[u] = j < L ? selkey(row[j], (uint32_t)j) : 0ull;
            c += (j < L && k[u] >= thr) ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t off = init_excl_scan(c, tot, red);
#pragma unroll
        for (int u = 0; u < kInitItems; ++u) {
            const int j = j0 + tid * kInitItems + u;
            if (j < L && k[u] >= thr) {
                const int slot = running + (int)off;
                kb[slot] = k[u];
                pb[slot] = j;
                list[off] = j;
                ++off;
            }
        }
        __syncthreads();
        for (int x = tid; x < (int)tot * RV; x += kInitThreads) {
            const int r = x / RV, cv = x - r * RV;
            const int j = list[r];
            const size_t src = ((size_t)b * Lmax + j) * Hkv * d + (size_t)g * d + 8 * cv;
            const size_t dst = (size_t)(running + r) * d + 8 * cv;
            *reinterpret_cast<u32x4 *>(Kb + dst) = *reinterpret_cast<const u32x4 *>(Kc + src);
            *reinterpret_cast<u32x4 *>(Vb + dst) = *reinterpret_cast<const u32x4 *>(Vc + src);
        }
        running += (int)tot;
        __syncthreads();  // the list is rewritten next
    }
    uint64_t kmin = 0;
    int smin = -1;
    if (running > 0) {
        // the keys just written are read back by other threads of this block
        __threadfence_block();
        __syncthreads();
        worst_key(kb, running, -1, 0ull, kInitThreads, kmin, smin, red_k, red_s);
    }
    if (tid == 0) {
        BgHdr h;
        h.n = running;
        h.len = L;
        h.min_slot = smin;
        h.pad = 0;
        h.min_key = kmin;
        hdr[bg] = h;
    }
}

// ---------------------------------------------------------------- attend --
template <int D>
__global__ __launch_bounds__(kThreads, 2) void state_attend_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    const float *__restrict__ dt_new, int Hq, int Hkv, int w, const BgHdr *__restrict__ hdr,
    const uint64_t *__restrict__ keys, const uint16_t *__restrict__ Ks, const uint16_t *__restrict__ Vs,
    float *__restrict__ pm, float *__restrict__ pl, float *__restrict__ po, uint64_t *__restrict__ pk,
    int32_t *__restrict__ ps, float qscale) {
    constexpr int NW = kThreads / 64;
    constexpr int KB = 32;          // slots per wave block
    constexpr int NS = D / 32;      // 32-wide head_dim slices
    constexpr int KP = D + 8;       // V row pitch in LDS (bf16)
    constexpr int RV = D / 8;       // 16-byte vectors per row
    constexpr int NU = KB * RV / 64;
    constexpr int NT = D / 16;      // output column tiles
    constexpr int NK = 2 * NS;
    static_assert(NW * KB * KP * 2 >= NW * 16 * D * 4, "the merge buffer fits in the row regions");
    __shared__ float l_dtl[kMaxSlotsPerWG];
    __shared__ __align__(16) uint16_t Vw[NW][KB * KP];
    __shared__ float mw[NW][16], lw[NW][16];
    __shared__ uint64_t red_k[NW];
    __shared__ int red_s[NW];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int nsplit = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int G = Hq / Hkv;
    const int col = lane & 15, grp = lane >> 4;
    const size_t bg = (size_t)b * Hkv + g;
    // the workgroup's range of slots does not depend on the header (only
    // its first n slots are kept), so its first requests need not wait for it
    const int per = (w + nsplit - 1) / nsplit;
    const int s0 = min(split * per, w);
    const int cnt_all = min(per, w - s0);
    const uint64_t *kb_keys = keys + bg * w;
    const uint16_t *Kb = Ks + bg * w * D;
    const uint16_t *Vb = Vs + bg * w * D;
    const uint16_t *kn_row = k_new + bg * D;
    const uint16_t *vn_row = v_new + bg * D;
    uint16_t *vw = Vw[wave];

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
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[t] = f32x4{};

    // rows of block kb (slot offsets from s0): K as the score MFMA's A
    // operand (lane (col, grp): slot 16c + col, columns 32s + 8grp .. +7), V
    // as whole rows for LDS (vector v = lane + 64u: row v / RV, column v % RV);
    // the admitted slot reads the new token's row
    u32x4 kr[NK], vr[NU], kn[NK], vn[NU];
    // slot offset x of a range of c slots, slot a holding the new token
    auto row_of = [&](const uint16_t *base, const uint16_t *nrow, int x, int c, int a) __attribute__((always_inline)) {
        const int s = s0 + min(x, c - 1);
        return s == a ? nrow : base + (size_t)s * D;
    };
    auto load_rows_of = [&](u32x4 (&kx)[NK], u32x4 (&vx)[NU], int kb, int c, int a) __attribute__((always_inline)) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const uint16_t *kp = row_of(Kb, kn_row, kb + 16 * cc + col, c, a);
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) kx[cc * NS + s2] = *reinterpret_cast<const u32x4 *>(kp + 32 * s2 + 8 * grp);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const uint16_t *vp = row_of(Vb, vn_row, kb + (lane + 64 * u) / RV, c, a);
            vx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + ((lane + 64 * u) % RV) * 8));
        }
    };
    // requested before the header: this wave's first block as if every slot
    // of the range were kept and none admitted, and the range's keys
    constexpr int KPT = kMaxSlotsPerWG / kThreads;
    int kb = wave * KB;
    if (kb < cnt_all) load_rows_of(kr, vr, kb, cnt_all, -1);
    uint64_t kv[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (i * kThreads < cnt_all) kv[i] = kb_keys[s0 + min(tid + i * kThreads, cnt_all - 1)];

    const BgHdr h = hdr[bg];
    const float dtn = dt_new[bg];
    const uint64_t key_new = selkey(dtn, (uint32_t)h.len);
    int n;
    const int adm = admit(h, key_new, w, n);
    const int cnt = max(0, min(n - s0, cnt_all));  // kept slots of the range after the step
    auto load_rows = [&](u32x4 (&kx)[NK], u32x4 (&vx)[NU], int kb) __attribute__((always_inline)) {
        load_rows_of(kx, vx, kb, cnt, adm);
    };
    // the first block again where the guess was wrong: it holds the admitted
    // slot, or slots past the kept ones (whose rows are not defined)
    if (kb < cnt && ((cnt != cnt_all && kb + KB > cnt) || (unsigned)(adm - (s0 + kb)) < (unsigned)KB))
        load_rows(kr, vr, kb);
    auto block = [&](const u32x4 (&kx)[NK], const u32x4 (&vx)[NU], int kb) __attribute__((always_inline)) {
        const int nb = min(KB, cnt - kb);
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
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kx[c * NS + s]), qf[s], sacc,
                                                               0, 0, 0);
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
    // the dt bias of the range's kept slots; the same pass finds the
    // smallest key of the range after the step (the admitted slot holding the
    // new key), the candidate for the next eviction
    uint64_t mk = ~0ull;
    int ms = -1;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int x = tid + i * kThreads;
        if (x < cnt) {
            const int s = s0 + x;
            const uint64_t ku = s == adm ? key_new : kv[i];
            l_dtl[x] = (s == adm ? dtn : key_dt(ku)) * kLog2e;
            if (ku < mk) {
                mk = ku;
                ms = s;
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)mk, o, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(mk >> 32), o, 64);
        const int os = __shfl_xor(ms, o, 64);
        const uint64_t ok = ((uint64_t)hi << 32) | lo;
        if (ok < mk) {
            mk = ok;
            ms = os;
        }
    }
    if (lane == 0) {
        red_k[wave] = mk;
        red_s[wave] = ms;
    }
    __syncthreads();  // l_dtl and the per-wave minima visible
    if (tid == 0) {
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) {
            if (red_k[w2] < mk) {
                mk = red_k[w2];
                ms = red_s[w2];
            }
        }
        pk[bg * nsplit + split] = mk;
        ps[bg * nsplit + split] = ms;
    }

    // this wave's blocks: kb = (wave + NW*k) * KB, two register sets in turn;
    // the next block is requested unconditionally (offsets clamp to the last
    // slot), so no request waits on a branch
    if (kb < cnt) {
        for (;;) {
            load_rows(kn, vn, kb + NW * KB);
            block(kr, vr, kb);
            kb += NW * KB;
            if (kb >= cnt) break;
            load_rows(kr, vr, kb + NW * KB);
            block(kn, vn, kb);
            kb += NW * KB;
            if (kb >= cnt) break;
        }
    }

    // merge the four waves into one partial per query head
    __syncthreads();  // the V regions are reused below
    float *om = reinterpret_cast<float *>(&Vw[0][0]);  // [NW][16][D]
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

// ------------------------------------------------------ combine + update --
// One workgroup per (batch, kv head), min(G * d, 1024) threads, a thread per
// (query head, output element) in turn: merges the partials into the output.  Then the
// step is applied to the state: the admitted key into its slot, the worst
// kept key taken from the attend workgroups' range minima (wave 0), the
// length advanced.
__global__ __launch_bounds__(1024) void state_combine_kernel(
    const float *__restrict__ pm, const float *__restrict__ pl, const float *__restrict__ po,
    const uint64_t *__restrict__ pk, const int32_t *__restrict__ ps, int nchunk, int d, int Hq, int Hkv, int w,
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new, const float *__restrict__ dt_new,
    BgHdr *__restrict__ hdr, uint64_t *__restrict__ keys, int32_t *__restrict__ pos, uint16_t *__restrict__ Ks,
    uint16_t *__restrict__ Vs, uint16_t *__restrict__ out) {
    constexpr int kGroup = 8;
    const size_t bg = blockIdx.x;  // b * Hkv + g
    const int tid = threadIdx.x, lane = tid & 63;
    const int G = Hq / Hkv;
    // the step's own inputs depend on nothing the merge computes: requested
    // together with the partials
    const BgHdr h = hdr[bg];
    const float dtn = dt_new[bg];
    const int ec = min(tid, d - 1);
    const uint16_t kn = k_new[bg * d + ec], vn = v_new[bg * d + ec];
    uint64_t mk = ~0ull;
    int ms = -1;
    if (tid < 64) {
        for (int x = lane; x < nchunk; x += 64) {
            const uint64_t k = pk[bg * nchunk + x];
            const int sl = ps[bg * nchunk + x];
            if (k < mk) {
                mk = k;
                ms = sl;
            }
        }
    }

    for (int x = tid; x < G * d; x += blockDim.x) {
        const int hh = x / d, e = x - hh * d;
        const size_t bh = bg * G + hh;  // b * Hq + g * G + hh
        const float *m = pm + bh * nchunk;
        const float *l = pl + bh * nchunk;
        const float *o = po + bh * nchunk * d + e;
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
            if (Mn == -INFINITY) continue;
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
        out[bh * d + e] = f32_to_bf16(den > 0.f ? num / den : 0.f);
    }

    const uint64_t key_new = selkey(dtn, (uint32_t)h.len);
    int n;
    const int adm = admit(h, key_new, w, n);
    if (adm >= 0) {
        const size_t dst = (bg * w + adm) * d;
        if (tid < d) {
            Ks[dst + tid] = kn;
            Vs[dst + tid] = vn;
        }
        if (tid == 0) {
            keys[bg * w + adm] = key_new;
            pos[bg * w + adm] = h.len;
        }
    }
    if (tid < 64) {
#pragma unroll
        for (int o2 = 32; o2 >= 1; o2 >>= 1) {
            const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)mk, o2, 64);
            const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(mk >> 32), o2, 64);
            const int os = __shfl_xor(ms, o2, 64);
            const uint64_t ok = ((uint64_t)hi << 32) | lo;
            if (ok < mk) {
                mk = ok;
                ms = os;
            }
        }
        if (tid == 0) {
            BgHdr nh;
            nh.n = n;
            nh.len = h.len + 1;
            nh.min_slot = ms;
            nh.pad = 0;
            nh.min_key = mk;
            hdr[bg] = nh;
        }
    }
}

// Kept positions (slot order) of every (batch, kv head), padded with -1.
__global__ __launch_bounds__(kThreads) void state_kept_kernel(const BgHdr *__restrict__ hdr,
                                                               const int32_t *__restrict__ pos, int Hkv, int w,
                                                               int32_t *__restrict__ kept_idx,
                                                               int32_t *__restrict__ lens) {
    const int g = blockIdx.x, b = blockIdx.y;
    const size_t bg = (size_t)b * Hkv + g;
    const BgHdr h = hdr[bg];
    for (int s = threadIdx.x; s < w; s += kThreads) kept_idx[bg * w + s] = s < h.n ? pos[bg * w + s] : -1;
    if (lens && threadIdx.x == 0) lens[bg] = h.len;
}

}  // namespace

size_t decode_state_bytes(int B, int Hkv, int d, int w) { return state_layout(B, Hkv, d, w).total; }

size_t decode_step_ws_bytes(int B, int Hq, int Hkv, int d, int w) {
    return step_ws_layout(B, Hq, Hkv, d, w).total;
}

hipError_t launch_decode_state_init(const void *Kc, const void *Vc, const float *dt_cache, const int32_t *cache_lens,
                                    int B, int Lmax, int Hkv, int d, int w, void *state, void *ws,
                                    hipStream_t stream) {
    const StateLayout sl = state_layout(B, Hkv, d, w);
    char *st = (char *)state;
    uint64_t *thr = (uint64_t *)ws;
    hipError_t e = launch_decode_thresholds(dt_cache, cache_lens, B, Lmax, Hkv, w, thr, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(state_init_kernel, dim3(Hkv, B), dim3(kInitThreads), 0, stream, (const uint16_t *)Kc,
                       (const uint16_t *)Vc, dt_cache, cache_lens, Lmax, Hkv, d, w, thr, (BgHdr *)(st + sl.hdr),
                       (uint64_t *)(st + sl.keys), (int32_t *)(st + sl.pos), (uint16_t *)(st + sl.K),
                       (uint16_t *)(st + sl.V));
    return hipGetLastError();
}

hipError_t launch_decode_step(const void *q, const void *k_new, const void *v_new, const float *dt_new, int B,
                              int Hq, int Hkv, int d, int w, void *state, void *out, void *ws, hipStream_t stream) {
    const StateLayout sl = state_layout(B, Hkv, d, w);
    const StepWs wl = step_ws_layout(B, Hq, Hkv, d, w);
    char *st = (char *)state;
    char *wsb = (char *)ws;
    BgHdr *hdr = (BgHdr *)(st + sl.hdr);
    uint64_t *keys = (uint64_t *)(st + sl.keys);
    int32_t *pos = (int32_t *)(st + sl.pos);
    uint16_t *Ks = (uint16_t *)(st + sl.K);
    uint16_t *Vs = (uint16_t *)(st + sl.V);
    float *pm = (float *)(wsb + wl.pm), *pl = (float *)(wsb + wl.pl), *po = (float *)(wsb + wl.po);
    uint64_t *pk = (uint64_t *)(wsb + wl.pk);
    int32_t *ps = (int32_t *)(wsb + wl.ps);
    const float qscale = (float)(1.0 / __builtin_sqrt((double)d) * 1.4426950408889634);
    const int nparts = parts_for(B, Hkv, w);
    const dim3 grid(nparts, Hkv, B);
    if (d == 128)
        hipLaunchKernelGGL(state_attend_kernel<128>, grid, dim3(kThreads), 0, stream, (const uint16_t *)q,
                           (const uint16_t *)k_new, (const uint16_t *)v_new, dt_new, Hq, Hkv, w, hdr, keys, Ks, Vs,
                           pm, pl, po, pk, ps, qscale);
    else
        hipLaunchKernelGGL(state_attend_kernel<64>, grid, dim3(kThreads), 0, stream, (const uint16_t *)q,
                           (const uint16_t *)k_new, (const uint16_t *)v_new, dt_new, Hq, Hkv, w, hdr, keys, Ks, Vs,
                           pm, pl, po, pk, ps, qscale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(state_combine_kernel, dim3(B * Hkv), dim3(min(Hq / Hkv * d, 1024)), 0, stream, pm, pl, po, pk,
                       ps, nparts, d, Hq, Hkv, w, (const uint16_t *)k_new, (const uint16_t *)v_new, dt_new, hdr, keys, pos, Ks, Vs,
                       (uint16_t *)out);
    return hipGetLastError();
}

hipError_t launch_decode_state_kept(const void *state, int B, int Hkv, int d, int w, int32_t *kept_idx,
                                    int32_t *lens, hipStream_t stream) {
    const StateLayout sl = state_layout(B, Hkv, d, w);
    const char *st = (const char *)state;
    hipLaunchKernelGGL(state_kept_kernel, dim3(Hkv, B), dim3(kThreads), 0, stream, (const BgHdr *)(st + sl.hdr),
                       (const int32_t *)(st + sl.pos), Hkv, w, kept_idx, lens);
    return hipGetLastError();
}

}  // namespace dma
