// select.hip -- index producer: the selection branch's block lists from
// compressed attention.
//
// The pages name the module's arguments (Flash-Sparse-Attention project
// page, "Quick start", step 2): compressed keys with kernel size 32 and
// stride 16, selection blocks of 64 tokens, topk blocks per list, one init
// block and two local blocks, but print no formula; each step below is the
// plainest reading of its name:
//   - compressed key of window c (positions [16c, 16c + 32) of a sequence):
//     the mean of the window's k rows, summed in fp32 in position order and
//     rounded to the 16-bit input format;
//   - compressed attention of query (t, qh): softmax over the windows that
//     end at or before t, of scale * q . kc;
//   - importance of block j for (t, kv head h): the probabilities of the
//     windows overlapping j (window c overlaps blocks c / 4 and, for
//     c % 4 == 3, c / 4 + 1), summed over the G query heads of h;
//   - list: init blocks, local blocks b, b-1, then the most important other
//     blocks of [0, b] (ties: lower id), -1 after them.
//
// Kernels: prep (window and tile offsets per sequence), compress (one thread
// per window, kv head and 8 channels), select (one workgroup per 16 tokens
// of a sequence and kv head: two passes over the visible windows in chunks
// of 64 -- row log-sum-exp, then the probabilities binned into the blocks in
// LDS -- then a wave-wide arg-max per list slot), orphans (rows of tokens
// outside every sequence).  Every sum has a fixed order: the lists are
// bitwise reproducible.
#include "device_common.h"

namespace nsa {

namespace {

constexpr int kSelTok = 16;          // tokens per workgroup
constexpr int kSelChunk = 64;        // compressed windows per chunk (16 blocks)
constexpr int kSelKs = 32, kSelStride = 16, kSelBs = 64;
constexpr int kSelMaxBlocks = 1024;  // blocks per sequence the LDS bins hold (L <= 65536)
constexpr int kSelStrad = kSelMaxBlocks / 16 + 1;
#ifndef NSA_SEL_WAVES
#define NSA_SEL_WAVES 12
#endif
constexpr int kLdsBytes = 160 * 1024;

// Dynamic LDS of the list kernel: query tile, per-wave running max and sum,
// row log-sum-exp, straddle slots, bins.
constexpr size_t sel_lds_bytes(int G, int D, int NW)
{
    return (size_t)kSelTok * G * (D + 8) * 2 +
           sizeof(float) * ((size_t)(2 * NW + 1) * kSelTok * G + kSelTok * kSelStrad + kSelTok * kSelMaxBlocks);
}
// Waves per workgroup of the list kernel: 12, or 8 where the per-wave
// partials of 12 would not fit the LDS (G 16 with d 128).
constexpr int sel_waves(int G, int D)
{
    return sel_lds_bytes(G, D, NSA_SEL_WAVES) <= kLdsBytes ? NSA_SEL_WAVES : 8;
}

// Lane-permuted copies by DPP (CTRL: a quad_perm or row-mirror code).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x)
{
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}

// Value of lane l ^ off (off < 16): quad permutes for 1 and 2, else a
// bpermute.
__device__ __forceinline__ float lane_xor(float x, int off)
{
    const int v = __float_as_int(x);
    if (off == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    if (off == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    return __shfl_xor(x, off, 64);
}

// One workgroup of 256 threads, after the sequence prep: compressed-window
// and 16-token-tile offsets of every sequence; flags sequences too long for
// the LDS bins.
__global__ __launch_bounds__(256) void k_sel_prep(Params p)
{
    __shared__ int sh[16];
    __shared__ int carry_c, carry_t, bad;
    const int tid = threadIdx.x;
    if (tid == 0) {
        carry_c = 0;
        carry_t = 0;
        bad = 0;
    }
    __syncthreads();
    const int n = p.B + 1;
    for (int base = 0; base < n; base += 256) {
        const int s = base + tid;
        int nc = 0, nt = 0;
        if (s >= 1 && s < n) {
            const int L = p.cus[s] - p.cus[s - 1];
            nc = L >= kSelKs ? (L - kSelKs) / kSelStride + 1 : 0;
            nt = (L + kSelTok - 1) / kSelTok;
            if (L > kSelMaxBlocks * kSelBs) atomicOr(&bad, 1);
        }
        const int ci = block_inclusive_scan<false>(nc, sh) + carry_c;
        const int ti = block_inclusive_scan<false>(nt, sh) + carry_t;
        if (s < n) {
            p.sel_cbase[s] = ci;
            p.sel_tbase[s] = ti;
        }
        __syncthreads();
        if (tid == 255) {
            carry_c = ci;
            carry_t = ti;
        }
        __syncthreads();
    }
    if (tid == 0 && bad) atomicOr(&p.status[kStatusError], kBadSelectLength);
}

// Compressed keys: thread per (window, kv head, 8 channels).
template <typename E, int D>
__global__ __launch_bounds__(256) void k_compress(Params p)
{
    using H = H16<E>;
    constexpr int CH = D / 8;
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= (int64_t)p.sel_cap * p.Hkv * CH) return;
    const int c8 = (int)(x % CH);
    const int64_t wh = x / CH;
    const int h = (int)(wh % p.Hkv);
    const int w = (int)(wh / p.Hkv);
    if (w >= p.sel_cbase[p.B]) return;
    int lo = 0, hi = p.B - 1;  // last sequence with cbase <= w
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.sel_cbase[mid] <= w) lo = mid; else hi = mid - 1;
    }
    const int64_t p0 = p.cus[lo] + (int64_t)(w - p.sel_cbase[lo]) * kSelStride;
    const u16* kr = reinterpret_cast<const u16*>(p.k) + (p0 * p.Hkv + h) * D + c8 * 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int a = 0; a < kSelKs; ++a) {  // position order
        const uint4 v = *reinterpret_cast<const uint4*>(kr + (int64_t)a * p.Hkv * D);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += H::to_f32((u16)(wd[e] & 0xFFFFu));
            acc[2 * e + 1] += H::to_f32((u16)(wd[e] >> 16));
        }
    }
    const f32x4 lo4 = {acc[0] / (float)kSelKs, acc[1] / (float)kSelKs, acc[2] / (float)kSelKs, acc[3] / (float)kSelKs};
    const f32x4 hi4 = {acc[4] / (float)kSelKs, acc[5] / (float)kSelKs, acc[6] / (float)kSelKs, acc[7] / (float)kSelKs};
    const uint2 a = cvt4<E>(lo4), b = cvt4<E>(hi4);
    *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.sel_kcmp) + ((int64_t)w * p.Hkv + h) * D + c8 * 8) =
        make_uint4(a.x, a.y, b.x, b.y);
}

// One workgroup (8 waves) per (16-token tile of a sequence, kv head).  Rows
// of the tile: r = token * G + head (16 G rows, G row tiles of 16).  The
// waves share the visible windows in chunks of 64 (wave w takes chunks w,
// w + 8, ..; the next chunk's compressed keys load while one computes) and
// run every row tile over their chunks; in the S^T = Kc Q^T accumulator,
// lane (n, gq) of key tile kt holds the 4 windows of block 16 m + 4 kt + gq
// for row n, so a block's partial importance never crosses lanes.
template <typename E, int D, int G>
__global__ __launch_bounds__(64 * sel_waves(G, D)) void k_select(Params p)
{
    using H = H16<E>;
    typedef typename H::v8 v8;
    constexpr int NW = sel_waves(G, D);
    constexpr int NT = 64 * NW;     // threads
    constexpr int R = kSelTok * G;  // rows
    constexpr int QP = D + 8;       // padded LDS row of the query tile
    constexpr int DS = D / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char sel_smem[];
    u16* sQ = reinterpret_cast<u16*>(sel_smem);                                  // [R][QP]
    float* sM = reinterpret_cast<float*>(sel_smem + R * QP * 2);                 // [NW][R]
    float* sL = sM + NW * R;                                                     // [NW][R]
    float* sLse = sL + NW * R;                                                   // [R]
    float* strad = sLse + R;                                                     // [16][kSelStrad]
    float* bins = strad + kSelTok * kSelStrad;                                   // [16][kSelMaxBlocks]

    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int tile = blockIdx.x, h = blockIdx.y;
    if (tile >= p.sel_tbase[p.B]) return;
    int s = 0;
    {
        int lo = 0, hi = p.B - 1;  // last sequence with tbase <= tile
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.sel_tbase[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        s = uni(lo);
    }
    const int c0 = uni(p.cus[s]), L = uni(p.cus[s + 1]) - c0;
    const int i0 = (tile - uni(p.sel_tbase[s])) * kSelTok;
    const int ntok = min(kSelTok, L - i0);
    const int i_last = i0 + ntok - 1;
    const int nbins = i_last / kSelBs + 1;
    const int topk = p.topk;
    int32_t* outrow0 = p.sel_out + ((int64_t)(c0 + i0) * p.Hkv + h) * topk;
    if (L > kSelMaxBlocks * kSelBs) {  // flagged by the prep: empty lists
        for (int x = tid; x < ntok * topk; x += NT)
            outrow0[(int64_t)(x / topk) * p.Hkv * topk + x % topk] = -1;
        return;
    }
    const int cb = uni(p.sel_cbase[s]), ncmp = uni(p.sel_cbase[s + 1]) - cb;
    const int nvis = i_last >= kSelKs - 1 ? min(ncmp, (i_last - (kSelKs - 1)) / kSelStride + 1) : 0;
    const int nch = (nvis + kSelChunk - 1) / kSelChunk;

    // query tile, bins and straddle slots
    const u16* qg = reinterpret_cast<const u16*>(p.q);
    for (int x = tid; x < R * (D / 8); x += NT) {
        const int r = x / (D / 8), c8 = x % (D / 8);
        const int tl = r / G, g = r % G;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (tl < ntok) v = *reinterpret_cast<const uint4*>(qg + ((int64_t)(c0 + i0 + tl) * p.Hq + h * G + g) * D + c8 * 8);
        *reinterpret_cast<uint4*>(&sQ[r * QP + c8 * 8]) = v;
    }
    for (int x = tid; x < kSelTok * nbins; x += NT) bins[(x / nbins) * kSelMaxBlocks + x % nbins] = 0.f;
    for (int x = tid; x < kSelTok * kSelStrad; x += NT) strad[x] = 0.f;
    for (int x = tid; x < NW * R; x += NT) {
        sM[x] = -INFINITY;
        sL[x] = 0.f;
    }
    __syncthreads();

    const u16* kc = reinterpret_cast<const u16*>(p.sel_kcmp);
    auto load_chunk = [&](int m, v8 (&kf)[4][DS]) {
        // windows past the sequence's last read window 0 (they are masked)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int w = m * kSelChunk + kt * 16 + n;
            const u16* src = kc + ((int64_t)(cb + (w < ncmp ? w : 0)) * p.Hkv + h) * D + gq * 8;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) kf[kt][ds] = *reinterpret_cast<const v8*>(src + ds * 32);
        }
    };
    // windows every token of the tile sees (those of its first token)
    const int wlim0 = i0 >= kSelKs - 1 ? min(ncmp, (i0 - (kSelKs - 1)) / kSelStride + 1) : 0;
    // S^T (64 windows x 16 rows) of row tile rt, scaled to log2 units and
    // masked: window w is visible to the row's token iff w < wlim (no mask
    // when the whole chunk is visible to the whole tile)
    auto scores = [&](const v8 (&kf)[4][DS], int rt, int m, f32x4 (&x)[4]) {
        v8 bq[DS];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) bq[ds] = *reinterpret_cast<const v8*>(&sQ[(rt * 16 + n) * QP + ds * 32 + gq * 8]);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) x[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) x[kt] = H::mfma(kf[kt][ds], bq[ds], x[kt]);
        if (m * kSelChunk + kSelChunk <= wlim0) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) x[kt] = x[kt] * p.scale_log2;
            return;
        }
        const int tl = (rt * 16 + n) / G;
        const int pos = i0 + tl;
        const int wlim = tl < ntok && pos >= kSelKs - 1 ? min(ncmp, (pos - (kSelKs - 1)) / kSelStride + 1) : 0;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int w = m * kSelChunk + kt * 16 + gq * 4 + i;
                x[kt][i] = w < wlim ? x[kt][i] * p.scale_log2 : -INFINITY;
            }
    };

    // pass 1: per-row running max and sum (log2 units) over this wave's
    // chunks, kept in this wave's slots of sM / sL (every lane of a row reads
    // them, its gq == 0 lane writes them)
    // the wave's chunks m = wave, wave + NW, ..: fn(m, keys of m) (each
    // chunk's keys load just before its use: with 12 waves per CU the other
    // waves cover the latency, and the registers of a second buffer would
    // cost occupancy)
    auto for_chunks = [&](auto&& fn) {
        for (int m = wave; m < nch; m += NW) {
            v8 ka[4][DS];
            load_chunk(m, ka);
            fn(m, ka);
        }
    };
    // (small G * D: the running state stays in registers, the row tiles
    // unrolled, and is written once)
    constexpr bool REGS = G * D <= 256;
    float rm[REGS ? G : 1], rl[REGS ? G : 1];
#pragma unroll
    for (int rt = 0; rt < (REGS ? G : 1); ++rt) {
        rm[rt] = -INFINITY;
        rl[rt] = 0.f;
    }
    auto pass1_tile = [&](const v8 (&kf)[4][DS], int m, int rt, float& mst, float& lst) {
        f32x4 x[4];
        scores(kf, rt, m, x);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[kt][i]);
        mx = xmax32(xmax16(mx));
        const float mnew = fmaxf(mst, mx);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(x[kt][i] - mref);
        sum = xsum32(xsum16(sum));
        lst = lst * __builtin_amdgcn_exp2f(mst - mref) + sum;
        mst = mnew;
    };
    for_chunks([&](int m, const v8 (&kf)[4][DS]) {
        if constexpr (REGS) {
#pragma unroll
            for (int rt = 0; rt < (REGS ? G : 1); ++rt) pass1_tile(kf, m, rt, rm[rt], rl[rt]);
        } else {
#pragma unroll 1
            for (int rt = 0; rt < G; ++rt) {
                const int slot = wave * R + rt * 16 + n;
                float mst = sM[slot], lst = sL[slot];
                pass1_tile(kf, m, rt, mst, lst);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (gq == 0) {
                    sL[slot] = lst;
                    sM[slot] = mst;
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
    });
    if constexpr (REGS) {
        if (gq == 0) {
#pragma unroll
            for (int rt = 0; rt < (REGS ? G : 1); ++rt) {
                sM[wave * R + rt * 16 + n] = rm[rt];
                sL[wave * R + rt * 16 + n] = rl[rt];
            }
        }
    }
    __syncthreads();
    for (int r = tid; r < R; r += NT) {  // combine the waves in order
        float M = -INFINITY;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sM[w * R + r]);
        const float Mref = M == -INFINITY ? 0.f : M;
        float Ls = 0.f;
        for (int w = 0; w < NW; ++w) Ls += sL[w * R + r] * __builtin_amdgcn_exp2f(sM[w * R + r] - Mref);
        sLse[r] = Ls > 0.f ? Mref + __log2f(Ls) : INFINITY;  // nothing visible: p = 0
    }
    __syncthreads();

    // pass 2: probabilities, summed over the G heads of each token, into the bins
    for_chunks([&](int m, const v8 (&kf)[4][DS]) {
#pragma unroll 1
        for (int rt = 0; rt < G; ++rt) {
            f32x4 x[4];
            scores(kf, rt, m, x);
            const float l2 = sLse[rt * 16 + n];
            float A[4], Bv[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                f32x4 e;
#pragma unroll
                for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(x[kt][i] - l2);
                A[kt] = ((e[0] + e[1]) + e[2]) + e[3];
                Bv[kt] = e[3];  // window 4j+3 also overlaps block j+1
            }
#pragma unroll
            for (int off = 1; off < G; off <<= 1)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    A[kt] += lane_xor(A[kt], off);
                    Bv[kt] += lane_xor(Bv[kt], off);
                }
            const int tl = (rt * 16 + n) / G;
            const bool writer = (n % G) == 0 && tl < ntok;
            if (writer) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const int j = m * 16 + kt * 4 + gq;
                    if (j < nbins) bins[tl * kSelMaxBlocks + j] = A[kt];
                }
            }
            // the block sums above are all stored before the straddles add
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (writer) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const int jj = kt * 4 + gq;  // block within the chunk
                    if (jj < 15) {
                        if (m * 16 + jj + 1 < nbins) bins[tl * kSelMaxBlocks + m * 16 + jj + 1] += Bv[kt];
                    } else {
                        strad[tl * kSelStrad + m + 1] = Bv[kt];
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    });
    __syncthreads();
    // straddles across chunk boundaries (block 16 m gets window 64 m - 1)
    for (int x = tid; x < kSelTok * nch; x += NT) {
        const int tl = x / nch, m = x % nch + 1;
        if (tl < ntok && m * 16 < nbins) bins[tl * kSelMaxBlocks + m * 16] += strad[tl * kSelStrad + m];
    }
    __syncthreads();

    // lists: wave w builds those of tokens w, w + NW, ..
    constexpr int VPL = kSelMaxBlocks / 64;  // candidate blocks per lane
    for (int tl = wave; tl < ntok; tl += NW) {
        const int b = (i0 + tl) / kSelBs;
        const int lo_local = b - p.sel_local + 1;
        auto forced = [&](int j) { return j < p.sel_init || (j >= lo_local && j <= b); };
        // forced ids first: init blocks ascending, then local blocks b, b-1, ..
        int nf = 0;
        int slot_id = -1;  // this lane's slot of the list
        for (int j = 0; j < p.sel_init && j <= b && nf < topk; ++j) {
            if (lane == nf) slot_id = j;
            ++nf;
        }
        for (int u = 0; u < p.sel_local && nf < topk; ++u) {
            const int j = b - u;
            if (j < 0 || j < p.sel_init) continue;  // outside [0, b] or already an init block
            if (lane == nf) slot_id = j;
            ++nf;
        }
        float v[VPL];
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const int j = lane + 64 * u;
            v[u] = j <= b && !forced(j) ? bins[tl * kSelMaxBlocks + j] : -INFINITY;
        }
        int nforced_valid = 0;  // forced ids inside [0, b]
        for (int j = 0; j <= b && j < p.sel_init; ++j) ++nforced_valid;
        for (int u = 0; u < p.sel_local; ++u) {
            const int j = b - u;
            if (j >= 0 && j >= p.sel_init) ++nforced_valid;
        }
        const int rounds = min(topk - nf, b + 1 - nforced_valid);
        // This lane's two best untaken candidates (value, slot u; strict
        // comparisons in ascending u keep the lowest id first among equal
        // values) and the slots already taken.  A pick promotes the second;
        // only a lane picked again after that rescans its slots.
        float a1, a2;
        int u1, u2;  // VPL: none
        unsigned taken = 0;
        bool known2;  // a2 is the second best of the untaken slots
        auto top2 = [&]() {
            a1 = a2 = -INFINITY;
            u1 = u2 = VPL;
#pragma unroll
            for (int u = 0; u < VPL; ++u) {
                // selects, not branches: the four stay in registers
                const float x = (taken >> u) & 1u ? -INFINITY : v[u];
                const bool g1 = x > a1, g2 = x > a2;
                const float n2 = g1 ? a1 : g2 ? x : a2;
                const int m2 = g1 ? u1 : g2 ? u : u2;
                a1 = g1 ? x : a1;
                u1 = g1 ? u : u1;
                a2 = n2;
                u2 = m2;
            }
            known2 = true;
        };
        top2();
        for (int r = 0; r < rounds; ++r) {
            // wave-wide largest value: DPP within rows (quad_perm [1,0,3,2],
            // [2,3,0,1], row_half_mirror, row_mirror), lane swaps across rows.
            // Importances are +0 or positive and unplaced slots -inf, so the
            // float order is the signed-integer order of the bits.
            int mi = __float_as_int(a1);
            mi = max(mi, dpp_i<0xB1>(mi));
            mi = max(mi, dpp_i<0x4E>(mi));
            mi = max(mi, dpp_i<0x141>(mi));
            mi = max(mi, dpp_i<0x140>(mi));
            {
                const auto s = __builtin_amdgcn_permlane16_swap((unsigned)mi, (unsigned)mi, false, false);
                mi = max((int)s[0], (int)s[1]);
            }
            {
                const auto s = __builtin_amdgcn_permlane32_swap((unsigned)mi, (unsigned)mi, false, false);
                mi = max((int)s[0], (int)s[1]);
            }
            mi = __builtin_amdgcn_readfirstlane(mi);
            const float m = __int_as_float(mi);
            if (m == -INFINITY) {  // no candidate left (only NaN importances remain)
                if (lane == nf + r) slot_id = -1;
                continue;
            }
            const uint64_t hit = __builtin_amdgcn_ballot_w64(__float_as_int(a1) == mi);
            int id;
            if (__builtin_popcountll(hit) == 1) {
                const int wl = __builtin_ctzll(hit);
                id = wl + 64 * __builtin_amdgcn_readlane(u1, wl);
            } else {
                // equal values in several lanes: the lowest of their ids
                int c = __float_as_int(a1) == mi ? lane + 64 * u1 : INT_MAX;
                c = min(c, dpp_i<0xB1>(c));
                c = min(c, dpp_i<0x4E>(c));
                c = min(c, dpp_i<0x141>(c));
                c = min(c, dpp_i<0x140>(c));
                {
                    const auto s = __builtin_amdgcn_permlane16_swap((unsigned)c, (unsigned)c, false, false);
                    c = min((int)s[0], (int)s[1]);
                }
                {
                    const auto s = __builtin_amdgcn_permlane32_swap((unsigned)c, (unsigned)c, false, false);
                    c = min((int)s[0], (int)s[1]);
                }
                id = __builtin_amdgcn_readfirstlane(c);
            }
            if (lane == nf + r) slot_id = id;
            const int wl = id & 63;
            const bool rescan = __builtin_amdgcn_readlane((int)known2, wl) == 0;
            if (lane == wl) {
                taken |= 1u << u1;
                a1 = a2;
                u1 = u2;
                known2 = false;
                if (rescan) top2();
            }
        }
        if (lane < topk) outrow0[(int64_t)tl * p.Hkv * topk + lane] = slot_id;
    }
}

// Lists of tokens outside every sequence: all -1.
__global__ __launch_bounds__(256) void k_sel_orphans(Params p)
{
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (t * Hkv + h) * topk + slot
    if (x >= p.T * p.Hkv * p.topk) return;
    const int64_t t = x / ((int64_t)p.Hkv * p.topk);
    if (seq_of_token(p.cus, p.B, t) < 0) p.sel_out[x] = -1;
}

template <typename E, int D, int G>
void launch_select_g(const Params& p, hipStream_t st)
{
    constexpr int NW = sel_waves(G, D);
    constexpr size_t lds = sel_lds_bytes(G, D, NW);
    static_assert(lds <= kLdsBytes, "list kernel LDS");
    const dim3 grid((unsigned)(p.T / kSelTok + p.B), (unsigned)p.Hkv);
    hipLaunchKernelGGL((k_select<E, D, G>), grid, dim3(64 * NW), lds, st, p);
}

template <typename E, int D>
void launch_compress_d(const Params& p, hipStream_t st)
{
    const unsigned cgrid = (unsigned)div_up((int64_t)p.sel_cap * p.Hkv * (D / 8), 256);
    if (cgrid) hipLaunchKernelGGL((k_compress<E, D>), dim3(cgrid), dim3(256), 0, st, p);
}

template <typename E, int D>
void launch_select_d(const Params& p, hipStream_t st)
{
    switch (p.G) {
    case 1: launch_select_g<E, D, 1>(p, st); break;
    case 2: launch_select_g<E, D, 2>(p, st); break;
    case 4: launch_select_g<E, D, 4>(p, st); break;
    case 8: launch_select_g<E, D, 8>(p, st); break;
    default: launch_select_g<E, D, 16>(p, st); break;
    }
}

}  // namespace

// The shapes this path takes (the host checks them before enqueueing).
bool select_supported(int D, int G, int bs, int ks, int stride)
{
    return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) && bs == kSelBs &&
           ks == kSelKs && stride == kSelStride;
}

int select_cap(int64_t T, int B) { return (int)(T / kSelStride + B); }

// Window and tile offsets per sequence (after the sequence prep).
hipError_t launch_sel_prep(const Params& p, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_sel_prep, dim3(1), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_compress(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    if (kind == kElemF16) {
        if (p.D == 64) launch_compress_d<_Float16, 64>(p, st);
        else launch_compress_d<_Float16, 128>(p, st);
    } else {
        if (p.D == 64) launch_compress_d<__bf16, 64>(p, st);
        else launch_compress_d<__bf16, 128>(p, st);
    }
    return hipGetLastError();
}

hipError_t launch_select(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    if (kind == kElemF16) {
        if (p.D == 64) launch_select_d<_Float16, 64>(p, st);
        else launch_select_d<_Float16, 128>(p, st);
    } else {
        if (p.D == 64) launch_select_d<__bf16, 64>(p, st);
        else launch_select_d<__bf16, 128>(p, st);
    }
    return hipGetLastError();
}

hipError_t launch_sel_orphans(const Params& p, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const unsigned ogrid = (unsigned)div_up(p.T * p.Hkv * p.topk, 256);
    hipLaunchKernelGGL(k_sel_orphans, dim3(ogrid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace nsa
