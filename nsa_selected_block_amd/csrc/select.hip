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
// per window, kv head and 8 channels), select (one workgroup per token tile
// of a sequence and kv head: every wave keeps its rows' queries in registers
// while the tile's visible windows stream through LDS in chunks of 64; a
// first pass gives each row's log-sum-exp, a second the probabilities, summed
// per block and over the G heads, that a sorted top-k list per token, held in
// registers, takes in ascending block order), orphans (rows of tokens outside
// every sequence).
// Every sum has a fixed order: the lists are bitwise reproducible.  No
// per-block table is kept, so sequences of any length are taken.
#include "device_common.h"

#include <float.h>

#include <type_traits>

namespace nsa {

namespace {

constexpr int kSelChunk = 64;  // compressed windows per chunk (16 blocks)
constexpr int kSelKs = 32, kSelStride = 16, kSelBs = 64;
constexpr int kSelWaves = 8;   // waves per workgroup of the list kernel

// One workgroup of 256 threads, after the sequence prep: compressed-window
// and token-tile offsets of every sequence.
__global__ __launch_bounds__(256) void k_sel_prep(Params p)
{
    __shared__ int sh[16];
    __shared__ int carry_c, carry_t;
    const int tid = threadIdx.x;
    if (tid == 0) {
        carry_c = 0;
        carry_t = 0;
    }
    __syncthreads();
    const int n = p.B + 1;
    for (int base = 0; base < n; base += 256) {
        const int s = base + tid;
        int nc = 0, nt = 0;
        if (s >= 1 && s < n) {
            const int L = p.cus[s] - p.cus[s - 1];
            nc = L >= kSelKs ? (L - kSelKs) / kSelStride + 1 : 0;
            nt = (L + p.sel_tok - 1) / p.sel_tok;
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
}

// Dispatch order of the list kernel's token tiles.  A tile's work grows with
// its tokens' position (it streams every window before them, twice), so the
// tiles go latest position first -- the heaviest workgroups start first and
// the light ones fill the tail.  Tile m of sequence s (local position m * TOK)
// gets rank sum over s' of max(0, nt_s' - m - 1) (the tiles further along
// than m) plus the number of sequences s' < s with a tile m: a permutation.
// One thread per tile; with more than kSelOrderMaxSeq sequences the ranks are
// left in tile order (the sum per tile is O(B)).
constexpr int kSelOrderMaxSeq = 1024;

__global__ __launch_bounds__(256) void k_sel_order(Params p, int32_t* __restrict__ order)
{
    const int x = blockIdx.x * 256 + threadIdx.x;
    const int ntiles = p.sel_tbase[p.B];
    if (x >= ntiles) return;
    if (p.B > kSelOrderMaxSeq) {
        order[x] = x;
        return;
    }
    int lo = 0, hi = p.B - 1;  // last sequence with tbase <= x
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.sel_tbase[mid] <= x) lo = mid; else hi = mid - 1;
    }
    const int m = x - p.sel_tbase[lo];
    int rank = 0;
    for (int s = 0; s < p.B; ++s) {
        const int nt = p.sel_tbase[s + 1] - p.sel_tbase[s];
        rank += max(0, nt - m - 1) + (s < lo && nt > m ? 1 : 0);
    }
    order[rank] = x;
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

// LDS image of a chunk of compressed keys: 64 rows of D 16-bit values; the
// 16-byte pieces of row r permuted by XOR with (r / 4) mod C, C = min(D / 8,
// 16).  Key tile kt of the list kernel takes rows 4 n + kt (n = 0 .. 15), one
// piece each: sixteen different pieces, so every bank once per read.
template <int D> __device__ __forceinline__ int sel_swz(int r) { return (r >> 2) & ((D / 8 < 16 ? D / 8 : 16) - 1); }

// Queue the loads of compressed-key rows [w0, w0 + 64) of kv head h into the
// LDS image dst (one 16-byte buffer load to LDS per lane, pieces permuted by
// sel_swz); rows past nvalid are outside the buffer range and read as zeros.
template <int D>
__device__ __forceinline__ void stage_chunk_lds(const Params& p, int h, int w0, int nvalid, u16* dst)
{
    typedef __attribute__((address_space(3))) void lds_void;
    constexpr int NCH = D / 8;        // chunks per row
    constexpr int RPI = 64 / NCH;     // rows per wave-load
    constexpr int NI = kSelChunk / RPI;
    const int64_t e0 = ((int64_t)w0 * p.Hkv + h) * D;
    const uint32_t bytes = nvalid > 0 ? (uint32_t)(((int64_t)(nvalid - 1) * p.Hkv + 1) * D * 2) : 0u;
    const auto rk = make_rsrc(reinterpret_cast<const u16*>(p.sel_kcmp) + e0, bytes);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rl = lane / NCH, pc = lane % NCH;
#pragma unroll
    for (int i = wave; i < NI; i += kSelWaves) {
        const int r = i * RPI + rl;
        const uint32_t rowb = (uint32_t)(r * p.Hkv * D * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + i * RPI * D), 16,
                                                 rowb + (uint32_t)((pc ^ sel_swz<D>(r)) * 16), 0, 0, 0);
    }
}

// DPP moves within 16-lane rows.  Controls: quad permutes 0x00 .. 0xFF,
// row_shl:N 0x100 + N, row_shr:N 0x110 + N (lane l reads lane l - N),
// row_ror:N 0x120 + N (lane l reads lane (l - N) mod 16), row_mirror 0x140.
// `upd` keeps `old` in lanes whose source lies outside the row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x)
{
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_upd(float old, float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_upd(int old, int x)
{
    return __builtin_amdgcn_update_dpp(old, x, CTRL, 0xF, 0xF, false);
}

// Every lane of a row gets the row's lane 15.
__device__ __forceinline__ float row_bcast_last(float x)
{
    x = dpp_mov<0xFF>(x);  // each quad its lane 3
    x = dpp_upd<0x104>(x, x);
    return dpp_upd<0x108>(x, x);
}

// Query rows of a 16-row tile per lane row of the pass-2 layout (lane row g:
// rows 4 g .. 4 g + 3): TPL tokens of G rows for G <= 4, else one token over
// G / 4 lane rows.
template <int G> struct SelShape {
    static constexpr int TPL = G >= 4 ? 1 : 4 / G;
};

// 16-row tiles per wave: two, or one where the lists (RM registers of 16
// slots per token slot) would take more than four registers per tile.
template <int G, int RM> struct SelTiles {
    static constexpr int NTL = SelShape<G>::TPL * RM <= 4 ? 2 : 1;
};

// One workgroup (8 waves) per (token tile of a sequence, kv head).  Rows of
// the tile: r = token * G + head, 16-row tiles; wave w owns tiles w, w + 8, ..
// and keeps their queries as MFMA operands in registers.  All waves walk the
// same chunks of 64 compressed windows, double buffered in LDS.  Key tile kt
// of a chunk holds windows 4 n + kt, n = 0 .. 15: key n of the four tiles are
// the four windows of block n of the chunk.
//   pass 1 (S^T = Kc Q^T; lane (n, g) holds keys 4 g .. 4 g + 3 for row n):
//           per-row running max and sum -> the row's log-sum-exp;
//   pass 2 (S = Q Kc^T; lane (n, g) holds rows 4 g .. 4 g + 3 for key n):
//           p = exp2(s - lse), summed over the token's heads in the lane (and
//           across lane rows for G = 8, 16), then over the four key tiles,
//           plus window 4 n - 1 from lane n - 1 (the window before the block
//           straddles into it): lane (n, g) has block n of the chunk for the
//           token of lane row g.
// Each token keeps its list in registers, in one lane row: RM registers of 16
// slots, sorted by (importance descending, id ascending) and aligned to the
// last slot, the slots before the list at +inf, empty ones at -1.  A block of
// the chunk is inserted, in ascending id, when it beats the token's last
// slot: every lane compares its entry with the block and shifts by one slot
// (row shift, and row rotate across registers) where the block goes ahead of
// it.  An equal importance stays behind the entries already there (they have
// smaller ids), so the list ends as the k best under (importance descending,
// id ascending).  Blocks the last slot rules out, by the threshold known at
// the start of the chunk, are never inserted.
template <typename E, int D, int G, int RM>
__global__ __launch_bounds__(64 * kSelWaves, 4) void k_select(Params p, const int32_t* __restrict__ order)
{
    using H = H16<E>;
    typedef typename H::v8 v8;
    constexpr int DS = D / 32;
    constexpr int IMG = kSelChunk * D;
    constexpr int NTL = SelTiles<G, RM>::NTL;
    constexpr int TPL = SelShape<G>::TPL;
    // two separate chunk buffers: the compiler then sees that the loads into
    // one never alias the reads of the other
    __shared__ __attribute__((aligned(16))) u16 kb0[IMG];
    __shared__ __attribute__((aligned(16))) u16 kb1[IMG];

    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int TOK = p.sel_tok, topk = p.topk;
    // workgroups in order of decreasing work (order: token tiles by position,
    // latest first), the kv heads of one tile side by side
    const int h = (int)(blockIdx.x % p.Hkv), rank = (int)(blockIdx.x / p.Hkv);
    if (rank >= p.sel_tbase[p.B]) return;
    const int tile = order[rank];
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
    const int i0 = (tile - uni(p.sel_tbase[s])) * TOK;
    const int ntok = min(TOK, L - i0);
    const int i_last = i0 + ntok - 1;
    const int cb = uni(p.sel_cbase[s]), ncmp = uni(p.sel_cbase[s + 1]) - cb;
    // windows visible to the token at local position i: 16 c + 31 <= i
    auto wlim_of = [&](int i) { return i >= kSelKs - 1 ? min(ncmp, (i - (kSelKs - 1)) / kSelStride + 1) : 0; };
    const int wlim0 = wlim_of(i0);
    const int nch1 = (wlim_of(i_last) + kSelChunk - 1) / kSelChunk;  // chunks with visible windows
    const int nch2 = i_last / kSelBs / 16 + 1;                      // chunks holding blocks <= b
    const int nrows = ntok * G;

    // this wave's row tiles: queries (rows past the tile's tokens read the
    // first token's row) and row validity
    bool tv[NTL];
    v8 bq[NTL][DS];
    const bool qflip = p.scale_log2 < 0.f;
    const float sl = fmaxf(fabsf(p.scale_log2), FLT_MIN);
    {
        const u16* qg = reinterpret_cast<const u16*>(p.q);
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            const int rt = wave + kSelWaves * j;
            tv[j] = rt * 16 < nrows;  // uniform
            const int r = rt * 16 + n;
            const int tl = r / G;
            const u16* qr = qg + ((int64_t)(c0 + i0 + (r < nrows ? tl : 0)) * p.Hq + h * G + r % G) * D + gq * 8;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                bq[j][ds] = *reinterpret_cast<const v8*>(qr + ds * 32);
                if (qflip) {  // a negative scale's sign goes into the queries (exact)
                    const uint4 u = __builtin_bit_cast(uint4, bq[j][ds]);
                    bq[j][ds] = __builtin_bit_cast(v8, make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u,
                                                                  u.z ^ 0x80008000u, u.w ^ 0x80008000u));
                }
            }
        }
    }
    // this lane's key rows: 4 n + kt, piece (4 ds + gq) ^ sel_swz
    const int kbase = 4 * n * D;
    const int ksw = sel_swz<D>(4 * n);
    // raw scores of this wave's tiles for the chunk in `cur`, windows not
    // visible to a row's token at -inf; TR: the transposed layout of pass 2
    auto scores = [&](auto tr, const u16* cur, int m, f32x4 (&x)[NTL][4]) {
        constexpr bool TR = decltype(tr)::value;
        int lo = kbase;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) x[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const v8 ak = *reinterpret_cast<const v8*>(&cur[lo + kt * D + ((4 * ds + gq) ^ ksw) * 8]);
#pragma unroll
                for (int j = 0; j < NTL; ++j)
                    x[j][kt] = TR ? H::mfma(bq[j][ds], ak, x[j][kt]) : H::mfma(ak, bq[j][ds], x[j][kt]);
            }
        if (m * kSelChunk + kSelChunk <= wlim0) return;  // every window visible to every token
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            const int rt = wave + kSelWaves * j;
            int wl[4];  // visible windows of the rows in x[j][.][i]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rt * 16 + (TR ? 4 * gq + i : n);
                wl[i] = r < nrows ? wlim_of(i0 + r / G) : 0;
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int w = m * kSelChunk + 4 * (TR ? n : 4 * gq + i) + kt;
                    x[j][kt][i] = w < wl[i] ? x[j][kt][i] : -INFINITY;
                }
        }
    };
    // chunks 0 .. nch-1 through the two buffers: chunk m is computed from
    // buffer m % 2 while chunk m + 1 loads into the other one
    auto stream = [&](int nch, auto&& body) {
        if (nch == 0) return;
        stage_chunk_lds<D>(p, h, cb, ncmp, kb0);
        auto step = [&](int m, const u16* cur, u16* nxt) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // chunk m in LDS; every wave done with chunk m - 1
            if (m + 1 < nch)
                stage_chunk_lds<D>(p, h, cb + (m + 1) * kSelChunk, ncmp - (m + 1) * kSelChunk, nxt);
            body(m, cur);
        };
        for (int m = 0; m < nch; m += 2) {
            step(m, kb0, kb1);
            if (m + 1 < nch) step(m + 1, kb1, kb0);
        }
        __syncthreads();  // the buffers are free again
    };

    // pass 1: each row's log-sum-exp (log2 units).  Every lane keeps a
    // reference mr and a sum lr of exp2(s - mr) over its own windows of the
    // row (the four lane rows hold a quarter of them each); the four are
    // combined at the end.  The reference moves only when a chunk's terms,
    // taken against it, sum past 2^64 (or are not finite: the first chunk,
    // where mr is -inf): then the chunk's max is found and the sum rescaled.
    // Terms below the reference by more than 126 flush to 0; they are below
    // 2^-126 of the sum, which holds the reference's own term (1).
    float mr[NTL], lr[NTL];
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        mr[j] = -INFINITY;
        lr[j] = 0.f;
    }
    stream(nch1, [&](int m, const u16* cur) {
        f32x4 x[NTL][4];
        scores(std::false_type{}, cur, m, x);
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            if (!tv[j]) continue;
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(fmaf(x[j][kt][i], sl, -mr[j]));
            const bool move = !(sum <= 0x1p64f);
            if (__ballot(move)) {  // rare: some lane's reference moves
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[j][kt][i]);
                const float mnew = fmaxf(mr[j], mx * sl);
                const float mref = mnew == -INFINITY ? 0.f : mnew;
                if (move) {
                    sum = lr[j] * __builtin_amdgcn_exp2f(mr[j] - mref);
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(fmaf(x[j][kt][i], sl, -mref));
                    lr[j] = sum;
                    mr[j] = mnew == -INFINITY ? -INFINITY : mref;
                    continue;
                }
            }
            lr[j] += sum;
        }
    });
    // log-sum-exp of rows 4 gq + v in the pass-2 layout (nothing visible:
    // +inf, so every p is 0)
    float lseT[NTL][4];
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        const float mrow = xmax32(xmax16(mr[j]));
        const float l = mrow == -INFINITY ? 0.f : xsum32(xsum16(lr[j] * __builtin_amdgcn_exp2f(mr[j] - mrow)));
        const float l2 = l > 0.f ? mrow + __log2f(l) : INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            lseT[j][v] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * gq + v) * 4, __float_as_int(l2)));
    }

    // The lists.  Token of (tile j, slot u) in lane row gq: (16 rt + 4 gq +
    // u G) / G; its own block b, its forced ids in [0, b] (init blocks, then
    // local ones), its list length kc (topk less those), the last id it may
    // choose (b - local).
    struct Tok {
        int t, b, nf, kc;
    };
    auto tok_of = [&](int j, int u) {
        Tok k;
        k.t = ((wave + kSelWaves * j) * 16 + 4 * gq + u * G) / G;
        k.b = (i0 + k.t) / kSelBs;
        k.nf = min(p.sel_init, k.b + 1);
        for (int w = 0; w < p.sel_local; ++w)
            if (k.b - w >= 0 && k.b - w >= p.sel_init) ++k.nf;
        k.kc = tv[j] && k.t < ntok ? topk - min(k.nf, topk) : 0;
        return k;
    };
    // registers below r0 hold no slot of any list (topk >= 1)
    const int r0 = RM == 1 ? 0 : RM - min(RM, (topk + 15) / 16);
    float lv[NTL][TPL][RM], thr[NTL][TPL], carry[NTL][TPL];
    int li[NTL][TPL][RM], blim[NTL][TPL];
#pragma unroll
    for (int j = 0; j < NTL; ++j)
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
            const Tok k = tok_of(j, u);
            blim[j][u] = k.kc > 0 ? k.b - p.sel_local : -1;
            const int pre = 16 * RM - k.kc;
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                lv[j][u][r] = 16 * r + n < pre ? INFINITY : -1.f;
                li[j][u][r] = -1;
            }
            thr[j][u] = k.kc > 0 ? -1.f : INFINITY;
            carry[j][u] = 0.f;
        }
    // insert block `id` of importance x (-inf: nothing) into the lists of
    // every lane row
    auto insert = [&](float (&Lv)[RM], int (&Li)[RM], float x, int id) {
#pragma unroll
        for (int r = RM - 1; r >= 0; --r) {
            if (r < r0) break;
            float pl;
            int pi;
            if (RM == 1) {  // lane 0 is a slot before the list (+inf): its shift-in is never taken
                pl = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Lv[0]), 0x111, 0xF, 0xF, true));
                pi = __builtin_amdgcn_mov_dpp(Li[0], 0x111, 0xF, 0xF, true);
            } else {
                const float tl = r == 0 ? INFINITY : dpp_mov<0x121>(Lv[r > 0 ? r - 1 : 0]);  // lane 0: slot before
                const int ti = r == 0 ? -1 : dpp_mov<0x121>(Li[r > 0 ? r - 1 : 0]);
                pl = dpp_upd<0x111>(tl, Lv[r]);
                pi = dpp_upd<0x111>(ti, Li[r]);
            }
            const bool keep = Lv[r] >= x, pk = pl >= x;
            Lv[r] = keep ? Lv[r] : pk ? x : pl;
            Li[r] = keep ? Li[r] : pk ? id : pi;
        }
    };
    // the blocks of chunk m from the probabilities (pass-2 layout)
    const int b_lo = i0 / kSelBs;  // smallest own block of the workgroup's tokens
    auto take = [&](int m, const f32x4 (&e)[NTL][4]) {
        const bool plain = m * 16 >= p.sel_init && m * 16 + 15 <= b_lo - p.sel_local;
        const int jb = m * 16 + n;  // this lane's block
        const bool idok = plain || jb >= p.sel_init;
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            if (!tv[j]) continue;
            // sum over the token's heads: hv[u][kt], window 4 n + kt
            float hv[TPL][4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (G == 1) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) hv[v % TPL][kt] = e[j][kt][v];
                } else if (G == 2) {
                    hv[0][kt] = e[j][kt][0] + e[j][kt][1];
                    hv[TPL - 1][kt] = e[j][kt][2] + e[j][kt][3];
                } else {
                    float t = (e[j][kt][0] + e[j][kt][1]) + (e[j][kt][2] + e[j][kt][3]);
                    if (G >= 8) t = xsum16(t);
                    if (G >= 16) t = xsum32(t);
                    hv[0][kt] = t;
                }
            }
#pragma unroll
            for (int u = 0; u < TPL; ++u) {
                // block n: windows 4 n .. 4 n + 3, and window 4 n - 1 (lane
                // n - 1's last, or the previous chunk's lane 15 for n = 0)
                const float sh = dpp_upd<0x111>(carry[j][u], hv[u][3]);
                const float z = ((hv[u][0] + hv[u][1]) + (hv[u][2] + hv[u][3])) + sh;
                carry[j][u] = dpp_mov<0x121>(hv[u][3]);
                const bool c = z > thr[j][u] && idok && (plain || jb <= blim[j][u]);
                const uint64_t cm = __ballot(c);
                if (cm == 0) continue;
                const float bm = c ? z : -INFINITY;
                // each lane row takes its own candidates, lowest id first: the
                // lane's row's candidate positions, one per step, its value
                // from that lane of the row (rows done insert -inf)
                uint32_t rm = (uint32_t)(cm >> (16 * gq)) & 0xFFFFu;
                do {
                    const int pos = __builtin_ctz(rm | 0x10000u);
                    const float xv = __int_as_float(
                        __builtin_amdgcn_ds_bpermute(((lane & 48) | (pos & 15)) << 2, __float_as_int(bm)));
                    insert(lv[j][u], li[j][u], rm ? xv : -INFINITY, m * 16 + pos);
                    rm &= rm - 1u;
                } while (__ballot(rm != 0));
                thr[j][u] = row_bcast_last(lv[j][u][RM - 1]);
            }
        }
    };

    // pass 2: chunks with visible windows, then (all probabilities 0) the
    // chunks that only hold blocks <= b.  Off the diagonal the products of
    // key tile kt + 1 issue between the exponentials of key tile kt.
    stream(nch1, [&](int m, const u16* cur) {
        f32x4 x[NTL][4];
        if (m * kSelChunk + kSelChunk <= wlim0) {
            int lo = kbase;
            asm volatile("" : "+v"(lo));
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                for (int j = 0; j < NTL; ++j) x[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    const v8 ak = *reinterpret_cast<const v8*>(&cur[lo + kt * D + ((4 * ds + gq) ^ ksw) * 8]);
#pragma unroll
                    for (int j = 0; j < NTL; ++j) x[j][kt] = H::mfma(bq[j][ds], ak, x[j][kt]);
                }
#pragma unroll
                for (int j = 0; j < NTL; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        x[j][kt][v] = __builtin_amdgcn_exp2f(fmaf(x[j][kt][v], sl, -lseT[j][v]));
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);  // this tile's key reads
#pragma unroll
                for (int i = 0; i < DS * NTL; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a product
                    if (kt > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4 * NTL * 2 / (DS * NTL), 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x002, 8 * NTL, 0);
        } else {
            scores(std::true_type{}, cur, m, x);
#pragma unroll
            for (int j = 0; j < NTL; ++j)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        x[j][kt][v] = __builtin_amdgcn_exp2f(fmaf(x[j][kt][v], sl, -lseT[j][v]));
        }
        take(m, x);
    });
    for (int m = nch1; m < nch2; ++m) {
        f32x4 z[NTL][4];
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) z[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        take(m, z);
    }

    // lists: forced ids (init blocks, then local blocks b, b - 1, ..), then
    // the list's slots in rank order (-1 where empty); one lane row per token
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        if (!tv[j]) continue;
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
            const Tok k = tok_of(j, u);
            if (k.t >= ntok || (4 * gq) % G != 0) continue;
            const int b = k.b;
            int32_t* out = p.sel_out + ((int64_t)(c0 + i0 + k.t) * p.Hkv + h) * topk;
            const int f = min(k.nf, topk);
            if (n == 0) {
                int o = 0;
                for (int jj = 0; jj < p.sel_init && jj <= b && o < topk; ++jj) out[o++] = jj;
                for (int w = 0; w < p.sel_local && o < topk; ++w) {
                    const int jj = b - w;
                    if (jj >= 0 && jj >= p.sel_init) out[o++] = jj;
                }
            }
            const int pre = 16 * RM - k.kc;
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int rank = 16 * r + n - pre;
                if (rank >= 0) out[f + rank] = li[j][u][r];
            }
        }
    }
}

// Lists of tokens outside every sequence: all -1.  One thread per token.
__global__ __launch_bounds__(256) void k_sel_orphans(Params p)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= p.T || seq_of_token(p.cus, p.B, t) >= 0) return;
    int32_t* o = p.sel_out + t * p.Hkv * p.topk;
    for (int x = 0; x < p.Hkv * p.topk; ++x) o[x] = -1;
}

// Registers per token list: one (16 slots) while a list never fills its
// register (topk < 16, or 16 with at least one forced id, so lane 0 stays a
// slot before the list), else four.
int select_regs(int topk, int init, int local) { return topk < 16 || (topk == 16 && (init > 0 || local > 0)) ? 1 : 4; }

template <typename E, int D, int G>
void launch_select_g(const Params& p, const int32_t* order, hipStream_t st)
{
    const dim3 grid((unsigned)((p.T / p.sel_tok + p.B) * p.Hkv));  // (tile rank, kv head), kv head fastest
    if (select_regs(p.topk, p.sel_init, p.sel_local) == 1)
        hipLaunchKernelGGL((k_select<E, D, G, 1>), grid, dim3(64 * kSelWaves), 0, st, p, order);
    else hipLaunchKernelGGL((k_select<E, D, G, 4>), grid, dim3(64 * kSelWaves), 0, st, p, order);
}

template <typename E, int D>
void launch_compress_d(const Params& p, hipStream_t st)
{
    const unsigned cgrid = (unsigned)div_up((int64_t)p.sel_cap * p.Hkv * (D / 8), 256);
    if (cgrid) hipLaunchKernelGGL((k_compress<E, D>), dim3(cgrid), dim3(256), 0, st, p);
}

template <typename E, int D>
void launch_select_d(const Params& p, const int32_t* order, hipStream_t st)
{
    switch (p.G) {
    case 1: launch_select_g<E, D, 1>(p, order, st); break;
    case 2: launch_select_g<E, D, 2>(p, order, st); break;
    case 4: launch_select_g<E, D, 4>(p, order, st); break;
    case 8: launch_select_g<E, D, 8>(p, order, st); break;
    default: launch_select_g<E, D, 16>(p, order, st); break;
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

// Token tiles of the list kernel at most: a tile holds at least 128 / G
// tokens (see select_tokens).
int64_t select_max_tiles(int64_t T, int B, int G) { return T / (128 / G > 0 ? 128 / G : 1) + B; }

// Tokens per token tile of the list kernel for group size G, topk and the
// forced ids: the rows (token x head) of eight waves of one or two 16-row
// tiles each (one where the lists would take more than four registers per
// tile and lane).
int select_tokens(int G, int topk, int init, int local)
{
    const int tpl = G >= 4 ? 1 : 4 / G;
    const int rm = select_regs(topk, init, local);
    const int rows = 16 * kSelWaves * (tpl * rm <= 4 ? 2 : 1);
    return rows / G;
}

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

hipError_t launch_select(const Params& p, int kind, int32_t* order, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const int64_t tiles = p.T / p.sel_tok + p.B;  // grid bound of the tile count
    hipLaunchKernelGGL(k_sel_order, dim3((unsigned)div_up(tiles, 256)), dim3(256), 0, st, p, order);
    if (kind == kElemF16) {
        if (p.D == 64) launch_select_d<_Float16, 64>(p, order, st);
        else launch_select_d<_Float16, 128>(p, order, st);
    } else {
        if (p.D == 64) launch_select_d<__bf16, 64>(p, order, st);
        else launch_select_d<__bf16, 128>(p, order, st);
    }
    return hipGetLastError();
}

hipError_t launch_sel_orphans(const Params& p, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const unsigned ogrid = (unsigned)div_up(p.T, 256);
    hipLaunchKernelGGL(k_sel_orphans, dim3(ogrid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace nsa
