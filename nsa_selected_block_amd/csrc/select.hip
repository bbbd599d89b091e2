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
// per block and over the G heads, that a running top-k per token takes in
// ascending block order), orphans (rows of tokens outside every sequence).
// Every sum has a fixed order: the lists are bitwise reproducible.  No
// per-block table is kept, so sequences of any length are taken.
#include "device_common.h"

#include <float.h>

namespace nsa {

namespace {

constexpr int kSelChunk = 64;  // compressed windows per chunk (16 blocks)
constexpr int kSelKs = 32, kSelStride = 16, kSelBs = 64;
constexpr int kSelWaves = 8;   // waves per workgroup of the list kernel
constexpr int kSelTiles = 2;   // 16-row tiles per wave
constexpr int kSelRows = 16 * kSelWaves * kSelTiles;  // rows (token x head) per workgroup
constexpr int kSelCandBytes = 64 * 1024;              // LDS for the running lists

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

// Queue the loads of compressed-key rows [w0, w0 + 64) of kv head h into the
// LDS image dst (one 16-byte buffer load to LDS per lane, chunks permuted by
// kswz); rows past nvalid are outside the buffer range and read as zeros.
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
                                                 rowb + (uint32_t)((pc ^ kswz<D>(r)) * 16), 0, 0, 0);
    }
}

// One workgroup (8 waves) per (token tile of a sequence, kv head).  Rows of
// the tile: r = token * G + head, 16-row tiles; wave w owns tiles w and w + 8
// and keeps their queries as MFMA B operands in registers.  All waves walk
// the same chunks of 64 compressed windows, double buffered in LDS; in the
// S^T = Kc Q^T accumulator lane (n, gq) of key tile kt holds the 4 windows of
// block 16 m + 4 kt + gq for row n, so a block's sum stays in the lane.
//   pass 1: per-row running max and sum -> the row's log-sum-exp;
//   pass 2: p = exp2(s - lse); per block the sum of its 4 windows plus the
//           window before it (which straddles the boundary), summed over the
//           G heads of the token; one lane per token takes the chunk's 16
//           blocks, in ascending id, into the token's running list of the
//           k best (LDS): a block enters when it is better than the worst
//           entry (importance larger; an equal one comes later, so has the
//           larger id, and stays out), so the list ends as the k best under
//           (importance descending, id ascending).
template <typename E, int D, int G>
__global__ __launch_bounds__(64 * kSelWaves) void k_select(Params p)
{
    using H = H16<E>;
    typedef typename H::v8 v8;
    constexpr int DS = D / 32;
    constexpr int IMG = kSelChunk * D;
    constexpr int NTL = kSelTiles;
    // two separate chunk buffers: the compiler then sees that the loads into
    // one never alias the reads of the other
    __shared__ __attribute__((aligned(16))) u16 kb0[IMG];
    __shared__ __attribute__((aligned(16))) u16 kb1[IMG];
    extern __shared__ __attribute__((aligned(16))) float sel_dyn[];

    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int TOK = p.sel_tok, topk = p.topk;
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

    // this wave's row tiles: queries, row validity, visible windows
    bool tv[NTL];
    int wl[NTL];
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
            wl[j] = r < nrows ? wlim_of(i0 + tl) : 0;
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
    const int ksw = kswz<D>(n);
    // raw scores S^T of this wave's tiles for the chunk in `cur`, windows not
    // visible to a row's token at -inf
    auto scores = [&](const u16* cur, int m, f32x4 (&x)[NTL][4]) {
        int lo = 0;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) x[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const v8 ak = *reinterpret_cast<const v8*>(&cur[lo + (kt * 16 + n) * D + ((4 * ds + gq) ^ ksw) * 8]);
#pragma unroll
                for (int j = 0; j < NTL; ++j)
                    if (tv[j]) x[j][kt] = H::mfma(ak, bq[j][ds], x[j][kt]);
            }
        if (m * kSelChunk + kSelChunk <= wlim0) return;  // every window visible to every token
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int w = m * kSelChunk + kt * 16 + gq * 4 + i;
                    x[j][kt][i] = w < wl[j] ? x[j][kt][i] : -INFINITY;
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

    // pass 1: each row's log-sum-exp (log2 units)
    float mr[NTL], lr[NTL];
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        mr[j] = -INFINITY;
        lr[j] = 0.f;
    }
    stream(nch1, [&](int m, const u16* cur) {
        f32x4 x[NTL][4];
        scores(cur, m, x);
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            if (!tv[j]) continue;
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[j][kt][i]);
            mx = xmax32(xmax16(mx)) * sl;
            const float mnew = fmaxf(mr[j], mx);
            const float mref = mnew == -INFINITY ? 0.f : mnew;
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(fmaf(x[j][kt][i], sl, -mref));
            sum = xsum32(xsum16(sum));
            lr[j] = lr[j] * __builtin_amdgcn_exp2f(mr[j] - mref) + sum;
            mr[j] = mnew;
        }
    });
    float lse2[NTL];  // nothing visible: +inf, so every p is 0
#pragma unroll
    for (int j = 0; j < NTL; ++j) lse2[j] = lr[j] > 0.f ? mr[j] + __log2f(lr[j]) : INFINITY;

    // The running lists.  The lanes n % G == 0 of a tile hold the head-summed
    // block sums of their token (lane row gq: blocks 16 m + 4 kt + gq); all
    // four lane rows keep the token's list length and threshold.  A block
    // joins the token's pending entries (LDS, lcap slots) when it beats the
    // threshold: the k-th best importance after the last compaction (-inf
    // while fewer than k are known).  A compaction (the whole wave, one token
    // at a time) keeps the k best under (importance descending, id
    // ascending), in that order, and raises the threshold; it runs when the
    // next chunk might not fit, and once at the end.
    const int lcap = p.sel_lcap;
    float* pv = sel_dyn;                                   // [TOK][lcap] importances
    int* pj = reinterpret_cast<int*>(pv + TOK * lcap);     // [TOK][lcap] block ids
    const bool lead = n % G == 0;
    int tok[NTL], bb[NTL], kc[NTL], cnt[NTL];
    float thr[NTL];
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        tok[j] = ((wave + kSelWaves * j) * 16 + n) / G;
        const bool ok = tv[j] && tok[j] < ntok;
        bb[j] = ok ? (i0 + tok[j]) / kSelBs : -1;
        // forced ids in [0, b]: init blocks, then local blocks not already taken
        int f = min(p.sel_init, bb[j] + 1);
        for (int u = 0; u < p.sel_local; ++u) {
            const int jj = bb[j] - u;
            if (jj >= 0 && jj >= p.sel_init) ++f;
        }
        kc[j] = ok ? topk - min(f, topk) : 0;
        cnt[j] = 0;
        thr[j] = -INFINITY;
    }
    auto forced = [&](int jb, int b) { return jb < p.sel_init || (jb <= b && jb > b - p.sel_local); };
    // Compaction of the list of the token whose lead lane (row 0) is `src` in
    // tile j: every lane takes two pending entries, kc rounds of a wave-wide
    // arg-max over (importance bits, then lowest id) write the winners back in
    // rank order; the token's lanes take the new length and threshold.
    auto compact = [&](int j, int src) {
        const int tl = __builtin_amdgcn_readlane(tok[j], src);
        const int c = __builtin_amdgcn_readlane(cnt[j], src);
        const int k = __builtin_amdgcn_readlane(kc[j], src);
        float* lv = pv + tl * lcap;
        int* lj = pj + tl * lcap;
        // (importances are +0 or positive: their bits order like the values)
        int va = lane < c ? __float_as_int(lv[lane]) : -1, ia = lane < c ? lj[lane] : INT_MAX;
        int vb = lane + 64 < c ? __float_as_int(lv[lane + 64]) : -1, ib = lane + 64 < c ? lj[lane + 64] : INT_MAX;
        const int keep = min(k, c);
        int last = 0;
        for (int r = 0; r < keep; ++r) {
            // this lane's better entry, then the wave's best value, then its lowest id
            const bool useb = vb > va || (vb == va && ib < ia);
            const int v1 = useb ? vb : va, i1 = useb ? ib : ia;
            int mv = v1;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mv = max(mv, __shfl_xor(mv, off, 64));
            int mi = v1 == mv ? i1 : INT_MAX;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mi = min(mi, __shfl_xor(mi, off, 64));
            if (lane == 0) {
                lv[r] = __int_as_float(mv);
                lj[r] = mi;
            }
            // the winner leaves its lane (ids are distinct)
            if (ia == mi && va == mv) va = -1, ia = INT_MAX;
            if (ib == mi && vb == mv) vb = -1, ib = INT_MAX;
            last = mv;
        }
        if (tok[j] == tl && lead) {
            cnt[j] = keep;
            thr[j] = keep == k ? __int_as_float(last) : -INFINITY;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // block sums of one chunk into the tokens' pending entries
    float carry[NTL];  // window 64 m - 1 of the row (straddles into block 16 m)
#pragma unroll
    for (int j = 0; j < NTL; ++j) carry[j] = 0.f;
    auto take = [&](int m, const f32x4 (&e)[NTL][4]) {
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            if (!tv[j]) continue;
            float A[4], W3[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                A[kt] = ((e[j][kt][0] + e[j][kt][1]) + e[j][kt][2]) + e[j][kt][3];
                W3[kt] = e[j][kt][3];
            }
            // window 4 j' - 1 of block j' = 16 m + 4 kt + gq sits in lane row
            // gq - 1 of the same kt, or lane row 3 of kt - 1 (previous chunk
            // for kt = 0, gq = 0)
            float s1[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) s1[kt] = __shfl(W3[kt], (lane + 48) & 63, 64);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) A[kt] += gq > 0 ? s1[kt] : kt > 0 ? s1[kt - 1] : carry[j];
            carry[j] = s1[3];
            // sum over the G heads of the token (lanes n .. n + G - 1)
#pragma unroll
            for (int off = 1; off < G; off <<= 1)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) A[kt] += lane_xor(A[kt], off);
            // room for this chunk's 16 blocks in every token's pending entries
            uint64_t full = __ballot(lead && gq == 0 && bb[j] >= 0 && cnt[j] + 16 > lcap);
            while (full) {
                compact(j, __builtin_ctzll(full));
                full &= full - 1;
            }
            const bool act = lead && bb[j] >= 0;
            const int bit0 = n;  // the token's lanes: n, n + 16, n + 32, n + 48
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int jb = m * 16 + kt * 4 + gq;
                const bool in = act && jb <= bb[j] && !forced(jb, bb[j]) && A[kt] > thr[j];
                const uint64_t mk = __ballot(in);
                const unsigned b4 = (unsigned)((mk >> bit0) & 1ull) | (unsigned)((mk >> (bit0 + 16)) & 1ull) << 1 |
                                    (unsigned)((mk >> (bit0 + 32)) & 1ull) << 2 | (unsigned)((mk >> (bit0 + 48)) & 1ull) << 3;
                if (in) {
                    const int at = tok[j] * lcap + cnt[j] + __builtin_popcount(b4 & ((1u << gq) - 1u));
                    pv[at] = A[kt];
                    pj[at] = jb;
                }
                if (act) cnt[j] += __builtin_popcount(b4);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // pass 2: chunks with visible windows, then (all probabilities 0) the
    // chunks that only hold blocks <= b
    stream(nch1, [&](int m, const u16* cur) {
        f32x4 x[NTL][4];
        scores(cur, m, x);
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[j][kt][i] = __builtin_amdgcn_exp2f(fmaf(x[j][kt][i], sl, -lse2[j]));
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

    // lists: forced ids (init blocks, then local blocks b, b - 1, ..), then the
    // k best in rank order (a last compaction of every token), then -1
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        if (!tv[j]) continue;
        uint64_t all = __ballot(lead && gq == 0 && bb[j] >= 0);
        while (all) {
            compact(j, __builtin_ctzll(all));
            all &= all - 1;
        }
        if (lead && gq == 0 && bb[j] >= 0) {
            const int tl = tok[j], b = bb[j];
            int32_t* out = p.sel_out + ((int64_t)(c0 + i0 + tl) * p.Hkv + h) * topk;
            int o = 0;
            for (int jj = 0; jj < p.sel_init && jj <= b && o < topk; ++jj) out[o++] = jj;
            for (int u = 0; u < p.sel_local && o < topk; ++u) {
                const int jj = b - u;
                if (jj >= 0 && jj >= p.sel_init) out[o++] = jj;
            }
            for (int r = 0; r < cnt[j]; ++r) out[o++] = pj[tl * lcap + r];
            while (o < topk) out[o++] = -1;
        }
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
    const size_t lds = 2 * sizeof(float) * (size_t)p.sel_tok * p.sel_lcap;
    const dim3 grid((unsigned)(p.T / p.sel_tok + p.B), (unsigned)p.Hkv);
    hipLaunchKernelGGL((k_select<E, D, G>), grid, dim3(64 * kSelWaves), lds, st, p);
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

// Pending-entry slots per token of the list kernel: the list (at most topk)
// plus one chunk's 16 blocks, in one or two entries per lane.
int select_list_cap(int topk) { return topk + 16 <= 64 ? 64 : 128; }

// Tokens per token tile of the list kernel for group size G and topk: the
// 256 rows of a workgroup, halved while the pending entries (importance and
// id per slot) would pass 64 KB; a whole number of 16-row tiles.
int select_tokens(int G, int topk)
{
    int tok = kSelRows / G;
    while (tok * G > 16 && (size_t)tok * select_list_cap(topk) * 8 > (size_t)kSelCandBytes) tok /= 2;
    return tok;
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
