// index.hip -- index inversion: per-token block lists -> per-block token lists.
//
// A key/value-outer schedule (Flash-Sparse-Attention project page,
// "Importance" and "Key features": the outer and inner loops are swapped so
// that the kv blocks are the outer loop) needs, for every kv block, the list
// of tokens that selected it.  This file builds that list as a CSR per
// (kv head, block) bucket with a stable counting sort, so the result is
// unique and bitwise reproducible; integer atomics only ever produce totals
// (LDS histograms, LDS bit masks), never positions.
//
//   prep     sanitised cu_seqlens, per-sequence block offsets, status reset
//   dense    (forward only) per (kv head, token block): the blocks every token
//            of the block keeps; those pairs skip the CSR and go to the
//            dense+merge kernel
//   count    per (token tile, kv head): LDS histogram of kept blocks
//   colscan  per bucket: exclusive prefix over tiles -> tile bases, totals
//   scan     exclusive prefix over buckets -> offsets; work items per bucket
//            and the item -> bucket map
//   scatter  per (token tile, kv head), one wave: 64 tokens per round, rank
//            within the round from an LDS bit mask per bucket
#include "internal.h"

namespace nsa {

namespace {

// Grids over (token range, kv head) pairs.  Workgroup i runs on XCD i % 8 and
// each XCD takes its workgroups in index order, so with the grid padded to a
// multiple of 8, logical id (i % 8) * (grid / 8) + i / 8 gives every XCD one
// contiguous run of logical ids, taken in order.  With the kv head fastest in
// the logical id, the kv heads of one token range run side by side on one XCD,
// and the block-index rows of a token (all kv heads adjacent in memory) are
// fetched once into that XCD's L2 instead of once per kv head.
__host__ __device__ inline int64_t xcd_grid(int64_t n) { return div_up(n, kNumXcd) * kNumXcd; }
__device__ __forceinline__ int64_t xcd_logical()
{
    const int64_t per = gridDim.x / kNumXcd;
    return (int64_t)(blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd;
}

// One workgroup of 256 threads.
__global__ __launch_bounds__(256) void k_prep(Params p)
{
    __shared__ int sh[16];
    __shared__ int carry_max, carry_sum, bad;
    const int tid = threadIdx.x;
    if (tid == 0) {
        p.status[kStatusError] = 0;
        p.status[kStatusNnz] = 0;
        p.status[kStatusItems] = 0;
        for (int x = 0; x < kNumXcd; ++x) p.status[kStatusQueue + x] = 0;
        carry_max = 0;
        carry_sum = 0;
        bad = 0;
    }
    __syncthreads();
    const int n = p.B + 1;
    const int T = (int)p.T;
    for (int base = 0; base < n; base += 256) {
        const int s = base + tid;
        int raw = s < n ? p.cu[s] : 0;
        int c = min(max(raw, 0), T);
        // sanitised value: running maximum, clamped to [0, T]
        int run = block_inclusive_scan<true>(s < n ? c : 0, sh);
        run = max(run, carry_max);
        int prev_raw = s < n && s > 0 ? p.cu[s - 1] : 0;
        bool b = s < n && ((s == 0 && raw != 0) || (s == n - 1 && raw != T) || (s > 0 && raw < prev_raw) ||
                           raw < 0 || raw > T);
        if (b) atomicOr(&bad, 1);
        if (s < n) p.cus[s] = run;
        // block count of sequence s-1 ends at run; store blocks of sequence s after
        __syncthreads();
        if (tid == 255) carry_max = run;
        __syncthreads();
    }
    // blkoff[s] = sum_{s' < s} ceil((cus[s'+1] - cus[s']) / bs)
    for (int base = 0; base < n; base += 256) {
        const int s = base + tid;
        int nb = 0;
        if (s >= 1 && s < n) nb = (int)div_up(p.cus[s] - p.cus[s - 1], p.bs);
        int inc = block_inclusive_scan<false>(nb, sh) + carry_sum;
        if (s < n) p.blkoff[s] = inc;
        __syncthreads();
        if (tid == 255) carry_sum = inc;
        __syncthreads();
    }
    if (tid == 0 && bad) p.status[kStatusError] |= kBadSeqlens;
}

// The LDS tables of the count and scatter kernels cover kIdxWindow buckets at
// a time; with more buckets per kv head (T / bs + B), a tile walks its
// tokens once per window of buckets.
template <int MAXK>
__global__ __launch_bounds__(256) void k_count(Params p)
{
    extern __shared__ int32_t hist[];  // [min(nbc, kIdxWindow)]
    const int64_t lg = xcd_logical();  // tile * Hkv + h
    const int tile = (int)(lg / p.Hkv), h = (int)(lg % p.Hkv), tid = threadIdx.x;
    if (tile >= p.ntiles) return;  // grid padding (uniform)
    const int64_t t0 = (int64_t)tile * p.tile_tokens;
    const int64_t t1 = min(p.T, t0 + p.tile_tokens);
    int bad = 0;
    int32_t* dst = p.tilecnt + ((size_t)h * p.ntiles + tile) * p.nbc;
    for (int g0 = 0; g0 < p.nbc; g0 += kIdxWindow) {
        const int gw = min(kIdxWindow, p.nbc - g0);
        for (int g = tid; g < gw; g += 256) hist[g] = 0;
        __syncthreads();
        for (int64_t t = t0 + tid; t < t1; t += 256) {
            const int s = seq_of_token(p.cus, p.B, t);
            if (s < 0) continue;
            const int c0 = p.cus[s];
            const int b = (int)((t - c0) / p.bs);
            const int nb = (int)div_up(p.cus[s + 1] - c0, p.bs);
            int32_t row[MAXK];
            load_row<MAXK>(p, t, h, row);
            if (g0 == 0) {
#pragma unroll
                for (int kk = 0; kk < MAXK; ++kk)
                    if (kk < p.topk && (row[kk] < -1 || row[kk] >= nb)) bad = 1;
            }
            const int base = p.blkoff[s];
            const uint64_t m = drop_dense<MAXK>(p, h, base + b, row, keep_mask<MAXK>(row, p.topk, b));
#pragma unroll
            for (int kk = 0; kk < MAXK; ++kk) {
                const int g = base + row[kk] - g0;
                if (((m >> kk) & 1) && g >= 0 && g < gw) atomicAdd(&hist[g], 1);
            }
        }
        __syncthreads();
        for (int g = tid; g < gw; g += 256) dst[g0 + g] = hist[g];
        __syncthreads();  // (the next window clears the table)
    }
    if (bad) atomicOr(&p.status[kStatusError], kBadBlockId);
}

// Dense sets: one wave per (kv head, global token block g).  A block id is
// dense for g when every token of token block g keeps it; candidates are the
// kept ids of the block's first token.  Ids are written ascending.
template <int MAXK>
__global__ __launch_bounds__(256) void k_dense(Params p)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t lg = xcd_logical() * 4 + wave;  // g * Hkv + h: kv heads of a token block together
    const int g = (int)(lg / p.Hkv), h = (int)(lg % p.Hkv);
    if (g >= p.nbc) return;  // grid padding (whole wave)
    const int64_t idx = (int64_t)h * p.nbc + g;  // storage order of the dense sets
    if (g >= p.blkoff[p.B]) {  // unused block capacity
        if (lane == 0) p.dense_cnt[idx] = 0;
        return;
    }
    int slo = 0, shi = p.B - 1;  // last sequence with blkoff <= g
    while (slo < shi) {
        int mid = (slo + shi + 1) >> 1;
        if (p.blkoff[mid] <= g) slo = mid; else shi = mid - 1;
    }
    const int b = g - p.blkoff[slo];
    const int64_t c0 = p.cus[slo];
    const int64_t t0 = c0 + (int64_t)b * p.bs;
    const int64_t t1 = min(c0 + (int64_t)(b + 1) * p.bs, (int64_t)p.cus[slo + 1]);
    int32_t row0[MAXK];
    load_row<MAXK>(p, t0, h, row0);
#pragma unroll
    for (int kk = 0; kk < MAXK; ++kk) row0[kk] = __builtin_amdgcn_readfirstlane(row0[kk]);  // one row for all lanes
    uint64_t dmask = keep_mask<MAXK>(row0, p.topk, b);
    for (int64_t tb = t0; tb < t1; tb += 64) {
        const int64_t t = tb + lane;
        int32_t row[MAXK];
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) row[kk] = -1;
        if (t < t1) load_row<MAXK>(p, t, h, row);
        // Every token of the block has the same block index b, so a
        // candidate (an id in [0, b]) is kept by token t exactly when it
        // appears among t's topk ids: no keep mask of t is needed.
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) {
            if (!((dmask >> kk) & 1)) continue;  // uniform
            const int c = row0[kk];
            bool have = t >= t1;
#pragma unroll
            for (int k2 = 0; k2 < MAXK; ++k2) have |= row[k2] == c;
            if (__ballot(!have)) dmask &= ~(1ull << kk);
        }
    }
    if (lane == 0) {
        p.dense_cnt[idx] = __popcll(dmask);
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) {
            if (!((dmask >> kk) & 1)) continue;
            int r = 0;
#pragma unroll
            for (int k2 = 0; k2 < MAXK; ++k2)
                r += ((dmask >> k2) & 1) && row0[k2] < row0[kk];
            p.dense_ids[idx * p.topk + r] = row0[kk];
        }
    }
}

// Exclusive prefix over the tiles of each (kv head, bucket) column of the
// tile table, and the column totals (the bucket sizes).
__global__ __launch_bounds__(256) void k_colscan(Params p)
{
    // 16 columns (h, g) per workgroup, each cut into 16 runs of tiles, one
    // thread per (column, run): run sums, their exclusive prefix in LDS, then
    // each run rewritten as running sums from its prefix
    __shared__ int sRun[16][16];
    const int col = threadIdx.x & 15, run = threadIdx.x >> 4;
    const int64_t idx = (int64_t)blockIdx.x * 16 + col;
    const bool ok = idx < (int64_t)p.Hkv * p.nbc;
    const int h = ok ? (int)(idx / p.nbc) : 0, g = ok ? (int)(idx % p.nbc) : 0;
    int32_t* colp = p.tilecnt + (size_t)h * p.ntiles * p.nbc + g;
    const int per = (p.ntiles + 15) / 16;
    const int t0 = min(p.ntiles, run * per), t1 = min(p.ntiles, t0 + per);
    int sum = 0;
    if (ok)
#pragma unroll 4
        for (int tile = t0; tile < t1; ++tile) sum += colp[(size_t)tile * p.nbc];
    sRun[run][col] = sum;
    __syncthreads();
    int base = 0;
    for (int r = 0; r < run; ++r) base += sRun[r][col];
    if (!ok) return;
#pragma unroll 4
    for (int tile = t0; tile < t1; ++tile) {
        const int c = colp[(size_t)tile * p.nbc];
        colp[(size_t)tile * p.nbc] = base;
        base += c;
    }
    if (run == 15) p.counts[idx] = base;
}

// One workgroup of 1024 threads; each thread owns a contiguous run of buckets.
__global__ __launch_bounds__(1024) void k_scan(Params p, int32_t* offsets)
{
    __shared__ int sh[16];
    const int n = p.Hkv * p.nbc;
    const int tid = threadIdx.x;
    const int per = (n + 1023) / 1024;
    const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
    int c_sum = 0, i_sum = 0;
    for (int b = b0; b < b1; ++b) {
        int c = p.counts[b];
        c_sum += c;
        i_sum += (c * p.G + p.item_rows - 1) / p.item_rows;
    }
    int c_inc = block_inclusive_scan<false>(c_sum, sh);
    int i_inc = block_inclusive_scan<false>(i_sum, sh);
    int c_run = c_inc - c_sum, i_run = i_inc - i_sum;
    for (int b = b0; b < b1; ++b) {
        int c = p.counts[b];
        offsets[b] = c_run;
        p.item_start[b] = i_run;
        const int ni = (c * p.G + p.item_rows - 1) / p.item_rows;
        if (p.item_bucket)  // the work-item -> bucket map of this thread's buckets
            for (int i = i_run; i < i_run + ni; ++i) p.item_bucket[i] = b;
        c_run += c;
        i_run += ni;
    }
    if (tid == 1023) {
        offsets[n] = c_inc;
        p.item_start[n] = i_inc;
        p.status[kStatusNnz] = c_inc;
        p.status[kStatusItems] = i_inc;
    }
}

// Work-item -> bucket map for the forward on a prebuilt index: one thread per
// bucket writes its items (the inversion's scan writes the map itself).
__global__ __launch_bounds__(256) void k_items(Params p)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= (int64_t)p.Hkv * p.nbc) return;
    const int i0 = p.item_start[b], i1 = p.item_start[b + 1];
    for (int i = i0; i < i1; ++i) p.item_bucket[i] = (int32_t)b;
}

// One wave per (token tile, kv head).  Entries of a bucket land in order of
// tile (tile bases), then round (running count), then lane (bit-mask rank);
// lanes are consecutive tokens, so every bucket list is ascending in t.  For
// the merges, each row's kept CSR positions are recorded too, in ascending
// block order and then -1 up to topk: partial results are stored in CSR order
// and the merges read them in that order.
template <int MAXK>
__global__ __launch_bounds__(64) void k_scatter(Params p, const int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ entries)
{
    extern __shared__ uint64_t smem64[];
    const int nw = min(p.nbc, kIdxWindow);
    uint64_t* mask = smem64;                                 // [nw]
    int32_t* run = reinterpret_cast<int32_t*>(smem64 + nw);  // [nw]
    const int64_t lg = xcd_logical();  // tile * Hkv + h
    const int tile = (int)(lg / p.Hkv), h = (int)(lg % p.Hkv), lane = threadIdx.x;
    if (tile >= p.ntiles) return;  // grid padding (uniform)
    const int32_t* tbase = p.tilecnt + ((size_t)h * p.ntiles + tile) * p.nbc;
    const int32_t* off = offsets + (size_t)h * p.nbc;
    const int64_t t0 = (int64_t)tile * p.tile_tokens;
    const int64_t t1 = min(p.T, t0 + p.tile_tokens);
    const uint64_t lower = (1ull << lane) - 1;
    for (int g0 = 0; g0 < p.nbc; g0 += kIdxWindow)  // windows of buckets (usually one)
    for (int64_t r0 = t0; r0 < t1; r0 += 64) {
        if (r0 == t0) {
            // run[g]: CSR position of the bucket's next entry from this tile
            // (bucket offset + tile base + entries of the earlier rounds)
            for (int g = lane; g < nw; g += 64) {
                mask[g] = 0;
                run[g] = g0 + g < p.nbc ? off[g0 + g] + tbase[g0 + g] : 0;
            }
            __syncthreads();
        }
        const int64_t t = r0 + lane;
        int s = t < t1 ? seq_of_token(p.cus, p.B, t) : -1;
        int32_t row[MAXK] = {};
        uint64_t m = 0;
        int gbase = 0;
        if (s >= 0) {
            const int c0 = p.cus[s];
            load_row<MAXK>(p, t, h, row);
            const int b = (int)((t - c0) / p.bs);
            gbase = p.blkoff[s];
            m = drop_dense<MAXK>(p, h, gbase + b, row, keep_mask<MAXK>(row, p.topk, b));
        }
        // rank of each kept slot among the row's kept blocks (kept ids are
        // distinct; the others compare as INT_MAX and rank nothing)
        int rk[MAXK], kid[MAXK];
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) kid[kk] = (m >> kk) & 1 ? row[kk] : INT_MAX;
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) {
            rk[kk] = 0;
#pragma unroll
            for (int k2 = 0; k2 < MAXK; ++k2) rk[kk] += kid[k2] < kid[kk];
        }
        int32_t* srow = p.slot_pos ? p.slot_pos + ((size_t)t * p.Hkv + h) * p.topk : nullptr;
        if (srow && t < t1 && g0 == 0)
            for (int r = __popcll(m); r < p.topk; ++r) srow[r] = -1;
        // this window's kept slots
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) {
            const int gl = gbase + row[kk] - g0;
            if (!(gl >= 0 && gl < nw)) m &= ~(1ull << kk);
        }
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk)
            if ((m >> kk) & 1) atomicOr((unsigned long long*)&mask[gbase + row[kk] - g0], 1ull << lane);
        __syncthreads();
        uint64_t last = 0;
        int cnt[MAXK];
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) {
            cnt[kk] = 0;
            if ((m >> kk) & 1) {
                const int g = gbase + row[kk];
                const uint64_t mk = mask[g - g0];
                const int pos = run[g - g0] + __popcll(mk & lower);
                entries[pos] = (int32_t)(t * p.topk + kk);
                if (srow) srow[rk[kk]] = pos;
                if ((mk >> lane) == 1ull) {
                    last |= 1ull << kk;
                    cnt[kk] = __popcll(mk);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk)
            if ((last >> kk) & 1) {
                const int gl = gbase + row[kk] - g0;
                run[gl] += cnt[kk];
                mask[gl] = 0;
            }
        __syncthreads();
    }
}

template <int MAXK>
hipError_t launch_index_t(const Params& p, int32_t* offsets, int32_t* entries, hipStream_t st)
{
    hipLaunchKernelGGL(k_prep, dim3(1), dim3(256), 0, st, p);
    const dim3 tiles((unsigned)xcd_grid((int64_t)p.ntiles * p.Hkv));  // (tile, kv head), kv head fastest
    const int nw = p.nbc < kIdxWindow ? p.nbc : kIdxWindow;
    const size_t lds_count = sizeof(int32_t) * nw;
    const size_t lds_scatter = (sizeof(uint64_t) + sizeof(int32_t)) * nw;
    hipError_t e = hipFuncSetAttribute((const void*)k_count<MAXK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_count);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)k_scatter<MAXK>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_scatter);
    if (e != hipSuccess) return e;
    const int64_t nbk = (int64_t)p.Hkv * p.nbc;
    if (p.dense_cnt)
        hipLaunchKernelGGL(k_dense<MAXK>, dim3((unsigned)xcd_grid(div_up(nbk, 4))), dim3(256), 0, st, p);
    if (p.T > 0) hipLaunchKernelGGL(k_count<MAXK>, tiles, dim3(256), lds_count, st, p);
    hipLaunchKernelGGL(k_colscan, dim3((unsigned)div_up(nbk, 16)), dim3(256), 0, st, p);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, p, offsets);  // (writes the item map too)
    if (p.T > 0)
        hipLaunchKernelGGL(k_scatter<MAXK>, tiles, dim3(64), lds_scatter, st, p,
                           (const int32_t*)offsets, entries);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Forward on a prebuilt index (offsets and entries that nsa_sel_build_index
// wrote for the same descriptor, cu_seqlens and block_idx).  What the
// forward derives from the inversion is rebuilt from them, memory-safely
// whatever they hold:
//   idx_offsets  sanitised offsets (clamped to [0, capacity], non-decreasing)
//                into the workspace, work items, nnz
//   idx_rows     every row's kept-position list set to -1
//   idx_entries  per bucket: its entries copied into the workspace; one that
//                is not a kept (t, slot) of the bucket's block in block_idx
//                becomes 0 (a valid token, whose partial nobody reads) and
//                sets a status bit; a valid one's CSR position goes to its
//                row's list at the rank of its block among the row's kept
//                blocks, as the inversion's scatter writes it
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_idx_offsets(Params p, const int32_t* __restrict__ offsets_in, int cap)
{
    __shared__ int sh[16];
    __shared__ int s_incl[1024];
    const int n = p.Hkv * p.nbc;
    const int tid = threadIdx.x;
    const int per = (n + 1 + 1023) / 1024;
    const int b0 = min(n + 1, tid * per), b1 = min(n + 1, b0 + per);
    int m = 0;
    for (int b = b0; b < b1; ++b) m = max(m, min(max(offsets_in[b], 0), cap));
    s_incl[tid] = block_inclusive_scan<true>(m, sh);
    __syncthreads();
    int run = tid > 0 ? s_incl[tid - 1] : 0;
    for (int b = b0; b < b1; ++b) {
        run = max(run, min(max(offsets_in[b], 0), cap));
        p.offsets[b] = run;
    }
    __syncthreads();  // (the block's global writes are visible to it after the barrier)
    const int32_t* s_off = p.offsets;
    const int c0 = min(n, b0), c1 = min(n, b1);  // buckets of this thread
    int i_sum = 0;
    for (int b = c0; b < c1; ++b) i_sum += ((s_off[b + 1] - s_off[b]) * p.G + p.item_rows - 1) / p.item_rows;
    const int i_inc = block_inclusive_scan<false>(i_sum, sh);
    int i_run = i_inc - i_sum;
    for (int b = c0; b < c1; ++b) {
        p.item_start[b] = i_run;
        i_run += ((s_off[b + 1] - s_off[b]) * p.G + p.item_rows - 1) / p.item_rows;
    }
    if (tid == 1023) {
        p.item_start[n] = i_inc;
        p.status[kStatusNnz] = s_off[n];
        p.status[kStatusItems] = i_inc;
    }
}

__global__ __launch_bounds__(256) void k_idx_rows(Params p)
{
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x < p.T * p.Hkv * p.topk) p.slot_pos[x] = -1;
}

// One workgroup per bucket: an entry is kept when it names a kept (t, slot)
// of the bucket's block in block_idx; any other entry becomes token 0 (its
// partial is never read) and sets the status bit.  The entries need not be
// ascending: the main kernel's causal-mask test looks at every row of a
// chunk, so any order of a bucket's entries gives the same result.
template <int MAXK>
__global__ __launch_bounds__(256) void k_idx_entries(Params p, const int32_t* __restrict__ entries_in)
{
    const int bkt = blockIdx.x;
    const int h = bkt / p.nbc, g = bkt - h * p.nbc;
    const int off0 = p.offsets[bkt], off1 = p.offsets[bkt + 1];
    int s = -1, j = 0, c0 = 0, L = 0;
    if (g < p.blkoff[p.B]) {  // a used bucket: sequence s, block j
        int lo = 0, hi = p.B - 1;  // last sequence with blkoff <= g
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.blkoff[mid] <= g) lo = mid; else hi = mid - 1;
        }
        s = lo;
        j = g - p.blkoff[s];
        c0 = p.cus[s];
        L = p.cus[s + 1] - c0;
    }
    int bad = 0;
    for (int pos = off0 + (int)threadIdx.x; pos < off1; pos += 256) {
        const int e = entries_in[pos];
        const int64_t t = e >= 0 ? e / p.topk : -1;
        const int slot = e >= 0 ? e - (int)t * p.topk : 0;
        bool ok = s >= 0 && t >= c0 && t < c0 + L;
        int rank = 0;
        if (ok) {
            int32_t row[MAXK];
            load_row<MAXK>(p, t, h, row);
            const uint64_t m = keep_mask<MAXK>(row, p.topk, (int)((t - c0) / p.bs));
            int rj = -1;
#pragma unroll
            for (int kk = 0; kk < MAXK; ++kk) {
                if (kk == slot) rj = row[kk];
                rank += ((m >> kk) & 1) && row[kk] < j;
            }
            ok = rj == j && ((m >> slot) & 1);
        }
        if (ok) p.slot_pos[((size_t)t * p.Hkv + h) * p.topk + rank] = pos;
        p.entries[pos] = ok ? e : 0;
        bad |= !ok;
    }
    if (bad) atomicOr(&p.status[kStatusError], kBadPrebuiltIndex);
}

template <int MAXK>
hipError_t launch_index_prebuilt_t(const Params& p, const int32_t* offsets_in, const int32_t* entries_in,
                                   int cap, hipStream_t st)
{
    hipLaunchKernelGGL(k_prep, dim3(1), dim3(256), 0, st, p);
    const int64_t nbk = (int64_t)p.Hkv * p.nbc;
    hipLaunchKernelGGL(k_idx_offsets, dim3(1), dim3(1024), 0, st, p, offsets_in, cap);
    hipLaunchKernelGGL(k_items, dim3((unsigned)div_up(nbk, 256)), dim3(256), 0, st, p);
    if (p.T > 0) {
        hipLaunchKernelGGL(k_idx_rows, dim3((unsigned)div_up(p.T * p.Hkv * p.topk, 256)), dim3(256), 0, st, p);
        hipLaunchKernelGGL(k_idx_entries<MAXK>, dim3((unsigned)nbk), dim3(256), 0, st, p, entries_in);
    }
    return hipGetLastError();
}

}  // namespace

// Forward on a prebuilt index: p.offsets, p.entries, p.item_start,
// p.item_bucket and p.slot_pos are the workspace's; offsets_in / entries_in
// the caller's (entries_in holds at least cap entries).
hipError_t launch_index_prebuilt(const Params& p, const int32_t* offsets_in, const int32_t* entries_in, int cap,
                                 hipStream_t st)
{
    if (p.topk <= 16) return launch_index_prebuilt_t<16>(p, offsets_in, entries_in, cap, st);
    if (p.topk <= 32) return launch_index_prebuilt_t<32>(p, offsets_in, entries_in, cap, st);
    return launch_index_prebuilt_t<64>(p, offsets_in, entries_in, cap, st);
}

// Status reset, sanitised cu_seqlens and per-sequence block offsets only.
hipError_t launch_prep(const Params& p, hipStream_t st)
{
    hipLaunchKernelGGL(k_prep, dim3(1), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_index(const Params& p, int32_t* offsets, int32_t* entries, hipStream_t st)
{
    if (p.topk <= 16) return launch_index_t<16>(p, offsets, entries, st);
    if (p.topk <= 32) return launch_index_t<32>(p, offsets, entries, st);
    return launch_index_t<64>(p, offsets, entries, st);
}

}  // namespace nsa
