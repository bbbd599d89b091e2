// internal.h -- shared definitions of the HIP selected-attention kernels.
//
// Private to the library: launch parameters, the workspace layout and the
// few device helpers every kernel needs (sequence lookup and the row filter
// that decides which block ids of a row are kept).  Nothing here is part of
// the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <limits.h>
#include <stdint.h>

namespace nsa {

// Element type of q, k, v and the outputs.
constexpr int kElemF32 = 0;
constexpr int kElemBF16 = 1;
constexpr int kElemF16 = 2;

// Status word bits (workspace status[0]).
constexpr int kBadSeqlens = 1;
constexpr int kBadBlockId = 2;
constexpr int kBadPrebuiltIndex = 8; // indexed forward: an entry that is not a kept (t, slot) of its bucket

// Slots of the int32 status area at the start of the workspace.
constexpr int kStatusError = 0;   // malformed-input bits
constexpr int kStatusNnz = 1;     // entries written by the inversion
constexpr int kStatusItems = 2;   // main-kernel work items
constexpr int kStatusQueue = 8;   // [8] per-XCD work-queue counters of the main kernel
constexpr int kStatusWords = 64;  // keep 256 B

// Gathered rows (bucket tokens x query heads of the group) per main-kernel
// work item (every item lies inside one bucket): the plan takes the largest
// of kItemRowsMax, its half, .. kItemRowsMin that still gives each of
// kItemPlanWgs workgroups at least kItemPlanPer items at the row count's upper
// bound (T * Hkv * topk * G): large items restage K / V less often, small
// ones balance the persistent workgroups' tails on small workloads.
constexpr int kItemRowsMax = 4096, kItemRowsMin = 1024;
constexpr int kItemPlanWgs = 512, kItemPlanPer = 4;
// Consecutive items a per-XCD work queue hands out before moving to the next
// group (keeps a bucket's items, and so its K/V block, on one XCD's L2).
constexpr int kQueueGroup = 16;
constexpr int kNumXcd = 8;

// Largest bucket count (per kv head) the inversion keeps in LDS.
constexpr int kIdxWindow = 12288;  // buckets per LDS pass of the index build (12 B each in the scatter)

struct Params {
    // shapes
    int64_t T;
    int B, Hq, Hkv, G, D, bs, topk;
    uint32_t g_mul, topk_mul;  // division by G / topk (see FastDiv)
    int g_shr, topk_shr;
    int nbc;          // buckets per kv head: T / bs + B
    int ntiles;       // token tiles of the inversion
    int tile_tokens;  // tokens per inversion tile
    int item_rows;    // gathered rows per main-kernel work item
    int main_grid;    // workgroups of the persistent main kernel
    int flags;
    float scale_log2; // scale * log2(e)
    int64_t max_items;

    // inputs
    const int32_t* cu;        // [B+1] as given
    const int32_t* block_idx; // [T][Hkv][topk]
    const void* q;
    const void* k;
    const void* v;

    // workspace / outputs
    int32_t* status;      // [kStatusWords]
    int32_t* cus;         // [B+1] sanitised cu_seqlens
    int32_t* blkoff;      // [B+1] block offsets of the sequences
    int32_t* tilecnt;     // [Hkv][ntiles][nbc] per-tile bucket counts -> bases
    int32_t* counts;      // [Hkv*nbc] bucket sizes
    int32_t* offsets;     // [Hkv*nbc+1]
    int32_t* item_start;  // [Hkv*nbc+1] first work item of each bucket
    int32_t* item_bucket; // [max_items] bucket of each work item
    int32_t* entries;     // [T*Hkv*topk] CSR entries t*topk + slot
    int32_t* slot_pos;    // [T*Hkv*topk] per (t, h): kept CSR positions by ascending block, then -1; or null
    int32_t* dense_cnt;   // [Hkv*nbc] blocks every token of a token block keeps, or null
    int32_t* dense_ids;   // [Hkv*nbc*topk] those blocks, ascending
    void* dense_o;        // [T*Hkv*G*D] bf16 dense partial per (t, h, head)
    float* dense_lse;     // [T*Hkv*G]
    float* part_lse;      // [nnz*G] partial lse, in CSR order
    void* part_o;         // [nnz*G*D] partial outputs, in CSR order
    void* out;            // [T][Hq][D] (forward output; read by the backward)
    float* lse;           // [T][Hq]    (forward output; read by the backward)

    // backward
    float scale;          // score scale
    int bwd_grid;         // workgroups of the backward main kernel
    int window;           // sliding-window branch: keys i - window < p <= i
    int dense_parts;      // row parts per token block of the dense / window kernel
    int fuse_merge;       // dense split: the dense kernel also merges its tokens' rows (G divides 16)
    const void* dout;     // [T][Hq][D] gradient of out
    float* delta;         // [T*Hq] rowsum(dout * out)
    void* dq_part;        // [nnz*G*D] bf16 per-slot dq / scale, in CSR order
    float* dkv_part;      // [2*bwd_grid][2][bs][D] fp32 dk / scale, dv of split buckets
    void* dq;             // [T][Hq][D]
    void* dk;             // [T][Hkv][D]
    void* dv;             // [T][Hkv][D]

    // index producer
    int sel_init, sel_local;  // forced init / local blocks per list
    int sel_cap;              // compressed-window capacity: T / stride + B
    int32_t* sel_cbase;       // [B+1] first compressed window of each sequence
    int32_t* sel_tbase;       // [B+1] first token tile of each sequence
    int sel_tok;              // tokens per token tile of the list kernel
    void* sel_kcmp;           // [sel_cap][Hkv][D] compressed keys (16-bit)
    int32_t* sel_out;         // [T][Hkv][topk] block lists
};

// Gathered rows per chunk of the backward main kernel; the rows a workgroup
// owns are a multiple of this.
constexpr int kBwdRows = 32;
// Most workgroups the backward main kernel launches (two dk/dv partial slots
// each in the workspace).
constexpr int kBwdMaxGrid = 1024;
// Threads of a backward main workgroup: one wave per 16 keys of the block, two
// at d = 256 (one per half of d for dK, dV).
__host__ __device__ constexpr int bwd_threads(int D, int bs) { return bs * 4 * (D > 128 ? 2 : 1); }

// Inclusive block-wide scan of one int per thread (blockDim.x = 64 * nw).
template <bool IS_MAX>
__device__ inline int block_inclusive_scan(int x, int* sh_waves)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x = IS_MAX ? max(x, y) : x + y;
    }
    if (lane == 63) sh_waves[wave] = x;
    __syncthreads();
    int base = IS_MAX ? INT_MIN : 0;
    for (int w = 0; w < wave; ++w) base = IS_MAX ? max(base, sh_waves[w]) : base + sh_waves[w];
    __syncthreads();
    return IS_MAX ? max(base, x) : base + x;
}

// Sequence of token t under the sanitised cu_seqlens: the s with
// cus[s] <= t < cus[s+1], or -1 for a token outside every sequence.
__device__ __forceinline__ int seq_of_token(const int32_t* __restrict__ cus, int B, int64_t t)
{
    if (B <= 0 || t < cus[0] || t >= cus[B]) return -1;
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cus[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Merges run one wave per (token, kv head) row, four waves per workgroup,
// over a grid that is a multiple of the XCD count.  Workgroup i runs on XCD
// i % 8; each XCD takes a contiguous range of the kv-head-major row order
// (one kv head per XCD at 8 kv heads), so the partials one XCD reads lie in
// one head's part of the CSR-ordered buffer.  Returns t * Hkv + h, or -1.
__host__ __device__ inline int64_t merge_grid(int64_t T, int Hkv) { return (T * Hkv + 4 * kNumXcd - 1) / (4 * kNumXcd) * kNumXcd; }
__device__ __forceinline__ int64_t merge_rowid(int64_t T, int Hkv)
{
    const int64_t per = gridDim.x / kNumXcd;
    const int64_t w = (blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd;
    const int64_t idx = w * 4 + (threadIdx.x >> 6);
    if (idx >= T * Hkv) return -1;
    const int64_t h = idx / T;
    return (idx - h * T) * Hkv + h;
}

// Which slots of a row are kept: bit k set iff 0 <= row[k] <= b and no
// earlier slot holds the same id.  `row` holds topk ids (topk <= 64).
template <int MAXK>
__device__ __forceinline__ uint64_t keep_mask(const int32_t* row, int topk, int b)
{
    uint64_t m = 0;
#pragma unroll
    for (int kk = 0; kk < MAXK; ++kk) {
        if (kk >= topk) break;
        int j = row[kk];
        bool keep = (j >= 0) && (j <= b);
#pragma unroll
        for (int k2 = 0; k2 < MAXK; ++k2) {
            if (k2 >= kk) break;
            keep = keep && (row[k2] != j);
        }
        if (keep) m |= (1ull << kk);
    }
    return m;
}

__host__ __device__ inline int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Division of 0 <= x < 2^31 by a fixed d >= 1 as a multiply-high and a shift
// (the round-up method for invariant integer division, Granlund and
// Montgomery, 1994): with s = ceil(log2 d) and m = floor(2^(31+s) / d) + 1,
// floor(x / d) = umulhi(x, m) >> (s - 1) for d >= 2, since the excess of m d
// over 2^(31+s) is at most d <= 2^s and x < 2^31.  d = 1 is passed through.
inline void fast_div_init(int d, uint32_t& mul, int& shr)
{
    if (d <= 1) {
        mul = 0;
        shr = 0;
        return;
    }
    int s = 0;
    while ((1ll << s) < d) ++s;
    mul = (uint32_t)((((uint64_t)1 << (31 + s)) / (uint64_t)d) + 1);
    shr = s - 1;
}
__device__ __forceinline__ int fast_div(int x, int d, uint32_t mul, int shr)
{
    return d == 1 ? x : (int)(__umulhi((uint32_t)x, mul) >> shr);
}

// Loads row (t, h) of block_idx into registers (-1 beyond topk).
template <int MAXK>
__device__ __forceinline__ void load_row(const Params& p, int64_t t, int h, int32_t (&row)[MAXK])
{
    const int32_t* src = p.block_idx + ((size_t)t * p.Hkv + h) * p.topk;
    if ((p.topk & 3) == 0) {
#pragma unroll
        for (int kk = 0; kk < MAXK; kk += 4) {
            if (kk < p.topk) {
                int4 v = *reinterpret_cast<const int4*>(src + kk);
                row[kk] = v.x; row[kk + 1] = v.y; row[kk + 2] = v.z; row[kk + 3] = v.w;
            } else {
                row[kk] = row[kk + 1] = row[kk + 2] = row[kk + 3] = -1;
            }
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk) row[kk] = kk < p.topk ? src[kk] : -1;
    }
}

// Clears from keep-mask m the slots whose block is in the dense set of
// (kv head h, global token block g): blocks every token of that token block
// keeps, which the dense+merge kernel handles instead of the CSR path.
template <int MAXK>
__device__ __forceinline__ uint64_t drop_dense(const Params& p, int h, int g, const int32_t (&row)[MAXK],
                                               uint64_t m)
{
    if (!p.dense_cnt || !m) return m;
    const size_t dk = (size_t)h * p.nbc + g;
    const int dc = p.dense_cnt[dk];
    for (int i = 0; i < dc; ++i) {
        const int dj = p.dense_ids[dk * p.topk + i];
#pragma unroll
        for (int kk = 0; kk < MAXK; ++kk)
            if (row[kk] == dj) m &= ~(1ull << kk);
    }
    return m;
}

}  // namespace nsa
