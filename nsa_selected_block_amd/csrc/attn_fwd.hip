// attn_fwd.hip -- main selected-attention kernel and partial-result merge.
//
// Main kernel (Flash-Sparse-Attention project page, "Key features",
// optimised-kernels row: the main batched query-to-KV kernel).  The kv block
// is the outer loop ("Importance": outer and inner loops swapped).  A work
// item is up to item_rows (1024, 2048 or 4096, planned per call) gathered
// rows (bucket token x query head of the GQA group) of one (kv head, kv
// block) bucket.  A persistent workgroup takes
// items from a per-XCD queue and stages the bucket's K and V block into LDS
// when the bucket changes; its waves run 16-row chunks on their own (see the
// kernel below).  Partial outputs are normalised 16-bit rows plus an fp32
// log-sum-exp, stored at the entry's CSR position, so an item writes one
// contiguous stream (the merge finds a row's partials through slot_pos).
// No atomics touch results (one integer counter per queue hands out work).
//
// Merge (same row: the reduction and online-softmax kernels).  One wave per
// (token, kv head) combines the row's partials in ascending block order:
// M = max lse_s, w_s = exp(lse_s - M), out = sum w_s o_s / sum w_s,
// lse = M + ln sum w_s.  In the 16-bit forward the blocks that every token of
// a token block keeps (at the workloads here: the init block and the two
// local blocks) skip the gather path: a dense kernel attends to them with
// whole query tiles and leaves one more partial per row for the merge.
#include "device_common.h"

#include <algorithm>
#include <atomic>
#include <float.h>

namespace nsa {

#ifndef NSA_MAIN_NT
#define NSA_MAIN_NT 1
#endif
// Row tiles (16 rows each) per wave chunk of the 16-bit main kernel.
constexpr int kMainNT = NSA_MAIN_NT;
#ifndef NSA_MAIN_WAVES
#define NSA_MAIN_WAVES 8
#endif
#ifndef NSA_MAIN_OCC
#define NSA_MAIN_OCC 4
#endif
// Waves per workgroup of the 16-bit main kernel (they share the staged K/V
// block) and the waves per SIMD it is compiled for.
constexpr int kMainWaves = NSA_MAIN_WAVES;
constexpr int kMainOcc = NSA_MAIN_OCC;

namespace {

// ---------------------------------------------------------------------------
// fp32 main kernel (VALU): one thread per gathered row, online softmax over
// the bucket's keys staged in LDS; one workgroup per 256 rows of a work item
// (item_rows / 256 workgroups per item).
// ---------------------------------------------------------------------------
static_assert(kItemRowsMin % 256 == 0, "work items of whole 256-row parts");

template <int D, int BS>
__global__ __launch_bounds__(256) void k_main_f32(Params p)
{
    __shared__ __attribute__((aligned(16))) float sK[BS * D];
    __shared__ __attribute__((aligned(16))) float sV[BS * D];
    const int parts = p.item_rows / 256;
    const int item = blockIdx.x / parts, part = blockIdx.x % parts;
    if (item >= p.status[kStatusItems]) return;
    const int bkt = p.item_bucket[item];
    const Bucket bk = decode_bucket(p, bkt);
    const int item_row0 = (item - p.item_start[bkt]) * p.item_rows;
    const int row0 = item_row0 + part * 256;
    const int row_end = min(row0 + 256, min(item_row0 + p.item_rows, bk.cnt * p.G));
    if (row0 >= row_end) return;  // (uniform: before the staging's barrier)
    const int tid = threadIdx.x;
    const int Hkv = p.Hkv, G = p.G;
    const float* kg = reinterpret_cast<const float*>(p.k);
    const float* vg = reinterpret_cast<const float*>(p.v);
    for (int x = tid; x < BS * (D / 4); x += 256) {
        const int key = x / (D / 4), c4 = x - key * (D / 4);
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (key < bk.nkeys) {
            const int64_t off = ((int64_t)(bk.c0 + bk.kbeg + key) * Hkv + bk.h) * D + c4 * 4;
            kv = *reinterpret_cast<const float4*>(kg + off);
            vv = *reinterpret_cast<const float4*>(vg + off);
        }
        *reinterpret_cast<float4*>(&sK[key * D + c4 * 4]) = kv;
        *reinterpret_cast<float4*>(&sV[key * D + c4 * 4]) = vv;
    }
    __syncthreads();
    for (int r = row0 + tid; r < row_end; r += 256) {
        const int ti = r / G, qq = r - ti * G;
        const int ent = p.entries[bk.off + ti];
        const int t = ent / p.topk;
        const int pos = t - bk.c0;
        const float* qrow = reinterpret_cast<const float*>(p.q) + ((int64_t)t * p.Hq + bk.h * G + qq) * D;
        float qv[D], acc[D];
#pragma unroll
        for (int e = 0; e < D; e += 4) {
            const float4 x = *reinterpret_cast<const float4*>(qrow + e);
            qv[e] = x.x; qv[e + 1] = x.y; qv[e + 2] = x.z; qv[e + 3] = x.w;
            acc[e] = acc[e + 1] = acc[e + 2] = acc[e + 3] = 0.f;
        }
        float m = -INFINITY, l = 0.f;
        const int kend = min(bk.nkeys, pos - bk.kbeg + 1);
        for (int key = 0; key < kend; ++key) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) s = fmaf(qv[e], sK[key * D + e], s);
            s *= p.scale_log2;
            const float mn = fmaxf(m, s);
            const float corr = exp2f(m - mn);
            const float w = exp2f(s - mn);
            l = l * corr + w;
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] = fmaf(w, sV[key * D + e], acc[e] * corr);
            m = mn;
        }
        const int64_t prow = (int64_t)(bk.off + ti) * G + qq;  // partial row, CSR order
        float* dst = reinterpret_cast<float*>(p.part_o) + prow * D;
        const float inv = 1.f / l;
#pragma unroll
        for (int e = 0; e < D; e += 4)
            *reinterpret_cast<float4*>(dst + e) =
                make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
        p.part_lse[prow] = (m + log2f(l)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Merge of one (token, kv head) row by one wave; 16-byte chunks of the G*D
// outputs.  Sparse slots are combined in ascending block order, in groups of
// kMergeGroup whose loads (non-temporal: each partial is read once) are all
// issued before any is used.  In the 16-bit forward with the dense split, the
// row's dense partial (dense_o / dense_lse; lse -inf when the token block has
// no dense blocks) starts the merge.  With LDS_DENSE the dense kernel merges
// its own tokens: the row's dense part is its normalised 16-bit tile rows in
// LDS (head qq at lo + qq * lp) and their lse values (ll[qq]; no dense part
// when ll is null), the same values the dense partial would hold.
// ---------------------------------------------------------------------------
constexpr int kMergeGroup = 16;

constexpr float kMergeLog2e = 1.4426950408889634f;

// Slot positions of several rows in one register, loaded by one wave load:
// lane l holds slot l mod S of row l / S, with S the power of two in
// {16, 32, 64} at or above topk (-1 past topk and past the rows), so a row's
// merge does not wait for its own load of them (the fused merge of the dense
// kernel: 2.77 -> 2.74 ms at the 64K+32K GQA-4 workload; the standalone
// merge with four rows per wave lost 6% against one wave per row).
__device__ __forceinline__ int merge_stride(int topk) { return topk <= 16 ? 16 : topk <= 32 ? 32 : 64; }

// NC: 16-byte chunks of the row per lane taken in one walk over the slots
// (rows of 2 KB: both halves' loads in flight together, kMergeGroup / NC
// slots per round); 1 walks the row 1 KB at a time.
template <typename ET, bool LDS_DENSE = false, int NC = 1>
__device__ __forceinline__ void merge_row(const Params& p, int64_t rowid, const u16* lo = nullptr, int lp = 0,
                                          const float* ll = nullptr, int sreg = -1, int sbase = -1)
{
    constexpr bool HALF = sizeof(ET) == 2;  // bf16 or fp16 partials (else fp32)
    constexpr int E = HALF ? 8 : 4;  // elements per 16-byte chunk
    constexpr int MG = kMergeGroup / NC;  // slots per load round
    const int lane = threadIdx.x & 63;
    const int G = p.G, D = p.D, GD = G * D, topk = p.topk;
    // the row's kept CSR positions in ascending block order, then -1 (written
    // by the index build, which also drops the dense set's blocks); the lanes
    // holding one are walked in order, so a -1 between them (only a prebuilt
    // index that lacks a kept slot leaves one) is skipped, never read
    // (sbase >= 0: they sit in lanes sbase .. sbase + topk - 1 of sreg)
    const int base = sbase >= 0 ? sbase : 0;
    const int spos = sbase >= 0 ? sreg : lane < topk ? p.slot_pos[rowid * topk + lane] : -1;
    const uint64_t kept = __ballot(spos >= 0 && lane >= base && lane < base + topk) >> base;
    const int n = __popcll(kept);
    const bool in_seq = p.dense_o && seq_of_token(p.cus, p.B, rowid / p.Hkv) >= 0;

    const char* pob = reinterpret_cast<const char*>(p.part_o);
    for (int c = 0; c * 64 * E < GD; c += NC) {
        int e[NC], ee[NC], qq[NC];
        bool active[NC];
        float M[NC], L[NC];
        float acc[NC][E];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            e[j] = ((c + j) * 64 + lane) * E;
            active[j] = e[j] < GD;
            ee[j] = active[j] ? e[j] : 0;
            qq[j] = ee[j] / D;
            M[j] = -INFINITY;
            L[j] = 0.f;
#pragma unroll
            for (int x = 0; x < E; ++x) acc[j][x] = 0.f;
            if constexpr (LDS_DENSE) {
                if (ll) {
                    M[j] = ll[qq[j]];
                    if (M[j] != -INFINITY) {
                        L[j] = 1.f;
                        const uint4 v4 = *reinterpret_cast<const uint4*>(lo + qq[j] * lp + (ee[j] - qq[j] * D));
                        const uint32_t wd[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            acc[j][2 * x] = H16<ET>::to_f32((u16)(wd[x] & 0xFFFFu));
                            acc[j][2 * x + 1] = H16<ET>::to_f32((u16)(wd[x] >> 16));
                        }
                    }
                }
            } else if (HALF && in_seq) {  // the dense part starts the merge
                M[j] = __builtin_nontemporal_load(&p.dense_lse[rowid * G + qq[j]]);
                if (M[j] != -INFINITY) {
                    L[j] = 1.f;
                    const uint32_t* src = reinterpret_cast<const uint32_t*>(
                        reinterpret_cast<const u16*>(p.dense_o) + rowid * GD + ee[j]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const uint32_t wd = __builtin_nontemporal_load(src + x);
                        if constexpr (HALF) {
                            acc[j][2 * x] = H16<ET>::to_f32((u16)(wd & 0xFFFFu));
                            acc[j][2 * x + 1] = H16<ET>::to_f32((u16)(wd >> 16));
                        }
                    }
                }
            }
        }
        uint64_t km = kept;
        for (int r0 = 0; r0 < n; r0 += MG) {
            float ls[MG][NC];
            uint4 raw[MG][NC];
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const int r = r0 + g;
                const int src_lane = km ? __builtin_ctzll(km) : 0;
                km &= km - 1;
                const int64_t pr = __builtin_amdgcn_readlane(spos, base + src_lane);
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    ls[g][j] = -INFINITY;
                    raw[g][j] = make_uint4(0, 0, 0, 0);
                    if (r < n) {
                        ls[g][j] = __builtin_nontemporal_load(&p.part_lse[pr * G + qq[j]]);
                        const uint32_t* src =
                            reinterpret_cast<const uint32_t*>(pob + (pr * GD + ee[j]) * (HALF ? 2 : 4));
                        raw[g][j] = make_uint4(__builtin_nontemporal_load(src), __builtin_nontemporal_load(src + 1),
                                               __builtin_nontemporal_load(src + 2),
                                               __builtin_nontemporal_load(src + 3));
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                float gm = M[j];
#pragma unroll
                for (int g = 0; g < MG; ++g) gm = fmaxf(gm, ls[g][j]);
                // weights e^(lse - M) as raw v_exp_f32 of (lse - M) log2 e (a
                // weight below 2^-126 flushes to 0)
                const float corr = M[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((M[j] - gm) * kMergeLog2e);
                L[j] *= corr;
#pragma unroll
                for (int x = 0; x < E; ++x) acc[j][x] *= corr;
                M[j] = gm;
#pragma unroll
                for (int g = 0; g < MG; ++g) {
                    if (r0 + g < n) {
                        const float w = __builtin_amdgcn_exp2f((ls[g][j] - M[j]) * kMergeLog2e);
                        L[j] += w;
                        const uint32_t wd[4] = {raw[g][j].x, raw[g][j].y, raw[g][j].z, raw[g][j].w};
                        if constexpr (HALF) {
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                acc[j][2 * x] = fmaf(w, H16<ET>::to_f32((u16)(wd[x] & 0xFFFFu)), acc[j][2 * x]);
                                acc[j][2 * x + 1] =
                                    fmaf(w, H16<ET>::to_f32((u16)(wd[x] >> 16)), acc[j][2 * x + 1]);
                            }
                        } else {
#pragma unroll
                            for (int x = 0; x < 4; ++x) acc[j][x] = fmaf(w, __uint_as_float(wd[x]), acc[j][x]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            if (!active[j]) continue;
            const float inv = L[j] > 0.f ? 1.f / L[j] : 0.f;
            const int64_t ooff = rowid * GD + e[j];
            if constexpr (HALF) {
                uint4 o;
                o.x = pack2h<ET>(acc[j][0] * inv, acc[j][1] * inv);
                o.y = pack2h<ET>(acc[j][2] * inv, acc[j][3] * inv);
                o.z = pack2h<ET>(acc[j][4] * inv, acc[j][5] * inv);
                o.w = pack2h<ET>(acc[j][6] * inv, acc[j][7] * inv);
                *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.out) + ooff) = o;
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + ooff) =
                    make_float4(acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv);
            }
            if (e[j] % D == 0) p.lse[rowid * G + qq[j]] = L[j] > 0.f ? M[j] + logf(L[j]) : -INFINITY;
        }
    }
}

// Rows narrower than a wave (G * D * element size < 1 KB: G = 1 or 2 at
// d = 128) leave most lanes of merge_row idle, and a wave merges one row at a
// time.  Lanes per row, when a group of them can hold a whole row (one 16-byte
// chunk per lane) and its topk slot positions: a power of two below 64, or 0.
__host__ __device__ inline int merge_group_lanes(int G, int D, int topk, bool half)
{
    const int lpr = G * D / (half ? 8 : 4);
    return lpr < 64 && 64 % lpr == 0 && G * D % (half ? 8 : 4) == 0 && topk <= lpr ? lpr : 0;
}

// Merge of 64 / LPR rows at once: lane group gi (lanes gi * LPR ..) merges the
// row `rowid` its lanes carry (-1: none), each lane one 16-byte chunk; `spos`
// is the lane's slot position of its row (slot lane % LPR; -1 past topk).  The
// same steps as merge_row, per lane: the dense part (LDS_DENSE: the row's
// tile rows at lo, their lse at ll; else dense_o / dense_lse), then the kept
// slots in ascending block order, in groups whose loads are all issued first.
template <typename ET, bool LDS_DENSE = false>
__device__ __forceinline__ void merge_rows_grp(const Params& p, int64_t rowid, int spos, int LPR,
                                               const u16* lo = nullptr, int lp = 0, const float* ll = nullptr)
{
    constexpr bool HALF = sizeof(ET) == 2;
    constexpr int E = HALF ? 8 : 4;
    const int lane = threadIdx.x & 63, gl = lane & (LPR - 1), gb = lane - gl;
    const int G = p.G, D = p.D, GD = G * D;
    const bool live = rowid >= 0;
    const int e = gl * E, qq = e / D;
    // this lane's row's kept slots: bits gb .. gb + LPR - 1 of the ballot
    const uint64_t all = __ballot(live && spos >= 0);
    uint64_t km = (all >> gb) & ((1ull << LPR) - 1);
    const int n = __popcll(km);
    float M = -INFINITY, L = 0.f;
    float acc[E];
#pragma unroll
    for (int x = 0; x < E; ++x) acc[x] = 0.f;
    if (live) {
        if constexpr (LDS_DENSE) {
            M = ll[qq];
            if (M != -INFINITY) {
                L = 1.f;
                const uint4 v4 = *reinterpret_cast<const uint4*>(lo + qq * lp + (e - qq * D));
                const uint32_t wd[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    acc[2 * x] = H16<ET>::to_f32((u16)(wd[x] & 0xFFFFu));
                    acc[2 * x + 1] = H16<ET>::to_f32((u16)(wd[x] >> 16));
                }
            }
        } else if (HALF && p.dense_o && seq_of_token(p.cus, p.B, rowid / p.Hkv) >= 0) {
            M = __builtin_nontemporal_load(&p.dense_lse[rowid * G + qq]);
            if (M != -INFINITY) {
                L = 1.f;
                const uint32_t* src = reinterpret_cast<const uint32_t*>(
                    reinterpret_cast<const u16*>(p.dense_o) + rowid * GD + e);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint32_t wd = __builtin_nontemporal_load(src + x);
                    if constexpr (HALF) {
                        acc[2 * x] = H16<ET>::to_f32((u16)(wd & 0xFFFFu));
                        acc[2 * x + 1] = H16<ET>::to_f32((u16)(wd >> 16));
                    }
                }
            }
        }
    }
    const char* pob = reinterpret_cast<const char*>(p.part_o);
    // (a uniform loop: every lane takes part in the permutes)
    for (int r0 = 0; __ballot(r0 < n) != 0; r0 += kMergeGroup) {
        float ls[kMergeGroup];
        uint4 raw[kMergeGroup];
#pragma unroll
        for (int g = 0; g < kMergeGroup; ++g) {
            const int r = r0 + g;
            const int src = km ? __builtin_ctzll(km) : 0;
            km &= km - 1;
            const int64_t pr = __builtin_amdgcn_ds_bpermute((gb + src) << 2, spos);
            ls[g] = -INFINITY;
            raw[g] = make_uint4(0, 0, 0, 0);
            if (r < n) {
                ls[g] = __builtin_nontemporal_load(&p.part_lse[pr * G + qq]);
                const uint32_t* sp = reinterpret_cast<const uint32_t*>(pob + (pr * GD + e) * (HALF ? 2 : 4));
                raw[g] = make_uint4(__builtin_nontemporal_load(sp), __builtin_nontemporal_load(sp + 1),
                                    __builtin_nontemporal_load(sp + 2), __builtin_nontemporal_load(sp + 3));
            }
        }
        float gm = M;
#pragma unroll
        for (int g = 0; g < kMergeGroup; ++g) gm = fmaxf(gm, ls[g]);
        const float corr = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((M - gm) * kMergeLog2e);
        L *= corr;
#pragma unroll
        for (int x = 0; x < E; ++x) acc[x] *= corr;
        M = gm;
#pragma unroll
        for (int g = 0; g < kMergeGroup; ++g) {
            if (r0 + g < n) {
                const float w = __builtin_amdgcn_exp2f((ls[g] - M) * kMergeLog2e);
                L += w;
                const uint32_t wd[4] = {raw[g].x, raw[g].y, raw[g].z, raw[g].w};
                if constexpr (HALF) {
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        acc[2 * x] = fmaf(w, H16<ET>::to_f32((u16)(wd[x] & 0xFFFFu)), acc[2 * x]);
                        acc[2 * x + 1] = fmaf(w, H16<ET>::to_f32((u16)(wd[x] >> 16)), acc[2 * x + 1]);
                    }
                } else {
#pragma unroll
                    for (int x = 0; x < 4; ++x) acc[x] = fmaf(w, __uint_as_float(wd[x]), acc[x]);
                }
            }
        }
    }
    if (!live) return;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int64_t ooff = rowid * GD + e;
    if constexpr (HALF) {
        uint4 o;
        o.x = pack2h<ET>(acc[0] * inv, acc[1] * inv);
        o.y = pack2h<ET>(acc[2] * inv, acc[3] * inv);
        o.z = pack2h<ET>(acc[4] * inv, acc[5] * inv);
        o.w = pack2h<ET>(acc[6] * inv, acc[7] * inv);
        *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.out) + ooff) = o;
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + ooff) =
            make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
    if (e % D == 0) p.lse[rowid * G + qq] = L > 0.f ? M + logf(L) : -INFINITY;
}

// Merge only: one wave per (token, kv head), or, for rows narrower than a
// wave, 64 / LPR rows per wave (LPR = merge_group_lanes, passed by the host).
// Rows are dealt as merge_rowid deals them: kv-head-major, one contiguous
// range per XCD.  NC: chunks per lane per walk over a row's slots (2 for rows
// of 2 KB).
template <typename ET, int NC>
__global__ __launch_bounds__(256) void k_merge(Params p, int LPR)
{
    if (LPR == 0) {
        const int64_t rowid = merge_rowid(p.T, p.Hkv);
        if (rowid < 0) return;
        merge_row<ET, false, NC>(p, rowid);
        return;
    }
    const int lane = threadIdx.x & 63, NR = 64 / LPR;
    const int64_t per = gridDim.x / kNumXcd;
    const int64_t w = (blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd;
    const int64_t idx = (w * 4 + (threadIdx.x >> 6)) * NR + lane / LPR;
    const int64_t nrows = p.T * p.Hkv;
    int64_t rowid = -1;
    if (idx < nrows) {
        const int64_t h = idx / p.T;
        rowid = (idx - h * p.T) * p.Hkv + h;
    }
    const int gl = lane & (LPR - 1);
    const int spos = rowid >= 0 && gl < p.topk ? p.slot_pos[rowid * p.topk + gl] : -1;
    merge_rows_grp<ET>(p, rowid, spos, LPR);
}

// ---------------------------------------------------------------------------
// Dense attention (bf16 / fp16).  One 8-wave workgroup per (kv head, token block).
// Two uses: the dense split of the selection branch (WINDOW false) and the
// sliding-window branch (WINDOW true: the key blocks covering
// i - window < p <= i for the block's tokens, written as the final out / lse;
// Flash-Sparse-Attention project page, "Quick start", window_size).
// The token block's rows (tokens x G heads) sit in MFMA registers, 16-row
// tiles per wave; the block's dense set -- the blocks every token of the
// token block keeps -- streams through LDS one key block at a time, double
// buffered: the next block's K and V rows go from HBM straight into the other
// LDS buffer (buffer loads to LDS, no registers) while this one is computed,
// with MFMA as in the main kernel and an online softmax across the blocks.
// The result is one more normalised
// partial per (token, kv head): dense_o (16-bit, written through an LDS tile
// as 16-byte linear stores) and dense_lse (natural log, -inf when the set is
// empty), which the merge starts from.
// ---------------------------------------------------------------------------
// Row tiles each wave of the dense / window kernel computes at once, and
// waves per workgroup: two tiles and 4 waves (every K / V^T fragment read
// from LDS feeds two MFMAs; 8 waves were slower for 64-key blocks, 0.73
// against 0.65 ms for the dense part of the 64K+32K GQA-4 workload).  Blocks
// of 128 keys go through LDS in 64-key granules (below), so two such
// workgroups fit a CU at d <= 128.
#ifndef NSA_DENSE128_WAVES
#define NSA_DENSE128_WAVES 4
#endif
#ifndef NSA_DENSE128_TILES
#define NSA_DENSE128_TILES 2
#endif
#ifndef NSA_DENSE_GRANULE
#define NSA_DENSE_GRANULE 64
#endif
__host__ __device__ constexpr int dense_tiles_per_wave(int bs, int d)
{
    return bs > 64 && d <= 128 ? NSA_DENSE128_TILES : bs <= 64 && d <= 128 ? 2 : 1;
}
__host__ __device__ constexpr int dense_waves(int bs, int d) { return bs > 64 && d <= 128 ? NSA_DENSE128_WAVES : 4; }
// Keys staged per LDS buffer: blocks of 128 keys go through in halves of 64
// (the online softmax runs over the halves as over blocks), so the two
// buffers take 64 KB at d = 128 and two workgroups fit a CU.
__host__ __device__ constexpr int dense_granule(int bs) { return bs > NSA_DENSE_GRANULE ? NSA_DENSE_GRANULE : bs; }


// Queue the loads of key block [kbeg, kbeg + BS) of sequence (c0, L), kv head
// h, into the LDS images dK, dV: one 16-byte buffer load to LDS per lane,
// wave w taking wave-loads w, w + NW, ..  Rows past the sequence end are
// outside the buffer range and read as zeros.
template <int D, int BS, int NW>
__device__ __forceinline__ void stage_block_lds(const Params& p, int h, int c0, int L, int kbeg, u16* dK, u16* dV)
{
    typedef __attribute__((address_space(3))) void lds_void;
    constexpr int NCH = D / 8;       // chunks per row
    constexpr int RPI = 64 / NCH;    // rows per wave-load
    constexpr int NI = BS / RPI;     // wave-loads per matrix
    const int nk = min(BS, L - kbeg);
    const int64_t e0 = ((int64_t)(c0 + kbeg) * p.Hkv + h) * D;
    const uint32_t bytes = nk > 0 ? (uint32_t)(((int64_t)(nk - 1) * p.Hkv + 1) * D * 2) : 0u;
    const auto rk = make_rsrc(reinterpret_cast<const u16*>(p.k) + e0, bytes);
    const auto rv = make_rsrc(reinterpret_cast<const u16*>(p.v) + e0, bytes);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rl = lane / NCH, pc = lane % NCH;
#pragma unroll
    for (int i = wave; i < NI; i += NW) {
        const int r = i * RPI + rl;
        const uint32_t rowb = (uint32_t)(r * p.Hkv * D * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dK + i * RPI * D), 16, rowb + (uint32_t)((pc ^ kswz<D>(r)) * 16), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dV + i * RPI * D), 16, rowb + (uint32_t)((pc ^ vswz<D>(r)) * 16), 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// 16-bit (bf16 / fp16) main kernel (persistent).  Workgroups of kMainWaves
// waves take items from per-XCD queues; the item's kv block is staged once
// per bucket into LDS (K and V images as the dense kernel lays them out:
// unpadded rows, 16-byte chunks XOR-permuted by row, loaded by buffer loads
// straight to LDS), and each wave runs chunks of NT 16-row tiles of gathered
// rows on its own:
//   - the chunk's query rows load straight into MFMA B-operand registers;
//   - S^T = K Q^T (A = K rows from LDS, one conflict-free 16-byte read each);
//   - masked softmax per row in registers, P normalised;
//   - O^T = V^T P^T, V^T operands by LDS transpose reads, P still in the
//     S^T accumulator layout;
//   - the 16-bit partial rows are transposed through a per-wave LDS tile and
//     leave as 1 KB runs of consecutive CSR rows, 16 bytes per lane.  (Stores
//     straight from the accumulator layout, after swapping 8-byte runs between
//     lane rows, write 64-byte pieces per row and instruction; measured at
//     4.2 ms against 3.2 ms for the main kernel on the 64K+32K GQA-4
//     workload.)
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int main_occupancy(int D, int NT) { return NT == 1 && D <= 128 ? kMainOcc : 2; }

template <typename E, int D, int BS, int NT>
__global__ __launch_bounds__(64 * kMainWaves)
__attribute__((amdgpu_waves_per_eu(main_occupancy(D, NT)))) void k_main_h(Params p)
{
    using H = H16<E>;
    typedef typename H::v8 v8;
    constexpr int CW = 16 * NT; // rows per wave chunk
    constexpr int KT = BS / 16; // key tiles of S^T
    constexpr int DS = D / 32;  // k-steps of S^T = K Q^T
    constexpr int KS = BS / 32; // k-steps of O^T = V^T P^T
    constexpr int DT = D / 16;  // d tiles of O^T
    constexpr int IMG = BS * D; // one K or V image (elements)
    static_assert(BS % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 sK[IMG];
    __shared__ __attribute__((aligned(16))) u16 sV[IMG];
    constexpr int OP = D + 8;   // padded LDS row of the per-wave output tile
    // rows of the output tile per pass: the whole chunk, or 4 where the K and
    // V images leave too little LDS (d 256 with 128-key blocks: 128 KB)
    constexpr int RP = 2 * IMG * 2 + kMainWaves * CW * OP * 2 > 160 * 1024 - 256 ? 4 : CW;
    __shared__ __attribute__((aligned(16))) u16 sO[kMainWaves][RP * OP];
    __shared__ int sItem[2];

    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int G = p.G, topk = p.topk;
    const int nitems = p.status[kStatusItems];
    const int xq = blockIdx.x % kNumXcd;
    const u16* qg = reinterpret_cast<const u16*>(p.q);
    u16* po = reinterpret_cast<u16*>(p.part_o);
    // K operand: row kt * 16 + n, chunk 4 ds + gq; V^T operand (transpose
    // reads): rows 32 ks + 4 gq + n / 4 and 16 below, columns 16 mt + 4 (n % 4)
    const int ksw = kswz<D>(n), vsw = vswz<D>(4 * gq + (n >> 2));
    const int vrow = (4 * gq + (n >> 2)) * D + (n & 1) * 4;

    int cur = -1;
    Bucket bk{};
    for (int iter = 0;; ++iter) {
        if (tid == 0) sItem[iter & 1] = queue_item(atomicAdd(&p.status[kStatusQueue + xq], 1), xq);
        __syncthreads();  // (also: every wave is done with the previous item's block)
        const int item = uni(sItem[iter & 1]);
        if (item >= nitems) break;
        const int bkt = uni(p.item_bucket[item]);
        if (bkt != cur) {
            bk = decode_bucket_uni(p, bkt);
            stage_block_lds<D, BS, kMainWaves>(p, bk.h, bk.c0, bk.kbeg + bk.nkeys, bk.kbeg, sK, sV);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            cur = bkt;
        }
        const int row0 = (item - uni(p.item_start[bkt])) * p.item_rows;
        const int row_end = min(row0 + p.item_rows, bk.cnt * G);

        // Software pipeline over the wave's chunks: the entry of chunk n + 2
        // and the query rows of chunk n + 1 are requested before chunk n's
        // partial output is stored.  Loads and stores share one in-order
        // completion counter, so a load issued after a store could only be
        // waited for together with that store; issued before it, the wait for
        // the next chunk's queries leaves the stores in flight.  Every memory
        // instruction of the loop is unconditional (buffer range checks
        // replace branches), so the compiler's wait counts stay exact.
        constexpr int STRIDE = kMainWaves * CW;
        const auto ents = make_rsrc(p.entries + bk.off, (uint32_t)bk.cnt * 4u);
        // rows of this lane in a chunk at c: c + 16 nt + n
        auto load_ent = [&](int c, int (&e)[NT]) {  // rows past the bucket read 0
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int ti = fast_div(c + 16 * nt + n, G, p.g_mul, p.g_shr);
                e[nt] = (int)__builtin_amdgcn_raw_buffer_load_b32(ents, (uint32_t)ti * 4u, 0, 0);
            }
        };
        // rows past the item's end read some valid token's queries (discarded)
        auto load_q = [&](int c, const int (&e)[NT], v8 (&dst)[NT][DS], int (&tok)[NT]) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int r = c + 16 * nt + n;
                tok[nt] = fast_div(e[nt], topk, p.topk_mul, p.topk_shr);
                const int qq = r - fast_div(r, G, p.g_mul, p.g_shr) * G;
                const u16* qr = qg + ((int64_t)tok[nt] * p.Hq + bk.h * G + qq) * D + gq * 8;
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) dst[nt][ds] = *reinterpret_cast<const v8*>(qr + ds * 32);
            }
        };
        int ent_cur[NT], ent_nx[NT], tok[NT];
        v8 bq[NT][DS];
        {
            const int c = row0 + wave * CW;
            load_ent(c, ent_cur);
            load_ent(c + STRIDE, ent_nx);
            load_q(c, ent_cur, bq, tok);
            // As many range-less (dropped) stores as a chunk issues after its
            // query loads: the wait for the queries before the first MFMA is
            // then the same on loop entry and on the back edge.
            const auto none = make_rsrc(po, 0u);
#pragma unroll
            for (int k = 0; k < NT + CW * D / 512; ++k)
                __builtin_amdgcn_raw_buffer_store_b32(0u, none, kBufOff + 64u * k, 0, 0);
        }

        for (int c = row0 + wave * CW; c < row_end; c += STRIDE) {
            // Re-read the K / V^T operands from LDS for every chunk rather than
            // letting them be hoisted into ~128 registers per lane: the empty asm
            // makes the offset opaque (the arrays stay in the LDS address space),
            // which keeps occupancy up.
            int lo = 0;
            asm volatile("" : "+v"(lo));
            int pos[NT];
            int pmin = INT_MAX;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bool row_ok = c + 16 * nt + n < row_end;
                pos[nt] = row_ok ? tok[nt] - bk.c0 : -1;
                pmin = min(pmin, row_ok ? pos[nt] : INT_MAX);
            }
            // Keys need a mask only where the block is a row's own block or is
            // cut by the sequence end; the test is uniform over the chunk and
            // takes its smallest token (the 4 lane groups hold the same rows),
            // so it holds for any order of a bucket's entries.
            const bool masked = bk.nkeys < BS || uni(row16_min(pmin)) < bk.kbeg + BS - 1;

            // S^T[key][row] = K Q^T
            f32x4 sacc[NT][KT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) sacc[nt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const v8 ak = *reinterpret_cast<const v8*>(&sK[lo + (kt * 16 + n) * D + ((4 * ds + gq) ^ ksw) * 8]);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) sacc[nt][kt] = H::mfma(ak, bq[nt][ds], sacc[nt][kt]);
                }

            // softmax over the block's keys (one row per lane column)
            float lse_v[NT];
            v8 bp[NT][KS];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float mx = -INFINITY;
                if (masked) {
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int key = kt * 16 + gq * 4 + i;
                            const bool vis = key < bk.nkeys && bk.kbeg + key <= pos[nt];
                            const float x = vis ? sacc[nt][kt][i] * p.scale_log2 : -INFINITY;
                            sacc[nt][kt][i] = x;
                            mx = fmaxf(mx, x);
                        }
                } else {
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = sacc[nt][kt][i] * p.scale_log2;
                            sacc[nt][kt][i] = x;
                            mx = fmaxf(mx, x);
                        }
                }
                mx = xmax32(xmax16(mx));
                const float mref = mx == -INFINITY ? 0.f : mx;
                float sum = 0.f;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // raw v_exp_f32 (results below 2^-126 flush to 0)
                        const float e = __builtin_amdgcn_exp2f(sacc[nt][kt][i] - mref);
                        sacc[nt][kt][i] = e;
                        sum += e;
                    }
                sum = xsum32(xsum16(sum));
                // P is normalised before PV (a row with no visible key: 0)
                const float inv = sum > 0.f ? __builtin_amdgcn_rcpf(sum) : 0.f;
                lse_v[nt] = (mref + __log2f(sum)) * kLn2;
                // P as the B operand of O^T = V^T P^T: k-slot 8 gq + i holds
                // key 32 ks + 4 gq + i (i < 4) or 32 ks + 16 + 4 gq + i - 4
                // (i >= 4), the order the V^T transpose reads deliver
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    bp[nt][ks] = cvt8<E>(sacc[nt][2 * ks] * inv, sacc[nt][2 * ks + 1] * inv);
            }

            // next chunks' loads (bq is free once S^T is done)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) ent_cur[nt] = ent_nx[nt];
            load_ent(c + 2 * STRIDE, ent_nx);
            load_q(c + STRIDE, ent_cur, bq, tok);

            // O^T[d][row] = V^T P^T
            f32x4 oacc[NT][DT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < DT; ++mt) oacc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mt = 0; mt < DT; ++mt) {
                    const int vo = lo + 32 * ks * D + vrow + ((2 * mt + ((n & 3) >> 1)) ^ vsw) * 8;
                    const v8 av = lds_tr_pair<v8>(&sV[vo], &sV[vo + 16 * D]);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) oacc[nt][mt] = H::mfma(av, bp[nt][ks], oacc[nt][mt]);
                }

            // Partial output (16-bit, normalised) and its lse (fp32, natural
            // log) at the chunk's CSR rows, which are consecutive; rows past
            // nrows fall outside the ranges and are dropped.  The partials are
            // read once, by the merge: they stream past the caches.
            const int nrows = min(CW, row_end - c);
            const auto lse_r = make_rsrc(p.part_lse + (int64_t)bk.off * G + c, (uint32_t)nrows * 4u);
            const auto out_r = make_rsrc(po + ((int64_t)bk.off * G + c) * D, (uint32_t)(nrows * D * 2));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse_v[nt]), lse_r,
                                                      gq == 0 ? (uint32_t)(16 * nt + n) * 4u : kBufOff, 0, 0);
            u16* tile = sO[wave];
#pragma unroll
            for (int r0 = 0; r0 < CW; r0 += RP) {  // rows [r0, r0 + RP) of the chunk
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int rr = 16 * nt + n - r0;
                    if (RP == CW || (rr >= 0 && rr < RP)) {
#pragma unroll
                        for (int mt = 0; mt < DT; ++mt)
                            *reinterpret_cast<uint2*>(&tile[rr * OP + mt * 16 + gq * 4]) = cvt4<E>(oacc[nt][mt]);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
                for (int k = 0; k < RP * CPR / 64; ++k) {
                    const int ch = k * 64 + lane;  // chunk of the tile
                    const int r = ch / CPR, cc = ch - r * CPR;
                    const u32x4 v4 = *reinterpret_cast<const u32x4*>(&tile[r * OP + cc * 8]);
                    __builtin_amdgcn_raw_buffer_store_b128(v4, out_r, (uint32_t)((r0 + r) * D + cc * 8) * 2u, 0,
                                                           kBufNT);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
    }
}

#ifndef NSA_DENSE128_OCC
#define NSA_DENSE128_OCC 2
#endif
// GRP: the fused merge takes rows narrower than a wave 64 / LPR at a time
// (merge_group_lanes); MNC: 16-byte chunks per lane the fused merge takes in
// one walk over a row's slots (2 for rows of 2 KB, G * D = 1024).  Separate
// instances, so the others keep their code.
template <typename E, int D, int BS, bool WINDOW, bool GRP = false, int MNC = 1>
__global__ __launch_bounds__(64 * dense_waves(BS, D))
__attribute__((amdgpu_waves_per_eu(BS > 64 && D <= 128 ? NSA_DENSE128_OCC : 2))) void k_dense_attn(Params p)
{
    using H = H16<E>;
    typedef typename H::v8 v8;
    constexpr int BL = dense_granule(BS);  // keys per staged granule
    constexpr int SUB = BS / BL;           // granules per block
    constexpr int KT = BL / 16, DS = D / 32, KS = BL / 32, DT = D / 16;
    constexpr int NW = dense_waves(BS, D);
    constexpr int NTHR = 64 * NW;
    constexpr int OP = D + 8;  // padded LDS row of a wave's output tile
    constexpr int IMG = BL * D;  // one K or V image
    constexpr int DNT = dense_tiles_per_wave(BS, D);
    static_assert(DNT <= 2, "output tiles");
    // buffer 0 also holds the waves' first output tiles, buffer 1 the second
    constexpr int SB0 = 2 * IMG > NW * 16 * OP ? 2 * IMG : NW * 16 * OP;
    constexpr int SB1 = DNT > 1 && NW * 16 * OP > 2 * IMG ? NW * 16 * OP : 2 * IMG;
    // two buffers, each a K image and then a V image; separate arrays, so the
    // compiler sees that loads into one never alias reads of the other
    __shared__ __attribute__((aligned(16))) u16 sb0[SB0];
    __shared__ __attribute__((aligned(16))) u16 sb1[SB1];
    __shared__ float sLt[WINDOW ? 1 : NW * DNT * 16];  // lse of the output tile rows (merge inside)
    u16 (*sO)[16 * OP] = reinterpret_cast<u16 (*)[16 * OP]>(sb0);  // after the last block
    u16 (*sO1)[16 * OP] = reinterpret_cast<u16 (*)[16 * OP]>(sb1);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    // Scores stay unscaled in the accumulators; the scale (sl, log2 units)
    // enters through the FMA that forms each exponent.  A negative scale's
    // sign goes into the query registers (exact), so sl > 0: the max of the
    // raw scores scales to the max of the scaled ones and a masked -inf stays
    // -inf; a zero scale becomes FLT_MIN (every exponent rounds alike, as the
    // exact uniform softmax has it).
    const bool qflip = p.scale_log2 < 0.f;
    const float sl = fmaxf(fabsf(p.scale_log2), FLT_MIN);
    const int G = p.G, Hkv = p.Hkv;
    // XCD-aware order: workgroup i runs on XCD i % 8; give each XCD a
    // contiguous run of (kv head, token block) so neighbouring token blocks,
    // which share dense blocks, meet in the same L2
    // a token block's rows are split into dense_parts row ranges of
    // NW * DNT tiles; the parts of one token block are adjacent in wid
    const int parts = p.dense_parts;
    const int total = p.Hkv * p.nbc * parts;
    const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
    const int wid = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
    if (wid >= total) return;
    const int part = wid % parts;
    const int h = (wid / parts) / p.nbc;
    const int g = wid / parts - h * p.nbc;
    if (g >= p.blkoff[p.B]) return;
    int slo = 0, shi = p.B - 1;  // last sequence with blkoff <= g
    while (slo < shi) {
        int mid = (slo + shi + 1) >> 1;
        if (p.blkoff[mid] <= g) slo = mid; else shi = mid - 1;
    }
    const int b = g - p.blkoff[slo];
    const int c0 = p.cus[slo], L = p.cus[slo + 1] - c0;
    const int i0 = b * BS;
    const int nrows = (min((b + 1) * BS, L) - i0) * G;
    const size_t dk = (size_t)h * p.nbc + g;
    // window: the blocks holding keys max(0, i0 - window + 1) .. last token
    const int jlo = WINDOW ? max(0, i0 - p.window + 1) / BS : 0;
    const int dcnt = WINDOW ? (i0 + nrows / G - 1) / BS - jlo + 1 : p.dense_cnt[dk];
    auto block_of = [&](int di) { return WINDOW ? jlo + di : p.dense_ids[dk * p.topk + di]; };
    // first key of granule gi (granules of a block are consecutive)
    auto gran_beg = [&](int gi) { return block_of(gi / SUB) * BS + (gi % SUB) * BL; };
    const int ngr = dcnt * SUB;
    // output row of tile row r (token i0 + r / G, head r % G); tokens of one kv
    // head are Hkv * G rows apart.  Dense split: the dense partial; window:
    // the branch's final out / lse.
    u16* o_dst = reinterpret_cast<u16*>(WINDOW ? p.out : p.dense_o);
    float* lse_dst = WINDOW ? p.lse : p.dense_lse;
    auto orow = [&](int r) { return ((int64_t)(c0 + i0 + r / G) * Hkv + h) * G + r % G; };
    const int nrt = (nrows + 15) / 16;  // 16-row tiles
    // dense split with the merge inside: each wave merges the tokens of its
    // own row tiles (G divides 16, so a token's heads share a tile)
    const bool fuse = !WINDOW && p.fuse_merge;
    if (dcnt == 0) {  // uniform: nothing every token keeps
        if (fuse) {
            for (int rt0 = part * NW * DNT; rt0 < nrt; rt0 += parts * NW * DNT)
                for (int j = 0; j < DNT; ++j) {
                    const int rt = rt0 + wave + NW * j;
                    if (rt >= nrt) break;
                    for (int r = rt * 16; r < min(rt * 16 + 16, nrows); r += G)
                        merge_row<E, true, MNC>(p, (int64_t)(c0 + i0 + r / G) * Hkv + h);
                }
        } else if (part == 0) {
            for (int r = tid; r < nrows; r += NTHR) lse_dst[orow(r)] = -INFINITY;
        }
        return;
    }
    // Each wave computes DNT row tiles at once (tiles wave, wave + NW, ...),
    // so every K / V^T fragment read from LDS feeds DNT MFMAs.
    auto load_q = [&](int rt, v8 (&dst)[DS]) {
        const int r = rt * 16 + n;
        const int ti = r < nrows ? r / G : 0, qq = r - (r / G) * G;
        const u16* qr = reinterpret_cast<const u16*>(p.q) + ((int64_t)(c0 + i0 + ti) * p.Hq + h * G + qq) * D + gq * 8;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) dst[ds] = *reinterpret_cast<const v8*>(qr + ds * 32);
    };
    for (int rt0 = part * NW * DNT; rt0 < nrt; rt0 += parts * NW * DNT) {
        v8 bq[DNT][DS];
        int pos[DNT];
        bool act[DNT];
#pragma unroll
        for (int j = 0; j < DNT; ++j) {
            const int rt = rt0 + wave + NW * j;
            act[j] = rt < nrt;
            const int r = rt * 16 + n;
            pos[j] = act[j] && r < nrows ? i0 + r / G : -1;
            load_q(act[j] ? rt : 0, bq[j]);  // in flight during the staging below
        }
        float m[DNT], l[DNT];
        f32x4 oacc[DNT][DT];
#pragma unroll
        for (int j = 0; j < DNT; ++j) {
            m[j] = -INFINITY;
            l[j] = 0.f;
#pragma unroll
            for (int mt = 0; mt < DT; ++mt) oacc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // K operand: row kt * 16 + n, chunk 4 ds + gq; V^T operand (transpose
        // reads): rows 32 ks + 4 gq + n / 4 and 16 below, columns 16 mt + 4 (n % 4)
        const int ksw = kswz<D>(n), vsw = vswz<D>(4 * gq + (n >> 2));
        const int vrow = (4 * gq + (n >> 2)) * D + (n & 1) * 4;
        if (rt0 != part * NW * DNT) __syncthreads();  // the previous pass's output tiles are out
        int kb_cur = gran_beg(0);
        stage_block_lds<D, BL, NW>(p, h, c0, L, kb_cur, sb0, sb0 + IMG);
        // block di: computed from buffer di % 2 while block di + 1 loads into
        // the other one
        auto step = [&](int di, const u16* cur, u16* nxt) {
            // (the next id is read before the wait: no load issued after the
            // staging may be waited for inside the block's math)
            const int kb_nx = di + 1 < ngr ? gran_beg(di + 1) : 0;
            // this wave's loads of block di are in LDS (and its query rows in
            // registers); after the barrier every wave's are, and every wave
            // is done with block di - 1, whose buffer takes block di + 1
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (di + 1 < ngr) stage_block_lds<D, BL, NW>(p, h, c0, L, kb_nx, nxt, nxt + IMG);
            if (qflip && di == 0) {  // (the query rows have arrived)
#pragma unroll
                for (int j = 0; j < DNT; ++j)
#pragma unroll
                    for (int ds = 0; ds < DS; ++ds) {
                        const uint4 u = __builtin_bit_cast(uint4, bq[j][ds]);
                        bq[j][ds] = __builtin_bit_cast(v8, make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u,
                                                                     u.z ^ 0x80008000u, u.w ^ 0x80008000u));
                    }
            }
            const int kbeg = kb_cur;
            kb_cur = kb_nx;
            if (!act[0]) return;
            {
                const int nkeys = min(BL, L - kbeg);
                // opaque LDS offset: keep the fragment loads next to their MFMAs.
                // Every read below indexes cur with one integer offset: the
                // compiler's proof that these reads do not touch the buffer
                // being loaded follows only a few pointer steps from the array.
                int lo = 0;
                asm volatile("" : "+v"(lo));
                f32x4 sacc[DNT][KT];
#pragma unroll
                for (int j = 0; j < DNT; ++j)
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) sacc[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) {
                        const v8 ak = *reinterpret_cast<const v8*>(&cur[lo + (kt * 16 + n) * D + ((4 * ds + gq) ^ ksw) * 8]);
#pragma unroll
                        for (int j = 0; j < DNT; ++j) sacc[j][kt] = H::mfma(ak, bq[j][ds], sacc[j][kt]);
                    }
                v8 bp[DNT][KS];
#pragma unroll
                for (int j = 0; j < DNT; ++j) {
                    // Keys need a mask only on the block's causal diagonal, at the
                    // window's lower edge and past the sequence end; the test is
                    // uniform over the wave's tile (rows 16 rt .. 16 rt + 15).
                    const int rt = rt0 + wave + NW * j;
                    const int pmin = i0 + (rt * 16) / G;
                    const int pmax = i0 + min(rt * 16 + 15, nrows - 1) / G;
                    const bool masked = nkeys < BL || kbeg + BL - 1 > pmin || rt * 16 + 15 >= nrows ||
                                        (WINDOW && kbeg <= pmax - p.window);
                    auto mask = [&]() {
                        if (!masked) return;
#pragma unroll
                        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int key = kt * 16 + gq * 4 + i;
                                const bool vis = key < nkeys && kbeg + key <= pos[j] &&
                                                 (!WINDOW || kbeg + key > pos[j] - p.window);
                                sacc[j][kt][i] = vis ? sacc[j][kt][i] : -INFINITY;
                            }
                    };
                    mask();
                    // The lane's max over its scores; the row's reference moves
                    // (to the row's max, when that passes it by more than 8, log2
                    // units) only when some lane's max passes it by more than 64
                    // or the reference is still -inf: then the exact path with
                    // the max over the row's 4 lane groups and the rescale.
                    // Otherwise the exponentials are taken against the reference
                    // as it stands: exponents up to 64 are exact enough in fp32
                    // and in the 16-bit P.
                    float mx = -INFINITY;
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[j][kt][i]);
                    mx *= sl;  // (sl > 0)
                    float mref = m[j];
                    if (__ballot(m[j] == -INFINITY || mx > m[j] + 64.f)) {
                        // over the row's 4 lane groups
                        mx = xmax32(xmax16(mx));
                        const bool move = m[j] == -INFINITY || mx > m[j] + 8.f;
                        const float mnew = move ? fmaxf(m[j], mx) : m[j];
                        mref = mnew == -INFINITY ? 0.f : mnew;
                        // raw v_exp_f32 (results below 2^-126 flush to 0)
                        const float corr = __builtin_amdgcn_exp2f(m[j] - mref);  // 0 while nothing was visible
                        l[j] *= corr;
                        m[j] = mnew;
                        if (__ballot(corr != 1.f)) {  // the reference moved for some row
#pragma unroll
                            for (int mt = 0; mt < DT; ++mt) oacc[j][mt] *= corr;
                        }
                    }
                    float sum = 0.f;
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float e = __builtin_amdgcn_exp2f(fmaf(sacc[j][kt][i], sl, -mref));
                            sacc[j][kt][i] = e;
                            sum += e;
                        }
                    l[j] += xsum32(xsum16(sum));
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            bp[j][ks][i] = static_cast<E>(sacc[j][2 * ks][i]);
                            bp[j][ks][4 + i] = static_cast<E>(sacc[j][2 * ks + 1][i]);
                        }
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int mt = 0; mt < DT; ++mt) {
                        const int vo = lo + IMG + 32 * ks * D + vrow + ((2 * mt + ((n & 3) >> 1)) ^ vsw) * 8;
                        const v8 av = lds_tr_pair<v8>(&cur[vo], &cur[vo + 16 * D]);
#pragma unroll
                        for (int j = 0; j < DNT; ++j) oacc[j][mt] = H::mfma(av, bp[j][ks], oacc[j][mt]);
                    }
            }
        };
        for (int di = 0; di < ngr; di += 2) {
            step(di, sb0, sb1);
            if (di + 1 < ngr) step(di + 1, sb1, sb0);
        }
        __syncthreads();  // the output tiles overwrite the K / V blocks
#pragma unroll
        for (int j = 0; j < DNT; ++j) {
            if (!act[j]) continue;
            const int rt = rt0 + wave + NW * j;
            const int r = rt * 16 + n;
            // normalised tile -> LDS -> 16 bytes per lane, each row's 256 B
            // contiguous (or, with the merge inside, kept for it)
            const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
            u16* tile = j == 0 ? sO[wave] : sO1[wave];
#pragma unroll
            for (int mt = 0; mt < DT; ++mt)
                *reinterpret_cast<uint2*>(&tile[n * OP + mt * 16 + gq * 4]) =
                    make_uint2(pack2h<E>(oacc[j][mt][0] * inv, oacc[j][mt][1] * inv),
                               pack2h<E>(oacc[j][mt][2] * inv, oacc[j][mt][3] * inv));
            const float lv = l[j] > 0.f ? (m[j] + __log2f(l[j])) * kLn2 : -INFINITY;
            if (fuse) {
                if (!WINDOW && gq == 0) sLt[(wave * DNT + j) * 16 + n] = lv;
                continue;
            }
            if (r < nrows && gq == 0) lse_dst[orow(r)] = lv;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
            for (int k = 0; k < 16 * CPR / 64; ++k) {
                const int c = k * 64 + lane;
                const int tr = c / CPR, cc = c - tr * CPR;  // tile row, chunk
                const uint4 v4 = *reinterpret_cast<const uint4*>(&tile[tr * OP + cc * 8]);
                const int rr = rt * 16 + tr;
                if (rr < nrows) *reinterpret_cast<uint4*>(o_dst + orow(rr) * D + cc * 8) = v4;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        if (fuse) {  // merge the tiles' tokens, dense part from LDS
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int S = merge_stride(p.topk), rpb = 64 / S;
            for (int j = 0; j < DNT; ++j) {
                if (!act[j]) continue;
                const int rt = rt0 + wave + NW * j;
                const u16* tile = j == 0 ? sO[wave] : sO1[wave];
                const int ntok = min(16, nrows - rt * 16 + G - 1) / G;  // the tile's tokens
                auto rowid_of = [&](int k) { return (int64_t)(c0 + i0 + (rt * 16 + k * G) / G) * Hkv + h; };
                if constexpr (GRP) {  // 64 / LPR tokens at once, one lane group each
                    const int LPR = merge_group_lanes(G, D, p.topk, true);
                    const int gi = lane / LPR, gl = lane & (LPR - 1);
                    for (int k0 = 0; k0 < ntok; k0 += 64 / LPR) {
                        const int k = k0 + gi;
                        const int64_t rowid = k < ntok ? rowid_of(k) : -1;
                        const int spos = rowid >= 0 && gl < p.topk ? p.slot_pos[rowid * p.topk + gl] : -1;
                        merge_rows_grp<E, true>(p, rowid, spos, LPR, tile + (k < ntok ? k : 0) * G * OP, OP,
                                                &sLt[(wave * DNT + j) * 16 + (k < ntok ? k : 0) * G]);
                    }
                    continue;
                }
                for (int k0 = 0; k0 < ntok; k0 += rpb) {  // slot positions of rpb tokens at once
                    const int kk = k0 + lane / S, sl = lane % S;
                    const int sreg = kk < ntok && sl < p.topk ? p.slot_pos[rowid_of(kk) * p.topk + sl] : -1;
                    for (int k = k0; k < k0 + rpb && k < ntok; ++k)
                        merge_row<E, true, MNC>(p, rowid_of(k), tile + k * G * OP, OP,
                                           &sLt[(wave * DNT + j) * 16 + k * G], sreg, (k - k0) * S);
                }
            }
            __syncthreads();  // the next row range's blocks overwrite the tiles
        }
    }
}

template <typename E, int D>
void launch_main_h(const Params& p, hipStream_t st)
{
    const unsigned grid = (unsigned)p.main_grid;
    switch (p.bs) {
    case 32: hipLaunchKernelGGL((k_main_h<E, D, 32, kMainNT>), dim3(grid), dim3(64 * kMainWaves), 0, st, p); break;
    case 64: hipLaunchKernelGGL((k_main_h<E, D, 64, kMainNT>), dim3(grid), dim3(64 * kMainWaves), 0, st, p); break;
    default: hipLaunchKernelGGL((k_main_h<E, D, 128, kMainNT>), dim3(grid), dim3(64 * kMainWaves), 0, st, p); break;
    }
}

// d = 256: 16-bit only (the host checks reject fp32)
template <typename E>
void launch_main_h256(const Params& p, hipStream_t st)
{
    const unsigned grid = (unsigned)p.main_grid;
    switch (p.bs) {
    case 32: hipLaunchKernelGGL((k_main_h<E, 256, 32, kMainNT>), dim3(grid), dim3(64 * kMainWaves), 0, st, p); break;
    case 64: hipLaunchKernelGGL((k_main_h<E, 256, 64, kMainNT>), dim3(grid), dim3(64 * kMainWaves), 0, st, p); break;
    default: hipLaunchKernelGGL((k_main_h<E, 256, 128, kMainNT>), dim3(grid), dim3(64 * kMainWaves), 0, st, p); break;
    }
}

template <int D>
void launch_main_d(const Params& p, hipStream_t st, int kind)
{
    if (kind == kElemBF16) {
        launch_main_h<__bf16, D>(p, st);
    } else if (kind == kElemF16) {
        launch_main_h<_Float16, D>(p, st);
    } else {
        const unsigned grid = (unsigned)(p.max_items * (p.item_rows / 256));
        switch (p.bs) {
        case 32: hipLaunchKernelGGL((k_main_f32<D, 32>), dim3(grid), dim3(256), 0, st, p); break;
        case 64: hipLaunchKernelGGL((k_main_f32<D, 64>), dim3(grid), dim3(256), 0, st, p); break;
        default: hipLaunchKernelGGL((k_main_f32<D, 128>), dim3(grid), dim3(256), 0, st, p); break;
        }
    }
}

template <typename E>
const void* main_h_ptr(int D, int bs)
{
    if (D == 256) return bs == 32 ? (const void*)k_main_h<E, 256, 32, kMainNT>
                       : bs == 64 ? (const void*)k_main_h<E, 256, 64, kMainNT>
                                  : (const void*)k_main_h<E, 256, 128, kMainNT>;
    if (D == 64) return bs == 32 ? (const void*)k_main_h<E, 64, 32, kMainNT>
                      : bs == 64 ? (const void*)k_main_h<E, 64, 64, kMainNT>
                                 : (const void*)k_main_h<E, 64, 128, kMainNT>;
    return bs == 32 ? (const void*)k_main_h<E, 128, 32, kMainNT>
         : bs == 64 ? (const void*)k_main_h<E, 128, 64, kMainNT>
                    : (const void*)k_main_h<E, 128, 128, kMainNT>;
}

}  // namespace

// Workgroups the persistent 16-bit main kernel launches: enough to fill
// every CU at the kernel's occupancy, a multiple of the XCD count.
int main_grid_size(int D, int bs, int kind)
{
    // per device and configuration; any thread may fill an entry (every
    // thread computes the same value)
    constexpr int kDevs = 16;
    static std::atomic<int> cached[kDevs][2][3][3];
    const int ki = kind == kElemF16 ? 1 : 0;
    const int di = D == 64 ? 0 : D == 128 ? 1 : 2, bi = bs == 32 ? 0 : bs == 64 ? 1 : 2;
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::atomic<int>* slot = dev >= 0 && dev < kDevs ? &cached[dev][ki][di][bi] : nullptr;
    if (slot) {
        const int g = slot->load(std::memory_order_relaxed);
        if (g) return g;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
    const void* fn = ki ? main_h_ptr<_Float16>(D, bs) : main_h_ptr<__bf16>(D, bs);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, 64 * kMainWaves, 0) != hipSuccess || per < 1) per = 1;
    int g = cus * per;
    g = (g + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (slot) slot->store(g, std::memory_order_relaxed);
    return g;
}

hipError_t launch_main(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0 || p.max_items == 0) return hipSuccess;
    if (p.D == 64) launch_main_d<64>(p, st, kind);
    else if (p.D == 128) launch_main_d<128>(p, st, kind);
    else if (kind == kElemF16) launch_main_h256<_Float16>(p, st);
    else launch_main_h256<__bf16>(p, st);
    return hipGetLastError();
}

template <typename E, int D, int BS, bool WINDOW>
void launch_dense_bs(const Params& p, hipStream_t st, unsigned grid)
{
    if constexpr (!WINDOW) {
        if (p.fuse_merge && merge_group_lanes(p.G, D, p.topk, true)) {
            hipLaunchKernelGGL((k_dense_attn<E, D, BS, false, true>), dim3(grid), dim3(64 * dense_waves(BS, D)), 0, st,
                               p);
            return;
        }
        if (p.fuse_merge && p.G * D == 1024) {  // rows of 2 KB: both halves in one walk
            hipLaunchKernelGGL((k_dense_attn<E, D, BS, false, false, 2>), dim3(grid), dim3(64 * dense_waves(BS, D)),
                               0, st, p);
            return;
        }
    }
    hipLaunchKernelGGL((k_dense_attn<E, D, BS, WINDOW>), dim3(grid), dim3(64 * dense_waves(BS, D)), 0, st, p);
}

template <typename E, int D, bool WINDOW>
void launch_dense_d(const Params& p, hipStream_t st, unsigned grid)
{
    switch (p.bs) {
    case 32: launch_dense_bs<E, D, 32, WINDOW>(p, st, grid); break;
    case 64: launch_dense_bs<E, D, 64, WINDOW>(p, st, grid); break;
    default: launch_dense_bs<E, D, 128, WINDOW>(p, st, grid); break;
    }
}

template <bool WINDOW>
void launch_dense_k(Params p, int kind, hipStream_t st)
{
    // row parts per token block: tiles of 16 rows, NW waves x DNT tiles each
    const int tiles = (int)div_up((int64_t)p.bs * p.G, 16);
    const int per_wg = dense_waves(p.bs, p.D) * dense_tiles_per_wave(p.bs, p.D);
    p.dense_parts = (int)div_up(tiles, per_wg);
    const unsigned grid = (unsigned)(div_up((int64_t)p.Hkv * p.nbc * p.dense_parts, kNumXcd) * kNumXcd);
    if (kind == kElemF16) {
        if (p.D == 64) launch_dense_d<_Float16, 64, WINDOW>(p, st, grid);
        else if (p.D == 128) launch_dense_d<_Float16, 128, WINDOW>(p, st, grid);
        else launch_dense_d<_Float16, 256, WINDOW>(p, st, grid);
    } else {
        if (p.D == 64) launch_dense_d<__bf16, 64, WINDOW>(p, st, grid);
        else if (p.D == 128) launch_dense_d<__bf16, 128, WINDOW>(p, st, grid);
        else launch_dense_d<__bf16, 256, WINDOW>(p, st, grid);
    }
}

// Tokens outside every sequence: out = 0, lse = -inf (window branch, and the
// forward whose dense kernel merges the tokens of every sequence).
template <typename E>
__global__ __launch_bounds__(256) void k_orphans(Params p)
{
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // t * Hq + qh
    if (row >= p.T * p.Hq) return;
    if (seq_of_token(p.cus, p.B, row / p.Hq) >= 0) return;
    p.lse[row] = -INFINITY;
    uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.out) + row * p.D);
    for (int c = 0; c < p.D / 8; ++c) o[c] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_dense(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0 || !p.dense_cnt) return hipSuccess;
    launch_dense_k<false>(p, kind, st);
    return hipGetLastError();
}

hipError_t launch_window(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    launch_dense_k<true>(p, kind, st);
    return hipGetLastError();
}

hipError_t launch_window_orphans(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const unsigned grid = (unsigned)div_up(p.T * p.Hq, 256);
    if (kind == kElemF16) hipLaunchKernelGGL(k_orphans<_Float16>, dim3(grid), dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_orphans<__bf16>, dim3(grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <typename ET>
void launch_merge_t(const Params& p, hipStream_t st)
{
    const int lpr = merge_group_lanes(p.G, p.D, p.topk, sizeof(ET) == 2);
    // waves: one per row, or one per 64 / lpr rows
    const int64_t rows = lpr ? div_up(p.T * p.Hkv, 64 / lpr) : p.T * p.Hkv;
    const unsigned mgrid = (unsigned)merge_grid(rows, 1);
    if (sizeof(ET) == 2 && p.G * p.D == 1024)  // rows of 2 KB: both halves in one walk over the slots
        hipLaunchKernelGGL((k_merge<ET, 2>), dim3(mgrid), dim3(256), 0, st, p, lpr);
    else hipLaunchKernelGGL((k_merge<ET, 1>), dim3(mgrid), dim3(256), 0, st, p, lpr);
}

hipError_t launch_merge(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    if (p.fuse_merge) {  // the dense kernel merged every token of a sequence
        const unsigned grid = (unsigned)div_up(p.T * p.Hq, 256);
        if (kind == kElemF16) hipLaunchKernelGGL(k_orphans<_Float16>, dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL(k_orphans<__bf16>, dim3(grid), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    if (kind == kElemBF16) launch_merge_t<__bf16>(p, st);
    else if (kind == kElemF16) launch_merge_t<_Float16>(p, st);
    else launch_merge_t<float>(p, st);
    return hipGetLastError();
}

}  // namespace nsa
