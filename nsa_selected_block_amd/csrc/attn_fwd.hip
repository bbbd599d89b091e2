// attn_fwd.hip -- main selected-attention kernel and partial-result merge.
//
// Main kernel (Flash-Sparse-Attention project page, "Key features",
// optimised-kernels row: the main batched query-to-KV kernel).  One work item
// is (kv head h, kv block j, chunk of the block's token list).  The K and V
// block is staged once in LDS, the queries of the chunk's tokens are
// gathered for every query head of the GQA group (rows = tokens x G), and
// S^T = K Q^T and O^T = V^T P^T run on bf16 MFMA (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation.  The score tile comes out of the first MFMA in
// exactly the lane layout the second MFMA takes as its B operand (after a
// permutation of the key index that A = V^T is loaded with as well), so P
// never leaves registers.  Each (token, head, slot) gets a normalised partial
// output and its log-sum-exp; no atomics.
//
// Merge kernel (same row: the reduction and online-softmax kernels).  One
// wave per (token, kv head) combines that row's partials in ascending block
// order: M = max lse_s, w_s = exp(lse_s - M), out = sum w_s o_s / sum w_s,
// lse = M + ln sum w_s, with coalesced 16-byte loads and stores.
#include "internal.h"

namespace nsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float bf16_to_f32(u16 x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ u16 f32_to_bf16(float x)
{
    __bf16 b = static_cast<__bf16>(x);  // round to nearest even
    return __builtin_bit_cast(u16, b);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Decoded work item of the main kernel.
struct Item {
    int h, j, c0, kbeg, nkeys, e0, ne;
};

// Returns false when this workgroup has no item (grid is an upper bound).
__device__ __forceinline__ bool decode_item(const Params& p, int item, Item& it)
{
    const int nitems = p.status[kStatusItems];
    if (item >= nitems) return false;
    const int nbk = p.Hkv * p.nbc;
    int lo = 0, hi = nbk - 1;  // last bucket with item_start <= item (never empty)
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (p.item_start[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int bkt = lo;
    it.h = bkt / p.nbc;
    const int g = bkt - it.h * p.nbc;
    int slo = 0, shi = p.B - 1;  // last sequence with blkoff <= g
    while (slo < shi) {
        int mid = (slo + shi + 1) >> 1;
        if (p.blkoff[mid] <= g) slo = mid; else shi = mid - 1;
    }
    it.j = g - p.blkoff[slo];
    it.c0 = p.cus[slo];
    const int L = p.cus[slo + 1] - it.c0;
    it.kbeg = it.j * p.bs;
    it.nkeys = min(p.bs, L - it.kbeg);
    const int chunk = item - p.item_start[bkt];
    it.e0 = p.offsets[bkt] + chunk * p.item_tokens;
    it.ne = min(p.item_tokens, p.offsets[bkt + 1] - it.e0);
    return true;
}

// ---------------------------------------------------------------------------
// bf16 main kernel: 4 waves, 128 gathered rows, each wave 32 rows (2 tiles).
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void k_main_bf16(Params p)
{
    constexpr int ROWS = kRowsBf16;
    constexpr int KP = D + 8;   // padded LDS row (elements) of K and Q
    constexpr int VP = BS + 8;  // padded LDS row of V^T
    constexpr int KT = BS / 16; // key tiles of S^T
    constexpr int DS = D / 32;  // k-steps of S^T = K Q^T
    constexpr int KS = BS / 32; // k-steps of O^T = V^T P^T
    constexpr int DT = D / 16;  // d tiles of O^T
    static_assert(BS % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 sK[BS * KP];
    __shared__ __attribute__((aligned(16))) u16 sVt[D * VP];
    __shared__ __attribute__((aligned(16))) u16 sQ[ROWS * KP];
    __shared__ int sPos[ROWS];      // local position of the row's token, -1 = padding
    __shared__ int sTok[ROWS];      // token id
    __shared__ int64_t sPart[ROWS]; // partial row: ((t*Hkv + h)*topk + slot)*G + head

    Item it;
    if (!decode_item(p, blockIdx.x, it)) return;
    const int tid = threadIdx.x;
    const int G = p.G;
    const int Hkv = p.Hkv;

    // row metadata
    for (int r = tid; r < ROWS; r += 256) {
        const int ti = r / G, qq = r - ti * G;
        int pos = -1, t = 0;
        int64_t prow = 0;
        if (ti < it.ne) {
            const int ent = p.entries[it.e0 + ti];
            t = ent / p.topk;
            const int slot = ent - t * p.topk;
            pos = t - it.c0;
            prow = ((int64_t)((int64_t)t * Hkv + it.h) * p.topk + slot) * G + qq;
        }
        sPos[r] = pos;
        sTok[r] = t;
        sPart[r] = prow;
    }

    // K block, row-major
    const u16* kg = reinterpret_cast<const u16*>(p.k);
    const u16* vg = reinterpret_cast<const u16*>(p.v);
    for (int x = tid; x < BS * (D / 8); x += 256) {
        const int key = x / (D / 8), c8 = x - key * (D / 8);
        uint4 val = make_uint4(0, 0, 0, 0);
        if (key < it.nkeys)
            val = *reinterpret_cast<const uint4*>(
                kg + ((int64_t)(it.c0 + it.kbeg + key) * Hkv + it.h) * D + c8 * 8);
        *reinterpret_cast<uint4*>(&sK[key * KP + c8 * 8]) = val;
    }
    // V block, transposed to [d][key] through an 8x8 register transpose
    for (int x = tid; x < (BS / 8) * (D / 8); x += 256) {
        const int k8 = x / (D / 8), c8 = x - k8 * (D / 8);
        uint32_t w[8][4];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int key = k8 * 8 + rr;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (key < it.nkeys)
                val = *reinterpret_cast<const uint4*>(
                    vg + ((int64_t)(it.c0 + it.kbeg + key) * Hkv + it.h) * D + c8 * 8);
            w[rr][0] = val.x; w[rr][1] = val.y; w[rr][2] = val.z; w[rr][3] = val.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int sh = (i & 1) * 16;
            uint32_t o[4];
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2)
                o[q2] = ((w[2 * q2][i >> 1] >> sh) & 0xFFFFu) | (((w[2 * q2 + 1][i >> 1] >> sh) & 0xFFFFu) << 16);
            *reinterpret_cast<uint4*>(&sVt[(c8 * 8 + i) * VP + k8 * 8]) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    __syncthreads();

    // gathered Q rows
    const u16* qg = reinterpret_cast<const u16*>(p.q);
    for (int x = tid; x < ROWS * (D / 8); x += 256) {
        const int r = x / (D / 8), c8 = x - r * (D / 8);
        uint4 val = make_uint4(0, 0, 0, 0);
        if (sPos[r] >= 0) {
            const int qh = it.h * G + (r % G);
            val = *reinterpret_cast<const uint4*>(qg + ((int64_t)sTok[r] * p.Hq + qh) * D + c8 * 8);
        }
        *reinterpret_cast<uint4*>(&sQ[r * KP + c8 * 8]) = val;
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;

    // S^T[key][row] = K Q^T
    f32x4 sacc[KT][2];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sacc[kt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
        bf16x8 bq[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            bq[nt] = *reinterpret_cast<const bf16x8*>(&sQ[(wave * 32 + nt * 16 + n) * KP + ds * 32 + gq * 8]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&sK[(kt * 16 + n) * KP + ds * 32 + gq * 8]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                sacc[kt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bq[nt], sacc[kt][nt], 0, 0, 0);
        }
    }

    // masked softmax over the block's keys, one row per lane column
    float mrow[2], lrow[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int pos = sPos[wave * 32 + nt * 16 + n];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kt * 16 + gq * 4 + i;
                const bool vis = key < it.nkeys && it.kbeg + key <= pos;
                const float x = vis ? sacc[kt][nt][i] * p.scale_log2 : -INFINITY;
                sacc[kt][nt][i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mref = mx == -INFINITY ? 0.f : mx;
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = exp2f(sacc[kt][nt][i] - mref);
                sacc[kt][nt][i] = e;
                sum += e;
            }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        mrow[nt] = mref;
        lrow[nt] = sum;
    }

    // O^T[d][row] = V^T P^T; key order inside a k-step: lane group gq holds
    // keys {4gq..4gq+3} and {16+4gq..16+4gq+3}, for both operands.
    f32x4 oacc[DT][2];
#pragma unroll
    for (int mt = 0; mt < DT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bf16x8 bp[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bp[nt][i] = static_cast<__bf16>(sacc[2 * ks][nt][i]);
                bp[nt][4 + i] = static_cast<__bf16>(sacc[2 * ks + 1][nt][i]);
            }
#pragma unroll
        for (int mt = 0; mt < DT; ++mt) {
            const u16* vr = &sVt[(mt * 16 + n) * VP + ks * 32 + gq * 4];
            const uint2 lo = *reinterpret_cast<const uint2*>(vr);
            const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
            const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bp[nt], oacc[mt][nt], 0, 0, 0);
        }
    }

    // normalised partial output (bf16) and its lse (fp32, natural log)
    u16* po = reinterpret_cast<u16*>(p.part_o);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int r = wave * 32 + nt * 16 + n;
        if (sPos[r] < 0) continue;
        const float inv = 1.f / lrow[nt];
        const int64_t prow = sPart[r];
        u16* dst = po + prow * D + gq * 4;
#pragma unroll
        for (int mt = 0; mt < DT; ++mt) {
            const uint2 v2 = make_uint2(pack2(oacc[mt][nt][0] * inv, oacc[mt][nt][1] * inv),
                                        pack2(oacc[mt][nt][2] * inv, oacc[mt][nt][3] * inv));
            *reinterpret_cast<uint2*>(dst + mt * 16) = v2;
        }
        if (gq == 0) p.part_lse[prow] = (mrow[nt] + __log2f(lrow[nt])) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// fp32 main kernel (VALU): one thread per gathered row, online softmax over
// the block's keys staged in LDS.
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void k_main_f32(Params p)
{
    __shared__ __attribute__((aligned(16))) float sK[BS * D];
    __shared__ __attribute__((aligned(16))) float sV[BS * D];
    Item it;
    if (!decode_item(p, blockIdx.x, it)) return;
    const int tid = threadIdx.x;
    const int Hkv = p.Hkv, G = p.G;
    const float* kg = reinterpret_cast<const float*>(p.k);
    const float* vg = reinterpret_cast<const float*>(p.v);
    for (int x = tid; x < BS * (D / 4); x += 256) {
        const int key = x / (D / 4), c4 = x - key * (D / 4);
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (key < it.nkeys) {
            const int64_t off = ((int64_t)(it.c0 + it.kbeg + key) * Hkv + it.h) * D + c4 * 4;
            kv = *reinterpret_cast<const float4*>(kg + off);
            vv = *reinterpret_cast<const float4*>(vg + off);
        }
        *reinterpret_cast<float4*>(&sK[key * D + c4 * 4]) = kv;
        *reinterpret_cast<float4*>(&sV[key * D + c4 * 4]) = vv;
    }
    __syncthreads();
    const int r = tid, ti = r / G, qq = r - ti * G;
    if (ti >= it.ne) return;
    const int ent = p.entries[it.e0 + ti];
    const int t = ent / p.topk, slot = ent - t * p.topk;
    const int pos = t - it.c0;
    const float* qrow = reinterpret_cast<const float*>(p.q) + ((int64_t)t * p.Hq + it.h * G + qq) * D;
    float qv[D], acc[D];
#pragma unroll
    for (int e = 0; e < D; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qrow + e);
        qv[e] = x.x; qv[e + 1] = x.y; qv[e + 2] = x.z; qv[e + 3] = x.w;
        acc[e] = acc[e + 1] = acc[e + 2] = acc[e + 3] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int kend = min(it.nkeys, pos - it.kbeg + 1);
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
    const int64_t prow = ((int64_t)((int64_t)t * Hkv + it.h) * p.topk + slot) * G + qq;
    float* dst = reinterpret_cast<float*>(p.part_o) + prow * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    p.part_lse[prow] = (m + log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Merge: one wave per (token, kv head); 16-byte chunks of the G*D outputs.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void k_merge(Params p)
{
    constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte chunk
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t rowid = (int64_t)blockIdx.x * 4 + wave;  // t*Hkv + h
    if (rowid >= p.T * p.Hkv) return;
    const int64_t t = rowid / p.Hkv;
    const int G = p.G, D = p.D, GD = G * D, topk = p.topk;
    const int s = seq_of_token(p.cus, p.B, t);
    const int b = s >= 0 ? (int)((t - p.cus[s]) / p.bs) : -1;

    // this lane's slot: kept iff 0 <= j <= b and no earlier slot has j
    const int j = lane < topk ? p.block_idx[rowid * topk + lane] : -1;
    bool keep = lane < topk && j >= 0 && j <= b;
    for (int k2 = 0; k2 < topk; ++k2) {
        const int o = __shfl(j, k2, 64);
        if (k2 < lane && o == j) keep = false;
    }
    const uint64_t kept = __ballot(keep);
    const int n = __popcll(kept);
    int rank = 0;  // position in ascending block order
    for (int k2 = 0; k2 < topk; ++k2) {
        const int o = __shfl(j, k2, 64);
        if (((kept >> k2) & 1) && o < j) ++rank;
    }

    const int64_t pbase = rowid * topk;  // partial rows of this (t, h)
    for (int c = 0; c * 64 * E < GD; ++c) {
        const int e = (c * 64 + lane) * E;
        const bool active = e < GD;
        const int qq = active ? e / D : 0;
        float M = -INFINITY;
        for (int r = 0; r < n; ++r) {
            const int slot = __ffsll((unsigned long long)__ballot(keep && rank == r)) - 1;
            M = fmaxf(M, p.part_lse[(pbase + slot) * G + qq]);
        }
        float acc[E];
#pragma unroll
        for (int x = 0; x < E; ++x) acc[x] = 0.f;
        float L = 0.f;
        for (int r = 0; r < n; ++r) {
            const int slot = __ffsll((unsigned long long)__ballot(keep && rank == r)) - 1;
            const float w = expf(p.part_lse[(pbase + slot) * G + qq] - M);
            L += w;
            if (active) {
                const int64_t off = (pbase + slot) * GD + e;
                if (BF16) {
                    const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(p.part_o) + off);
                    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        acc[2 * x] = fmaf(w, bf16_to_f32((u16)(wd[x] & 0xFFFFu)), acc[2 * x]);
                        acc[2 * x + 1] = fmaf(w, bf16_to_f32((u16)(wd[x] >> 16)), acc[2 * x + 1]);
                    }
                } else {
                    const float4 v4 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.part_o) + off);
                    acc[0] = fmaf(w, v4.x, acc[0]);
                    acc[1] = fmaf(w, v4.y, acc[1]);
                    acc[2] = fmaf(w, v4.z, acc[2]);
                    acc[3] = fmaf(w, v4.w, acc[3]);
                }
            }
        }
        if (!active) continue;
        const float inv = n > 0 ? 1.f / L : 0.f;
        const int64_t ooff = rowid * GD + e;
        if (BF16) {
            uint4 o;
            o.x = pack2(acc[0] * inv, acc[1] * inv);
            o.y = pack2(acc[2] * inv, acc[3] * inv);
            o.z = pack2(acc[4] * inv, acc[5] * inv);
            o.w = pack2(acc[6] * inv, acc[7] * inv);
            *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.out) + ooff) = o;
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + ooff) =
                make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        }
        if (e % D == 0) p.lse[rowid * G + qq] = n > 0 ? M + logf(L) : -INFINITY;
    }
}

template <int D>
hipError_t launch_main_d(const Params& p, hipStream_t st, bool bf16, unsigned grid)
{
    if (bf16) {
        switch (p.bs) {
        case 32: hipLaunchKernelGGL((k_main_bf16<D, 32>), dim3(grid), dim3(256), 0, st, p); break;
        case 64: hipLaunchKernelGGL((k_main_bf16<D, 64>), dim3(grid), dim3(256), 0, st, p); break;
        case 128: hipLaunchKernelGGL((k_main_bf16<D, 128>), dim3(grid), dim3(256), 0, st, p); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.bs) {
        case 32: hipLaunchKernelGGL((k_main_f32<D, 32>), dim3(grid), dim3(256), 0, st, p); break;
        case 64: hipLaunchKernelGGL((k_main_f32<D, 64>), dim3(grid), dim3(256), 0, st, p); break;
        case 128: hipLaunchKernelGGL((k_main_f32<D, 128>), dim3(grid), dim3(256), 0, st, p); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_main(const Params& p, bool bf16, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const unsigned grid = (unsigned)p.max_items;
    return grid == 0 ? hipSuccess
         : p.D == 64 ? launch_main_d<64>(p, st, bf16, grid)
         : p.D == 128 ? launch_main_d<128>(p, st, bf16, grid)
         : hipErrorInvalidValue;
}

hipError_t launch_merge(const Params& p, bool bf16, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const unsigned mgrid = (unsigned)div_up(p.T * p.Hkv, 4);
    if (bf16) hipLaunchKernelGGL(k_merge<true>, dim3(mgrid), dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_merge<false>, dim3(mgrid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace nsa
