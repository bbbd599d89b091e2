// attn_bwd.hip -- gradients of selected-block attention (bf16 / fp16).
//
// The forward is trained through as well as run for prefill (Flash-Sparse-
// Attention project page, "Key features", training-and-inference row, and
// "Quick start", step 4: a loss on the output, then backward).  With
// P_rp = exp(scale * q_r . k_p - lse_r) over the keys p the forward attends
// to, and D_r = dout_r . out_r:
//   dP_rp = dout_r . v_p,  dS_rp = P_rp (dP_rp - D_r),
//   dq_r = scale * sum_p dS_rp k_p,
//   dk_p = scale * sum_r dS_rp q_r,  dv_p = sum_r P_rp dout_r.
// Every (row, kv block) pair contributes independently once lse and D are
// known, so the backward keeps the forward's kv-outer schedule over the same
// inverted index ("Importance": kv blocks outer, queries inner):
//
//   delta   D_r for every (token, query head) row.
//   main    The gathered rows of all buckets, in CSR order, are cut into one
//           contiguous range per workgroup.  A workgroup walks its range
//           bucket by bucket: each wave owns 16 keys of the block and keeps
//           their K and V rows in registers and their dK, dV sums in MFMA
//           accumulators; 32-row chunks of the gathered q and dout are staged
//           in LDS (row-major and transposed), and the chunk's dS goes
//           through LDS so that dq over all the block's keys comes out as one
//           partial per (row, slot), stored at the row's CSR position.
//           dk, dv of a bucket that lies inside one range are final there;
//           the at most two buckets a range shares with its neighbours leave
//           fp32 partial sums.
//   finish  Buckets split across ranges: partial sums in range order; empty
//           buckets: zeros.
//   merge   dq of each (token, kv head): its kept slots' partials summed in
//           ascending block order.
// No atomics touch results, and every sum has a fixed order, so results are
// bitwise reproducible and do not depend on the order of ids within a row.
#include "device_common.h"

#include <algorithm>
#include <atomic>

namespace nsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Rows of the backward main kernel's range for workgroup w: [w*C, (w+1)*C)
// clipped to [0, R), C a multiple of kBwdRows.
__device__ __forceinline__ int64_t bwd_range_rows(int R, int W)
{
    const int64_t per = div_up(R, W);
    return div_up(per, kBwdRows) * kBwdRows;
}

// ---------------------------------------------------------------------------
// delta[t*Hq + qh] = sum_e dout * out (fp32); tokens outside every sequence
// get delta 0 and zero dk, dv rows (no bucket covers them).
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(256) void k_bwd_delta(Params p)
{
    using H = H16<E>;
    constexpr int LPR = D / 8;       // lanes per row, 16 bytes each
    constexpr int RPB = 256 / LPR;   // rows per workgroup
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;  // t*Hq + qh
    const int l = tid % LPR;
    const bool active = row < p.T * p.Hq;
    float acc = 0.f;
    if (active) {
        const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(p.out) + row * D + l * 8);
        const uint4 b = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(p.dout) + row * D + l * 8);
        const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            acc = fmaf(H::to_f32((u16)(wa[x] & 0xFFFFu)), H::to_f32((u16)(wb[x] & 0xFFFFu)), acc);
            acc = fmaf(H::to_f32((u16)(wa[x] >> 16)), H::to_f32((u16)(wb[x] >> 16)), acc);
        }
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (!active) return;
    const int64_t t = row / p.Hq;
    const int qh = (int)(row - t * p.Hq);
    const bool orphan = seq_of_token(p.cus, p.B, t) < 0;
    if (l == 0) p.delta[row] = orphan ? 0.f : acc;
    if (orphan && qh % p.G == 0) {
        const int64_t kr = (t * p.Hkv + qh / p.G) * D + l * 8;
        *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.dk) + kr) = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.dv) + kr) = make_uint4(0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// Main backward kernel.  BS/16 key groups of waves; a wave of key group w owns
// keys [16w, 16w+16) of the current block.  At d = 256 each key group has two
// waves, one per half of d for dK and dV (both compute the group's S and dP
// over all of d: twice the S/dP MFMA work, but the dK/dV accumulators stay at
// the d = 128 register count).  Per 32-row chunk (rows c..c+31 of the range,
// one bucket):
//   S = Q K_w^T, dP = dO V_w^T   (A = Q, dO rows from LDS; B = K_w, V_w rows
//                                 held in registers)
//   P = exp2(S scale log2e - lse log2e) masked, dS = P (dP - delta)
//   dV_w^T += dO^T P, dK_w^T += Q^T dS   (the S accumulator of two 16-row
//        tiles is the B operand of a 32-row k-step once the rows inside the
//        step are permuted: k-slot 8g+i holds row 4g+i for i < 4 and row
//        16+4g+i-4 for i >= 4; A = dO^T, Q^T read from LDS in that order)
//   dS -> LDS; dq^T = K^T dS^T over all BS keys, d tiles split across
//        waves: each wave keeps the K^T operands of its d tiles in registers
//        for the whole bucket and reads each dS tile once per chunk; dq goes
//        through an LDS tile to contiguous 16-byte stores.
// Loads run ahead of the math in three stages: once chunk n's rows are in
// LDS, the gathered q / dout rows and lse / delta of chunk n+1 are issued
// (their row indices come from the CSR entries by lane shuffles, not through
// LDS, so no barrier precedes them) together with the CSR entries of chunk
// n+2; no load waits on another inside a chunk and the chunk's MFMA work
// overlaps the next chunk's HBM traffic.
// ---------------------------------------------------------------------------

// LDS tiles without padding; the 16-byte pieces of a row are permuted by an
// XOR with a function of the row.  The LDS has 64 banks of 4 bytes.  A
// 16-byte read serves 16 lanes per cycle: the lanes of one half-wave whose
// quad index (lane / 4 mod 8) has the same bit parity; an 8-byte transpose
// read serves each half-wave in one cycle.  (Both measured: pairs of lanes
// swapped in otherwise conflict-free patterns, bank-conflict counter.)
// q / dout tiles (32 rows of D values): piece c of row r sits at c ^ qsw(r).
// The operand reads take row 16 rt + n, piece 4 ds + g; the transpose reads
// take rows 4 g + n / 4 (+ 16), pieces 2 mt, 2 mt + 1: with qsw(r) = 2 (r mod
// 8) (D >= 128; rows of 64 banks) or r & 6 (D = 64; rows of 32 banks) both
// read every bank once per cycle.
template <int D> __device__ __forceinline__ int qsw(int r) { return D >= 128 ? 2 * (r & 7) : (r & 6); }
template <int D> __device__ __forceinline__ int qoff(int r, int c) { return r * D + ((c ^ qsw<D>(r)) << 3); }
// dS tile (32 rows of BS keys): piece c of row r at c ^ ssw(r); the dq
// operand reads take row 16 j + n, piece 4 ks + g.
template <int BS> __device__ __forceinline__ int ssw(int r)
{
    return BS == 32 ? ((r >> 2) & 2) : BS == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int BS> __device__ __forceinline__ int soff(int r, int c) { return r * BS + ((c ^ ssw<BS>(r)) << 3); }
// dq tile (32 rows of D values; 8-byte writes from the MFMA results, 16-byte
// row reads): at D = 128 unpadded, piece c of row r at c ^ (r mod 16) ^ (r /
// 16) (measured: the 8-byte writes then take the time of 16-byte ones);
// otherwise rows padded by 16 bytes.
template <int D> __device__ __forceinline__ int dqoff(int r, int c)
{
    return D == 128 ? r * D + ((c ^ (r & 15) ^ (r >> 4)) << 3) : r * (D + 8) + (c << 3);
}

// Rows [c, cend) of the range in bucket b (decoded in bk); c == cend past
// the end of the range.
struct Chunk {
    int c, cend, b;
    Bucket bk;
};

__device__ __forceinline__ Chunk next_chunk(const Params& p, const Chunk& ch, int xe, int G)
{
    Chunk nx = ch;
    nx.c = ch.cend;
    if (nx.c >= xe) {
        nx.cend = nx.c;
        return nx;
    }
    if (nx.c >= (ch.bk.off + ch.bk.cnt) * G) {  // next non-empty bucket
        int b = ch.b + 1;
        while (uni(p.offsets[b + 1]) == uni(p.offsets[b])) ++b;
        nx.b = b;
        nx.bk = decode_bucket_uni(p, b);
    }
    nx.cend = min(min(nx.c + kBwdRows, (nx.bk.off + nx.bk.cnt) * G), xe);
    return nx;
}

template <typename E, int D, int BS>
__global__ __launch_bounds__(bwd_threads(D, BS)) __attribute__((amdgpu_waves_per_eu(2))) void k_bwd_main(Params p)
{
    using H = H16<E>;
    typedef typename H::v8 v8;
    constexpr int NWK = BS / 16;          // key groups
    constexpr int NDH = D > 128 ? 2 : 1;  // waves per key group (halves of d for dK, dV)
    constexpr int NW = NWK * NDH;
    constexpr int NTHR = 64 * NW;
    static_assert(NTHR == bwd_threads(D, BS), "threads");
    constexpr int RC = kBwdRows;
    constexpr int DS = D / 32;       // k-steps over d (S, dP)
    constexpr int MT = D / 16;       // d tiles (dK, dV, dq)
    constexpr int MTH = MT / NDH;    // d tiles of one wave's dK, dV
    constexpr int NTR = RC / 16;     // row tiles per chunk
    constexpr int KSQ = BS / 32;     // k-steps over keys (dq)
    // dq tiles of a wave: d tiles mt = wave + NW * mi (mi < MPW) for every
    // row tile, or, with fewer d tiles than waves, d tile wave % MT for
    // NTW of the row tiles
    constexpr int MPW = MT >= NW ? MT / NW : 1;
    constexpr int NTW = MT >= NW ? NTR : NTR * MT / NW;
    static_assert(MT % NW == 0 || (NW % MT == 0 && NW <= MT * NTR), "dq tiles per wave");
    constexpr int KTP = BS + 8;      // row pitch of sKt
    constexpr int RG = RC / 4;       // row groups of 4 per chunk
    constexpr int NSTG = 2 * RG * (D / 8);   // staging tasks: 4 rows x 16 B of Q or dO
    constexpr int SPT = (NSTG + NTHR - 1) / NTHR;
    static_assert(RC == 32 && NTR == 2, "one 32-row k-step per chunk");
    static_assert(BS % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 sKt[D * KTP];
    __shared__ __attribute__((aligned(16))) u16 sQ[RC * D];
    __shared__ __attribute__((aligned(16))) u16 sdO[RC * D];
    __shared__ __attribute__((aligned(16))) u16 sdS[RC * BS];
    __shared__ __attribute__((aligned(16))) u16 sdQ[RC * (D == 128 ? D : D + 8)];
    __shared__ __attribute__((aligned(16))) float sLse[RC];
    __shared__ __attribute__((aligned(16))) float sDel[RC];
    __shared__ __attribute__((aligned(16))) int sPos[RC];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int kw = wave % NWK, dh = wave / NWK;  // key group, half of d
    const int n = lane & 15, g = lane >> 4;
    const int G = p.G, Hkv = p.Hkv, Hq = p.Hq, topk = p.topk;
    const int nbk = Hkv * p.nbc;
    const int R = uni(p.status[kStatusNnz]) * G;
    const int W = gridDim.x;
    const int64_t C = bwd_range_rows(R, W);
    const int64_t xb64 = (int64_t)blockIdx.x * C;
    const int xb = xb64 < R ? (int)xb64 : R;
    const int xe = (int64_t)xb + C < R ? (int)(xb + C) : R;
    if (xb >= xe) return;

    const u16* qg = reinterpret_cast<const u16*>(p.q);
    const u16* dog = reinterpret_cast<const u16*>(p.dout);
    const u16* kg = reinterpret_cast<const u16*>(p.k);
    const u16* vg = reinterpret_cast<const u16*>(p.v);

    // This thread's staging task(s): 4 rows (4*rg ..) x 16 bytes (column
    // chunk c8) of Q (mat 0) or dO (mat 1); c8 varies fastest across lanes.
    // Threads beyond the task count repeat a task's loads (no extra HBM
    // traffic) so that every load is unconditional, and skip its LDS writes.
    int t_mat[SPT], t_rg[SPT], t_c8[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int y = (tid + NTHR * i) % NSTG;
        const int z = y % (NSTG / 2);
        t_mat[i] = y / (NSTG / 2);
        t_c8[i] = z % (D / 8);
        t_rg[i] = z / (D / 8);
    }
    const int mrow = tid % RC;  // row whose entry / lse / delta this thread fetches

    // chunk n (computed now), n+1 (rows in flight), n+2 (entries in flight)
    Chunk ch0;
    {
        const int v = xb / G;  // first bucket: the last b with offsets[b] <= xb / G
        int lo = 0, hi = nbk - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (uni(p.offsets[mid]) <= v) lo = mid; else hi = mid - 1;
        }
        ch0.b = lo;
        ch0.bk = decode_bucket_uni(p, lo);
        ch0.c = xb;
        ch0.cend = min(min(xb + RC, (ch0.bk.off + ch0.bk.cnt) * G), xe);
    }
    Chunk ch1 = next_chunk(p, ch0, xe, G);
    Chunk ch2 = next_chunk(p, ch1, xe, G);

    // Stage A: the CSR entry of row mrow of a chunk (entry of row x is x / G).
    auto load_entry = [&](const Chunk& ch) -> int {
        const int xr = ch.c + mrow;
        return p.entries[xr < ch.cend ? fast_div(xr, G, p.g_mul, p.g_shr) : 0];
    };
    // Entry -> token t and row index (t Hq + query head; T Hq < 2^31) of
    // row mrow of chunk ch, both -1 past the chunk's end.
    auto decode = [&](const Chunk& ch, int ent, int& t, int& rix) {
        const int xr = ch.c + mrow;
        const int e = fast_div(xr, G, p.g_mul, p.g_shr);
        t = xr < ch.cend ? fast_div(ent, topk, p.topk_mul, p.topk_shr) : -1;
        rix = t >= 0 ? t * Hq + ch.bk.h * G + (xr - e * G) : -1;
    };
    // Stage B: q / dout rows, lse and delta of a chunk's rows, kept raw in
    // registers until the chunk is committed.  Lane r mod 32 of every wave
    // holds row r's index; the staging lanes take theirs by lane shuffles.
    uint4 pf[SPT][4];
    int pf_valid[SPT];
    float m_lse = 0.f, m_del = 0.f;
    int m_t = -1;
    auto load_rows = [&](int t, int rix) {
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const u16* src = t_mat[i] ? dog : qg;
            int vmask = 0;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int rv = __shfl(rix, 4 * t_rg[i] + rr, 64);
                vmask |= (rv >= 0) << rr;
                const uint32_t row = (uint32_t)(rv >= 0 ? rv : 0);
                pf[i][rr] = *reinterpret_cast<const uint4*>(src + (size_t)row * D + t_c8[i] * 8);
            }
            pf_valid[i] = vmask;
        }
        const uint32_t qr = (uint32_t)(rix >= 0 ? rix : 0);
        m_lse = p.lse[qr];
        m_del = p.delta[qr];
        m_t = t;
    };

    // prologue: rows of chunk 0 in flight, entries of chunk 1 in flight
    {
        int t0, r0;
        decode(ch0, load_entry(ch0), t0, r0);
        load_rows(t0, r0);
    }
    int ent_nx = load_entry(ch1);

    int cur_b = -1;       // bucket whose K, V are staged
    Bucket cur_bk{};
    v8 kreg[DS], vreg[DS];
    v8 ktr[MPW][KSQ];  // K^T of this wave's dq d tiles over the block's keys
    bool kt_stale = false;
    f32x4 dKt[MTH], dVt[MTH];  // d tiles dh * MTH + mi
    const int key = 16 * kw + n;

    // dK, dV of this wave's keys for the segment of bucket cur_b: final if the
    // bucket lies inside this range, else a partial sum in one of the range's
    // two slots (first slot: the bucket began at or before the range).
    auto flush = [&]() {
        const int bs0 = cur_bk.off * G, bs1 = (cur_bk.off + cur_bk.cnt) * G;
        if (bs0 >= xb && bs1 <= xe) {
            if (key < cur_bk.nkeys) {
                const int64_t kr = ((int64_t)(cur_bk.c0 + cur_bk.kbeg + key) * Hkv + cur_bk.h) * D + 4 * g;
                u16* dkr = reinterpret_cast<u16*>(p.dk) + kr;
                u16* dvr = reinterpret_cast<u16*>(p.dv) + kr;
#pragma unroll
                for (int mi = 0; mi < MTH; ++mi) {
                    const int mt = dh * MTH + mi;
                    *reinterpret_cast<uint2*>(dkr + 16 * mt) =
                        make_uint2(pack2h<E>(dKt[mi][0] * p.scale, dKt[mi][1] * p.scale),
                                   pack2h<E>(dKt[mi][2] * p.scale, dKt[mi][3] * p.scale));
                    *reinterpret_cast<uint2*>(dvr + 16 * mt) =
                        make_uint2(pack2h<E>(dVt[mi][0], dVt[mi][1]), pack2h<E>(dVt[mi][2], dVt[mi][3]));
                }
            }
        } else {
            const int slot = bs0 <= xb ? 2 * (int)blockIdx.x : 2 * (int)blockIdx.x + 1;
            float* base = p.dkv_part + (size_t)slot * 2 * BS * D;
#pragma unroll
            for (int mi = 0; mi < MTH; ++mi) {
                const int mt = dh * MTH + mi;
                *reinterpret_cast<f32x4*>(&base[key * D + 16 * mt + 4 * g]) = dKt[mi];
                *reinterpret_cast<f32x4*>(&base[(BS + key) * D + 16 * mt + 4 * g]) = dVt[mi];
            }
        }
    };

    // dq partial rows [dq_c, dq_cend) (their CSR row positions) from the LDS
    // tile: contiguous 16-byte stores, streamed past the caches (the merge
    // reads each once)
    int dq_c = 0, dq_cend = 0;
    auto store_dq = [&]() {
        constexpr int CPR = D / 8;
        constexpr int NIT = (RC * CPR + NTHR - 1) / NTHR;
        const int nrows = dq_cend - dq_c;
        u16* base = reinterpret_cast<u16*>(p.dq_part) + (int64_t)dq_c * D;
        uint4 tile[NIT];  // every LDS read first, then the stores
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int x = tid + NTHR * it, r = x / CPR, cc = x - r * CPR;
            if ((RC * CPR) % NTHR == 0 || x < RC * CPR)
                tile[it] = *reinterpret_cast<const uint4*>(&sdQ[dqoff<D>(r, cc)]);
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int x = tid + NTHR * it, r = x / CPR, cc = x - r * CPR;
            if (((RC * CPR) % NTHR == 0 || x < RC * CPR) && r < nrows) {
                const uint4 v4 = tile[it];
                uint32_t* dst = reinterpret_cast<uint32_t*>(base + (int64_t)r * D + cc * 8);
                __builtin_nontemporal_store(v4.x, dst);
                __builtin_nontemporal_store(v4.y, dst + 1);
                __builtin_nontemporal_store(v4.z, dst + 2);
                __builtin_nontemporal_store(v4.w, dst + 3);
            }
        }
    };

    while (ch0.c < xe) {
        // registers -> LDS: chunk n's rows
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            if (NSTG % NTHR == 0 || tid + NTHR * i < NSTG) {
                u16* rm = t_mat[i] ? sdO : sQ;
                const int rg = t_rg[i], c8 = t_c8[i];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint32_t mk = 0u - (uint32_t)((pf_valid[i] >> rr) & 1);  // rows past the chunk: zeros
                    const uint4 v4 = make_uint4(pf[i][rr].x & mk, pf[i][rr].y & mk, pf[i][rr].z & mk, pf[i][rr].w & mk);
                    *reinterpret_cast<uint4*>(&rm[qoff<D>(4 * rg + rr, c8)]) = v4;
                }
            }
        }
        if (tid < RC) {
            sPos[tid] = m_t >= 0 ? m_t - ch0.bk.c0 : -1;
            sLse[tid] = m_lse * kLog2e;
            sDel[tid] = m_del;
        }
        // issue chunk n+1's rows and chunk n+2's entries
        {
            int t1, r1;
            decode(ch1, ent_nx, t1, r1);
            load_rows(t1, r1);
        }
        ent_nx = load_entry(ch2);

        // a new bucket: finish the previous segment, stage this block (after
        // every wave's last read of the previous block's K^T)
        if (ch0.b != cur_b) {
            if (cur_b >= 0) {
                flush();
                __syncthreads();
            }
            cur_b = ch0.b;
            cur_bk = ch0.bk;
            const int kc = key < cur_bk.nkeys ? key : 0;
            const int64_t kr = ((int64_t)(cur_bk.c0 + cur_bk.kbeg + kc) * Hkv + cur_bk.h) * D + 8 * g;
            uint4 kv4[DS], vv4[DS];
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                kv4[ds] = *reinterpret_cast<const uint4*>(kg + kr + 32 * ds);
                vv4[ds] = *reinterpret_cast<const uint4*>(vg + kr + 32 * ds);
            }
            for (int y = tid; y < (BS / 8) * (D / 8); y += NTHR) {
                const int k8 = y / (D / 8), c8 = y - k8 * (D / 8);
                uint32_t w[8][4];
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    const int kk = k8 * 8 + rr;
                    uint4 val = make_uint4(0, 0, 0, 0);
                    if (kk < cur_bk.nkeys)
                        val = *reinterpret_cast<const uint4*>(
                            kg + ((int64_t)(cur_bk.c0 + cur_bk.kbeg + kk) * Hkv + cur_bk.h) * D + c8 * 8);
                    w[rr][0] = val.x; w[rr][1] = val.y; w[rr][2] = val.z; w[rr][3] = val.w;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int sh = (i & 1) * 16;
                    uint32_t o[4];
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2)
                        o[q2] = ((w[2 * q2][i >> 1] >> sh) & 0xFFFFu) | (((w[2 * q2 + 1][i >> 1] >> sh) & 0xFFFFu) << 16);
                    *reinterpret_cast<uint4*>(&sKt[(c8 * 8 + i) * KTP + k8 * 8]) = make_uint4(o[0], o[1], o[2], o[3]);
                }
            }
            const bool kin0 = key < cur_bk.nkeys;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                kreg[ds] = __builtin_bit_cast(v8, kin0 ? kv4[ds] : make_uint4(0, 0, 0, 0));
                vreg[ds] = __builtin_bit_cast(v8, kin0 ? vv4[ds] : make_uint4(0, 0, 0, 0));
            }
#pragma unroll
            for (int mi = 0; mi < MTH; ++mi) {
                dKt[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
                dVt[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            kt_stale = true;
        }
        __syncthreads();
        if (kt_stale) {  // the staged K^T -> this wave's dq operands
#pragma unroll
            for (int mi = 0; mi < MPW; ++mi) {
                const int mt = MT >= NW ? wave + NW * mi : wave % MT;
#pragma unroll
                for (int ks = 0; ks < KSQ; ++ks)
                    ktr[mi][ks] = *reinterpret_cast<const v8*>(&sKt[(16 * mt + n) * KTP + 32 * ks + 8 * g]);
            }
            kt_stale = false;
        }

        store_dq();  // the previous chunk's dq tile (nothing on the first chunk)

        const int kpos = cur_bk.kbeg + key;
        const bool kin = key < cur_bk.nkeys;

        // S and dP: rows 16*rt + 4g + i of the chunk, key 16*kw + n
        f32x4 sacc[NTR], pacc[NTR];
#pragma unroll
        for (int rt = 0; rt < NTR; ++rt) {
            sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            pacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // The two MFMA clusters run at raised wave priority: with two waves
        // per SIMD from different workgroups, the one that has MFMA work
        // issues it ahead of the other's LDS and VALU work (9.92 -> 9.78 ms
        // at the 64K+32K GQA-4 workload).  Row tile 0's products come first,
        // and the softmax stays inside the raised-priority region, so that
        // tile 0's exponentials can issue between tile 1's products (1%).
        // operand reads: row 16 rt + n, piece 4 ds + g, i.e. element
        // 16 rt D + (av ^ 32 ds) with av the ds = 0 offset of row n (the XOR
        // keeps the offset inside the row); av is recomputed per chunk so
        // that the read addresses are not all held in registers
        int av = qoff<D>(n, g);
        asm volatile("" : "+v"(av));
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int rt = 0; rt < NTR; ++rt)
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const int lr = 16 * rt * D + (av ^ (32 * ds));
                const v8 aq = *reinterpret_cast<const v8*>(&sQ[lr]);
                const v8 ao = *reinterpret_cast<const v8*>(&sdO[lr]);
                sacc[rt] = H::mfma(aq, kreg[ds], sacc[rt]);
                pacc[rt] = H::mfma(ao, vreg[ds], pacc[rt]);
            }

        uint32_t wP[4], wdS[4];  // P, dS as 16-bit pairs: element 4 rt + i
#pragma unroll
        for (int rt = 0; rt < NTR; ++rt) {
            const float4 l4 = *reinterpret_cast<const float4*>(&sLse[16 * rt + 4 * g]);
            const float4 d4 = *reinterpret_cast<const float4*>(&sDel[16 * rt + 4 * g]);
            const int4 p4 = *reinterpret_cast<const int4*>(&sPos[16 * rt + 4 * g]);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
            const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
            f32x4 pr, ds;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool vis = kin && kpos <= pv[i];
                // raw v_exp_f32: P below 2^-126 flushes to 0
                pr[i] = vis ? __builtin_amdgcn_exp2f(fmaf(sacc[rt][i], p.scale_log2, -lv[i])) : 0.f;
                ds[i] = pr[i] * (pacc[rt][i] - dv[i]);
            }
            const uint2 hp = cvt4<E>(pr), hd = cvt4<E>(ds);
            wP[2 * rt] = hp.x;
            wP[2 * rt + 1] = hp.y;
            wdS[2 * rt] = hd.x;
            wdS[2 * rt + 1] = hd.y;
        }
        __builtin_amdgcn_s_setprio(0);
        const v8 bP = __builtin_bit_cast(v8, make_uint4(wP[0], wP[1], wP[2], wP[3]));
        const v8 bdS = __builtin_bit_cast(v8, make_uint4(wdS[0], wdS[1], wdS[2], wdS[3]));

        // dV^T += dO^T P, dK^T += Q^T dS over the chunk's 32 rows.  The A
        // operands (dO^T, Q^T in the permuted row order) come straight from
        // the row-major tiles through LDS transpose reads: in each 16-lane
        // group, lane i receives element i % 4 of the 4-element runs that
        // lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 point at, so lane
        // (n, g) points at row 4g + n / 4 (then 16 + 4g + n / 4), columns
        // 16 mt + 4 (n % 4) .. + 3: piece 2 mt + (n / 2) % 2, element 4 (n % 2).
        // Row 4g + n / 4 + 16 has the row's permutation (qsw depends on the
        // row mod 8), so its offsets are those of row 4g + n / 4 plus 16 D;
        // piece 2 mt + b at (2 mt + b) ^ qsw = 2 mt ^ (b ^ qsw): the offset
        // of column 16 mt + 4 (n % 4) is tv ^ 16 mt.
        const int ra = 4 * g + (n >> 2);
        int tv = ra * D + ((((n >> 1) & 1) ^ qsw<D>(ra)) << 3) + 4 * (n & 1);
        asm volatile("" : "+v"(tv));
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int mi = 0; mi < MTH; ++mi) {
            const int mt = dh * MTH + mi;
            const int oa = tv ^ (16 * mt), ob = oa + 16 * D;
            const v8 ao = lds_tr_pair<v8>(&sdO[oa], &sdO[ob]);
            const v8 aq = lds_tr_pair<v8>(&sQ[oa], &sQ[ob]);
            dVt[mi] = H::mfma(ao, bP, dVt[mi]);
            dKt[mi] = H::mfma(aq, bdS, dKt[mi]);
        }

        __builtin_amdgcn_s_setprio(0);
        // dS (16-bit) -> LDS, row-major [row][key], by the first wave of each
        // key group
        if (dh == 0) {
            const uint32_t* wv = wdS;
#pragma unroll
            for (int rt = 0; rt < NTR; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 4 * rt + i;
                    sdS[soff<BS>(16 * rt + 4 * g + i, key >> 3) + (key & 7)] = (u16)(wv[e >> 1] >> ((e & 1) * 16));
                }
        }
        __syncthreads();

        // dq^T[e][row] = sum over the block's keys of K^T[e][key] dS[row][key]
        // (sdQ was last read by the previous chunk's stores, before this
        // chunk's second barrier)
        {
            const int nt0 = MT >= NW ? 0 : (wave / MT) * NTW;
            v8 bd[NTW][KSQ];
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int ks = 0; ks < KSQ; ++ks)
                    bd[j][ks] = *reinterpret_cast<const v8*>(&sdS[soff<BS>(16 * (nt0 + j) + n, 4 * ks + g)]);
#pragma unroll
            for (int mi = 0; mi < MPW; ++mi) {
                const int mt = MT >= NW ? wave + NW * mi : wave % MT;
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSQ; ++ks) acc = H::mfma(ktr[mi][ks], bd[j][ks], acc);
                    *reinterpret_cast<uint2*>(&sdQ[dqoff<D>(16 * (nt0 + j) + n, 2 * mt + (g >> 1)) + 4 * (g & 1)]) =
                        make_uint2(pack2h<E>(acc[0], acc[1]), pack2h<E>(acc[2], acc[3]));
                }
            }
        }

        // the tile is stored after the next chunk's first barrier
        dq_c = ch0.c;
        dq_cend = ch0.cend;

        ch0 = ch1;
        ch1 = ch2;
        ch2 = next_chunk(p, ch2, xe, G);
    }
    __syncthreads();
    store_dq();
    flush();
}

// ---------------------------------------------------------------------------
// dk, dv of buckets not finished by the main kernel: split buckets sum their
// ranges' partial slots in range order; empty buckets write zeros.  One
// workgroup per bucket.
// ---------------------------------------------------------------------------
template <typename E, int D, int BS>
__global__ __launch_bounds__(256) void k_bwd_dkv_finish(Params p)
{
    const int bkt = blockIdx.x;
    const Bucket bk = decode_bucket(p, bkt);
    if (bk.nkeys <= 0) return;
    const int G = p.G;
    const int R = p.status[kStatusNnz] * G;
    const int64_t C = bwd_range_rows(R, p.bwd_grid);
    const int bs0 = bk.off * G, bs1 = (bk.off + bk.cnt) * G;
    int wlo = 0, whi = -1;  // ranges holding the bucket's rows
    if (bk.cnt > 0) {
        wlo = (int)(bs0 / C);
        whi = (int)((bs1 - 1) / C);
        if (wlo == whi) return;  // finished by the main kernel
    }
    for (int y = threadIdx.x; y < BS * (D / 4); y += 256) {
        const int key = y / (D / 4), e4 = (y - key * (D / 4)) * 4;
        if (key >= bk.nkeys) continue;
        float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
        for (int w = wlo; w <= whi; ++w) {
            const int slot = (int64_t)bs0 <= (int64_t)w * C ? 2 * w : 2 * w + 1;
            const float* base = p.dkv_part + (size_t)slot * 2 * BS * D;
            const float4 a = *reinterpret_cast<const float4*>(&base[key * D + e4]);
            const float4 c = *reinterpret_cast<const float4*>(&base[(BS + key) * D + e4]);
            sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
            sv.x += c.x; sv.y += c.y; sv.z += c.z; sv.w += c.w;
        }
        const int64_t kr = ((int64_t)(bk.c0 + bk.kbeg + key) * p.Hkv + bk.h) * D + e4;
        *reinterpret_cast<uint2*>(reinterpret_cast<u16*>(p.dk) + kr) =
            make_uint2(pack2h<E>(sk.x * p.scale, sk.y * p.scale), pack2h<E>(sk.z * p.scale, sk.w * p.scale));
        *reinterpret_cast<uint2*>(reinterpret_cast<u16*>(p.dv) + kr) =
            make_uint2(pack2h<E>(sv.x, sv.y), pack2h<E>(sv.z, sv.w));
    }
}

// ---------------------------------------------------------------------------
// dq of one (token, kv head) row per wave: the kept slots' partials (CSR
// positions from slot_pos, already in ascending block order) summed in that
// order, times scale.
// Rows with no kept slot (and tokens outside every sequence) get zeros.
// Rows narrower than a wave (G * D < 512: G 1 or 2 at d 128) would leave
// most lanes idle: there each wave takes 64 / LPR rows, one group of LPR
// lanes per row (8 elements per lane), the same sums in the same order.
// ---------------------------------------------------------------------------
constexpr int kDqGroup = 8;

// Lanes per row of the grouped dq merge (a power of two below 64 whose lanes
// hold the row and its topk slot positions), or 0: one wave per row.
__host__ __device__ inline int dq_group_lanes(int G, int D, int topk)
{
    const int lpr = G * D / 8;
    return lpr < 64 && 64 % lpr == 0 && topk <= lpr ? lpr : 0;
}

template <typename E>
__global__ __launch_bounds__(256) void k_bwd_dq_merge(Params p, int LPR)
{
    using H = H16<E>;
    if (LPR) {
        const int lane = threadIdx.x & 63, gl = lane & (LPR - 1), gb = lane - gl;
        const int GD = p.G * p.D, topk = p.topk;
        // rows dealt as merge_rowid deals them, 64 / LPR per wave
        const int64_t per = gridDim.x / kNumXcd;
        const int64_t w = (blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd;
        const int64_t idx = (w * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;
        int64_t rowid = -1;
        if (idx < p.T * p.Hkv) {
            const int64_t h = idx / p.T;
            rowid = (idx - h * p.T) * p.Hkv + h;
        }
        const int spos = rowid >= 0 && gl < topk ? p.slot_pos[rowid * topk + gl] : -1;
        uint64_t km = (__ballot(spos >= 0) >> gb) & ((1ull << LPR) - 1);  // this row's kept slots
        const int nk = __popcll(km);
        const int e = gl * 8;
        const u16* part = reinterpret_cast<const u16*>(p.dq_part);
        float acc[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = 0.f;
        for (int r0 = 0; __ballot(r0 < nk) != 0; r0 += kDqGroup) {  // (uniform: every lane permutes)
            uint4 raw[kDqGroup];
#pragma unroll
            for (int q2 = 0; q2 < kDqGroup; ++q2) {
                const int src = km ? __builtin_ctzll(km) : 0;
                km &= km - 1;
                const int64_t pr = __builtin_amdgcn_ds_bpermute((gb + src) << 2, spos);
                raw[q2] = make_uint4(0, 0, 0, 0);
                if (r0 + q2 < nk) {
                    const uint32_t* sp = reinterpret_cast<const uint32_t*>(part + pr * GD + e);
                    raw[q2] = make_uint4(__builtin_nontemporal_load(sp), __builtin_nontemporal_load(sp + 1),
                                         __builtin_nontemporal_load(sp + 2), __builtin_nontemporal_load(sp + 3));
                }
            }
#pragma unroll
            for (int q2 = 0; q2 < kDqGroup; ++q2) {
                if (r0 + q2 < nk) {
                    const uint32_t wd[4] = {raw[q2].x, raw[q2].y, raw[q2].z, raw[q2].w};
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        acc[2 * x] += H::to_f32((u16)(wd[x] & 0xFFFFu));
                        acc[2 * x + 1] += H::to_f32((u16)(wd[x] >> 16));
                    }
                }
            }
        }
        if (rowid < 0) return;
        uint4 o;
        o.x = pack2h<E>(acc[0] * p.scale, acc[1] * p.scale);
        o.y = pack2h<E>(acc[2] * p.scale, acc[3] * p.scale);
        o.z = pack2h<E>(acc[4] * p.scale, acc[5] * p.scale);
        o.w = pack2h<E>(acc[6] * p.scale, acc[7] * p.scale);
        *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.dq) + rowid * GD + e) = o;
        return;
    }
    const int64_t rowid = merge_rowid(p.T, p.Hkv);
    if (rowid < 0) return;
    const int lane = threadIdx.x & 63;
    const int G = p.G, D = p.D, GD = G * D, topk = p.topk;
    // the row's kept CSR positions in ascending block order, then -1
    const int spos = lane < topk ? p.slot_pos[rowid * topk + lane] : -1;
    const uint64_t kept = __ballot(spos >= 0);
    const int nk = __popcll(kept);

    const u16* part = reinterpret_cast<const u16*>(p.dq_part);
    for (int c = 0; c * 64 * 8 < GD; ++c) {
        const int e = (c * 64 + lane) * 8;
        const bool active = e < GD;
        const int ee = active ? e : 0;
        float acc[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = 0.f;
        uint64_t km = kept;
        for (int r0 = 0; r0 < nk; r0 += kDqGroup) {
            uint4 raw[kDqGroup];
#pragma unroll
            for (int q2 = 0; q2 < kDqGroup; ++q2) {
                const int r = r0 + q2;
                const int src_lane = km ? __builtin_ctzll(km) : 0;
                km &= km - 1;
                const int64_t pr = __builtin_amdgcn_readlane(spos, src_lane);
                raw[q2] = make_uint4(0, 0, 0, 0);
                if (r < nk) {
                    const uint32_t* src = reinterpret_cast<const uint32_t*>(part + pr * GD + ee);
                    raw[q2] = make_uint4(__builtin_nontemporal_load(src), __builtin_nontemporal_load(src + 1),
                                         __builtin_nontemporal_load(src + 2), __builtin_nontemporal_load(src + 3));
                }
            }
#pragma unroll
            for (int q2 = 0; q2 < kDqGroup; ++q2) {
                if (r0 + q2 < nk) {
                    const uint32_t wd[4] = {raw[q2].x, raw[q2].y, raw[q2].z, raw[q2].w};
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        acc[2 * x] += H::to_f32((u16)(wd[x] & 0xFFFFu));
                        acc[2 * x + 1] += H::to_f32((u16)(wd[x] >> 16));
                    }
                }
            }
        }
        if (!active) continue;
        uint4 o;
        o.x = pack2h<E>(acc[0] * p.scale, acc[1] * p.scale);
        o.y = pack2h<E>(acc[2] * p.scale, acc[3] * p.scale);
        o.z = pack2h<E>(acc[4] * p.scale, acc[5] * p.scale);
        o.w = pack2h<E>(acc[6] * p.scale, acc[7] * p.scale);
        *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.dq) + rowid * GD + e) = o;
    }
}

// d = 256: blocks of 32 or 64 keys only (the host checks reject 128).
template <typename E>
const void* bwd_main_ptr(int D, int bs)
{
    if (D == 64) return bs == 32 ? (const void*)k_bwd_main<E, 64, 32>
                      : bs == 64 ? (const void*)k_bwd_main<E, 64, 64> : (const void*)k_bwd_main<E, 64, 128>;
    if (D == 256) return bs == 32 ? (const void*)k_bwd_main<E, 256, 32> : (const void*)k_bwd_main<E, 256, 64>;
    return bs == 32 ? (const void*)k_bwd_main<E, 128, 32>
         : bs == 64 ? (const void*)k_bwd_main<E, 128, 64> : (const void*)k_bwd_main<E, 128, 128>;
}

template <typename E, int D>
void launch_bwd_main_d(const Params& p, hipStream_t st)
{
    const unsigned grid = (unsigned)p.bwd_grid;
    if (p.bs == 32) {
        hipLaunchKernelGGL((k_bwd_main<E, D, 32>), dim3(grid), dim3(bwd_threads(D, 32)), 0, st, p);
    } else if (D == 256 || p.bs == 64) {
        hipLaunchKernelGGL((k_bwd_main<E, D, 64>), dim3(grid), dim3(bwd_threads(D, 64)), 0, st, p);
    } else if constexpr (D != 256) {
        hipLaunchKernelGGL((k_bwd_main<E, D, 128>), dim3(grid), dim3(bwd_threads(D, 128)), 0, st, p);
    }
}

template <typename E, int D>
void launch_bwd_finish_d(const Params& p, hipStream_t st)
{
    const unsigned nbk = (unsigned)((int64_t)p.Hkv * p.nbc);
    if (p.bs == 32) {
        hipLaunchKernelGGL((k_bwd_dkv_finish<E, D, 32>), dim3(nbk), dim3(256), 0, st, p);
    } else if (D == 256 || p.bs == 64) {
        hipLaunchKernelGGL((k_bwd_dkv_finish<E, D, 64>), dim3(nbk), dim3(256), 0, st, p);
    } else if constexpr (D != 256) {
        hipLaunchKernelGGL((k_bwd_dkv_finish<E, D, 128>), dim3(nbk), dim3(256), 0, st, p);
    }
}

template <typename E>
void launch_bwd_delta_t(const Params& p, hipStream_t st)
{
    const int64_t rows = p.T * p.Hq;
    if (p.D == 64) hipLaunchKernelGGL((k_bwd_delta<E, 64>), dim3((unsigned)div_up(rows, 32)), dim3(256), 0, st, p);
    else if (p.D == 128) hipLaunchKernelGGL((k_bwd_delta<E, 128>), dim3((unsigned)div_up(rows, 16)), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_bwd_delta<E, 256>), dim3((unsigned)div_up(rows, 8)), dim3(256), 0, st, p);
}

template <typename E>
void launch_bwd_main_t(const Params& p, hipStream_t st)
{
    if (p.D == 64) launch_bwd_main_d<E, 64>(p, st);
    else if (p.D == 128) launch_bwd_main_d<E, 128>(p, st);
    else launch_bwd_main_d<E, 256>(p, st);
}

template <typename E>
void launch_bwd_dq_merge_t(const Params& p, hipStream_t st)
{
    if (p.D == 64) launch_bwd_finish_d<E, 64>(p, st);
    else if (p.D == 128) launch_bwd_finish_d<E, 128>(p, st);
    else launch_bwd_finish_d<E, 256>(p, st);
    const int lpr = dq_group_lanes(p.G, p.D, p.topk);
    const int64_t rows = lpr ? div_up(p.T * p.Hkv, 64 / lpr) : p.T * p.Hkv;  // waves
    hipLaunchKernelGGL((k_bwd_dq_merge<E>), dim3((unsigned)merge_grid(rows, 1)), dim3(256), 0, st, p, lpr);
}

}  // namespace

// Workgroups of the backward main kernel: every CU filled at the kernel's
// occupancy, a multiple of the XCD count, at most kBwdMaxGrid.
int bwd_grid_size(int D, int bs, int kind)
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
    const void* fn = ki ? bwd_main_ptr<_Float16>(D, bs) : bwd_main_ptr<__bf16>(D, bs);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, bwd_threads(D, bs), 0) != hipSuccess || per < 1) per = 1;
    int g = cus * per;
    g = (g + kNumXcd - 1) / kNumXcd * kNumXcd;
    g = std::min(g, kBwdMaxGrid);
    if (slot) slot->store(g, std::memory_order_relaxed);
    return g;
}

hipError_t launch_bwd_delta(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    if (kind == kElemF16) launch_bwd_delta_t<_Float16>(p, st);
    else launch_bwd_delta_t<__bf16>(p, st);
    return hipGetLastError();
}

hipError_t launch_bwd_main(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    if (kind == kElemF16) launch_bwd_main_t<_Float16>(p, st);
    else launch_bwd_main_t<__bf16>(p, st);
    return hipGetLastError();
}

// dk / dv finish, then the dq merge.
hipError_t launch_bwd_dq_merge(const Params& p, int kind, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    if (kind == kElemF16) launch_bwd_dq_merge_t<_Float16>(p, st);
    else launch_bwd_dq_merge_t<__bf16>(p, st);
    return hipGetLastError();
}

}  // namespace nsa
