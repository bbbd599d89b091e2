// attn_bwd.hip -- gradients of selected-block attention (bf16).
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
template <int D>
__global__ __launch_bounds__(256) void k_bwd_delta(Params p)
{
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
            acc = fmaf(bf16_to_f32((u16)(wa[x] & 0xFFFFu)), bf16_to_f32((u16)(wb[x] & 0xFFFFu)), acc);
            acc = fmaf(bf16_to_f32((u16)(wa[x] >> 16)), bf16_to_f32((u16)(wb[x] >> 16)), acc);
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
// Main backward kernel.  BS/16 waves; wave w owns keys [16w, 16w+16) of the
// current block.  Per 32-row chunk (rows c..c+31 of the range, one bucket):
//   S = Q K_w^T, dP = dO V_w^T   (A = Q, dO rows from LDS; B = K_w, V_w rows
//                                 held in registers)
//   P = exp2(S scale log2e - lse log2e) masked, dS = P (dP - delta)
//   dV_w^T += dO^T P, dK_w^T += Q^T dS   (the S accumulator of two 16-row
//        tiles is the B operand of a 32-row k-step once the rows inside the
//        step are permuted: k-slot 8g+i holds row 4g+i for i < 4 and row
//        16+4g+i-4 for i >= 4; A = dO^T, Q^T read from LDS in that order)
//   dS -> LDS; dq^T = K^T dS^T over all BS keys, tiles split across waves,
//        through an LDS tile to contiguous 16-byte stores.
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(BS * 4) void k_bwd_main(Params p)
{
    constexpr int NW = BS / 16;
    constexpr int NTHR = 64 * NW;
    constexpr int RC = kBwdRows;
    constexpr int DS = D / 32;       // k-steps over d (S, dP)
    constexpr int MT = D / 16;       // d tiles (dK, dV, dq)
    constexpr int NTR = RC / 16;     // row tiles per chunk
    constexpr int KSQ = BS / 32;     // k-steps over keys (dq)
    constexpr int NDQ = (MT * NTR + NW - 1) / NW;  // dq tiles per wave
    constexpr int QP = D + 8;        // row pitch (elements) of sQ, sdO, sdQ
    constexpr int TP = RC + 8;       // row pitch of sQt, sdOt
    constexpr int KTP = BS + 8;      // row pitch of sKt
    constexpr int SP = BS + 8;       // row pitch of sdS
    constexpr int NSTG = 2 * (RC / 4) * (D / 8);   // staging tasks: 4 rows x 16 B of Q or dO
    constexpr int SPT = (NSTG + NTHR - 1) / NTHR;
    static_assert(RC == 32 && NTR == 2, "one 32-row k-step per chunk");
    static_assert(BS % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 sKt[D * KTP];
    __shared__ __attribute__((aligned(16))) u16 sQ[RC * QP];
    __shared__ __attribute__((aligned(16))) u16 sdO[RC * QP];
    __shared__ __attribute__((aligned(16))) u16 sQt[D * TP];
    __shared__ __attribute__((aligned(16))) u16 sdOt[D * TP];
    __shared__ __attribute__((aligned(16))) u16 sdS[RC * SP];
    __shared__ __attribute__((aligned(16))) u16 sdQ[RC * QP];
    __shared__ __attribute__((aligned(16))) float sLse[RC];
    __shared__ __attribute__((aligned(16))) float sDel[RC];
    __shared__ __attribute__((aligned(16))) int sPos[RC];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int G = p.G, Hkv = p.Hkv, Hq = p.Hq, topk = p.topk;
    const int nbk = Hkv * p.nbc;
    const int R = p.status[kStatusNnz] * G;
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

    // first bucket: the last b with offsets[b] <= xb / G (it is non-empty)
    int b;
    {
        const int v = xb / G;
        int lo = 0, hi = nbk - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.offsets[mid] <= v) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }

    uint4 pf[SPT][4];
    float pf_lse = 0.f, pf_del = 0.f;
    int pf_pos = -1;

    for (int x = xb; x < xe;) {
        const Bucket bk = decode_bucket(p, b);
        const int bs0 = bk.off * G, bs1 = (bk.off + bk.cnt) * G;
        const int s1 = min(bs1, xe);
        const int h = bk.h;

        // Gathered q / dout rows [c, c+RC) of this bucket (zeros past cend)
        // and the rows' lse, delta and position, into registers.
        auto prefetch = [&](int c, int cend) {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int y = tid + NTHR * i;
                if (y < NSTG) {
                    const int mat = y / (NSTG / 2), z = y - mat * (NSTG / 2);
                    const int rg = z / (D / 8), c8 = z - rg * (D / 8);
                    const u16* src = mat ? dog : qg;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int xr = c + 4 * rg + rr;
                        pf[i][rr] = make_uint4(0, 0, 0, 0);
                        if (xr < cend) {
                            const int rl = xr - bs0, ti = rl / G, qq = rl - ti * G;
                            const int t = p.entries[bk.off + ti] / topk;
                            pf[i][rr] = *reinterpret_cast<const uint4*>(
                                src + ((int64_t)t * Hq + h * G + qq) * D + c8 * 8);
                        }
                    }
                }
            }
            if (tid < RC) {
                const int xr = c + tid;
                pf_pos = -1; pf_lse = 0.f; pf_del = 0.f;
                if (xr < cend) {
                    const int rl = xr - bs0, ti = rl / G, qq = rl - ti * G;
                    const int t = p.entries[bk.off + ti] / topk;
                    const int64_t qr = (int64_t)t * Hq + h * G + qq;
                    pf_pos = t - bk.c0;
                    pf_lse = p.lse[qr] * kLog2e;
                    pf_del = p.delta[qr];
                }
            }
        };
        // registers -> LDS: row-major and transposed ([d][row]) copies
        auto commit = [&]() {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int y = tid + NTHR * i;
                if (y < NSTG) {
                    const int mat = y / (NSTG / 2), z = y - mat * (NSTG / 2);
                    const int rg = z / (D / 8), c8 = z - rg * (D / 8);
                    u16* rm = mat ? sdO : sQ;
                    u16* tr = mat ? sdOt : sQt;
                    uint32_t w[4][4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        *reinterpret_cast<uint4*>(&rm[(4 * rg + rr) * QP + c8 * 8]) = pf[i][rr];
                        w[rr][0] = pf[i][rr].x; w[rr][1] = pf[i][rr].y;
                        w[rr][2] = pf[i][rr].z; w[rr][3] = pf[i][rr].w;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int sh = (j & 1) * 16;
                        const uint32_t e0 = (w[0][j >> 1] >> sh) & 0xFFFFu, e1 = (w[1][j >> 1] >> sh) & 0xFFFFu;
                        const uint32_t e2 = (w[2][j >> 1] >> sh) & 0xFFFFu, e3 = (w[3][j >> 1] >> sh) & 0xFFFFu;
                        *reinterpret_cast<uint2*>(&tr[(c8 * 8 + j) * TP + 4 * rg]) =
                            make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
                    }
                }
            }
            if (tid < RC) {
                sPos[tid] = pf_pos;
                sLse[tid] = pf_lse;
                sDel[tid] = pf_del;
            }
        };

        prefetch(x, s1);

        // This wave's K and V rows (B operands of S and dP); K^T into LDS.
        const int key = 16 * wave + n;
        const bool kin = key < bk.nkeys;
        const int kpos = bk.kbeg + key;
        bf16x8 kreg[DS], vreg[DS];
        {
            const int64_t kr = ((int64_t)(bk.c0 + kpos) * Hkv + h) * D + 8 * g;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = kv4;
                if (kin) {
                    kv4 = *reinterpret_cast<const uint4*>(kg + kr + 32 * ds);
                    vv4 = *reinterpret_cast<const uint4*>(vg + kr + 32 * ds);
                }
                kreg[ds] = __builtin_bit_cast(bf16x8, kv4);
                vreg[ds] = __builtin_bit_cast(bf16x8, vv4);
            }
        }
        for (int y = tid; y < (BS / 8) * (D / 8); y += NTHR) {
            const int k8 = y / (D / 8), c8 = y - k8 * (D / 8);
            uint32_t w[8][4];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int kk = k8 * 8 + rr;
                uint4 val = make_uint4(0, 0, 0, 0);
                if (kk < bk.nkeys)
                    val = *reinterpret_cast<const uint4*>(kg + ((int64_t)(bk.c0 + bk.kbeg + kk) * Hkv + h) * D + c8 * 8);
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

        f32x4 dKt[MT], dVt[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            dKt[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dVt[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        for (int c = x; c < s1; c += RC) {
            commit();
            __syncthreads();
            if (c + RC < s1) prefetch(c + RC, s1);

            // S and dP: rows 16*rt + 4g + i of the chunk, key 16*wave + n
            f32x4 sacc[NTR], pacc[NTR];
#pragma unroll
            for (int rt = 0; rt < NTR; ++rt) {
                sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                pacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int rt = 0; rt < NTR; ++rt) {
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sQ[(16 * rt + n) * QP + 32 * ds + 8 * g]);
                    const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&sdO[(16 * rt + n) * QP + 32 * ds + 8 * g]);
                    sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kreg[ds], sacc[rt], 0, 0, 0);
                    pacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, vreg[ds], pacc[rt], 0, 0, 0);
                }

            bf16x8 bP, bdS;
            float dsv[NTR][4];
#pragma unroll
            for (int rt = 0; rt < NTR; ++rt) {
                const float4 l4 = *reinterpret_cast<const float4*>(&sLse[16 * rt + 4 * g]);
                const float4 d4 = *reinterpret_cast<const float4*>(&sDel[16 * rt + 4 * g]);
                const int4 p4 = *reinterpret_cast<const int4*>(&sPos[16 * rt + 4 * g]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
                const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool vis = kin && kpos <= pv[i];
                    const float pr = vis ? exp2f(fmaf(sacc[rt][i], p.scale_log2, -lv[i])) : 0.f;
                    const float ds = pr * (pacc[rt][i] - dv[i]);
                    bP[4 * rt + i] = static_cast<__bf16>(pr);
                    bdS[4 * rt + i] = static_cast<__bf16>(ds);
                    dsv[rt][i] = ds;
                }
            }

            // dV^T += dO^T P, dK^T += Q^T dS over the chunk's 32 rows
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u16* ro = &sdOt[(16 * mt + n) * TP + 4 * g];
                const u16* rq = &sQt[(16 * mt + n) * TP + 4 * g];
                const uint2 olo = *reinterpret_cast<const uint2*>(ro);
                const uint2 ohi = *reinterpret_cast<const uint2*>(ro + 16);
                const uint2 qlo = *reinterpret_cast<const uint2*>(rq);
                const uint2 qhi = *reinterpret_cast<const uint2*>(rq + 16);
                const bf16x8 ao = __builtin_bit_cast(bf16x8, make_uint4(olo.x, olo.y, ohi.x, ohi.y));
                const bf16x8 aq = __builtin_bit_cast(bf16x8, make_uint4(qlo.x, qlo.y, qhi.x, qhi.y));
                dVt[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, bP, dVt[mt], 0, 0, 0);
                dKt[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bdS, dKt[mt], 0, 0, 0);
            }

            // dS (bf16, the same rounding as bdS) -> LDS, row-major [row][key].
            // (Converted from the float: a bit_cast of a vector element is
            // compiled as a read of element 0.)
#pragma unroll
            for (int rt = 0; rt < NTR; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sdS[(16 * rt + 4 * g + i) * SP + key] = f32_to_bf16(dsv[rt][i]);
            __syncthreads();

            // dq^T[e][row] = sum over the block's keys of K^T[e][key] dS[row][key]
#pragma unroll
            for (int i = 0; i < NDQ; ++i) {
                const int idx = wave + NW * i;
                if (idx < MT * NTR) {
                    const int mt = idx % MT, nt = idx / MT;
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSQ; ++ks) {
                        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&sKt[(16 * mt + n) * KTP + 32 * ks + 8 * g]);
                        const bf16x8 bd = *reinterpret_cast<const bf16x8*>(&sdS[(16 * nt + n) * SP + 32 * ks + 8 * g]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bd, acc, 0, 0, 0);
                    }
                    *reinterpret_cast<uint2*>(&sdQ[(16 * nt + n) * QP + 16 * mt + 4 * g]) =
                        make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
                }
            }
            __syncthreads();

            // dq partial rows c.. (their CSR row positions): contiguous 16-byte stores
            {
                constexpr int CPR = D / 8;
                const int nrows = min(RC, s1 - c);
                u16* base = reinterpret_cast<u16*>(p.dq_part) + (int64_t)c * D;
                for (int ch = tid; ch < RC * CPR; ch += NTHR) {
                    const int r = ch / CPR, cc = ch - r * CPR;
                    if (r < nrows) {  // read once, by the merge: stream past the caches
                        const uint4 v4 = *reinterpret_cast<const uint4*>(&sdQ[r * QP + cc * 8]);
                        uint32_t* dst = reinterpret_cast<uint32_t*>(base + (int64_t)r * D + cc * 8);
                        __builtin_nontemporal_store(v4.x, dst);
                        __builtin_nontemporal_store(v4.y, dst + 1);
                        __builtin_nontemporal_store(v4.z, dst + 2);
                        __builtin_nontemporal_store(v4.w, dst + 3);
                    }
                }
            }
        }

        // dK, dV of this wave's keys: final if the bucket lies inside this
        // range, else a partial sum in one of the range's two slots.
        if (bs0 >= xb && bs1 <= xe) {
            if (kin) {
                const int64_t kr = ((int64_t)(bk.c0 + kpos) * Hkv + h) * D + 4 * g;
                u16* dkr = reinterpret_cast<u16*>(p.dk) + kr;
                u16* dvr = reinterpret_cast<u16*>(p.dv) + kr;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    *reinterpret_cast<uint2*>(dkr + 16 * mt) =
                        make_uint2(pack2(dKt[mt][0] * p.scale, dKt[mt][1] * p.scale),
                                   pack2(dKt[mt][2] * p.scale, dKt[mt][3] * p.scale));
                    *reinterpret_cast<uint2*>(dvr + 16 * mt) =
                        make_uint2(pack2(dVt[mt][0], dVt[mt][1]), pack2(dVt[mt][2], dVt[mt][3]));
                }
            }
        } else {
            const int slot = bs0 <= xb ? 2 * (int)blockIdx.x : 2 * (int)blockIdx.x + 1;
            float* base = p.dkv_part + (size_t)slot * 2 * BS * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                *reinterpret_cast<f32x4*>(&base[key * D + 16 * mt + 4 * g]) = dKt[mt];
                *reinterpret_cast<f32x4*>(&base[(BS + key) * D + 16 * mt + 4 * g]) = dVt[mt];
            }
        }

        x = s1;
        if (x < xe) {
            ++b;
            while (p.offsets[b + 1] == p.offsets[b]) ++b;  // skip empty buckets
        }
    }
}

// ---------------------------------------------------------------------------
// dk, dv of buckets not finished by the main kernel: split buckets sum their
// ranges' partial slots in range order; empty buckets write zeros.  One
// workgroup per bucket.
// ---------------------------------------------------------------------------
template <int D, int BS>
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
            make_uint2(pack2(sk.x * p.scale, sk.y * p.scale), pack2(sk.z * p.scale, sk.w * p.scale));
        *reinterpret_cast<uint2*>(reinterpret_cast<u16*>(p.dv) + kr) =
            make_uint2(pack2(sv.x, sv.y), pack2(sv.z, sv.w));
    }
}

// ---------------------------------------------------------------------------
// dq of one (token, kv head) row per wave: the kept slots' partials (CSR
// positions from slot_pos) summed in ascending block order, times scale.
// Rows with no kept slot (and tokens outside every sequence) get zeros.
// ---------------------------------------------------------------------------
constexpr int kDqGroup = 8;

template <int MAXK>
__global__ __launch_bounds__(256) void k_bwd_dq_merge(Params p)
{
    const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t*Hkv + h
    if (rowid >= p.T * p.Hkv) return;
    const int lane = threadIdx.x & 63;
    const int64_t t = rowid / p.Hkv;
    const int G = p.G, D = p.D, GD = G * D, topk = p.topk;
    const int s = seq_of_token(p.cus, p.B, t);
    const int b = s >= 0 ? (int)((t - p.cus[s]) / p.bs) : -1;

    const int j = lane < topk ? p.block_idx[rowid * topk + lane] : -1;
    bool keep = lane < topk && j >= 0 && j <= b;
#pragma unroll
    for (int k2 = 0; k2 < MAXK; ++k2) {
        if (k2 >= topk) break;
        const int o = __shfl(j, k2, 64);
        if (k2 < lane && o == j) keep = false;
    }
    const int spos = keep ? p.slot_pos[rowid * topk + lane] : 0;
    const uint64_t kept = __ballot(keep);
    const int nk = __popcll(kept);
    int rank = 0;
#pragma unroll
    for (int k2 = 0; k2 < MAXK; ++k2) {
        if (k2 >= topk) break;
        const int o = __shfl(j, k2, 64);
        if (((kept >> k2) & 1) && o < j) ++rank;
    }

    const u16* part = reinterpret_cast<const u16*>(p.dq_part);
    for (int c = 0; c * 64 * 8 < GD; ++c) {
        const int e = (c * 64 + lane) * 8;
        const bool active = e < GD;
        const int ee = active ? e : 0;
        float acc[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = 0.f;
        for (int r0 = 0; r0 < nk; r0 += kDqGroup) {
            uint4 raw[kDqGroup];
#pragma unroll
            for (int q2 = 0; q2 < kDqGroup; ++q2) {
                const int r = r0 + q2;
                const int slot = __ffsll((unsigned long long)__ballot(keep && rank == r)) - 1;
                const int64_t pr = __shfl(spos, slot < 0 ? 0 : slot, 64);
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
                        acc[2 * x] += bf16_to_f32((u16)(wd[x] & 0xFFFFu));
                        acc[2 * x + 1] += bf16_to_f32((u16)(wd[x] >> 16));
                    }
                }
            }
        }
        if (!active) continue;
        uint4 o;
        o.x = pack2(acc[0] * p.scale, acc[1] * p.scale);
        o.y = pack2(acc[2] * p.scale, acc[3] * p.scale);
        o.z = pack2(acc[4] * p.scale, acc[5] * p.scale);
        o.w = pack2(acc[6] * p.scale, acc[7] * p.scale);
        *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.dq) + rowid * GD + e) = o;
    }
}

template <int D, int BS>
const void* bwd_main_fn() { return (const void*)k_bwd_main<D, BS>; }

const void* bwd_main_ptr(int D, int bs)
{
    if (D == 64) return bs == 32 ? bwd_main_fn<64, 32>() : bs == 64 ? bwd_main_fn<64, 64>() : bwd_main_fn<64, 128>();
    return bs == 32 ? bwd_main_fn<128, 32>() : bs == 64 ? bwd_main_fn<128, 64>() : bwd_main_fn<128, 128>();
}

template <int D>
void launch_bwd_d(const Params& p, hipStream_t st)
{
    const unsigned nbk = (unsigned)((int64_t)p.Hkv * p.nbc);
    const unsigned grid = (unsigned)p.bwd_grid;
    switch (p.bs) {
    case 32:
        hipLaunchKernelGGL((k_bwd_main<D, 32>), dim3(grid), dim3(128), 0, st, p);
        hipLaunchKernelGGL((k_bwd_dkv_finish<D, 32>), dim3(nbk), dim3(256), 0, st, p);
        break;
    case 64:
        hipLaunchKernelGGL((k_bwd_main<D, 64>), dim3(grid), dim3(256), 0, st, p);
        hipLaunchKernelGGL((k_bwd_dkv_finish<D, 64>), dim3(nbk), dim3(256), 0, st, p);
        break;
    default:
        hipLaunchKernelGGL((k_bwd_main<D, 128>), dim3(grid), dim3(512), 0, st, p);
        hipLaunchKernelGGL((k_bwd_dkv_finish<D, 128>), dim3(nbk), dim3(256), 0, st, p);
        break;
    }
}

}  // namespace

// Workgroups of the backward main kernel: every CU filled at the kernel's
// occupancy, a multiple of the XCD count, at most kBwdMaxGrid.
int bwd_grid_size(int D, int bs)
{
    static int cached[2][3] = {{0}};
    const int di = D == 64 ? 0 : 1, bi = bs == 32 ? 0 : bs == 64 ? 1 : 2;
    if (cached[di][bi]) return cached[di][bi];
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, bwd_main_ptr(D, bs), bs * 4, 0) != hipSuccess ||
        per < 1)
        per = 1;
    int g = cus * per;
    g = (g + kNumXcd - 1) / kNumXcd * kNumXcd;
    g = std::min(g, kBwdMaxGrid);
    cached[di][bi] = g;
    return g;
}

hipError_t launch_bwd_delta(const Params& p, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const int64_t rows = p.T * p.Hq;
    if (p.D == 64) hipLaunchKernelGGL(k_bwd_delta<64>, dim3((unsigned)div_up(rows, 32)), dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_bwd_delta<128>, dim3((unsigned)div_up(rows, 16)), dim3(256), 0, st, p);
    return hipGetLastError();
}

// Main kernel and the dk / dv finish.
hipError_t launch_bwd_main(const Params& p, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    if (p.D == 64) launch_bwd_d<64>(p, st);
    else launch_bwd_d<128>(p, st);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_merge(const Params& p, hipStream_t st)
{
    if (p.T == 0) return hipSuccess;
    const unsigned grid = (unsigned)div_up(p.T * p.Hkv, 4);
    if (p.topk <= 16) hipLaunchKernelGGL(k_bwd_dq_merge<16>, dim3(grid), dim3(256), 0, st, p);
    else if (p.topk <= 32) hipLaunchKernelGGL(k_bwd_dq_merge<32>, dim3(grid), dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_bwd_dq_merge<64>, dim3(grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace nsa
